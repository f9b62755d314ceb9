"""Guard on the compiled kernels (CPU only): no MFMA reads, as its
accumulator input, the result of an MFMA of another shape issued a few
instructions earlier.

On the MI355X such a chain (a 16x16x16 bf16 product feeding a 16x16x32 bf16
accumulator three instructions later) read a stale accumulator: the affected
tiles of the chunk-pair chain came out wrong while the same source compiled
with the two products seven or more instructions apart was right.  The
compiler's hazard model treats an exactly overlapping accumulator as
forwarded and inserts no wait.  This test compiles every HIP source to gfx950
assembly with the library's own flags and fails if any kernel holds such a
chain within WINDOW instructions, so that a source or compiler change that
brings one back is caught before it runs.
"""
import os
import re
import subprocess

import pytest

from linear_attention_token_fwd_amd import build

WINDOW = 8  # instructions after the first product


def _regs(tok):
    m = re.fullmatch(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.fullmatch(r"([va])(\d+)", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def mixed_chains(asm: str, window: int = WINDOW):
    """(function, first, second) for every MFMA whose accumulator input (the
    fourth operand) overlaps the destination of an MFMA of another opcode
    issued at most `window` instructions before it."""
    found, func, body = [], None, []

    def scan():
        for i, a in enumerate(body):
            if not a.startswith("v_mfma"):
                continue
            op_a, rest_a = a.split(None, 1)
            dst = _regs(rest_a.split(",")[0].strip())
            for b in body[i + 1:i + 1 + window]:
                if not b.startswith("v_mfma"):
                    continue
                op_b, rest_b = b.split(None, 1)
                ops = [o.strip() for o in rest_b.split(",")]
                if op_b != op_a and len(ops) > 3 and _regs(ops[3]) & dst:
                    found.append((func, a, b))

    for raw in asm.splitlines():
        s = raw.strip()
        m = re.match(r"^(_Z\w+):", s)
        if m:
            if func:
                scan()
            func, body = m.group(1), []
        elif s and not s.startswith((";", ".")) and func:
            body.append(s.split(";")[0].strip())
    if func:
        scan()
    return found


def test_scanner_finds_a_planted_chain():
    asm = "\n".join([
        "_Zkern:",
        "v_mfma_f32_16x16x16_bf16 a[4:7], v[18:19], v[180:181], 0",
        "v_accvgpr_read_b32 v20, a1",
        "v_mfma_f32_16x16x32_bf16 a[0:3], v[96:99], v[24:27], a[4:7]",
        "v_mfma_f32_16x16x32_bf16 a[0:3], v[96:99], v[24:27], a[0:3]",  # same shape: forwarded, allowed
    ])
    got = mixed_chains(asm)
    assert len(got) == 1 and got[0][2].endswith("a[4:7]")
    assert mixed_chains(asm, window=0) == []


@pytest.mark.slow
@pytest.mark.parametrize("source", [os.path.basename(s) for s in build.SOURCES])
def test_no_mixed_accumulator_chains(source, tmp_path):
    out = tmp_path / (source + ".s")
    flags = [f for f in build.FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [build.HIPCC, *flags, "--cuda-device-only", "-S", "-I", os.path.join(build.ROOT, "include"),
           "-o", str(out), os.path.join(build.CSRC, source)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    asm = out.read_text()
    assert "v_mfma" in asm
    chains = mixed_chains(asm)
    assert not chains, "\n".join(f"{f}:\n  {a}\n  {b}" for f, a, b in chains[:10])

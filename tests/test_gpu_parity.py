"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Bars: relative L2 error <= 1e-2 with bf16 I/O and <= 1e-4 with fp32 I/O, on
the output y and on the final state(s); in addition every single token-head
of y must be within 5x the bar.
"""
import numpy as np
import pytest
import torch

import gdn_inputs
import oracle
from tests.gpu_common import check, compare_workload, run_gpu, say

pytestmark = pytest.mark.gpu

W = gdn_inputs.WORKLOADS


@pytest.mark.parametrize("wid", [0, 1, 2, 3, 4])
def test_reduced_workload(wid):
    """Each workload's distributions at T = 5 chunks + a 37-token tail, 2 heads."""
    w = W[wid]
    compare_workload(w, T=64 * 5 + 37, H=2)


@pytest.mark.parametrize("wid", [0, 1, 2, 3, 4])
def test_full_workload(wid):
    """Each workload at its full size, all heads compared."""
    compare_workload(W[wid])


def test_cfg_pair_batch():
    """A classifier-free-guidance pair as one call: B = 2 at the full
    480x832 length (T = 32760, H = 12, d = 128), every head of both rows."""
    compare_workload(W[1], B=2, seed=4242)


@pytest.mark.parametrize("wid", [0, 1])
@pytest.mark.parametrize("T", [1, 2, 3, 4, 63, 64, 65, 129])
def test_edge_lengths(wid, T):
    """Short sequences (inside the conv window, one chunk, chunk boundaries),
    two batch rows, three heads, a random initial state."""
    w = W[wid]
    inp = gdn_inputs.generate(w, T=T, H=3, B=2, seed=77 + T)
    inp["S0"] = (0.05 * np.random.default_rng(T).standard_normal((2, 3, w.D, w.D))).astype(np.float32)
    inp["norm_w"] = (1 + 0.3 * np.random.default_rng(5).standard_normal((3, w.D))).astype(np.float32)
    say(f"case: edge T={T} workload {wid}")
    y, s = run_gpu(inp, w.dtype)
    ry, rs, _ = oracle.inputs_for(inp)
    check("y", y, ry, w.dtype)
    check("S_T", s, rs, w.dtype)


def test_bf16_d64():
    w = gdn_inputs.Workload(90, "bf16 d64", 1, 1000, 4, 64, "bf16")
    compare_workload(w)


F32_D128 = gdn_inputs.Workload(92, "fp32 d128", 1, 32760, 12, 128, "f32")


@pytest.mark.parametrize("T,H,reverse", [(64 * 5 + 37, 2, False), (64 * 5 + 37, 2, True), (1, 3, False)])
def test_f32_d128(T, H, reverse):
    """fp32 I/O with d = 128 (the fp32 MFMA path at the model's head size),
    to the fp32 bar."""
    compare_workload(F32_D128, T=T, H=H, reverse=reverse)


def test_f32_d128_full_length():
    """fp32 I/O, d = 128, at the full 480x832 length: T = 32760, H = 12."""
    compare_workload(F32_D128)


@pytest.mark.parametrize("dtype,D", [("f32", 64), ("f32", 128), ("bf16", 64)])
@pytest.mark.parametrize("T", [64 * 5 + 37, 64 * 140 + 11])
def test_bidir_dtypes(dtype, D, T):
    """The bidirectional plan with the other operand types and head sizes
    (one range, and two ranges of 70 and 71 chunks), two heads, a random
    initial state shared by both directions."""
    w = gdn_inputs.Workload(94, f"bidir {dtype} d{D}", 1, T, 2, D, dtype, has_S0=True, bidirectional=True)
    compare_workload(w, seed=700 + T + D)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("T", [65, 128, 192, 64 * 199 + 5, 64 * 345])
def test_chunk_count_shapes(D, T):
    """bf16 chunk counts that exercise the state chain's loop (register sets
    used in turn) and its range hand-over: 2 chunks with a 1-token second
    chunk (65), 2 and 3 full chunks (128, 192), two ranges (200 chunks),
    three ranges (345 chunks); two heads, a random initial state, forward and
    reversed."""
    w = gdn_inputs.Workload(93, f"bf16 d{D}", 1, T, 2, D, "bf16")
    for reverse in (False, True):
        inp = gdn_inputs.generate(w, seed=500 + T + D)
        inp["S0"] = (0.05 * np.random.default_rng(T).standard_normal((1, 2, D, D))).astype(np.float32)
        say(f"case: chunk counts T={T} D={D} reverse={reverse}")
        y, s = run_gpu(inp, "bf16", reverse=reverse)
        ry, rs, _ = oracle.inputs_for(inp, reverse=reverse)
        check("y", y, ry, "bf16")
        check("S_T", s, rs, "bf16")


@pytest.mark.parametrize("wid", [0, 1])
def test_reverse_scan(wid):
    compare_workload(W[wid], T=64 * 3 + 5, H=2, reverse=True)


def test_deterministic():
    inp = gdn_inputs.generate(1, T=1000, H=3)
    y1, s1 = run_gpu(inp, "bf16")
    y2, s2 = run_gpu(inp, "bf16")
    assert np.array_equal(y1, y2) and np.array_equal(s1, s2)


def test_closed_form_pure_decay():
    """b = 0: S_t = (prod a) S0, so S_T is S0 scaled by the total decay and y is
    the normalised decayed readout; checked on the GPU path."""
    w = W[1]
    inp = gdn_inputs.generate(w, T=300, H=2, seed=5)
    inp["beta"][:] = 0.0
    S0 = (0.1 * np.random.default_rng(3).standard_normal((1, 2, 128, 128))).astype(np.float32)
    inp["S0"] = S0
    y, s = run_gpu(inp, "bf16")
    decay = np.exp(np.sum(inp["log_a"][0].astype(np.float64), axis=0))  # [H]
    np.testing.assert_allclose(s[0], decay[:, None, None] * S0[0], rtol=2e-3, atol=1e-7)
    ry, _, _ = oracle.inputs_for(inp)
    check("y", y, ry, "bf16")


def test_closed_form_exact_retrieval():
    """a = 1, b = 1, identity conv taps and one-hot keys: the state is a lookup
    table, S_T e_i = v^ of the last token whose key is e_i."""
    D, T, H = 64, 96, 1
    rng = np.random.default_rng(9)
    keys = np.concatenate([rng.permutation(D), rng.permutation(D)[:32]])
    inp = dict(
        q=np.eye(D, dtype=np.float32)[rng.integers(0, D, T)][None, :, None] * 2.0,
        k=np.eye(D, dtype=np.float32)[keys][None, :, None] * 2.0,
        v=rng.standard_normal((1, T, H, D)).astype(np.float32),
        gate=rng.standard_normal((1, T, H, D)).astype(np.float32),
        log_a=np.zeros((1, T, H), np.float32), beta=np.ones((1, T, H), np.float32),
        conv_q=np.tile(np.array([0, 0, 0, 1], np.float32), (D, 1)),
        conv_k=np.tile(np.array([0, 0, 0, 1], np.float32), (D, 1)),
        conv_v=np.tile(np.array([0, 0, 0, 1], np.float32), (D, 1)),
        norm_w=np.ones((1, D), np.float32), S0=None)
    _, s = run_gpu(inp, "f32")
    vhat = inp["v"][0, :, 0].astype(np.float64)
    vhat = vhat / (1 + np.exp(-vhat))
    for col in range(D):
        last = max(t for t in range(T) if keys[t] == col)
        np.testing.assert_allclose(s[0, 0, :, col], vhat[last], rtol=1e-4, atol=1e-5)


def test_errors_leave_outputs_untouched():
    import linear_attention_token_fwd_amd as gdn
    inp = gdn_inputs.generate(1, T=100, H=2)
    d = gdn.to_device(inp, dtype=torch.bfloat16)
    out = torch.full((1, 100, 2, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    small = torch.empty(1024, dtype=torch.uint8, device="cuda")
    with pytest.raises(gdn.GdnError) as e:
        gdn.gdn_fwd(d["q"], d["k"], d["v"], d["log_a"], d["beta"], d["gate"], d["conv_q"],
                    d["conv_k"], d["conv_v"], out=out, workspace=small)
    assert e.value.status == gdn.GDN_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())


VARLEN_LENGTHS = [1, 63, 64, 65, 200, 7, 129, 3]


def _varlen_inputs(w, lengths, seed):
    """Sequences of the given lengths sharing the layer's weights, packed
    along the token axis; each with its own random initial state."""
    base = gdn_inputs.generate(w, T=max(lengths), H=3, seed=seed)
    seqs = []
    for i, L in enumerate(lengths):
        d = gdn_inputs.generate(w, T=L, H=3, seed=seed + 1 + i)
        for key in ("conv_q", "conv_k", "conv_v", "norm_w"):
            d[key] = base[key]
        d["S0"] = (0.05 * np.random.default_rng(seed + 100 + i).standard_normal((1, 3, w.D, w.D))).astype(np.float32)
        seqs.append(d)
    packed = {key: np.concatenate([d[key] for d in seqs], axis=1)
              for key in ("q", "k", "v", "gate", "log_a", "beta")}
    for key in ("conv_q", "conv_k", "conv_v", "norm_w"):
        packed[key] = base[key]
    packed["S0"] = np.concatenate([d["S0"] for d in seqs], axis=0)
    cu = np.concatenate([[0], np.cumsum(lengths)]).tolist()
    return seqs, packed, cu


@pytest.mark.parametrize("wid,reverse", [(0, False), (1, False), (1, True)])
def test_varlen_batch(wid, reverse):
    """Sequences of different lengths (inside the conv window, one chunk,
    chunk boundaries, several chunks) in one call: every sequence against the
    oracle on that sequence alone, and bit-identical to gdn_fwd on it."""
    import linear_attention_token_fwd_amd as gdn
    w = W[wid]
    seqs, packed, cu = _varlen_inputs(w, VARLEN_LENGTHS, seed=500 + wid)
    say(f"case: varlen workload {wid} lengths {VARLEN_LENGTHS} reverse={reverse}")
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    d = gdn.to_device(packed, dtype=dt)
    total = cu[-1]
    out = torch.full((1, total, 3, w.D), float("nan"), dtype=dt, device="cuda")
    S_T = torch.full((len(seqs), 3, w.D, w.D), float("nan"), dtype=torch.float32, device="cuda")
    gdn.gdn_fwd_varlen(d["q"], d["k"], d["v"], d["log_a"], d["beta"], d["gate"], d["conv_q"], d["conv_k"],
                       d["conv_v"], cu, norm_w=d["norm_w"], S0=d["S0"], reverse=reverse, out=out, S_T=S_T)
    torch.cuda.synchronize()
    y = out.double().cpu().numpy()
    s = S_T.double().cpu().numpy()
    for i, seq in enumerate(seqs):
        ys = y[:, cu[i]:cu[i + 1]]
        ry, rs, _ = oracle.inputs_for(seq, reverse=reverse)
        check(f"y[{i}] (T={VARLEN_LENGTHS[i]})", ys, ry, w.dtype)
        check(f"S_T[{i}]", s[i:i + 1], rs, w.dtype)
        y1, s1 = run_gpu(seq, w.dtype, reverse=reverse)
        assert np.array_equal(ys, y1) and np.array_equal(s[i:i + 1], s1), f"sequence {i} differs from gdn_fwd alone"


def test_varlen_long_and_short():
    """Two sequences of very different lengths at the model's shape (d = 128,
    12 heads): 4096 and 37 tokens."""
    import linear_attention_token_fwd_amd as gdn
    w = W[1]
    lengths = [4096, 37]
    base = gdn_inputs.generate(w, T=4096 + 37, seed=808)
    cu = [0, 4096, 4133]
    d = gdn.to_device(base, dtype=torch.bfloat16)
    say(f"case: varlen lengths {lengths}, H=12")
    out, S_T = gdn.gdn_fwd_varlen(d["q"], d["k"], d["v"], d["log_a"], d["beta"], d["gate"], d["conv_q"],
                                  d["conv_k"], d["conv_v"], cu, norm_w=d["norm_w"])
    torch.cuda.synchronize()
    y = out.double().cpu().numpy()
    s = S_T.double().cpu().numpy()
    for i in range(2):
        seq = {key: (val[:, cu[i]:cu[i + 1]] if key in ("q", "k", "v", "gate", "log_a", "beta") else val)
               for key, val in base.items()}
        ry, rs, _ = oracle.inputs_for(seq)
        check(f"y[{i}]", y[:, cu[i]:cu[i + 1]], ry, "bf16")
        check(f"S_T[{i}]", s[i:i + 1], rs, "bf16")


MULTI_RANGE_LENGTHS = [30000, 37, 12000, 64]


@pytest.mark.parametrize("reverse", [False, True])
def test_varlen_multi_range(reverse):
    """A variable-length batch whose longest sequence spans several chunk
    ranges of the launch plan while the others end inside the first and the
    second range: lengths 30000 (3 ranges of about 156 chunks), 37, 12000
    (ends in the second range) and 64 at the model's shape
    (H = 12, d = 128, bf16), as in a batch of two videos of different lengths
    with two short prompts.  Each sequence against the oracle on that
    sequence alone, and bit-identical to gdn_fwd on it alone (the final state
    of a sequence that ends early is written by the range it ends in)."""
    import linear_attention_token_fwd_amd as gdn
    w = W[1]
    lengths = MULTI_RANGE_LENGTHS
    H = 12
    rng = np.random.default_rng(9090)
    seqs = []
    base = gdn_inputs.generate(w, T=64, H=H, seed=9091)
    for i, L in enumerate(lengths):
        d = gdn_inputs.generate(w, T=L, H=H, seed=9100 + i)
        for key in ("conv_q", "conv_k", "conv_v", "norm_w"):
            d[key] = base[key]
        d["S0"] = (0.05 * rng.standard_normal((1, H, w.D, w.D))).astype(np.float32)
        seqs.append(d)
    packed = {key: np.concatenate([d[key] for d in seqs], axis=1) for key in ("q", "k", "v", "gate", "log_a", "beta")}
    for key in ("conv_q", "conv_k", "conv_v", "norm_w"):
        packed[key] = base[key]
    packed["S0"] = np.concatenate([d["S0"] for d in seqs], axis=0)
    cu = np.concatenate([[0], np.cumsum(lengths)]).tolist()
    say(f"case: varlen multi-range lengths {lengths} H={H} d=128 bf16 reverse={reverse}")
    d = gdn.to_device(packed, dtype=torch.bfloat16)
    out = torch.full((1, cu[-1], H, w.D), float("nan"), dtype=torch.bfloat16, device="cuda")
    S_T = torch.full((len(lengths), H, w.D, w.D), float("nan"), dtype=torch.float32, device="cuda")
    gdn.gdn_fwd_varlen(d["q"], d["k"], d["v"], d["log_a"], d["beta"], d["gate"], d["conv_q"], d["conv_k"],
                       d["conv_v"], cu, norm_w=d["norm_w"], S0=d["S0"], reverse=reverse, out=out, S_T=S_T)
    torch.cuda.synchronize()
    y = out.double().cpu().numpy()
    s = S_T.double().cpu().numpy()
    for i, seq in enumerate(seqs):
        ys = y[:, cu[i]:cu[i + 1]]
        ry, rs, _ = oracle.inputs_for(seq, reverse=reverse)
        check(f"y[{i}] (T={lengths[i]})", ys, ry, "bf16")
        check(f"S_T[{i}]", s[i:i + 1], rs, "bf16")
        y1, s1 = run_gpu(seq, "bf16", reverse=reverse)
        assert np.array_equal(ys, y1) and np.array_equal(s[i:i + 1], s1), f"sequence {i} differs from gdn_fwd alone"


@pytest.mark.parametrize("T,B", [(1, 1), (64, 1), (100, 2), (64 * 9, 1), (64 * 9 + 24, 2), (64 * 300 + 24, 1),
                                 (64 * 520 + 5, 1)])
def test_bidir_shapes(T, B):
    """The bidirectional variant (both scans co-scheduled, outputs summed in
    fp32 and stored once, each scan writing the accumulator on the half of
    the tokens it reaches first): one chunk range and several, lengths that
    are and are not multiples of 64 (the two scans' chunk boundaries differ),
    a batch of two."""
    w = W[4]
    compare_workload(w, T=T, H=2, B=B)

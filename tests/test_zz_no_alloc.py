"""gdn_fwd_noalloc (the entry point that allocates nothing) against gdn_fwd.

Two calls in a row through the C ABI, the second with a smaller input, each
equal to gdn_fwd on the same inputs (same kernels and launch plan, so bit for
bit) and within the bf16 bar of the oracle; NaN-poisoned outputs must be
fully overwritten.  A size beyond the library's 64 MiB array is refused with
GDN_ERR_WORKSPACE and leaves the outputs untouched.
"""
import ctypes

import numpy as np
import pytest
import torch

import gdn_inputs
import oracle
from tests.gpu_common import check, say

pytestmark = pytest.mark.gpu


def _call_noalloc(lib, gdn, d, out, S_T, stream):
    p = gdn.make_params(d["q"], d["k"], d["v"], d["log_a"], d["beta"], d["gate"], d["conv_q"], d["conv_k"],
                        d["conv_v"], d["norm_w"], d["S0"], out, S_T, None)
    return lib.gdn_fwd_noalloc(ctypes.byref(p), ctypes.c_void_p(stream.cuda_stream))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_equals_gdn_fwd_twice(dtype):
    import linear_attention_token_fwd_amd as gdn
    lib = gdn.load()
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    w = gdn_inputs.Workload(95, f"{dtype} d128", 1, 1, 1, 128, dtype)
    stream = torch.cuda.current_stream()
    for T, H, seed in ((64 * 40 + 17, 6, 951), (64 * 7 + 3, 3, 952)):
        inp = gdn_inputs.generate(w, T=T, H=H, seed=seed)
        inp["S0"] = (0.05 * np.random.default_rng(seed).standard_normal((1, H, 128, 128))).astype(np.float32)
        say(f"case: gdn_fwd_noalloc {dtype} T={T} H={H}")
        d = gdn.to_device(inp, dtype=dt)
        out = torch.full((1, T, H, 128), float("nan"), dtype=dt, device="cuda")
        S_T = torch.full((1, H, 128, 128), float("nan"), dtype=torch.float32, device="cuda")
        assert _call_noalloc(lib, gdn, d, out, S_T, stream) == gdn.GDN_OK
        ref_y, ref_s = gdn.gdn_fwd(d["q"], d["k"], d["v"], d["log_a"], d["beta"], d["gate"], d["conv_q"],
                                   d["conv_k"], d["conv_v"], d["norm_w"], d["S0"])
        torch.cuda.synchronize()
        assert torch.equal(out, ref_y) and torch.equal(S_T, ref_s), "differs from gdn_fwd"
        ry, rs, _ = oracle.inputs_for(inp)
        check("y", out.double().cpu().numpy(), ry, dtype)
        check("S_T", S_T.double().cpu().numpy(), rs, dtype)


def test_noalloc_refuses_too_large():
    import linear_attention_token_fwd_amd as gdn
    lib = gdn.load()
    w = gdn_inputs.WORKLOADS[1]
    T, H = 64 * 80, 8  # 80 chunks x 8 heads: about 75 MiB of workspace
    inp = gdn_inputs.generate(w, T=T, H=H, seed=953)
    d = gdn.to_device(inp, dtype=torch.bfloat16)
    assert gdn.gdn_fwd_workspace_bytes(1, T, H, 128) > (64 << 20)
    out = torch.full((1, T, H, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    st = _call_noalloc(lib, gdn, d, out, None, torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert st == gdn.GDN_ERR_WORKSPACE
    assert bool((out == 7.0).all())

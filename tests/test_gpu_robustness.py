"""Failure handling and resumption of the layer forward on the GPU.

* Non-finite inputs: a NaN or an infinity planted in one input returns
  normally (no hang, no fault) and spreads exactly where the recurrence
  carries it: the oracle's non-finite outputs are non-finite on the GPU, the
  values the oracle keeps finite match it within the bar, and the only other
  non-finite values are the tokens of the planted token's own 64-token chunk
  that precede it (the chunked form multiplies whole chunks at once, and a
  product with a NaN is NaN even where the other factor is 0).
* Split and resume: the layer over [0, t) and then over [t, T) started from
  the first call's final state equals one call over [0, T) within the bar
  (identity conv taps, so the conv needs no history across the split).
* A call on a side stream with no workspace passed: the binding allocates
  the workspace on that stream's pool, so memory taken and written on the
  current stream right after the call cannot reuse it while the call runs.
"""
import numpy as np
import pytest
import torch

import gdn_inputs
import oracle
from tests.gpu_common import check, rel_l2, run_gpu, say

pytestmark = pytest.mark.gpu

W = gdn_inputs.WORKLOADS
T_NF, H_NF = 64 * 5 + 21, 2
T_BAD, H_BAD, CH_BAD = 64 * 2 + 23, 1, 5   # the planted token, head and channel
SPREAD_V_BLOCK = True


NONFINITE = [("q", np.nan), ("k", np.nan), ("v", np.nan), ("gate", np.nan), ("log_a", np.nan),
             ("beta", np.nan), ("v", np.inf), ("gate", -np.inf), ("k", np.inf)]


@pytest.mark.parametrize("wid", [0, 1])
@pytest.mark.parametrize("name,val", NONFINITE, ids=[f"{n}={v}" for n, v in NONFINITE])
def test_nonfinite_input_propagates(wid, name, val):
    w = W[wid]
    inp = gdn_inputs.generate(w, T=T_NF, H=H_NF, seed=313)
    arr = inp[name]
    if arr.ndim == 4:
        arr[0, T_BAD, H_BAD, CH_BAD] = val
    else:
        arr[0, T_BAD, H_BAD] = val
    say(f"case: non-finite {name}={val} at token {T_BAD}, head {H_BAD}, workload {wid}")
    y, s = run_gpu(inp, w.dtype)
    with np.errstate(invalid="ignore", over="ignore"):
        ry, rs, _ = oracle.inputs_for(inp)
    ry_bad, rs_bad = ~np.isfinite(ry), ~np.isfinite(rs)
    y_bad, s_bad = ~np.isfinite(y), ~np.isfinite(s)
    assert ry_bad.any(), "the planted value must reach the output"
    # what the recurrence carries is non-finite on the GPU too
    assert np.all(y_bad[ry_bad]), "y: finite where the oracle is not"
    assert np.all(s_bad[rs_bad]), "S_T: finite where the oracle is not"
    # extra non-finite values only in the planted chunk, before the planted token
    extra = y_bad & ~ry_bad
    c0 = (T_BAD // 64) * 64
    where = np.argwhere(extra)
    assert np.all((where[:, 1] >= c0) & (where[:, 1] < T_BAD) & (where[:, 2] == H_BAD)), \
        f"y non-finite outside the planted chunk: {where[:5]}"
    s_extra = np.argwhere(s_bad & ~rs_bad)
    if name == "v" and SPREAD_V_BLOCK:
        # the value tiles are moved into the MFMA layout by products with 0/1
        # matrices, so a NaN in one channel may reach the other channels of
        # its 16-channel block of the state
        blk = CH_BAD // 16
        assert np.all((s_extra[:, 1] == H_BAD) & (s_extra[:, 2] // 16 == blk)), s_extra[:5]
    else:
        assert s_extra.size == 0, f"S_T non-finite where the oracle is finite: {s_extra[:5]}"
    # the finite rest matches the oracle
    ok = ~(y_bad | ry_bad)
    e = rel_l2(y[ok], ry[ok])
    say(f"  y over {int(ok.sum())} finite values: rel-L2 {e:.2e}; non-finite {int(y_bad.sum())} "
        f"(oracle {int(ry_bad.sum())}); S_T non-finite {int(s_bad.sum())}")
    assert e <= (1e-2 if w.dtype == "bf16" else 1e-4)
    ok_s = ~(s_bad | rs_bad)
    if ok_s.any():
        es = rel_l2(s[ok_s], rs[ok_s])
        assert es <= (1e-2 if w.dtype == "bf16" else 1e-4)


@pytest.mark.parametrize("wid,t_split", [(0, 1000), (1, 1000), (1, 64 * 9), (1, 1)])
def test_split_and_resume(wid, t_split):
    """[0, t) then [t, T) seeded with the first part's final state equals one
    call over [0, T); identity conv taps (the conv carries no state across
    the split) and a random initial state."""
    w = W[wid]
    T, H = 2500, 2
    inp = gdn_inputs.generate(w, T=T, H=H, seed=515)
    ident = np.tile(np.array([0, 0, 0, 1], np.float32), (H * w.D, 1))
    for key in ("conv_q", "conv_k", "conv_v"):
        inp[key] = ident.copy()
    inp["S0"] = (0.05 * np.random.default_rng(516).standard_normal((1, H, w.D, w.D))).astype(np.float32)
    say(f"case: split at {t_split} of T={T}, workload {wid}")
    y, s = run_gpu(inp, w.dtype)
    per_tok = ("q", "k", "v", "gate", "log_a", "beta")
    first = {k: (v[:, :t_split] if k in per_tok else v) for k, v in inp.items()}
    y1, s1 = run_gpu(first, w.dtype)
    second = {k: (v[:, t_split:] if k in per_tok else v) for k, v in inp.items()}
    second["S0"] = s1.astype(np.float32)
    y2, s2 = run_gpu(second, w.dtype)
    ys = np.concatenate([y1, y2], axis=1)
    check("y split vs whole", ys, y, w.dtype)
    check("S_T split vs whole", s2, s, w.dtype)
    ry, rs, _ = oracle.inputs_for(inp)
    check("y split vs oracle", ys, ry, w.dtype)
    check("S_T split vs oracle", s2, rs, w.dtype)


def test_side_stream_without_workspace():
    """gdn_fwd and gdn_bwd on a side stream with no workspace, followed at
    once by allocations written on the current stream: results equal the
    same calls made on the current stream."""
    import linear_attention_token_fwd_amd as gdn
    w = W[1]
    T, H = 64 * 40 + 3, 4
    inp = gdn_inputs.generate(w, T=T, H=H, seed=616)
    d = gdn.to_device(inp, dtype=torch.bfloat16)
    args = (d["q"], d["k"], d["v"], d["log_a"], d["beta"], d["gate"], d["conv_q"], d["conv_k"], d["conv_v"],
            d["norm_w"], d["S0"])
    y_ref, s_ref = gdn.gdn_fwd(*args)
    grads = gdn_inputs.generate_grads(w, seed=617, T=T, H=H)
    dy = torch.from_numpy(grads["dy"]).to(torch.bfloat16).cuda()
    g_ref = gdn.gdn_bwd(*args, dy)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    for rep in range(3):
        side.wait_stream(torch.cuda.current_stream())
        y, s = gdn.gdn_fwd(*args, stream=side)
        g = gdn.gdn_bwd(*args, dy, stream=side)
        # memory taken and overwritten on the current stream while the side stream runs
        junk = [torch.full((64 << 20,), 3.0, device="cuda") for _ in range(8)]
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        del junk
        assert torch.equal(y, y_ref) and torch.equal(s, s_ref), f"forward differs (rep {rep})"
        for n, t in g_ref.items():
            if t is not None:
                assert torch.equal(g[n], t), f"d{n} differs (rep {rep})"
    say("  side-stream calls equal the current-stream calls")

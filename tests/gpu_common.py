"""Shared helpers of the GPU tests: run the HIP path through the C ABI and the
oracle on the same seeded inputs, and compare."""
from __future__ import annotations

import sys

import numpy as np

import gdn_inputs
import oracle

TOL = {"bf16": 1e-2, "f32": 1e-4}


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def rel_l2(x, ref) -> float:
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(x - ref) / max(np.linalg.norm(ref), 1e-300))


def torch_dtype(dtype: str):
    import torch
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def run_gpu(inp: dict, dtype: str, reverse=False, bidir=False, poison=True):
    """Run the HIP path; returns numpy float64 (y, S_T[, S_T_rev])."""
    import torch
    import linear_attention_token_fwd_amd as gdn
    d = gdn.to_device(inp, dtype=torch_dtype(dtype))
    B, T, H, D = inp["q"].shape
    out = torch.empty((B, T, H, D), dtype=torch_dtype(dtype), device="cuda")
    S_T = torch.empty((B, H, D, D), dtype=torch.float32, device="cuda")
    if poison:  # every element must be overwritten
        out.fill_(float("nan"))
        S_T.fill_(float("nan"))
    args = (d["q"], d["k"], d["v"], d["log_a"], d["beta"], d["gate"], d["conv_q"], d["conv_k"],
            d["conv_v"], d["norm_w"], d["S0"])
    if bidir:
        S_T_rev = torch.empty_like(S_T)
        if poison:
            S_T_rev.fill_(float("nan"))
        gdn.gdn_fwd_bidir(*args, out=out, S_T=S_T, S_T_rev=S_T_rev)
        torch.cuda.synchronize()
        return (out.double().cpu().numpy(), S_T.double().cpu().numpy(),
                S_T_rev.double().cpu().numpy())
    gdn.gdn_fwd(*args, out=out, S_T=S_T, reverse=reverse)
    torch.cuda.synchronize()
    return out.double().cpu().numpy(), S_T.double().cpu().numpy()


def check(name, got, ref, dtype):
    """rel-L2 over the compared heads within the bar, and every token-head
    within 5x the bar, so one bad chunk or head cannot hide in the total."""
    tol = TOL[dtype]
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    e = rel_l2(got, ref)
    say(f"  {name}: rel-L2 {e:.3e} (bar {tol:g})")
    assert e <= tol, f"{name}: rel-L2 {e:.3e} > {tol:g}"
    if got.ndim == 4 and name.startswith("y"):
        num = np.linalg.norm(got - ref, axis=-1)
        den = np.maximum(np.linalg.norm(ref, axis=-1), 1e-30)
        worst = float(np.max(num / den))
        assert worst <= 5 * tol, f"{name}: worst token-head rel error {worst:.3e}"
    return e


def compare_workload(w, T=None, H=None, B=None, heads=None, seed=None, threads=0, reverse=False):
    """Parity of one workload (optionally resized) on all outputs."""
    inp = gdn_inputs.generate(w, seed=seed, T=T, H=H, B=B)
    say(f"case: workload {w.id} B={inp['q'].shape[0]} T={inp['q'].shape[1]} H={inp['q'].shape[2]} "
        f"D={w.D} {w.dtype} bidir={w.bidirectional} reverse={reverse} heads={heads}")
    errs = {}
    if w.bidirectional:
        y, s, sr = run_gpu(inp, w.dtype, bidir=True)
        ry, rs, rsr, _ = oracle.inputs_for(inp, heads=heads, threads=threads, bidir=True)
        hs = slice(None) if heads is None else heads
        errs["y"] = check("y", y[:, :, hs], ry[:, :, hs], w.dtype)
        errs["S_T"] = check("S_T fwd", s[:, hs], rs[:, hs], w.dtype)
        errs["S_T_rev"] = check("S_T rev", sr[:, hs], rsr[:, hs], w.dtype)
    else:
        y, s = run_gpu(inp, w.dtype, reverse=reverse)
        ry, rs, _ = oracle.inputs_for(inp, heads=heads, threads=threads, reverse=reverse)
        hs = slice(None) if heads is None else heads
        errs["y"] = check("y", y[:, :, hs], ry[:, :, hs], w.dtype)
        errs["S_T"] = check("S_T", s[:, hs], rs[:, hs], w.dtype)
    return errs

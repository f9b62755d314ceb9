"""Parity of the backward pass (gdn_bwd, through the C ABI) with the fp64
backward oracle (oracle/bwd.py: torch.autograd on the layer forward written
token by token).

Bars, per gradient: relative L2 error <= 1e-2 with bf16 I/O and <= 1e-4 with
fp32 I/O.  Every output buffer starts as NaN, so an element the library
fails to write fails the test.
"""
import numpy as np
import pytest
import torch

import gdn_inputs
from oracle import bwd as obwd
from tests.gpu_common import TOL, rel_l2, say, torch_dtype

pytestmark = pytest.mark.gpu

W = gdn_inputs.WORKLOADS


def _workload(dtype, D):
    return gdn_inputs.Workload(91, f"{dtype} d{D}", 1, 1000, 2, D, dtype)


def run_bwd(inp, grads, dtype, reverse=False):
    """The library's gradients as float64 numpy arrays (keyed like the oracle)."""
    import linear_attention_token_fwd_amd as gdn
    d = gdn.to_device(inp, dtype=torch_dtype(dtype))
    dy = torch.from_numpy(grads["dy"]).to(torch_dtype(dtype)).cuda()
    dS = None if grads["dS_T"] is None else torch.from_numpy(grads["dS_T"]).cuda()
    B, T, H, D = inp["q"].shape
    io = torch_dtype(dtype)
    out = {n: torch.full((B, T, H, D), float("nan"), dtype=io, device="cuda") for n in ("q", "k", "v", "gate")}
    out.update({n: torch.full((B, T, H), float("nan"), device="cuda") for n in ("log_a", "beta")})
    out.update({n: torch.full((H * D, 4), float("nan"), device="cuda") for n in ("conv_q", "conv_k", "conv_v")})
    out["norm_w"] = torch.full((H, D), float("nan"), device="cuda")
    out["S0"] = torch.full((B, H, D, D), float("nan"), device="cuda")
    g = gdn.gdn_bwd(d["q"], d["k"], d["v"], d["log_a"], d["beta"], d["gate"], d["conv_q"], d["conv_k"],
                    d["conv_v"], d["norm_w"], d["S0"], dy, dS, out=out, reverse=reverse)
    torch.cuda.synchronize()
    return {n: g[n].double().cpu().numpy() for n in obwd.NAMES}


def oracle_grads(inp, grads):
    ref_in = {n: inp.get(n) for n in obwd.NAMES}
    _, _, ref = obwd.backward(ref_in, grads["dy"], grads["dS_T"])
    # the library reports the gradient at norm_w = ones and at S0 = 0 as well
    if ref["norm_w"] is None or ref["S0"] is None:
        filled = dict(ref_in)
        if filled["norm_w"] is None:
            filled["norm_w"] = np.ones(inp["q"].shape[2:], np.float32)
        if filled["S0"] is None:
            B, _, H, D = inp["q"].shape
            filled["S0"] = np.zeros((B, H, D, D), np.float32)
        _, _, ref2 = obwd.backward(filled, grads["dy"], grads["dS_T"])
        ref["norm_w"], ref["S0"] = ref2["norm_w"], ref2["S0"]
    return ref


def compare(got, ref, dtype, label):
    bar = TOL[dtype]
    errs = {n: rel_l2(got[n], ref[n]) for n in obwd.NAMES}
    say(f"{label}: " + ", ".join(f"{n} {e:.1e}" for n, e in errs.items()))
    for n in obwd.NAMES:
        assert np.isfinite(got[n]).all(), (label, n, "not finite (unwritten)")
        assert errs[n] <= bar, (label, n, errs[n])


CASES = [
    # dtype, D, T, H, B, S0, norm_w, dS_T
    ("bf16", 128, 64 * 3 + 17, 2, 1, True, True, True),
    ("bf16", 128, 64, 1, 2, False, False, True),
    ("bf16", 64, 150, 2, 2, True, True, False),
    ("f32", 64, 64 * 2 + 5, 2, 2, True, True, True),
    ("f32", 128, 100, 1, 1, False, True, True),
    ("f32", 64, 3, 2, 1, True, False, True),
    ("bf16", 128, 1, 1, 1, True, True, True),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-d{c[1]}-T{c[2]}-H{c[3]}-B{c[4]}" for c in CASES])
def test_bwd_matches_oracle(case):
    dtype, D, T, H, B, with_s0, with_nw, with_ds = case
    w = _workload(dtype, D)
    seed = 300 + T + D
    inp = gdn_inputs.generate(w, T=T, H=H, B=B, seed=seed)
    rng = np.random.default_rng(seed)
    inp["S0"] = (0.1 * rng.standard_normal((B, H, D, D))).astype(np.float32) if with_s0 else None
    inp["norm_w"] = (1 + 0.3 * rng.standard_normal((H, D))).astype(np.float32) if with_nw else None
    grads = gdn_inputs.generate_grads(w, seed=seed + 1, T=T, H=H, B=B, state=with_ds)
    say(f"case: bwd {dtype} D={D} T={T} H={H} B={B}")
    got = run_bwd(inp, grads, dtype)
    ref = oracle_grads(inp, grads)
    compare(got, ref, dtype, f"{dtype} D={D} T={T}")


TOKEN_WISE = ("q", "k", "v", "gate", "log_a", "beta")


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64)])
def test_bwd_reverse_is_the_flipped_layer(dtype, D):
    """reverse = 1 is the layer on the time-reversed sequence with its output
    in input order, so its gradients are the oracle's on the flipped inputs
    and dy, flipped back along time (the weights' and S0's as they are)."""
    w = _workload(dtype, D)
    T, H, B = 64 * 2 + 22, 2, 2
    inp = gdn_inputs.generate(w, T=T, H=H, B=B, seed=900 + D)
    rng = np.random.default_rng(901)
    inp["S0"] = (0.1 * rng.standard_normal((B, H, D, D))).astype(np.float32)
    inp["norm_w"] = (1 + 0.3 * rng.standard_normal((H, D))).astype(np.float32)
    grads = gdn_inputs.generate_grads(w, seed=902, T=T, H=H, B=B)
    say(f"case: bwd reverse {dtype} D={D} T={T}")
    got = run_bwd(inp, grads, dtype, reverse=True)

    def flip(a):
        return np.ascontiguousarray(a[:, ::-1])
    finp = {n: (flip(a) if n in TOKEN_WISE else a) for n, a in inp.items()}
    ref = oracle_grads(finp, dict(dy=flip(grads["dy"]), dS_T=grads["dS_T"]))
    ref = {n: (flip(a) if n in TOKEN_WISE else a) for n, a in ref.items()}
    compare(got, ref, dtype, f"reverse {dtype} D={D} T={T}")


def test_bwd_full_size_causal():
    """At the full 480x832 size (T = 32760, H = 12, d = 128, bf16), with dy
    zero from token 200 on and dS_T = 0: every gradient equals the oracle's
    on the first 200 tokens (the loss does not see the rest), and the
    per-token gradients from token 200 on are exactly zero."""
    w = W[1]
    t1 = 200
    inp = gdn_inputs.generate(w, seed=1234)
    grads = gdn_inputs.generate_grads(w, seed=1235, t_end=t1, state=False)
    say("case: bwd full size T=32760 H=12 d=128, dy zero from t=200")
    got = run_bwd(inp, grads, "bf16")
    for n in ("q", "k", "v", "gate", "log_a", "beta"):
        tail = got[n][:, t1:]
        assert np.isfinite(tail).all() and (tail == 0).all(), n
    short = {n: (None if a is None else (a[:, :t1] if n in ("q", "k", "v", "gate", "log_a", "beta") else a))
             for n, a in inp.items()}
    g_short = dict(dy=grads["dy"][:, :t1], dS_T=None)
    ref = oracle_grads(short, g_short)
    head = {n: (got[n][:, :t1] if n in ("q", "k", "v", "gate", "log_a", "beta") else got[n]) for n in obwd.NAMES}
    compare(head, ref, "bf16", "full size, first 200 tokens")


def test_bwd_ranges_match_single_pass():
    """The call splits the chains into ranges (about 64 chunks each) on two
    streams; the timed call runs every kernel once over all chunks on one
    stream.  At the full size (512 chunks: 8 ranges), with dy and dS_T dense,
    every gradient of the two must be identical, bit for bit."""
    import ctypes
    import linear_attention_token_fwd_amd as gdn
    from bench import HipEvents
    w = W[1]
    inp = gdn_inputs.generate(w, seed=4321)
    grads = gdn_inputs.generate_grads(w, seed=4322)
    say("case: bwd ranges vs single pass, T=32760 H=12 d=128")
    d = gdn.to_device(inp, dtype=torch.bfloat16)
    dy = torch.from_numpy(grads["dy"]).to(torch.bfloat16).cuda()
    dS = torch.from_numpy(grads["dS_T"]).cuda()
    B, T, H, D = inp["q"].shape
    lib = gdn.load()

    def outputs():
        o = {n: torch.full((B, T, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
             for n in ("q", "k", "v", "gate")}
        o.update({n: torch.full((B, T, H), float("nan"), device="cuda") for n in ("log_a", "beta")})
        o.update({n: torch.full((H * D, 4), float("nan"), device="cuda") for n in ("conv_q", "conv_k", "conv_v")})
        o["norm_w"] = torch.full((H, D), float("nan"), device="cuda")
        o["S0"] = torch.full((B, H, D, D), float("nan"), device="cuda")
        return o

    ws = torch.empty(gdn.gdn_bwd_workspace_bytes(B, T, H, D), dtype=torch.uint8, device="cuda")
    args = (d["q"], d["k"], d["v"], d["log_a"], d["beta"], d["gate"], d["conv_q"], d["conv_k"], d["conv_v"],
            d["norm_w"], d["S0"], dy, dS)
    o1, o2 = outputs(), outputs()
    stream = torch.cuda.current_stream().cuda_stream
    p1 = gdn.bwd_params(*args, o1, ws)
    assert lib.gdn_bwd(ctypes.byref(p1), ctypes.c_void_p(stream)) == gdn.GDN_OK
    torch.cuda.synchronize()
    ev = HipEvents()
    n = 2 * lib.gdn_bwd_launch_count()
    evs = ev.create(n)
    p2 = gdn.bwd_params(*args, o2, ws)
    assert lib.gdn_bwd_timed(ctypes.byref(p2), evs, n, ctypes.c_void_p(stream)) == gdn.GDN_OK
    torch.cuda.synchronize()
    for name in obwd.NAMES:
        a, b = o1[name], o2[name]
        assert torch.isfinite(a).all(), name
        assert torch.equal(a, b), name


def test_bwd_graph_replays():
    """The backward captured in a HIP graph (torch.cuda.graph on a side
    stream; the call's fork onto the library stream and the join back are
    captured with it) at 131 chunks (3 ranges).  Every replay, with eager
    backward calls and synchronisations in between, must equal the eager
    call bit for bit."""
    import linear_attention_token_fwd_amd as gdn
    w = _workload("bf16", 64)
    T, H, B, D = 64 * 130 + 7, 2, 1, 64
    inp = gdn_inputs.generate(w, T=T, H=H, B=B, seed=71)
    grads = gdn_inputs.generate_grads(w, seed=72, T=T, H=H, B=B)
    d = gdn.to_device(inp, dtype=torch.bfloat16)
    dy = torch.from_numpy(grads["dy"]).to(torch.bfloat16).cuda()
    dS = torch.from_numpy(grads["dS_T"]).cuda()
    args = (d["q"], d["k"], d["v"], d["log_a"], d["beta"], d["gate"], d["conv_q"], d["conv_k"], d["conv_v"],
            d["norm_w"], d["S0"], dy, dS)
    ws = torch.empty(gdn.gdn_bwd_workspace_bytes(B, T, H, D), dtype=torch.uint8, device="cuda")
    eager = {n: t.clone() for n, t in gdn.gdn_bwd(*args, workspace=ws).items() if t is not None}
    torch.cuda.synchronize()
    out = {n: torch.empty_like(t) for n, t in eager.items()}
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        gdn.gdn_bwd(*args, out=out, workspace=ws, stream=side)  # warm-up on the side stream
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=side):
        gdn.gdn_bwd(*args, out=out, workspace=ws, stream=side)
    for rep in range(3):
        for t in out.values():
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same = all(torch.equal(out[n], eager[n]) for n in eager)
        say(f"  replay {rep}: every gradient equal {same}")
        assert same, f"replay {rep} differs from the eager call"
        gdn.gdn_bwd(*args, workspace=ws)  # eager work between the replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("reverse", [False, True])
def test_bwd_varlen_equals_each_sequence(reverse):
    """Three sequences of different lengths packed along the token axis: each
    one's per-token gradients and dS0 equal gdn_bwd on that sequence alone,
    bit for bit (its chunks past the end are identity steps of both chains);
    the weight gradients equal the sums of the single calls' to rounding."""
    import linear_attention_token_fwd_amd as gdn
    w = _workload("bf16", 64)
    lens = (150, 64 * 3 + 5, 70)
    H, D = 2, 64
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(int)
    total = int(cu[-1])
    inp = gdn_inputs.generate(w, T=total, H=H, B=1, seed=81)
    rng = np.random.default_rng(82)
    S0 = (0.1 * rng.standard_normal((len(lens), H, D, D))).astype(np.float32)
    grads = gdn_inputs.generate_grads(w, seed=83, T=total, H=H, B=1)
    dS_T = rng.standard_normal((len(lens), H, D, D)).astype(np.float32)
    say(f"case: bwd varlen lengths {lens} reverse={reverse}")
    d = gdn.to_device(inp, dtype=torch.bfloat16)
    dy = torch.from_numpy(grads["dy"]).to(torch.bfloat16).cuda()
    S0_d, dS_d = torch.from_numpy(S0).cuda(), torch.from_numpy(dS_T).cuda()
    tok = ("q", "k", "v", "gate", "log_a", "beta")
    got = gdn.gdn_bwd_varlen(d["q"][0], d["k"][0], d["v"][0], d["log_a"][0], d["beta"][0], d["gate"][0],
                             d["conv_q"], d["conv_k"], d["conv_v"], d["norm_w"], S0_d, dy[0], dS_d, list(cu),
                             reverse=reverse)
    torch.cuda.synchronize()
    wsum = {n: 0.0 for n in ("conv_q", "conv_k", "conv_v", "norm_w")}
    for b, n_b in enumerate(lens):
        sl = slice(int(cu[b]), int(cu[b + 1]))
        one = gdn.gdn_bwd(*[d[n][:, sl].contiguous() if n in tok else d[n]
                            for n in ("q", "k", "v", "log_a", "beta", "gate", "conv_q", "conv_k", "conv_v", "norm_w")],
                          S0_d[b:b + 1].contiguous(), dy[:, sl].contiguous(), dS_d[b:b + 1].contiguous(),
                          reverse=reverse)
        torch.cuda.synchronize()
        for n in tok:
            assert torch.equal(got[n][sl], one[n][0]), (b, n)
        assert torch.equal(got["S0"][b], one["S0"][0]), (b, "S0")
        for n in wsum:
            wsum[n] = wsum[n] + one[n].double()
    for n, ref in wsum.items():
        assert rel_l2(got[n].double().cpu().numpy(), ref.cpu().numpy()) < 1e-5, n


def _varlen_bwd_case(lens, H, D, dtype, seed):
    w = _workload(dtype, D)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(int)
    total = int(cu[-1])
    inp = gdn_inputs.generate(w, T=total, H=H, B=1, seed=seed)
    rng = np.random.default_rng(seed + 1)
    S0 = (0.1 * rng.standard_normal((len(lens), H, D, D))).astype(np.float32)
    grads = gdn_inputs.generate_grads(w, seed=seed + 2, T=total, H=H, B=1)
    dS_T = rng.standard_normal((len(lens), H, D, D)).astype(np.float32)
    return inp, S0, grads, dS_T, cu


def _run_varlen_bwd(inp, S0, grads, dS_T, cu, dtype, reverse):
    import linear_attention_token_fwd_amd as gdn
    d = gdn.to_device(inp, dtype=torch_dtype(dtype))
    dy = torch.from_numpy(grads["dy"]).to(torch_dtype(dtype)).cuda()
    S0_d, dS_d = torch.from_numpy(S0).cuda(), torch.from_numpy(dS_T).cuda()
    got = gdn.gdn_bwd_varlen(d["q"][0], d["k"][0], d["v"][0], d["log_a"][0], d["beta"][0], d["gate"][0],
                             d["conv_q"], d["conv_k"], d["conv_v"], d["norm_w"], S0_d, dy[0], dS_d, list(cu),
                             reverse=reverse)
    torch.cuda.synchronize()
    return d, dy, S0_d, dS_d, got


@pytest.mark.parametrize("reverse", [False, True])
def test_bwd_varlen_multi_range_equals_each_sequence(reverse):
    """The backward of a variable-length batch at the model's shape (H = 12,
    d = 128, bf16) whose longest sequence spans several chain ranges (about
    64 chunks each) while the others end inside the first and the third:
    lengths 20000, 37, 9000, 64.  Each sequence's per-token gradients and dS0
    equal gdn_bwd on that sequence alone, bit for bit; the weight gradients
    equal the sums of the single calls' to rounding."""
    import linear_attention_token_fwd_amd as gdn
    lens = (20000, 37, 9000, 64)
    inp, S0, grads, dS_T, cu = _varlen_bwd_case(lens, 12, 128, "bf16", 1201)
    say(f"case: bwd varlen multi-range lengths {lens} H=12 d=128 bf16 reverse={reverse}")
    d, dy, S0_d, dS_d, got = _run_varlen_bwd(inp, S0, grads, dS_T, cu, "bf16", reverse)
    tok = ("q", "k", "v", "gate", "log_a", "beta")
    wsum = {n: 0.0 for n in ("conv_q", "conv_k", "conv_v", "norm_w")}
    for b in range(len(lens)):
        sl = slice(int(cu[b]), int(cu[b + 1]))
        one = gdn.gdn_bwd(*[d[n][:, sl].contiguous() if n in tok else d[n]
                            for n in ("q", "k", "v", "log_a", "beta", "gate", "conv_q", "conv_k", "conv_v", "norm_w")],
                          S0_d[b:b + 1].contiguous(), dy[:, sl].contiguous(), dS_d[b:b + 1].contiguous(),
                          reverse=reverse)
        torch.cuda.synchronize()
        for n in tok:
            assert torch.isfinite(got[n][sl]).all(), (b, n)
            assert torch.equal(got[n][sl], one[n][0]), (b, n)
        assert torch.equal(got["S0"][b], one["S0"][0]), (b, "S0")
        for n in wsum:
            wsum[n] = wsum[n] + one[n].double()
        del one
    for n, ref in wsum.items():
        assert rel_l2(got[n].double().cpu().numpy(), ref.cpu().numpy()) < 1e-5, n


def test_bwd_varlen_multi_range_matches_oracle():
    """The same structure at d = 64, one head, against the fp64 autograd
    oracle on each sequence alone: lengths 9000 (141 chunks, three chain
    ranges), 37, 5000 (ends inside the second range) and 64."""
    lens = (9000, 37, 5000, 64)
    H, D = 1, 64
    inp, S0, grads, dS_T, cu = _varlen_bwd_case(lens, H, D, "bf16", 1301)
    say(f"case: bwd varlen multi-range lengths {lens} H={H} d={D} bf16 vs oracle")
    _, _, _, _, got = _run_varlen_bwd(inp, S0, grads, dS_T, cu, "bf16", False)
    tok = ("q", "k", "v", "gate", "log_a", "beta")
    wsum = {n: 0.0 for n in ("conv_q", "conv_k", "conv_v", "norm_w")}
    for b in range(len(lens)):
        sl = slice(int(cu[b]), int(cu[b + 1]))
        seq = {n: (inp[n][:, sl] if n in tok else inp[n]) for n in obwd.NAMES if n != "S0"}
        seq["S0"] = S0[b:b + 1]
        ref = oracle_grads(seq, {"dy": grads["dy"][:, sl], "dS_T": dS_T[b:b + 1]})
        for n in tok:
            e = rel_l2(got[n][sl].double().cpu().numpy(), ref[n][0])
            say(f"  seq {b} (T={lens[b]}) d{n} rel-L2 {e:.2e}")
            assert e <= TOL["bf16"], (b, n, e)
        e = rel_l2(got["S0"][b].double().cpu().numpy(), ref["S0"][0])
        assert e <= TOL["bf16"], (b, "S0", e)
        for n in wsum:
            wsum[n] = wsum[n] + ref[n]
    for n, ref in wsum.items():
        e = rel_l2(got[n].double().cpu().numpy(), ref)
        say(f"  d{n} (sum over sequences) rel-L2 {e:.2e}")
        assert e <= TOL["bf16"], (n, e)

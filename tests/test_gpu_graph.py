"""HIP graphs.  The layer and the whole token mixer captured in a HIP graph
(through torch.cuda.graph on a side stream) and replayed: the call's fork
onto the library's streams and the join back are captured with it.  Every
replay, with eager work and synchronisations in between, must equal the
eager call bit for bit.  The library's own graph cache (calls on a stream
other than the null stream record their launches the second time and
replay them after) must equal direct launches bit for bit as well."""
import numpy as np
import pytest
import torch

import gdn_inputs
import linear_attention_token_fwd_amd as gdn
import oracle
from tests.gpu_common import TOL, rel_l2, say

pytestmark = pytest.mark.gpu


def _dev(a, dt=torch.float32):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(dt).contiguous()


def test_layer_graph_replays():
    w = gdn_inputs.WORKLOADS[1]
    inp = gdn_inputs.generate(w, T=64 * 9 + 13, H=3, seed=61)
    d = gdn.to_device(inp, dtype=torch.bfloat16)
    B, T, H, D = inp["q"].shape
    args = (d["q"], d["k"], d["v"], d["log_a"], d["beta"], d["gate"], d["conv_q"], d["conv_k"], d["conv_v"],
            d["norm_w"], d["S0"])
    ws = torch.empty(gdn.gdn_fwd_workspace_bytes(B, T, H, D), dtype=torch.uint8, device="cuda")
    eager_y, eager_s = gdn.gdn_fwd(*args, workspace=ws)
    torch.cuda.synchronize()
    eager_y, eager_s = eager_y.clone(), eager_s.clone()

    out = torch.empty_like(eager_y)
    S_T = torch.empty_like(eager_s)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        gdn.gdn_fwd(*args, out=out, S_T=S_T, workspace=ws, stream=side)  # warm-up on the side stream
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=side):
        gdn.gdn_fwd(*args, out=out, S_T=S_T, workspace=ws, stream=side)
    for rep in range(4):
        out.fill_(float("nan"))
        S_T.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say(f"  replay {rep}: y equal {bool(torch.equal(out, eager_y))}, S_T equal {bool(torch.equal(S_T, eager_s))}")
        assert torch.equal(out, eager_y) and torch.equal(S_T, eager_s), f"replay {rep} differs from the eager call"
        gdn.gdn_fwd(*args, workspace=ws)  # eager work between the replays
        torch.cuda.synchronize()


def test_mixer_graph_replays():
    mw = gdn_inputs.MIXER_WORKLOADS[0]
    inp = gdn_inputs.generate_mixer(mw, T=300, seed=62)
    H, D = mw.H, mw.D
    tensors = dict(x=_dev(inp["x"], torch.bfloat16), w_in=_dev(inp["w_in"], torch.bfloat16), A_log=_dev(inp["A_log"]),
                   conv_q=_dev(inp["conv_q"]), conv_k=_dev(inp["conv_k"]), conv_v=_dev(inp["conv_v"]),
                   w_out=_dev(inp["w_out"], torch.bfloat16))
    extra = dict(b_in=_dev(inp["b_in"]), b_out=_dev(inp["b_out"]), norm_w=_dev(inp["norm_w"]))
    B, T, C = inp["x"].shape
    ws = torch.empty(gdn.gdn_mixer_workspace_bytes(B, T, H, D, C), dtype=torch.uint8, device="cuda")

    def call(out=None, S_T=None, stream=None):
        return gdn.gdn_mixer_fwd(tensors["x"], tensors["w_in"], tensors["A_log"], tensors["conv_q"],
                                 tensors["conv_k"], tensors["conv_v"], tensors["w_out"], H, D, out=out, S_T=S_T,
                                 workspace=ws, stream=stream, **extra)

    eager_o, eager_s = call()
    torch.cuda.synchronize()
    eager_o, eager_s = eager_o.clone(), eager_s.clone()
    out = torch.empty_like(eager_o)
    S_T = torch.empty_like(eager_s)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(out, S_T, side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=side):
        call(out, S_T, side)
    for rep in range(4):
        out.fill_(float("nan"))
        S_T.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager_o) and torch.equal(S_T, eager_s), f"replay {rep} differs from the eager call"
        call()
        torch.cuda.synchronize()
    say("  mixer: 4 replays equal to the eager call")


def _layer_case(T, H, seed):
    w = gdn_inputs.WORKLOADS[1]
    inp = gdn_inputs.generate(w, T=T, H=H, seed=seed)
    d = gdn.to_device(inp, dtype=torch.bfloat16)
    args = (d["q"], d["k"], d["v"], d["log_a"], d["beta"], d["gate"], d["conv_q"], d["conv_k"], d["conv_v"],
            d["norm_w"], d["S0"])
    return inp, d, args


def _side_call(fn, side):
    """Run fn on the side stream, ordered after the current stream's work, and wait."""
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        r = fn()
    torch.cuda.synchronize()
    return r


def test_graph_cache_replays_equal_direct_launches():
    """On a side stream the library records a call's launches the second
    time it sees them and replays them afterwards; every call must equal the
    direct launch on the null stream bit for bit, also after the inputs
    change in place (a replay reads the buffers' current contents) and after
    older graphs are evicted."""
    gdn.gdn_set_graph_cache_limit(0)  # start empty
    gdn.gdn_set_graph_cache_limit(2)
    side = torch.cuda.Stream()
    try:
        inp, d, args = _layer_case(64 * 9 + 13, 3, 71)
        B, T, H, D = inp["q"].shape
        ws = torch.empty(gdn.gdn_fwd_workspace_bytes(B, T, H, D), dtype=torch.uint8, device="cuda")
        direct_y, direct_s = gdn.gdn_fwd(*args, workspace=ws)  # null stream: direct launches
        torch.cuda.synchronize()
        direct_y, direct_s = direct_y.clone(), direct_s.clone()
        assert gdn.gdn_graph_cache_count() == 0
        out = torch.empty_like(direct_y)
        S_T = torch.empty_like(direct_s)
        expect_count = [0, 1, 1, 1]  # first sighting direct, second recorded, then replays
        for i, n in enumerate(expect_count):
            out.fill_(float("nan"))
            S_T.fill_(float("nan"))
            _side_call(lambda: gdn.gdn_fwd(*args, out=out, S_T=S_T, workspace=ws, stream=side), side)
            say(f"  call {i}: graphs {gdn.gdn_graph_cache_count()}, y equal {bool(torch.equal(out, direct_y))}")
            assert gdn.gdn_graph_cache_count() == n
            assert torch.equal(out, direct_y) and torch.equal(S_T, direct_s), f"call {i} differs"

        # new contents in the same buffers: the replay must see them
        inp2, d2, _ = _layer_case(T, H, 72)
        for name in ("q", "k", "v", "log_a", "beta", "gate", "conv_q", "conv_k", "conv_v", "norm_w"):
            d[name].copy_(d2[name])
        torch.cuda.synchronize()
        ry, rs = gdn.gdn_fwd(*args, workspace=ws)
        torch.cuda.synchronize()
        ry, rs = ry.clone(), rs.clone()
        assert not torch.equal(ry, direct_y)
        _side_call(lambda: gdn.gdn_fwd(*args, out=out, S_T=S_T, workspace=ws, stream=side), side)
        assert gdn.gdn_graph_cache_count() == 1
        assert torch.equal(out, ry) and torch.equal(S_T, rs), "replay after an in-place input change differs"
        ref_y, ref_s, _ = oracle.inputs_for(inp2)
        ey = rel_l2(out.double().cpu().numpy(), ref_y)
        es = rel_l2(S_T.double().cpu().numpy(), ref_s)
        say(f"  replay vs oracle: y {ey:.2e}, S_T {es:.2e}")
        assert ey <= TOL["bf16"] and es <= TOL["bf16"]

        # three more configurations, each called three times, with a limit of two graphs
        for T2, H2, seed in ((64 * 3, 2, 73), (64 * 5 + 1, 1, 74), (64 * 2 + 40, 4, 75)):
            _, _, a2 = _layer_case(T2, H2, seed)
            ws2 = torch.empty(gdn.gdn_fwd_workspace_bytes(1, T2, H2, 128), dtype=torch.uint8, device="cuda")
            dy, ds = gdn.gdn_fwd(*a2, workspace=ws2)
            torch.cuda.synchronize()
            dy, ds = dy.clone(), ds.clone()
            o2 = torch.empty_like(dy)
            s2 = torch.empty_like(ds)
            for i in range(3):
                o2.fill_(float("nan"))
                _side_call(lambda: gdn.gdn_fwd(*a2, out=o2, S_T=s2, workspace=ws2, stream=side), side)
                assert torch.equal(o2, dy) and torch.equal(s2, ds), f"T={T2} H={H2} call {i} differs"
            assert gdn.gdn_graph_cache_count() <= 2
        say(f"  after eviction: graphs {gdn.gdn_graph_cache_count()}")

        # the first configuration again (its graph was evicted): still equal
        for i in range(3):
            out.fill_(float("nan"))
            _side_call(lambda: gdn.gdn_fwd(*args, out=out, S_T=S_T, workspace=ws, stream=side), side)
            assert torch.equal(out, ry) and torch.equal(S_T, rs), f"re-recorded call {i} differs"
    finally:
        gdn.gdn_set_graph_cache_limit(8)


def test_graph_cache_varlen_and_mixer():
    """The variable-length call and the mixer's layer stage take the same
    graph path: three calls on a side stream equal the direct launch."""
    gdn.gdn_set_graph_cache_limit(0)
    gdn.gdn_set_graph_cache_limit(8)
    side = torch.cuda.Stream()
    lens = [1, 63, 64, 65, 200, 7]
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    inp, d, _ = _layer_case(cu[-1], 2, 76)
    vargs = (d["q"], d["k"], d["v"], d["log_a"], d["beta"], d["gate"], d["conv_q"], d["conv_k"], d["conv_v"], cu)
    ws = torch.empty(gdn.gdn_fwd_varlen_workspace_bytes(cu, 2, 128), dtype=torch.uint8, device="cuda")
    dy, ds = gdn.gdn_fwd_varlen(*vargs, norm_w=d["norm_w"], workspace=ws)
    torch.cuda.synchronize()
    dy, ds = dy.clone(), ds.clone()
    out = torch.empty_like(dy)
    S_T = torch.empty_like(ds)
    for i in range(3):
        out.fill_(float("nan"))
        _side_call(lambda: gdn.gdn_fwd_varlen(*vargs, norm_w=d["norm_w"], out=out, S_T=S_T, workspace=ws,
                                              stream=side), side)
        assert torch.equal(out, dy) and torch.equal(S_T, ds), f"varlen call {i} differs"
    assert gdn.gdn_graph_cache_count() == 1
    say("  varlen: 3 side-stream calls equal the direct launch")

    mw = gdn_inputs.MIXER_WORKLOADS[0]
    minp = gdn_inputs.generate_mixer(mw, T=300, seed=77)
    H, D = mw.H, mw.D
    t = dict(x=_dev(minp["x"], torch.bfloat16), w_in=_dev(minp["w_in"], torch.bfloat16), A_log=_dev(minp["A_log"]),
             conv_q=_dev(minp["conv_q"]), conv_k=_dev(minp["conv_k"]), conv_v=_dev(minp["conv_v"]),
             w_out=_dev(minp["w_out"], torch.bfloat16))
    extra = dict(b_in=_dev(minp["b_in"]), b_out=_dev(minp["b_out"]), norm_w=_dev(minp["norm_w"]))
    B, T, C = minp["x"].shape
    mws = torch.empty(gdn.gdn_mixer_workspace_bytes(B, T, H, D, C), dtype=torch.uint8, device="cuda")

    def call(out=None, S_T=None, stream=None):
        return gdn.gdn_mixer_fwd(t["x"], t["w_in"], t["A_log"], t["conv_q"], t["conv_k"], t["conv_v"], t["w_out"],
                                 H, D, out=out, S_T=S_T, workspace=mws, stream=stream, **extra)

    do, dsm = call()
    torch.cuda.synchronize()
    do, dsm = do.clone(), dsm.clone()
    mo = torch.empty_like(do)
    ms = torch.empty_like(dsm)
    for i in range(3):
        mo.fill_(float("nan"))
        _side_call(lambda: call(mo, ms, side), side)
        assert torch.equal(mo, do) and torch.equal(ms, dsm), f"mixer call {i} differs"
    assert gdn.gdn_graph_cache_count() == 2
    say("  mixer: 3 side-stream calls equal the direct launch")

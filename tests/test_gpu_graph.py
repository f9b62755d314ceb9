"""The layer and the whole token mixer captured in a HIP graph (through
torch.cuda.graph on a side stream) and replayed: the call's fork onto the
library's streams and the join back are captured with it.  Every replay,
with eager work and synchronisations in between, must equal the eager call
bit for bit."""
import numpy as np
import pytest
import torch

import gdn_inputs
import linear_attention_token_fwd_amd as gdn
from tests.gpu_common import say

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

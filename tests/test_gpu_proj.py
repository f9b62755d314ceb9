"""Parity of the token mixer projections (gdn_in_proj, gdn_out_proj, through
the C ABI) with the fp64 projection oracle.

Bars.  The products run on bf16 operands with fp32 accumulation, so:
  * bf16 outputs (q, k, v, gate, the output projection) must sit within one
    bf16 rounding of the exact value: |got - ref| <= 2^-8 |ref| + 1e-4, and
    rel-L2 <= 4e-3 over the tensor;
  * fp32 outputs (beta, log a) must match to |got - ref| <= 2e-5 + 1e-5 |ref|
    (fp32 accumulation over C products), rel-L2 <= 1e-5.
"""
import ctypes

import numpy as np
import pytest
import torch

import gdn_inputs
import linear_attention_token_fwd_amd as gdn
from oracle import proj as oproj
from tests.gpu_common import rel_l2, say

pytestmark = pytest.mark.gpu

MW = gdn_inputs.MIXER_WORKLOADS


def _dev(a, dtype=torch.float32):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(dtype).contiguous()


def check_bf16(name, got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    e = rel_l2(got, ref)
    worst = float(np.max(np.abs(got - ref) - (2.0 ** -8 * np.abs(ref) + 1e-4)))
    say(f"  {name}: rel-L2 {e:.3e}, worst excess over one bf16 rounding {worst:.2e}")
    assert e <= 4e-3, f"{name}: rel-L2 {e:.3e}"
    assert worst <= 0, f"{name}: an element is off by more than one bf16 rounding"


def check_f32(name, got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    e = rel_l2(got, ref)
    worst = float(np.max(np.abs(got - ref) - (2e-5 + 1e-5 * np.abs(ref))))
    say(f"  {name}: rel-L2 {e:.3e}, worst excess {worst:.2e}")
    assert e <= 1e-5, f"{name}: rel-L2 {e:.3e}"
    assert worst <= 0, f"{name}: element error above the bound"


def run_in_proj(inp, H, D):
    """gdn_in_proj on NaN-poisoned outputs (every element must be written)."""
    x = _dev(inp["x"], torch.bfloat16)
    w_in = _dev(inp["w_in"], torch.bfloat16)
    B, T, C = inp["x"].shape
    q, k, v, g = (torch.full((B, T, H, D), float("nan"), dtype=torch.bfloat16, device="cuda") for _ in range(4))
    beta, log_a = (torch.full((B, T, H), float("nan"), dtype=torch.float32, device="cuda") for _ in range(2))
    A_log, b_in = _dev(inp["A_log"]), _dev(inp["b_in"])
    p = gdn.in_proj_params(x, w_in, b_in, A_log, H, D, q, k, v, g, beta, log_a)
    st = gdn.load().gdn_in_proj(ctypes.byref(p), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == gdn.GDN_OK, gdn.gdn_status_string(st)
    torch.cuda.synchronize()
    return [t.double().cpu().numpy() for t in (q, k, v, g, beta, log_a)]


def compare_in_proj(inp, H, D, rows=None):
    got = run_in_proj(inp, H, D)
    x = inp["x"]
    if rows is not None:  # the oracle on sampled token rows only
        x = x.reshape(-1, x.shape[-1])[rows][None]
        got = [g.reshape(-1, *g.shape[2:])[rows][None] for g in got]
    ref = oproj.in_proj(x, inp["w_in"], inp["b_in"], inp["A_log"], H, D)
    for name, g, r in zip(("q", "k", "v", "gate"), got[:4], ref[:4]):
        check_bf16(name, g, r)
    check_f32("beta", got[4], ref[4])
    check_f32("log_a", got[5], ref[5])


@pytest.mark.parametrize("bias", [True, False])
def test_in_proj_small(bias):
    """H = 3 heads of 64 (odd gate columns), C = 192, T = 700: ragged row
    tiles and a 6-column last column tile."""
    w = MW[0]
    say(f"case: in_proj {w.name} bias={bias}")
    compare_in_proj(gdn_inputs.generate_mixer(w, bias=bias), w.H, w.D)


@pytest.mark.parametrize("B,T", [(2, 300), (1, 1), (1, 257)])
def test_in_proj_model_width(B, T):
    """The 1.3B model's width (C = 1536, H = 12, d = 128) at short lengths."""
    w = MW[1]
    say(f"case: in_proj C=1536 B={B} T={T}")
    compare_in_proj(gdn_inputs.generate_mixer(w, T=T, B=B, seed=50 + T), w.H, w.D)


def test_in_proj_full_size_sampled():
    """T = 32760 at C = 1536, in the launch the benchmark times; the oracle
    checks 1500 sampled token rows, the last rows included."""
    w = MW[1]
    inp = gdn_inputs.generate_mixer(w)
    M = w.B * w.T
    rows = np.unique(np.concatenate([np.random.default_rng(9).choice(M, 1480, replace=False),
                                     np.arange(M - 20, M)]))
    say(f"case: in_proj full size {w.name}, {len(rows)} sampled rows")
    compare_in_proj(inp, w.H, w.D, rows=rows)


def run_out_proj(y, w_out, b_out):
    B, T, H, D = y.shape
    C = w_out.shape[0]
    out = torch.full((B, T, C), float("nan"), dtype=torch.bfloat16, device="cuda")
    gdn.gdn_out_proj(_dev(y, torch.bfloat16), _dev(w_out, torch.bfloat16), _dev(b_out), out=out)
    torch.cuda.synchronize()
    return out.double().cpu().numpy()


@pytest.mark.parametrize("wid,T,bias", [(0, 700, True), (0, 700, False), (1, 300, True), (1, 1, True)])
def test_out_proj(wid, T, bias):
    w = MW[wid]
    inp = gdn_inputs.generate_mixer(w, T=T, bias=bias, seed=70 + T)
    y = gdn_inputs.round_bf16(np.random.default_rng(T).standard_normal((w.B, T, w.H, w.D), dtype=np.float32))
    say(f"case: out_proj {w.name} T={T} bias={bias}")
    check_bf16("out", run_out_proj(y, inp["w_out"], inp["b_out"]), oproj.out_proj(y, inp["w_out"], inp["b_out"]))


def test_out_proj_full_size_sampled():
    w = MW[1]
    inp = gdn_inputs.generate_mixer(w)
    y = gdn_inputs.round_bf16(np.random.default_rng(1).standard_normal((w.B, w.T, w.H, w.D), dtype=np.float32))
    say(f"case: out_proj full size {w.name}")
    got = run_out_proj(y, inp["w_out"], inp["b_out"]).reshape(w.T, -1)
    rows = np.unique(np.concatenate([np.random.default_rng(4).choice(w.T, 1480, replace=False),
                                     np.arange(w.T - 20, w.T)]))
    ref = oproj.out_proj(y[:, rows], inp["w_out"], inp["b_out"])[0]
    check_bf16("out", got[rows], ref)


def test_projections_deterministic():
    w = MW[0]
    inp = gdn_inputs.generate_mixer(w)
    a = run_in_proj(inp, w.H, w.D)
    b = run_in_proj(inp, w.H, w.D)
    assert all(np.array_equal(x, y, equal_nan=False) for x, y in zip(a, b))


def test_in_proj_errors_leave_outputs_untouched():
    w = MW[0]
    inp = gdn_inputs.generate_mixer(w)
    x = _dev(inp["x"], torch.bfloat16)
    w_in = _dev(inp["w_in"], torch.bfloat16)
    A_log = _dev(inp["A_log"])
    B, T, C = inp["x"].shape
    H, D = w.H, w.D
    q, k, v, g = (torch.full((B, T, H, D), 7.0, dtype=torch.bfloat16, device="cuda") for _ in range(4))
    beta, log_a = (torch.full((B, T, H), 7.0, dtype=torch.float32, device="cuda") for _ in range(2))
    lib = gdn.load()
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def status(mutate):
        p = gdn.in_proj_params(x, w_in, None, A_log, H, D, q, k, v, g, beta, log_a)
        mutate(p)
        return lib.gdn_in_proj(ctypes.byref(p), s)

    assert status(lambda p: setattr(p, "C", 160)) == gdn.GDN_ERR_UNSUPPORTED       # C % 64 != 0
    assert status(lambda p: setattr(p, "x", p.x + 2)) == gdn.GDN_ERR_ALIGNMENT
    assert status(lambda p: setattr(p, "q", None)) == gdn.GDN_ERR_INVALID_ARG
    assert status(lambda p: setattr(p, "k", p.q)) == gdn.GDN_ERR_INVALID_ARG       # outputs overlap
    assert status(lambda p: setattr(p, "beta", p.w_in)) == gdn.GDN_ERR_INVALID_ARG  # output over an input
    torch.cuda.synchronize()
    for t in (q, k, v, g, beta, log_a):
        assert bool(torch.all(t == 7.0))


def run_mixer(inp, H, D, S0=None):
    B, T, C = inp["x"].shape
    out = torch.full((B, T, C), float("nan"), dtype=torch.bfloat16, device="cuda")
    S_T = torch.full((B, H, D, D), float("nan"), dtype=torch.float32, device="cuda")
    gdn.gdn_mixer_fwd(_dev(inp["x"], torch.bfloat16), _dev(inp["w_in"], torch.bfloat16), _dev(inp["A_log"]),
                      _dev(inp["conv_q"]), _dev(inp["conv_k"]), _dev(inp["conv_v"]),
                      _dev(inp["w_out"], torch.bfloat16), H, D, b_in=_dev(inp["b_in"]), b_out=_dev(inp["b_out"]),
                      norm_w=_dev(inp["norm_w"]), S0=_dev(S0), out=out, S_T=S_T)
    torch.cuda.synchronize()
    return out.double().cpu().numpy(), S_T.double().cpu().numpy()


def compare_mixer(inp, H, D, S0=None):
    got, s = run_mixer(inp, H, D, S0)
    ref, rs, _ = oproj.mixer(inp["x"], inp["w_in"], inp["b_in"], inp["A_log"], inp["conv_q"], inp["conv_k"],
                             inp["conv_v"], inp["norm_w"], inp["w_out"], inp["b_out"], H, D, S0=S0)
    assert np.all(np.isfinite(got)) and np.all(np.isfinite(s))
    e, es = rel_l2(got, ref), rel_l2(s, rs)
    rows = np.linalg.norm(got - ref, axis=-1) / np.maximum(np.linalg.norm(ref, axis=-1), 1e-30)
    say(f"  mixer out rel-L2 {e:.3e}, S_T rel-L2 {es:.3e}, worst token row {rows.max():.3e} (bar 1e-2)")
    assert e <= 1e-2 and es <= 1e-2 and rows.max() <= 5e-2


@pytest.mark.parametrize("T", [700, 1, 65])
def test_mixer_small(T):
    """The whole mixer (in_proj, layer, out_proj) at H = 3, d = 64, C = 192,
    with a random initial state and norm weight."""
    w = MW[0]
    inp = gdn_inputs.generate_mixer(w, T=T, seed=90 + T)
    inp["norm_w"] = (1 + 0.3 * np.random.default_rng(T).standard_normal((w.H, w.D))).astype(np.float32)
    S0 = (0.05 * np.random.default_rng(T + 1).standard_normal((1, w.H, w.D, w.D))).astype(np.float32)
    say(f"case: mixer {w.name} T={T}")
    compare_mixer(inp, w.H, w.D, S0)


def test_mixer_full_size():
    """The 1.3B model's token mixer at T = 32760 (the configuration the
    benchmark's mixer line times), every token against the oracle."""
    w = MW[1]
    say(f"case: mixer full size {w.name}")
    compare_mixer(gdn_inputs.generate_mixer(w), w.H, w.D)


def test_mixer_batch_d128_no_bias():
    """The mixer with two batch rows, heads of 128 and no biases (H = 2,
    C = 256, T = 130: a ragged last chunk and a ragged row tile)."""
    w = gdn_inputs.MixerWorkload(98, "B2 T130 H2 d128 C256", 2, 130, 2, 128, 256)
    inp = gdn_inputs.generate_mixer(w, bias=False, seed=31)
    say(f"case: mixer {w.name}, no bias")
    compare_mixer(inp, w.H, w.D)


def test_mixer_staged_equals_three_stages():
    """The mixer runs its out-projection beside the layer, split by the
    layer's chunk ranges and batch rows; its outputs must equal, bit for bit,
    the three stages called one after another (gdn_in_proj, gdn_fwd,
    gdn_out_proj).  B = 2, T = 24349 (381 chunks: three ranges and a ragged
    last chunk), H = 3, d = 64, C = 192, with a random initial state; on a
    side stream, three calls in a row (launched directly, recorded as a
    launch graph, replayed)."""
    w = gdn_inputs.MixerWorkload(97, "B2 T24349 H3 d64 C192", 2, 24349, 3, 64, 192)
    inp = gdn_inputs.generate_mixer(w, seed=41)
    H, D = w.H, w.D
    B, T, C = inp["x"].shape
    say(f"case: mixer {w.name}, against its three stages")
    x, w_in, w_out = (_dev(inp[n], torch.bfloat16) for n in ("x", "w_in", "w_out"))
    A_log, b_in, b_out, norm_w = (_dev(inp[n]) for n in ("A_log", "b_in", "b_out", "norm_w"))
    conv_q, conv_k, conv_v = (_dev(inp[n]) for n in ("conv_q", "conv_k", "conv_v"))
    S0 = _dev((0.05 * np.random.default_rng(42).standard_normal((B, H, D, D))).astype(np.float32))
    q, k, v, g, beta, log_a = gdn.gdn_in_proj(x, w_in, A_log, H, D, b_in=b_in)
    y, s_ref = gdn.gdn_fwd(q, k, v, log_a, beta, g, conv_q, conv_k, conv_v, norm_w, S0)
    o_ref = gdn.gdn_out_proj(y, w_out, b_out)
    torch.cuda.synchronize()
    ws = torch.empty(gdn.gdn_mixer_workspace_bytes(B, T, H, D, C), dtype=torch.uint8, device="cuda")
    out, S_T = torch.empty_like(o_ref), torch.empty_like(s_ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        out.fill_(float("nan"))
        S_T.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            gdn.gdn_mixer_fwd(x, w_in, A_log, conv_q, conv_k, conv_v, w_out, H, D, b_in=b_in, b_out=b_out,
                              norm_w=norm_w, S0=S0, out=out, S_T=S_T, workspace=ws, stream=side)
        torch.cuda.synchronize()
        assert torch.equal(out, o_ref) and torch.equal(S_T, s_ref), f"call {rep} differs from the three stages"
    say("  3 calls equal to the three stages, bit for bit")

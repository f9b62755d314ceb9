"""Pins of the backward oracle (oracle/bwd.py), on the CPU.

* Its forward, written again in torch fp64, equals the C oracle's layer.
* Its gradients equal central finite differences of the same scalar, input by
  input, on a tiny layer.
* The b = 0 closed form: then S_T = (prod_t a_t) S0, so for L = <dS_T, S_T>
  the gradient w.r.t. S0 is (prod a) dS_T, every d log a_t equals L, and q,
  k, v and the gate get no gradient.
* Planted mistakes in the forward (the delta term's sign, the decay, the
  conv taps' order) make it disagree with the C oracle.
"""
import numpy as np
import pytest
import torch

import gdn_inputs
import oracle
from oracle import bwd


def _small(wid, T, H, seed):
    inp = gdn_inputs.generate(gdn_inputs.WORKLOADS[wid], T=T, H=H, seed=seed)
    return {n: inp.get(n) for n in bwd.NAMES}


def _rel(a, b):
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / np.linalg.norm(np.asarray(b)))


@pytest.mark.parametrize("wid", [0, 3])
def test_forward_matches_c_oracle(wid):
    inp = _small(wid, 70, 2, 11)
    y_c, s_c, _ = oracle.gdn_fwd(*[inp[n] for n in bwd.NAMES])
    with torch.no_grad():
        y_t, s_t = bwd.forward(*[bwd._t(inp[n]) for n in bwd.NAMES])
    assert _rel(y_t.numpy(), y_c) < 1e-12
    assert _rel(s_t.numpy(), s_c) < 1e-12


def _tiny(seed):
    rng = np.random.default_rng(seed)
    B, T, H, D = 1, 6, 1, 4
    return {
        "q": rng.standard_normal((B, T, H, D)), "k": rng.standard_normal((B, T, H, D)),
        "v": rng.standard_normal((B, T, H, D)), "gate": rng.standard_normal((B, T, H, D)),
        "log_a": -rng.uniform(0.05, 0.8, (B, T, H)), "beta": rng.uniform(0.1, 0.9, (B, T, H)),
        "conv_q": rng.normal(0, 0.5, (H * D, 4)), "conv_k": rng.normal(0, 0.5, (H * D, 4)),
        "conv_v": rng.normal(0, 0.5, (H * D, 4)), "norm_w": rng.uniform(0.5, 1.5, (H, D)),
        "S0": rng.normal(0, 0.3, (B, H, D, D)),
    }


def test_gradients_match_finite_differences():
    inp = _tiny(5)
    rng = np.random.default_rng(6)
    dy = rng.standard_normal(inp["v"].shape)
    dS = rng.standard_normal(inp["S0"].shape)
    _, _, grads = bwd.backward(inp, dy, dS)
    for name in bwd.NAMES:
        x = inp[name]
        e = rng.standard_normal(x.shape)
        h = 1e-5
        plus = dict(inp, **{name: x + h * e})
        minus = dict(inp, **{name: x - h * e})
        fd = (bwd.loss(plus, dy, dS) - bwd.loss(minus, dy, dS)) / (2 * h)
        an = float((grads[name] * e).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_b0_closed_form():
    inp = _tiny(7)
    inp["beta"] = np.zeros_like(inp["beta"])
    rng = np.random.default_rng(8)
    dS = rng.standard_normal(inp["S0"].shape)
    dy = np.zeros(inp["v"].shape)
    _, S_T, grads = bwd.backward(inp, dy, dS)
    decay = np.exp(inp["log_a"].sum())
    assert np.allclose(S_T, decay * inp["S0"], rtol=1e-13, atol=0)
    L = float((dS * S_T).sum())
    assert np.allclose(grads["S0"], decay * dS, rtol=1e-13, atol=0)
    assert np.allclose(grads["log_a"], L, rtol=1e-12, atol=1e-15)
    for name in ("q", "k", "v", "gate", "conv_q", "conv_k", "conv_v", "norm_w"):
        assert np.abs(grads[name]).max() == 0.0, name


# ---- planted mistakes: each version of the forward must miss the C oracle
def _mutant_forward(kind):
    def conv_silu(x, w):
        B, T, H, D = x.shape
        wv = w.reshape(H, D, 4)
        xp = torch.cat([x.new_zeros(B, 3, H, D), x], dim=1)
        taps = range(3, -1, -1) if kind == "taps" else range(4)
        z = sum(wv[:, :, j] * xp[:, jj:jj + T] for j, jj in zip(range(4), taps))
        return z * torch.sigmoid(z)

    def fwd(q, k, v, log_a, beta, gate, conv_q, conv_k, conv_v, norm_w=None, S0=None):
        qh = bwd.l2_normalize(conv_silu(q, conv_q), 1e-6)
        kh = bwd.l2_normalize(conv_silu(k, conv_k), 1e-6)
        vh = conv_silu(v, conv_v)
        B, T, H, Dk = qh.shape
        S = S0 if S0 is not None else qh.new_zeros(B, H, vh.shape[3], Dk)
        a = torch.exp(log_a) if kind != "decay" else torch.ones_like(log_a)
        sign = -1.0 if kind == "sign" else 1.0
        outs = []
        for t in range(T):
            kt = kh[:, t].unsqueeze(-1)
            at, bt = a[:, t, :, None, None], beta[:, t, :, None, None]
            S = at * S - sign * (at * bt) * ((S @ kt) @ kt.transpose(-1, -2)) \
                + bt * (vh[:, t].unsqueeze(-1) @ kt.transpose(-1, -2))
            outs.append((S @ qh[:, t].unsqueeze(-1)).squeeze(-1))
        o = torch.stack(outs, dim=1)
        y = o / torch.sqrt((o * o).mean(-1, keepdim=True) + 1e-6) * torch.sigmoid(gate) * gate
        return y * norm_w if norm_w is not None else y, S
    return fwd


@pytest.mark.parametrize("kind", ["sign", "decay", "taps"])
def test_planted_mistakes_miss_the_c_oracle(kind):
    inp = _small(3, 70, 2, 12)
    y_c, _, _ = oracle.gdn_fwd(*[inp[n] for n in bwd.NAMES])
    with torch.no_grad():
        y_m, _ = _mutant_forward(kind)(*[bwd._t(inp[n]) for n in bwd.NAMES])
    assert _rel(y_m.numpy(), y_c) > 1e-3

"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each ``pin_*`` function takes an ``oracle.Oracle`` and asserts.  The same
functions run against the real oracle (test_oracle_pins.py) and against
mutated copies of its source (test_oracle_mutants.py), which must each fail
at least one pin.

What pins what:
  * conv + SiLU: an impulse response (taps come out reversed in time and
    causal), numpy.convolve as the textbook causal convolution, the logistic
    function from scipy for SiLU, and identity taps;
  * L2 normalisation: unit norm and direction at eps = 0; where eps sits
    (added to the sum of squares, inside the root);
  * gated delta rule: the closed form with b = 0 (pure decay of S0); exact
    retrieval with a = b = 1 and one-hot keys; the two facts that define one
    delta-rule step (what the new state does to k_t and to every vector
    orthogonal to k_t); a one-token case with explicit matrices; the
    contraction bound; agreement with an independent chunked (WY) model at
    several chunk lengths; split/resume and identity padding;
  * gated RMS normalisation: torch's rms_norm (a library routine) times SiLU
    of the gate, and the constant-vector closed form;
  * the layer driver: composition of the parts on gathered per-head arrays,
    head permutation, time reversal, palindromes for the bidirectional
    variant, head subsets and thread counts, and independence of the final
    state from q and the gate.
"""
from __future__ import annotations

import numpy as np
from scipy.special import expit

from oracle.chunked import chunked_delta_rule


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


def _silu(z):
    return z * expit(z)


def _unit_rows(rng, T, D):
    x = rng.standard_normal((T, D))
    return x / np.linalg.norm(x, axis=1, keepdims=True)


# ------------------------------------------------------------------ conv
def pin_conv_impulse(o):
    rng = np.random.default_rng(1)
    T, D, t0 = 12, 3, 4
    w = rng.standard_normal((D, 4))
    x = np.zeros((T, D))
    x[t0, :] = 1.0
    pre = np.zeros((T, D))
    for jp in range(4):  # output at t0 + jp sees the impulse through tap 3 - jp
        pre[t0 + jp, :] = w[:, 3 - jp]
    np.testing.assert_allclose(o.short_conv_silu(x, w), _silu(pre), rtol=1e-14, atol=1e-300)


def pin_conv_vs_numpy(o):
    rng = np.random.default_rng(2)
    T, D = 50, 5
    x = rng.standard_normal((T, D))
    w = rng.standard_normal((D, 4))
    pre = np.stack([np.convolve(x[:, c], w[c, ::-1])[:T] for c in range(D)], axis=1)
    np.testing.assert_allclose(o.short_conv_silu(x, w), _silu(pre), rtol=1e-12, atol=1e-14)


def pin_conv_identity_and_silu(o):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((40, 4)) * 3
    w = np.tile([0.0, 0.0, 0.0, 1.0], (4, 1))
    y = o.short_conv_silu(x, w)
    np.testing.assert_allclose(y, _silu(x), rtol=1e-14, atol=1e-300)
    # silu(z) - silu(-z) = z for the logistic-gated linear unit
    np.testing.assert_allclose(y - o.short_conv_silu(-x, w), x, rtol=1e-13, atol=1e-14)


# ------------------------------------------------------------------ L2
def pin_l2(o):
    rng = np.random.default_rng(4)
    x = rng.standard_normal((30, 16)) * 5
    y = o.l2_normalize(x, eps=0.0)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(y * np.linalg.norm(x, axis=1, keepdims=True), x, rtol=1e-13)
    eps = 1e-6
    tiny = np.full((1, 4), np.sqrt(eps) / 2.0)  # |x|^2 = eps
    np.testing.assert_allclose(np.linalg.norm(o.l2_normalize(tiny, eps)), 1 / np.sqrt(2), rtol=1e-12)
    assert np.all(o.l2_normalize(np.zeros((2, 4)), eps) == 0.0)


# ------------------------------------------------------------------ recurrence
def _rand_rec(rng, T, D, S0=True):
    q = _unit_rows(rng, T, D)
    k = _unit_rows(rng, T, D)
    v = rng.standard_normal((T, D))
    la = -0.3 * rng.random(T)
    be = rng.random(T)
    s0 = rng.standard_normal((D, D)) if S0 else None
    return q, k, v, la, be, s0


def pin_decay_closed_form(o):
    rng = np.random.default_rng(5)
    T, D = 25, 8
    q, k, v, la, _, S0 = _rand_rec(rng, T, D)
    out, ST, hist = o.delta_rule(q, k, v, la, np.zeros(T), S0, return_states=True)
    decay = np.exp(np.cumsum(la))
    for t in range(T):
        np.testing.assert_allclose(hist[t], decay[t] * S0, rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(out[t], decay[t] * (S0 @ q[t]), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(ST, decay[-1] * S0, rtol=1e-13)


def pin_delta_step_facts(o):
    """For unit k_t: S_t k_t = a(1-b) S_{t-1} k_t + b v_t, and S_t x = a S_{t-1} x
    for every x orthogonal to k_t; together they fix S_t.  o_t = S_t q_t."""
    rng = np.random.default_rng(6)
    T, D = 20, 8
    q, k, v, la, be, S0 = _rand_rec(rng, T, D)
    out, _, hist = o.delta_rule(q, k, v, la, be, S0, return_states=True)
    prev = S0
    for t in range(T):
        a, b = np.exp(la[t]), be[t]
        St = hist[t]
        np.testing.assert_allclose(St @ k[t], a * (1 - b) * (prev @ k[t]) + b * v[t],
                                   rtol=1e-11, atol=1e-12)
        x = rng.standard_normal(D)
        x -= (x @ k[t]) * k[t]
        np.testing.assert_allclose(St @ x, a * (prev @ x), rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(out[t], St @ q[t], rtol=1e-12, atol=1e-13)
        prev = St


def pin_exact_retrieval(o):
    """a = b = 1 with one-hot keys: the state is a lookup table that maps each
    key to the value last written under it."""
    rng = np.random.default_rng(7)
    D = 8
    keys = np.concatenate([rng.permutation(D), rng.permutation(D)[:5]])
    T = len(keys)
    k = np.eye(D)[keys]
    v = rng.standard_normal((T, D))
    q = np.eye(D)[rng.integers(0, D, T)]
    _, ST = o.delta_rule(q, k, v, np.zeros(T), np.ones(T), rng.standard_normal((D, D)))
    for col in range(D):
        last = max(t for t in range(T) if keys[t] == col)
        np.testing.assert_allclose(ST[:, col], v[last], rtol=0, atol=1e-14)


def pin_one_token_explicit(o):
    rng = np.random.default_rng(8)
    D = 6
    q, k, v, la, be, S0 = _rand_rec(rng, 1, D)
    a, b = np.exp(la[0]), be[0]
    S1 = a * S0 @ (np.eye(D) - b * np.outer(k[0], k[0])) + b * np.outer(v[0], k[0])
    out, ST = o.delta_rule(q, k, v, la, be, S0)
    np.testing.assert_allclose(ST, S1, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(out[0], S1 @ q[0], rtol=1e-13, atol=1e-14)


def pin_contraction(o):
    rng = np.random.default_rng(9)
    T, D = 60, 8
    q, k, v, la, be, S0 = _rand_rec(rng, T, D)
    _, _, hist = o.delta_rule(q, k, v, la, be, S0, return_states=True)
    prev = np.linalg.norm(S0, 2)
    for t in range(T):
        cur = np.linalg.norm(hist[t], 2)
        assert cur <= np.exp(la[t]) * prev + be[t] * np.linalg.norm(v[t]) + 1e-12
        prev = cur


def pin_chunked_agreement(o):
    rng = np.random.default_rng(10)
    D = 8
    for T in (1, 7, 63, 64, 65, 130, 200):
        q, k, v, la, be, S0 = _rand_rec(rng, T, D)
        ref_o, ref_S = o.delta_rule(q, k, v, la, be, S0)
        for C in (1, 3, 16, 64, T):
            co, cS = chunked_delta_rule(q, k, v, la, be, S0, C)
            assert _rel(co, ref_o) < 1e-12, (T, C, _rel(co, ref_o))
            assert _rel(cS, ref_S) < 1e-12, (T, C)


def pin_resume_and_padding(o):
    rng = np.random.default_rng(11)
    T, D, cut = 90, 8, 37
    q, k, v, la, be, S0 = _rand_rec(rng, T, D)
    o_all, S_all = o.delta_rule(q, k, v, la, be, S0)
    o1, S1 = o.delta_rule(q[:cut], k[:cut], v[:cut], la[:cut], be[:cut], S0)
    o2, S2 = o.delta_rule(q[cut:], k[cut:], v[cut:], la[cut:], be[cut:], S1)
    assert np.array_equal(np.concatenate([o1, o2]), o_all)
    assert np.array_equal(S2, S_all)
    pad = 11
    qp = np.concatenate([q, _unit_rows(rng, pad, D)])
    kp = np.concatenate([k, _unit_rows(rng, pad, D)])
    vp = np.concatenate([v, rng.standard_normal((pad, D))])
    _, Sp = o.delta_rule(qp, kp, vp, np.concatenate([la, np.zeros(pad)]),
                         np.concatenate([be, np.zeros(pad)]), S0)
    assert np.array_equal(Sp, S_all)


# ------------------------------------------------------------------ RMS norm
def pin_rmsnorm_torch(o):
    import torch
    rng = np.random.default_rng(12)
    T, D = 33, 16
    x = rng.standard_normal((T, D)) * 2
    g = rng.standard_normal((T, D)) * 2
    w = rng.standard_normal(D)
    eps = 1e-6
    ref = (torch.nn.functional.rms_norm(torch.from_numpy(x), (D,), torch.from_numpy(w), eps)
           * torch.nn.functional.silu(torch.from_numpy(g))).numpy()
    np.testing.assert_allclose(o.gated_rmsnorm(x, g, w, eps), ref, rtol=1e-12, atol=1e-14)


def pin_rmsnorm_constant(o):
    rng = np.random.default_rng(13)
    D = 8
    g = rng.standard_normal((2, D))
    w = rng.standard_normal(D)
    x = np.stack([np.full(D, 3.5), np.full(D, -0.25)])
    y = o.gated_rmsnorm(x, g, w, eps=0.0)
    np.testing.assert_allclose(y, np.sign(x) * w * _silu(g), rtol=1e-13)
    assert np.all(o.gated_rmsnorm(np.zeros((1, D)), g[:1], w, eps=1e-6) == 0.0)


# ------------------------------------------------------------------ layer driver
def _layer_inputs(rng, B=2, T=70, H=3, D=8, S0=True):
    f = np.float32
    return dict(
        q=rng.standard_normal((B, T, H, D)).astype(f),
        k=rng.standard_normal((B, T, H, D)).astype(f),
        v=rng.standard_normal((B, T, H, D)).astype(f),
        log_a=(-0.3 * rng.random((B, T, H))).astype(f),
        beta=rng.random((B, T, H)).astype(f),
        gate=rng.standard_normal((B, T, H, D)).astype(f),
        conv_q=(0.5 * rng.standard_normal((H * D, 4))).astype(f),
        conv_k=(0.5 * rng.standard_normal((H * D, 4))).astype(f),
        conv_v=(0.5 * rng.standard_normal((H * D, 4))).astype(f),
        norm_w=(1 + 0.5 * rng.standard_normal((H, D))).astype(f),
        S0=(0.3 * rng.standard_normal((B, H, D, D))).astype(f) if S0 else None,
    )


def _run(o, d, **kw):
    return o.gdn_fwd(d["q"], d["k"], d["v"], d["log_a"], d["beta"], d["gate"], d["conv_q"],
                     d["conv_k"], d["conv_v"], d["norm_w"], d["S0"], **kw)


def pin_layer_composition(o):
    rng = np.random.default_rng(14)
    d = _layer_inputs(rng)
    B, T, H, D = d["q"].shape
    y, ST, _ = _run(o, d)
    for b in range(B):
        for h in range(H):
            wsl = slice(h * D, (h + 1) * D)
            qh = o.l2_normalize(o.short_conv_silu(d["q"][b, :, h], d["conv_q"][wsl]))
            kh = o.l2_normalize(o.short_conv_silu(d["k"][b, :, h], d["conv_k"][wsl]))
            vh = o.short_conv_silu(d["v"][b, :, h], d["conv_v"][wsl])
            out, S = o.delta_rule(qh, kh, vh, d["log_a"][b, :, h], d["beta"][b, :, h],
                                  d["S0"][b, h])
            yh = o.gated_rmsnorm(out, d["gate"][b, :, h], d["norm_w"][h])
            np.testing.assert_allclose(y[b, :, h], yh, rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(ST[b, h], S, rtol=1e-12, atol=1e-14)


def pin_layer_head_permutation(o):
    rng = np.random.default_rng(15)
    d = _layer_inputs(rng, B=1, T=40, H=4)
    y, ST, _ = _run(o, d)
    perm = np.array([2, 0, 3, 1])
    D = d["q"].shape[3]
    wperm = (perm[:, None] * D + np.arange(D)[None, :]).reshape(-1)
    p = dict(d)
    for key in ("q", "k", "v", "gate", "log_a", "beta"):
        p[key] = d[key][:, :, perm]
    for key in ("conv_q", "conv_k", "conv_v"):
        p[key] = d[key][wperm]
    p["norm_w"] = d["norm_w"][perm]
    p["S0"] = d["S0"][:, perm]
    y2, ST2, _ = _run(o, p)
    assert np.array_equal(y2, y[:, :, perm])
    assert np.array_equal(ST2, ST[:, perm])


def pin_layer_reverse(o):
    rng = np.random.default_rng(16)
    d = _layer_inputs(rng, B=2, T=50, H=2)
    yr, Sr, _ = _run(o, d, reverse=True)
    f = dict(d)
    for key in ("q", "k", "v", "gate", "log_a", "beta"):
        f[key] = np.ascontiguousarray(d[key][:, ::-1])
    yf, Sf, _ = _run(o, f)
    assert np.array_equal(yr, yf[:, ::-1])
    assert np.array_equal(Sr, Sf)


def pin_layer_palindrome_bidir(o):
    rng = np.random.default_rng(17)
    d = _layer_inputs(rng, B=1, T=31, H=2, S0=False)
    for key in ("q", "k", "v", "gate", "log_a", "beta"):
        half = d[key][:, :16]
        d[key] = np.ascontiguousarray(np.concatenate([half, half[:, :15][:, ::-1]], axis=1))
    y, sf, sr, _ = o.gdn_fwd_bidir(d["q"], d["k"], d["v"], d["log_a"], d["beta"], d["gate"],
                                   d["conv_q"], d["conv_k"], d["conv_v"], d["norm_w"], None)
    yf, _, _ = _run(o, d)
    np.testing.assert_allclose(y, yf + yf[:, ::-1], rtol=1e-14)
    np.testing.assert_allclose(sr, sf, rtol=1e-14)


def pin_layer_subset_threads_independence(o):
    rng = np.random.default_rng(18)
    d = _layer_inputs(rng, B=2, T=45, H=3)
    y, ST, _ = _run(o, d, threads=3)
    y1, ST1, _ = _run(o, d, threads=1)
    assert np.array_equal(y, y1) and np.array_equal(ST, ST1)
    ys, STs, _ = _run(o, d, heads=[2, 0])
    assert np.array_equal(ys[:, :, [2, 0]], y[:, :, [2, 0]])
    assert np.all(np.isnan(ys[:, :, 1]))
    # the final state never sees q or the gate
    e = dict(d)
    e["q"] = rng.standard_normal(d["q"].shape).astype(np.float32)
    e["gate"] = rng.standard_normal(d["gate"].shape).astype(np.float32)
    _, ST2, _ = _run(o, e)
    assert np.array_equal(ST2, ST)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]

"""Pins of the projection oracle (oracle/proj.py) against facts that do not
come from it, and planted mistakes that the pins must catch (CPU only).

What pins what:
  * the linear layer: a brute-force triple loop on tiny shapes; identity and
    scaled-identity weights; bias only;
  * the column routing of the stacked in-projection: a weight with a single
    non-zero row must light up exactly one (tensor, head, channel);
  * sigmoid: scipy's logistic function (a library routine), sigmoid(0) = 1/2,
    the symmetry s(z) + s(-z) = 1, no overflow at |z| = 800;
  * softplus: log1p(e^z) written out for moderate z, softplus(0) = ln 2,
    softplus(z) - softplus(-z) = z, the limits at z = +-800;
  * the decay: log a = -exp(A_h) ln 2 at z = 0, a in (0, 1], monotone in A_h;
  * the output projection: brute force, identity weight, bias only.
"""
from __future__ import annotations

import math
import types

import numpy as np
import pytest
from scipy.special import expit

import oracle.proj as proj_module


def _rng(seed=0):
    return np.random.default_rng(seed)


def _brute_linear(x, w, b):
    M, K = x.shape
    N = w.shape[0]
    out = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            s = 0.0
            for k in range(K):
                s += float(x[m, k]) * float(w[n, k])
            out[m, n] = s + (float(b[n]) if b is not None else 0.0)
    return out


# ---------------------------------------------------------------- the pins
def pin_linear_brute_force(P):
    r = _rng(1)
    x, w, b = r.normal(size=(5, 7)), r.normal(size=(3, 7)), r.normal(size=3)
    np.testing.assert_allclose(P.linear(x, w, b), _brute_linear(x, w, b), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(P.linear(x, w), _brute_linear(x, w, None), rtol=1e-13, atol=1e-13)


def pin_in_proj_identity(P):
    # C = H D; the q rows are I, the k rows 2 I, the v rows -I, the gate rows 3 I
    B, T, H, D = 2, 3, 2, 4
    C = H * D
    x = _rng(2).normal(size=(B, T, C))
    eye = np.eye(C)
    w = np.concatenate([eye, 2 * eye, -eye, 3 * eye, np.zeros((2 * H, C))])
    q, k, v, g, beta, log_a = P.in_proj(x, w, None, np.zeros(H), H, D)
    xs = x.reshape(B, T, H, D)
    np.testing.assert_array_equal(q, xs)
    np.testing.assert_array_equal(k, 2 * xs)
    np.testing.assert_array_equal(v, -xs)
    np.testing.assert_array_equal(g, 3 * xs)
    np.testing.assert_array_equal(beta, np.full((B, T, H), 0.5))
    np.testing.assert_allclose(log_a, np.full((B, T, H), -math.log(2.0)), rtol=1e-15)


def pin_in_proj_routing(P):
    B, T, H, D, C = 1, 2, 3, 4, 5
    HD = H * D
    N = 4 * HD + 2 * H
    x = np.ones((B, T, C))
    A = np.log(np.array([0.02, 0.05, 0.08]))
    for row in range(N):
        w = np.zeros((N, C))
        w[row, row % C] = 0.7
        q, k, v, g, beta, log_a = P.in_proj(x, w, None, A, H, D)
        parts = [q, k, v, g]
        for i, t in enumerate(parts):
            expect = np.zeros((B, T, H, D))
            if row < 4 * HD and row // HD == i:
                hh, cc = divmod(row % HD, D)
                expect[:, :, hh, cc] = 0.7
            np.testing.assert_array_equal(t, expect)
        eb = np.full((B, T, H), 0.5)
        ea = np.broadcast_to(-np.exp(A) * math.log(2.0), (B, T, H)).copy()
        if 4 * HD <= row < 4 * HD + H:
            eb[:, :, row - 4 * HD] = expit(0.7)
        if 4 * HD + H <= row:
            h = row - 4 * HD - H
            ea[:, :, h] = -np.exp(A[h]) * math.log1p(math.exp(0.7))
        np.testing.assert_allclose(beta, eb, rtol=1e-14)
        np.testing.assert_allclose(log_a, ea, rtol=1e-14)


def pin_in_proj_bias_only(P):
    B, T, H, D, C = 2, 2, 2, 2, 3
    N = 4 * H * D + 2 * H
    b = _rng(3).normal(size=N)
    A = np.array([-3.0, -2.0])
    q, k, v, g, beta, log_a = P.in_proj(np.zeros((B, T, C)), _rng(4).normal(size=(N, C)), b, A, H, D)
    HD = H * D
    for i, t in enumerate((q, k, v, g)):
        np.testing.assert_array_equal(t, np.broadcast_to(b[i * HD:(i + 1) * HD].reshape(H, D), t.shape))
    np.testing.assert_allclose(beta, np.broadcast_to(expit(b[4 * HD:4 * HD + H]), beta.shape), rtol=1e-14)
    za = b[4 * HD + H:]
    np.testing.assert_allclose(log_a, np.broadcast_to(-np.exp(A) * np.log1p(np.exp(za)), log_a.shape),
                               rtol=1e-14)


def pin_sigmoid(P):
    z = np.concatenate([np.linspace(-30, 30, 121), [-800.0, 800.0]])
    s = P.sigmoid(z)
    np.testing.assert_allclose(s, expit(z), rtol=1e-14, atol=0)
    assert P.sigmoid(np.array(0.0)) == 0.5
    np.testing.assert_allclose(s + P.sigmoid(-z), 1.0, rtol=1e-15)
    assert np.all(np.isfinite(s)) and np.all((s >= 0) & (s <= 1))


def pin_softplus(P):
    z = np.linspace(-30, 30, 121)
    np.testing.assert_allclose(P.softplus(z), np.log1p(np.exp(z)), rtol=1e-13)
    assert abs(P.softplus(np.array(0.0)) - math.log(2.0)) < 1e-16
    np.testing.assert_allclose(P.softplus(z) - P.softplus(-z), z, atol=1e-13)
    assert P.softplus(np.array(800.0)) == 800.0
    assert 0.0 <= P.softplus(np.array(-800.0)) < 1e-300


def pin_decay_range(P):
    B, T, H, D, C = 1, 50, 4, 2, 3
    N = 4 * H * D + 2 * H
    r = _rng(5)
    A = np.log(np.array([0.01, 0.03, 0.1, 1.0]))
    x = r.normal(scale=3.0, size=(B, T, C))
    w = r.normal(size=(N, C))
    *_, beta, log_a = P.in_proj(x, w, None, A, H, D)
    assert np.all(log_a <= 0) and np.all(np.exp(log_a) > 0) and np.all(np.exp(log_a) <= 1)
    assert np.all((beta > 0) & (beta < 1))
    # a larger rate decays more for the same input
    *_, _, log_a2 = P.in_proj(x, w, None, A + 0.5, H, D)
    assert np.all(log_a2 <= log_a)
    np.testing.assert_allclose(log_a2, log_a * math.exp(0.5), rtol=1e-14)


def pin_out_proj(P):
    B, T, H, D, C = 2, 3, 2, 3, 4
    r = _rng(6)
    y = r.normal(size=(B, T, H, D))
    w = r.normal(size=(C, H * D))
    b = r.normal(size=C)
    out = P.out_proj(y, w, b)
    np.testing.assert_allclose(out.reshape(B * T, C), _brute_linear(y.reshape(B * T, H * D), w, b),
                               rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(P.out_proj(y, np.eye(H * D)), y.reshape(B, T, H * D))
    np.testing.assert_array_equal(P.out_proj(np.zeros_like(y), w, b), np.broadcast_to(b, (B, T, C)))


PINS = [pin_linear_brute_force, pin_in_proj_identity, pin_in_proj_routing, pin_in_proj_bias_only,
        pin_sigmoid, pin_softplus, pin_decay_range, pin_out_proj]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_projection_oracle_pin(pin):
    pin(proj_module)


# ------------------------------------------------------------- the mutants
MUTANTS = {
    "weight reshaped, not transposed": ("z = x @ w.T", "z = x @ w.reshape(w.shape[::-1])"),
    "bias dropped": ("        z = z + np.asarray(b, np.float64)", "        z = z"),
    "sigmoid sign": ("1.0 / (1.0 + e), e / (1.0 + e)", "e / (1.0 + e), 1.0 / (1.0 + e)"),
    "softplus as exp": ("np.logaddexp(0.0, np.asarray(z, np.float64))", "np.exp(np.asarray(z, np.float64))"),
    "rate without exp": ("-np.exp(np.asarray(A_log, np.float64))", "-np.asarray(A_log, np.float64)"),
    "decay sign": ("log_a = -np.exp(", "log_a = np.exp("),
    "b and a columns swapped": ("z_b = z[:, 4 * HD:4 * HD + H]", "z_b = z[:, 4 * HD + H:4 * HD + 2 * H]"),
    "k and v blocks swapped": ("parts = [z[:, i * HD:(i + 1) * HD].reshape(B, T, H, D) for i in range(4)]",
                               "parts = [z[:, j * HD:(j + 1) * HD].reshape(B, T, H, D) for j in (0, 2, 1, 3)]"),
    "head-major channels": ("parts = [z[:, i * HD:(i + 1) * HD].reshape(B, T, H, D) for i in range(4)]",
                            "parts = [z[:, i * HD:(i + 1) * HD].reshape(B, T, D, H).swapaxes(2, 3) for i in range(4)]"),
    "out proj without bias": ("return linear(y.reshape(B * T, H * D), w_out, b_out)",
                              "return linear(y.reshape(B * T, H * D), w_out)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_projection_mutant_is_caught(name):
    src = open(proj_module.__file__).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"snippet for '{name}' must occur exactly once"
    mod = types.ModuleType(f"proj_mutant_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    failed = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod)
        except Exception:  # an assertion or a crash both count as caught
            failed.append(pin.__name__)
    assert failed, f"mutant '{name}' passed every pin"


def test_mixer_oracle_composition():
    """The mixer oracle hands the projections' outputs to the layer oracle and
    the layer's output to the output projection: with an identity output
    weight (C = H D) and no output bias its output is the layer's y; with
    b = sigmoid(-800) = 0 (no writes) the final state is S0 decayed by
    exp(sum log a) (the closed form of the delta rule without updates)."""
    import gdn_inputs
    import oracle
    H, D = 2, 8
    w = gdn_inputs.MixerWorkload(99, "tiny", 1, 23, H, D, H * D)
    inp = gdn_inputs.generate_mixer(w, seed=3)
    C = H * D
    N = 4 * C + 2 * H
    inp["b_in"][4 * C:4 * C + H] = -800.0
    inp["w_in"][4 * C:4 * C + H] = 0.0
    S0 = np.random.default_rng(1).normal(size=(1, H, D, D))
    out, S_T, y = proj_module.mixer(inp["x"], inp["w_in"], inp["b_in"], inp["A_log"], inp["conv_q"],
                                    inp["conv_k"], inp["conv_v"], inp["norm_w"], np.eye(C), None, H, D, S0=S0)
    assert out.shape == (1, 23, C) and N == inp["w_in"].shape[0]
    np.testing.assert_array_equal(out, y.reshape(1, 23, C))
    q, k, v, g, beta, log_a = proj_module.in_proj(inp["x"], inp["w_in"], inp["b_in"], inp["A_log"], H, D)
    y2, _, _ = oracle.gdn_fwd(q, k, v, log_a, beta, g, inp["conv_q"], inp["conv_k"], inp["conv_v"],
                              inp["norm_w"], S0)
    np.testing.assert_array_equal(y, y2)
    decay = np.exp(np.sum(log_a.astype(np.float32).astype(np.float64)[0], axis=0))  # [H]
    np.testing.assert_allclose(S_T[0], decay[:, None, None] * S0.astype(np.float32)[0], rtol=1e-6)

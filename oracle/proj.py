"""fp64 CPU oracle of the token mixer's projections.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no
code with the HIP library and never imports it.

What it computes.  The GDN token mixer takes its per-token inputs from the
hidden states through linear projections and returns its output through one:
the LinMorph project page ("Why learn the initialization?") builds the GDN
parameters from the pretrained query, key, value and output projections, and
names the GDN-specific groups (update gates, decay terms) that have no
softmax counterpart; the T3-Video page's Table 1 counts the "QKV proj." and
"O proj." MACs of Wan2.1-T2V-1.3B.  Neither page prints formulas, so this
module takes the plain reading:

* a projection is a linear layer, ``z = x W^T + b`` (the weight stored as
  [out_features, in_features]); numpy's fp64 matrix product is the step;
* the in-projection stacks six such layers, for q, k, v, the output gate,
  the update-gate logit and the decay input;
* the update gate is ``b = sigmoid(z_b)``, in (0, 1);
* the decay is ``log a = -exp(A_h) * softplus(z_a)`` with a per-head rate
  A_h, so ``a = exp(log a)`` lies in (0, 1]; ``softplus(z) = log(1 + e^z)``.
"""
from __future__ import annotations

import numpy as np


def linear(x, w, b=None):
    """z = x W^T + b in fp64.  x [..., K], w [N, K], b [N] or None."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    z = x @ w.T
    if b is not None:
        z = z + np.asarray(b, np.float64)
    return z


def sigmoid(z):
    """1 / (1 + e^-z), evaluated without overflow on either side."""
    z = np.asarray(z, np.float64)
    e = np.exp(-np.abs(z))
    return np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def softplus(z):
    """log(1 + e^z) (numpy's log-add-exp of 0 and z)."""
    return np.logaddexp(0.0, np.asarray(z, np.float64))


def in_proj(x, w_in, b_in, A_log, H, D):
    """The layer's per-token inputs from the hidden states.

    x [B, T, C]; w_in [4 H D + 2 H, C] with rows q (H D), k (H D), v (H D),
    gate (H D), b logit (H), decay input (H); b_in [4 H D + 2 H] or None;
    A_log [H].  Returns fp64 (q, k, v, gate) [B, T, H, D] and (beta, log_a)
    [B, T, H].
    """
    x = np.asarray(x, np.float64)
    B, T, C = x.shape
    HD = H * D
    z = linear(x.reshape(B * T, C), w_in, b_in)
    assert z.shape[1] == 4 * HD + 2 * H
    parts = [z[:, i * HD:(i + 1) * HD].reshape(B, T, H, D) for i in range(4)]
    z_b = z[:, 4 * HD:4 * HD + H].reshape(B, T, H)
    z_a = z[:, 4 * HD + H:4 * HD + 2 * H].reshape(B, T, H)
    beta = sigmoid(z_b)
    log_a = -np.exp(np.asarray(A_log, np.float64)) * softplus(z_a)
    return parts[0], parts[1], parts[2], parts[3], beta, log_a


def out_proj(y, w_out, b_out=None):
    """out [B, T, C] = y [B, T, H, D] (as [B T, H D]) W_out^T + b_out."""
    y = np.asarray(y, np.float64)
    B, T, H, D = y.shape
    return linear(y.reshape(B * T, H * D), w_out, b_out).reshape(B, T, -1)


def mixer(x, w_in, b_in, A_log, conv_q, conv_k, conv_v, norm_w, w_out, b_out, H, D, S0=None,
          eps_l2=1e-6, eps_norm=1e-6, threads=0):
    """The whole token mixer: in_proj, the GDN layer (the C oracle, forward
    scan), out_proj.  The layer oracle takes its inputs as float32 (it is
    built for the exact values a device receives), so the projection outputs
    are rounded to float32 at that boundary, a relative change of at most
    2^-24.  Returns (out [B, T, C], S_T [B, H, D, D], y [B, T, H, D]), fp64."""
    from oracle import gdn_fwd
    q, k, v, g, beta, log_a = in_proj(x, w_in, b_in, A_log, H, D)
    y, S_T, _ = gdn_fwd(q, k, v, log_a, beta, g, conv_q, conv_k, conv_v, norm_w, S0, eps_l2, eps_norm,
                        threads=threads)
    return out_proj(y, w_out, b_out), S_T, y

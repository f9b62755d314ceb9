"""fp64 CPU oracle of the GDN layer's backward pass: the gradients of the
layer forward with respect to every input.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no
code with the HIP library and never imports it.

What it computes.  The pages train the GDN modules that replace softmax
attention (LinMorph project page, "Abstract": progressive distillation and
joint recovery of the converted blocks), which needs the gradient of the
layer.  The gradient is the derivative of the forward's definition, so this
module writes the forward out once more, token by token, in torch fp64 (the
same steps as the C oracle in ``gdn_oracle.c``: causal depthwise 4-tap
convolution and SiLU on q, k, v; L2 normalisation of q and k; the gated delta
rule S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T with o_t = S_t q_t;
the gated RMS normalisation y_t = o_t / sqrt(mean(o_t^2) + eps) * w *
SiLU(gate_t)), and takes torch.autograd's gradient of the scalar

    L = <dy, y> + <dS_T, S_T>

with respect to q, k, v, log a, b, gate, the three conv weights, the norm
weight and S0.  Autograd is the library step here: it differentiates exactly
the operations written below, up to fp64 rounding.  The forward is pinned to
the C oracle, and the gradients to central finite differences and to the
closed form of the b = 0 case (tests/test_bwd_oracle.py).  Tap j of a conv
weight multiplies x_{t-3+j}; positions before the sequence start are zeros.
The loop over tokens makes this oracle slow: it is meant for short sequences.
"""
from __future__ import annotations

import numpy as np
import torch

NAMES = ("q", "k", "v", "log_a", "beta", "gate", "conv_q", "conv_k", "conv_v", "norm_w", "S0")


def conv_silu(x, w):
    """SiLU of the causal depthwise 4-tap convolution.  x [B, T, H, D],
    w [H*D, 4] (tap 3 on the current token)."""
    B, T, H, D = x.shape
    wv = w.reshape(H, D, 4)
    xp = torch.cat([x.new_zeros(B, 3, H, D), x], dim=1)
    z = sum(wv[:, :, j] * xp[:, j:j + T] for j in range(4))
    return z * torch.sigmoid(z)


def l2_normalize(x, eps):
    return x / torch.sqrt((x * x).sum(-1, keepdim=True) + eps)


def forward(q, k, v, log_a, beta, gate, conv_q, conv_k, conv_v, norm_w=None, S0=None,
            eps_l2=1e-6, eps_norm=1e-6):
    """The layer forward in torch fp64.  Shapes as for the C oracle: q, k
    [B, T, H, Dk]; v, gate [B, T, H, Dv]; log_a, beta [B, T, H]; conv_*
    [H*D, 4]; norm_w [H, Dv] or None; S0 [B, H, Dv, Dk] or None.
    Returns (y [B, T, H, Dv], S_T [B, H, Dv, Dk])."""
    qh = l2_normalize(conv_silu(q, conv_q), eps_l2)
    kh = l2_normalize(conv_silu(k, conv_k), eps_l2)
    vh = conv_silu(v, conv_v)
    B, T, H, Dk = qh.shape
    Dv = vh.shape[3]
    S = S0 if S0 is not None else qh.new_zeros(B, H, Dv, Dk)
    a = torch.exp(log_a)
    outs = []
    for t in range(T):
        kt = kh[:, t].unsqueeze(-1)                  # [B, H, Dk, 1]
        at = a[:, t, :, None, None]
        bt = beta[:, t, :, None, None]
        Sk = S @ kt                                   # [B, H, Dv, 1]
        S = at * S - (at * bt) * (Sk @ kt.transpose(-1, -2)) \
            + bt * (vh[:, t].unsqueeze(-1) @ kt.transpose(-1, -2))
        outs.append((S @ qh[:, t].unsqueeze(-1)).squeeze(-1))   # [B, H, Dv]
    o = torch.stack(outs, dim=1)                      # [B, T, H, Dv]
    r = 1.0 / torch.sqrt((o * o).mean(-1, keepdim=True) + eps_norm)
    y = o * r * torch.sigmoid(gate) * gate
    if norm_w is not None:
        y = y * norm_w
    return y, S


def _t(a):
    return None if a is None else torch.tensor(np.asarray(a, np.float64), dtype=torch.float64)


def backward(inp: dict, dy, dS_T=None, eps_l2=1e-6, eps_norm=1e-6):
    """Gradients of L = <dy, y> + <dS_T, S_T> (dS_T None: zero).  inp holds
    the forward's inputs under NAMES (norm_w and S0 may be None).  Returns
    (y, S_T, grads) as fp64 numpy arrays, grads keyed by NAMES (None for an
    input that is None)."""
    leaves = {n: _t(inp.get(n)) for n in NAMES}
    for t in leaves.values():
        if t is not None:
            t.requires_grad_(True)
    y, S_T = forward(*[leaves[n] for n in NAMES], eps_l2=eps_l2, eps_norm=eps_norm)
    L = (y * _t(dy)).sum()
    if dS_T is not None:
        L = L + (S_T * _t(dS_T)).sum()
    live = [n for n in NAMES if leaves[n] is not None]
    grads = torch.autograd.grad(L, [leaves[n] for n in live], allow_unused=True)
    out = {n: None for n in NAMES}
    for n, g in zip(live, grads):
        out[n] = np.zeros(leaves[n].shape) if g is None else g.detach().numpy()
    return y.detach().numpy(), S_T.detach().numpy(), out


def loss(inp: dict, dy, dS_T=None, eps_l2=1e-6, eps_norm=1e-6) -> float:
    """The scalar L = <dy, y> + <dS_T, S_T> of the forward (no gradients)."""
    with torch.no_grad():
        y, S_T = forward(*[_t(inp.get(n)) for n in NAMES], eps_l2=eps_l2, eps_norm=eps_norm)
        L = (y * _t(dy)).sum()
        if dS_T is not None:
            L = L + (S_T * _t(dS_T)).sum()
    return float(L)

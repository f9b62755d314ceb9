"""fp64 model of the chunked (WY) form of the gated delta rule.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  This model exists to
pin the token-by-token oracle by brute force: for any chunk length C the
chunked form must reproduce the sequential recurrence up to fp64 rounding, so
a wrong sign, index or transpose in either one shows up as a disagreement.

Algebra (own derivation; the pages print no GDN equations).  Inside one chunk
with entry state S0 (Dv x Dk), local tokens r = 0..n-1, g_r = sum_{i<=r}
log a_i and gamma_r = exp(g_r):
  * write the step as S_r = a_r S_{r-1} + u_r k_r^T with the pseudo-value
    u_r = b_r (v_r - a_r S_{r-1} k_r);
  * unrolling gives S_r = gamma_r S0 + sum_{j<=r} exp(g_r - g_j) u_j k_j^T;
  * substituting back: (I + A) U = diag(b) V - diag(b * gamma) K S0^T with
    A_ij = b_i exp(g_i - g_j) k_i.k_j for i > j (strictly lower);
  * so U = Tinv diag(b) V - Tinv diag(b * gamma) K S0^T, Tinv = (I + A)^-1;
  * o_r = S_r q_r = gamma_r S0 q_r + sum_{j<=r} exp(g_r - g_j) (q_r.k_j) u_j;
  * the exit state is S_n = gamma_n S0 + U^T diag(exp(g_n - g)) K.
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular


def chunked_delta_rule(q, k, v, log_a, beta, S0=None, C=64):
    """Same contract as ``oracle.delta_rule`` (one head), computed chunk by
    chunk with the WY form above.  Returns (o [T, Dv], S_T [Dv, Dk])."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    la = np.asarray(log_a, np.float64).reshape(-1)
    be = np.asarray(beta, np.float64).reshape(-1)
    T, Dk = k.shape
    Dv = v.shape[1]
    S = np.zeros((Dv, Dk)) if S0 is None else np.array(S0, np.float64, copy=True)
    o = np.empty((T, Dv))
    for start in range(0, T, C):
        stop = min(start + C, T)
        n = stop - start
        Q, K, V, b = q[start:stop], k[start:stop], v[start:stop], be[start:stop]
        g = np.cumsum(la[start:stop])
        gam = np.exp(g)
        r_idx = np.arange(n)[:, None]
        j_idx = np.arange(n)[None, :]
        # exp(g_r - g_j) where j <= r, 0 elsewhere (never exponentiate j > r)
        diff = np.where(j_idx <= r_idx, g[:, None] - g[None, :], -np.inf)
        decay = np.exp(diff)
        A = np.where(j_idx < r_idx, b[:, None] * decay * (K @ K.T), 0.0)
        Tinv = solve_triangular(np.eye(n) + A, np.eye(n), lower=True, unit_diagonal=True)
        W = Tinv @ ((b * gam)[:, None] * K)
        U_tilde = Tinv @ (b[:, None] * V)
        U = U_tilde - W @ S.T
        P = decay * (Q @ K.T)
        o[start:stop] = gam[:, None] * (Q @ S.T) + P @ U
        S = gam[-1] * S + U.T @ (np.exp(g[-1] - g)[:, None] * K)
    return o, S

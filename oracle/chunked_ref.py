"""fp64 chunked (WY / UT-transform) form of the gated delta rule.

TEST INFRASTRUCTURE ONLY.  A second, independent fp64 formulation of the same
recurrence, used to pin the token-by-token oracle: both must agree to rounding.
It works on one (sequence, value head) with already normalised q, k and
post-conv v; it does no conv, no normalisation and no output gate.

Derivation (no page prints it; it follows from the delta rule in the hyper.ai
story on Qwen3-Next and the chunk size 64 given as FLA_CHUNK_SIZE in the SGLang
cookbook's Mamba Radix Cache tip).  Inside a chunk, with S the state on entry,
write u_t = b_t (v_t - a_t S_{t-1} k_t), so S_t = a_t S_{t-1} + u_t k_t^T.
With G the inclusive cumulative sum of g inside the chunk and
Gamma[t, i] = exp(G_t - G_i) for i <= t:
    S_t = exp(G_t) S + sum_{i<=t} Gamma[t, i] u_i k_i^T
    u_t + b_t sum_{i<t} Gamma[t, i] (k_t . k_i) u_i = b_t v_t - b_t exp(G_t) S k_t
so with A = strictly_lower(diag(b) (K K^T * Gamma)) and T = (I + A)^-1:
    U = T diag(b) V - T diag(b exp(G)) K S^T
    O = diag(exp(G)) Q S^T + lower_incl_diag(Q K^T * Gamma) U
    S <- exp(G_n) S + U^T diag(exp(G_n - G)) K
"""
from __future__ import annotations

import numpy as np


def chunked_head(q, k, v, g, beta, S0=None, chunk=64):
    """q, k: [T, dk]; v: [T, dv]; g, beta: [T]; S0: [dv, dk].  fp64.

    Returns (o [T, dv], S_final [dv, dk]).
    """
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    g, beta = np.asarray(g, np.float64), np.asarray(beta, np.float64)
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dv, dk)) if S0 is None else np.array(S0, np.float64)
    o = np.zeros((T, dv))
    for s in range(0, T, chunk):
        e = min(T, s + chunk)
        Q, Kc, V, b = q[s:e], k[s:e], v[s:e], beta[s:e]
        G = np.cumsum(g[s:e])
        n = e - s
        diff = G[:, None] - G[None, :]
        mask_incl = np.tril(np.ones((n, n), dtype=bool))
        Gam = np.where(mask_incl, np.exp(np.where(mask_incl, diff, 0.0)), 0.0)
        A = np.tril(b[:, None] * (Kc @ Kc.T) * Gam, -1)
        Tm = np.linalg.solve(np.eye(n) + A, np.eye(n))
        W = Tm @ ((b * np.exp(G))[:, None] * Kc)
        Ut = Tm @ (b[:, None] * V)
        U = Ut - W @ S.T
        P = (Q @ Kc.T) * Gam
        o[s:e] = np.exp(G)[:, None] * (Q @ S.T) + P @ U
        S = np.exp(G[-1]) * S + U.T @ (np.exp(G[-1] - G)[:, None] * Kc)
    return o, S


def chunk_affine_map(k, v, g, beta):
    """Affine map of one chunk: S_out = S_in @ M + B (fp64)."""
    k, v = np.asarray(k, np.float64), np.asarray(v, np.float64)
    g, b = np.asarray(g, np.float64), np.asarray(beta, np.float64)
    n, dk = k.shape
    G = np.cumsum(g)
    diff = G[:, None] - G[None, :]
    mask_incl = np.tril(np.ones((n, n), dtype=bool))
    Gam = np.where(mask_incl, np.exp(np.where(mask_incl, diff, 0.0)), 0.0)
    A = np.tril(b[:, None] * (k @ k.T) * Gam, -1)
    Tm = np.linalg.solve(np.eye(n) + A, np.eye(n))
    W = Tm @ ((b * np.exp(G))[:, None] * k)
    Ut = Tm @ (b[:, None] * v)
    dec = np.exp(G[-1] - G)[:, None] * k
    M = np.exp(G[-1]) * np.eye(dk) - W.T @ dec
    B = Ut.T @ dec
    return M, B

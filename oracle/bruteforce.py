"""Whole-sequence materialised form of the gated delta rule (numpy + scipy).

TEST INFRASTRUCTURE ONLY (an independent cross-check of the C oracle).

Unrolling the token recurrence of "Optimization: Qwen3 next autoregressive
pass (#17996)" (build_delta_net_autoregressive) over a whole sequence of T
tokens gives, with G_t = sum_{s<=t} g_s, Gamma[t][s] = exp(G_t - G_s) (s <= t),
A = strict_lower(diag(beta) (K K^T) * Gamma):

    (I + A) U = diag(beta) (V - diag(exp(G)) K S0)        (U: the deltas)
    O   = diag(exp(G)) Q S0 + (Q K^T * Gamma_incl) U
    S_T = exp(G_T) S0 + K^T diag(exp(G_T - G)) U

(q, k normalised, q scaled), i.e. the chunked form of the pages' chunked graph
with a single chunk spanning the whole sequence.  The unit-lower triangular
system is solved with scipy.linalg.solve_triangular, a textbook routine.
Cost O(T^2 d + T^3): use for T <= a few hundred.
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular


def _norm(x, eps, factor=1.0):
    x = np.asarray(x, np.float64)
    return x * (factor / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps))


def materialised_head(q, k, v, g, beta, s0, scale, eps):
    """One (sequence, value head): q, k [T, d_k], v [T, d_v], g, beta [T]."""
    Q = _norm(q, eps, scale)
    K = _norm(k, eps)
    V = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    b = np.asarray(beta, np.float64)
    S0 = np.asarray(s0, np.float64)
    T = Q.shape[0]
    G = np.cumsum(g)
    diff = G[:, None] - G[None, :]
    incl = np.tril(np.ones((T, T), bool))
    Gam = np.where(incl, np.exp(np.where(incl, diff, 0.0)), 0.0)
    A = np.tril(b[:, None] * (K @ K.T) * Gam, -1)
    rhs = b[:, None] * (V - np.exp(G)[:, None] * (K @ S0))
    U = solve_triangular(np.eye(T) + A, rhs, lower=True, unit_diagonal=True)
    O = np.exp(G)[:, None] * (Q @ S0) + ((Q @ K.T) * Gam) @ U
    ST = np.exp(G[-1]) * S0 + K.T @ (np.exp(G[-1] - G)[:, None] * U)
    return O, ST


def materialised(q, k, v, g, beta, cu_seqlens, s0=None, scale=None, eps=1e-6):
    """Packed varlen batch (same layout as the C oracle); returns (out, s_final)."""
    T, H_k, d_k = q.shape
    H_v, d_v = v.shape[1], v.shape[2]
    r = H_v // H_k
    if scale is None:
        scale = 1.0 / np.sqrt(d_k)
    N = len(cu_seqlens) - 1
    out = np.zeros((T, H_v, d_v))
    sf = np.zeros((N, H_v, d_k, d_v))
    for s in range(N):
        a, e = int(cu_seqlens[s]), int(cu_seqlens[s + 1])
        for h in range(H_v):
            S0 = np.zeros((d_k, d_v)) if s0 is None else s0[s, h]
            if e == a:
                sf[s, h] = S0
                continue
            hk = h // r
            O, ST = materialised_head(q[a:e, hk], k[a:e, hk], v[a:e, h],
                                      g[a:e, h], beta[a:e, h], S0, scale, eps)
            out[a:e, h] = O
            sf[s, h] = ST
    return out, sf

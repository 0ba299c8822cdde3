"""The chunked (UT/WY) form of the KDA recurrence, in fp64 NumPy.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).  It is a second, different
algorithm for the same result as the token loop in kda_oracle.c: the prefill
"builds the cumulative gate and calls chunk_kda_fwd" (page "[Feature][KDA]
Add Kimi K3 KDA execution", KDA execution step 3), i.e. it works a chunk of C
tokens at a time.  Agreement of the two, at every chunk size on tiny inputs,
pins the token loop and checks the chunk algebra the GPU kernels use.

Derivation (own; exact up to rounding).  In one chunk, positions r = 1..n,
G_r = sum_{s<=r} g_s per key channel (inclusive cumulative gate).  Unrolling
S_r = Diag(e^{g_r}) S_{r-1} + k_r d_r^T with d_r = beta_r (v_r - (Diag(e^{g_r})
S_{r-1})^T k_r) gives, with

  Kt_r = e^{G_r} * k_r,  Qt_r = e^{G_r} * q_r,  Kh_s = e^{-G_s} * k_s,
  Kb_s = e^{G_n - G_s} * k_s,
  M    = strict_lower(Diag(beta) Kt Kh^T),
  T    = (I + M)^{-1} Diag(beta),   W = T Kt,   U_v = T V,

the chunk's rank-one writes  D = U_v - W S_0,
its outputs                  O = scale (Qt S_0 + incl_lower(Qt Kh^T) D),
and the state at its end     S_n = Diag(e^{G_n}) S_0 + Kb^T D.

The triangular solve uses scipy's solve_triangular (a library step).
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular


def chunk_prefill_head(q, k, v, g, beta, S0, chunk: int, scale: float = 1.0):
    """One (sequence, head): q,k,g [L,dk]; v [L,dv]; beta [L]; S0 [dk,dv].
    Returns (o [L,dv], S_L [dk,dv])."""
    q, k, v, g = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g))
    beta = np.asarray(beta, dtype=np.float64)
    S = np.array(S0, dtype=np.float64, copy=True)
    L = q.shape[0]
    o = np.zeros((L, v.shape[1]))
    for c0 in range(0, L, chunk):
        c1 = min(c0 + chunk, L)
        qc, kc, vc, gc, bc = q[c0:c1], k[c0:c1], v[c0:c1], g[c0:c1], beta[c0:c1]
        n = c1 - c0
        G = np.cumsum(gc, axis=0)
        Kt = np.exp(G) * kc
        Qt = np.exp(G) * qc
        Kh = np.exp(-G) * kc
        Kb = np.exp(G[-1] - G) * kc
        M = np.tril(bc[:, None] * (Kt @ Kh.T), -1)
        T = solve_triangular(np.eye(n) + M, np.diag(bc), lower=True, unit_diagonal=True)
        W = T @ Kt
        Uv = T @ vc
        D = Uv - W @ S
        P = np.tril(Qt @ Kh.T)
        o[c0:c1] = scale * (Qt @ S + P @ D)
        S = np.exp(G[-1])[:, None] * S + Kb.T @ D
    return o, S


def chunk_prefill(q, k, v, g, beta, cu_seqlens, pool, slots, has_init=None,
                  chunk: int = 64, scale: float = 1.0):
    """Varlen wrapper with the same pool semantics as the token-loop oracle
    (slot < 0 = padding: zero output, no state I/O; empty sequence = no-op).
    Returns (o, new pool)."""
    q, k, v, g, beta = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, beta))
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    slots = np.asarray(slots, dtype=np.int64)
    pool = np.array(pool, dtype=np.float64, copy=True)
    T, H, _ = q.shape
    o = np.zeros((T, H, v.shape[2]))
    for i in range(len(slots)):
        t0, t1 = int(cu[i]), int(cu[i + 1])
        if slots[i] < 0 or t1 == t0:
            continue
        for h in range(H):
            S0 = pool[slots[i], h] if (has_init is None or has_init[i]) else np.zeros(pool.shape[2:])
            oo, S = chunk_prefill_head(q[t0:t1, h], k[t0:t1, h], v[t0:t1, h], g[t0:t1, h],
                                       beta[t0:t1, h], S0, chunk, scale)
            o[t0:t1, h] = oo
            pool[slots[i], h] = S
    return o, pool

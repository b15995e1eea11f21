"""Chunked (WY / UT-transform) form of the gated delta rule in float64 numpy.

Test-side only.  It restates the chunk algebra that the GPU prefill follows,
independently of both the oracle and the HIP code, so that the tests can show
that the chunked form reaches the sequential recurrence (up to rounding) for
any chunk size, including a ragged last chunk.

For one value head and a chunk with entry state S0 (d_v x d_k), rows t, s of
the chunk, G_t = sum_{r<=t} g_r, gamma_t = exp(G_t), D_ts = exp(G_t - G_s):

* u_t + beta_t sum_{s<t} D_ts (k_t . k_s) u_s = beta_t (v_t - gamma_t S0 k_t),
  i.e. (I + A) U = R with A = strict_lower(diag(beta) (D * K K^T)) and
  R = diag(beta) (V - diag(gamma) K S0^T);  U = (I + A)^{-1} R;
* O = diag(gamma) Q S0^T + (tril(D) * Q K^T) U;
* S_end = gamma_last S0 + U^T diag(D_last,.) K.
"""
from __future__ import annotations

import numpy as np


def chunked_recurrence(q, k, v, g, beta, z, S0, C: int):
    """Same contract as ``oracle.recurrence`` (float64 in and out)."""
    q, k, v, g, beta, z = (np.asarray(a, np.float64) for a in (q, k, v, g, beta, z))
    B, T, H_k, d_k = q.shape
    H_v, d_v = v.shape[2], v.shape[3]
    G_ = H_v // H_k
    S_all = np.array(S0, np.float64, copy=True)
    O_all = np.zeros((B, T, H_v, d_v))
    for b in range(B):
        for h in range(H_v):
            kh = h // G_
            S = S_all[b, h]
            for c0 in range(0, T, C):
                c1 = min(T, c0 + C)
                K = k[b, c0:c1, kh]
                Q = q[b, c0:c1, kh]
                V = v[b, c0:c1, h]
                bt = beta[b, c0:c1, h]
                G = np.cumsum(g[b, c0:c1, h])
                gam = np.exp(G)
                n = c1 - c0
                lower = np.tril(np.ones((n, n), bool))
                D = np.where(lower, np.exp(np.where(lower, G[:, None] - G[None, :], 0.0)), 0.0)
                A = np.tril(bt[:, None] * D * (K @ K.T), -1)
                R = bt[:, None] * (V - gam[:, None] * (K @ S.T))
                U = np.linalg.solve(np.eye(n) + A, R)
                O_all[b, c0:c1, h] = gam[:, None] * (Q @ S.T) + (D * (Q @ K.T)) @ U
                S = gam[-1] * S + U.T @ (np.exp(G[-1] - G)[:, None] * K)
            S_all[b, h] = S
    y = O_all / (1.0 + np.exp(-z))
    return y, S_all, O_all

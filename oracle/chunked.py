"""Chunk-by-chunk restatement of the KDA recurrence (numpy, fp64).

TEST INFRASTRUCTURE ONLY.  This is the second oracle path: it regroups the
state update of the Chimera paper's method step (5),
    S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
    o_t = S_t^T q_t,
into chunks of C tokens.  Inside a chunk, with G_r = sum_{u<=r} log alpha_u
(per key channel) and the exact pairwise decay D_rs = exp(G_r - G_s):

    A_rs = sum_c k_r[c] k_s[c] D_rs[c]            (s <  r)
    B_rs = sum_c q_r[c] k_s[c] D_rs[c]            (s <= r)
    Tm   = (I + Diag(beta) A)^-1
    W    = Tm Diag(beta) (exp(G) * K)
    U    = Tm Diag(beta) V - W S
    O    = (exp(G) * Q) S + B U
    S   <- Diag(exp(G_last)) S + (exp(G_last - G) * K)^T U

It is used only to show that this regrouping equals the recurrence (for any
chunk size, ragged tails included); the HIP kernels implement the same
regrouping with their own factorisation of the decays.
"""
from __future__ import annotations

import numpy as np
import scipy.linalg


def kda_chunked(q, k, v, alpha, beta, S0=None, C: int = 64):
    q, k, v, alpha, beta = (np.asarray(a, dtype=np.float64) for a in (q, k, v, alpha, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    ST = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else np.array(S0[b, h], dtype=np.float64)
            for n0 in range(0, T, C):
                sl = slice(n0, min(T, n0 + C))
                Q, K, V = q[b, sl, h], k[b, sl, h], v[b, sl, h]
                be = beta[b, sl, h]
                n = Q.shape[0]
                G = np.cumsum(np.log(alpha[b, sl, h]), axis=0)           # [n, dk]
                diff = G[:, None, :] - G[None, :, :]                     # [r, s, c]
                lower_incl = np.tril(np.ones((n, n), dtype=bool))
                D = np.where(lower_incl[:, :, None], np.exp(np.minimum(diff, 0.0)), 0.0)
                A = np.einsum("rc,sc,rsc->rs", K, K, D) * np.tril(np.ones((n, n)), -1)
                Bm = np.einsum("rc,sc,rsc->rs", Q, K, D)
                L = np.eye(n) + be[:, None] * A
                rhs = np.concatenate([be[:, None] * np.exp(G) * K, be[:, None] * V], axis=1)
                X = scipy.linalg.solve_triangular(L, rhs, lower=True, unit_diagonal=True)
                W, Ut = X[:, :dk], X[:, dk:]
                U = Ut - W @ S
                o[b, sl, h] = (np.exp(G) * Q) @ S + Bm @ U
                S = np.exp(G[-1])[:, None] * S + (np.exp(G[-1][None, :] - G) * K).T @ U
            ST[b, h] = S
    return o, ST

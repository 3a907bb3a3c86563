"""fp64 gradients of the conv + KDA token mixer (numpy).

TEST INFRASTRUCTURE ONLY, under the rules of the rest of ``oracle/``: only
``tests/``, ``__graft_entry__.smoke()`` and bench.py's CPU-baseline leg may
import it, and it shares no code with the HIP path.

``kda_recurrence_backward`` is the reverse-mode adjoint of the recurrence of
the Chimera paper's method step (5), written out token by token, in the
order of the forward steps
    S' = Diag(alpha_t) S_{t-1};  r = S'^T k_t;  u = beta_t (v_t - r);
    S_t = S' + k_t u^T;  o_t = S_t^T q_t
taken backwards for a loss L with dL/do = dO and dL/dS_T = dS_T.  The forward
states it needs are recomputed from checkpoints every ``ckpt`` tokens.

``short_conv_backward`` is the adjoint of the modality-aware depthwise conv:
each output is a sum of tap * input terms, so each input receives tap * dy of
every output it feeds, and each tap the sum of input * dy over the outputs.

``kda_chunked_backward`` restates the same gradients chunk by chunk (the
algebra the GPU backward implements); it exists only to be checked against the
token-level adjoint, never to produce expected values.
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def _f64(a) -> np.ndarray:
    if hasattr(a, "detach"):
        a = a.detach().cpu().double().numpy()
    return np.array(a, dtype=np.float64)


def kda_recurrence_backward(q, k, v, alpha, beta, dO, S0=None, dST=None, ckpt: int = 64):
    """Gradients of L = sum(dO * o) + sum(dST * S_T) through the KDA recurrence.

    q, k, alpha [B,T,H,dk]; v, dO [B,T,H,dv]; beta [B,T,H]; S0, dST [B,H,dk,dv] or None.
    Returns dict dq, dk, dv, dalpha, dbeta, dS0 (fp64, the input shapes).
    """
    q, k, v, alpha, beta, dO = (_f64(a) for a in (q, k, v, alpha, beta, dO))
    B, T, H, dkk = q.shape
    dvv = v.shape[-1]
    out = {"dq": np.zeros_like(q), "dk": np.zeros_like(k), "dv": np.zeros_like(v),
           "dalpha": np.zeros_like(alpha), "dbeta": np.zeros_like(beta), "dS0": np.zeros((B, H, dkk, dvv))}
    for b in range(B):
        for h in range(H):
            S = np.zeros((dkk, dvv)) if S0 is None else _f64(S0)[b, h].copy()
            # forward: states at the start of every checkpoint segment
            starts = list(range(0, T, ckpt))
            cp = {}
            for t in range(T):
                if t in starts:
                    cp[t] = S.copy()
                Sp = alpha[b, t, h][:, None] * S
                u = beta[b, t, h] * (v[b, t, h] - Sp.T @ k[b, t, h])
                S = Sp + np.outer(k[b, t, h], u)
            dS = np.zeros((dkk, dvv)) if dST is None else _f64(dST)[b, h].copy()
            for s0 in reversed(starts):
                s1 = min(T, s0 + ckpt)
                # recompute S_{t-1} for t in the segment
                prev = [cp[s0]]
                for t in range(s0, s1 - 1):
                    Sp = alpha[b, t, h][:, None] * prev[-1]
                    u = beta[b, t, h] * (v[b, t, h] - Sp.T @ k[b, t, h])
                    prev.append(Sp + np.outer(k[b, t, h], u))
                for t in range(s1 - 1, s0 - 1, -1):
                    Sm = prev[t - s0]                       # S_{t-1}
                    a_t, k_t, v_t, q_t, be = alpha[b, t, h], k[b, t, h], v[b, t, h], q[b, t, h], beta[b, t, h]
                    Sp = a_t[:, None] * Sm
                    r = Sp.T @ k_t
                    u = be * (v_t - r)
                    St = Sp + np.outer(k_t, u)
                    # o_t = S_t^T q_t
                    dS = dS + np.outer(q_t, dO[b, t, h])
                    out["dq"][b, t, h] = St @ dO[b, t, h]
                    # S_t = S' + k u^T
                    dSp = dS.copy()
                    dk_t = dS @ u
                    du = dS.T @ k_t
                    # u = beta (v - r), r = S'^T k
                    out["dbeta"][b, t, h] = du @ (v_t - r)
                    out["dv"][b, t, h] = be * du
                    dr = -be * du
                    dSp += np.outer(k_t, dr)
                    dk_t = dk_t + Sp @ dr
                    out["dk"][b, t, h] = dk_t
                    # S' = Diag(alpha) S_{t-1}
                    out["dalpha"][b, t, h] = np.sum(dSp * Sm, axis=1)
                    dS = a_t[:, None] * dSp
            out["dS0"][b, h] = dS
    return out


def _vis_taps(causal_t: int):
    P = 2 if causal_t else 1
    for a in range(3):
        for bb in range(3):
            for e in range(3):
                yield (a * 3 + bb) * 3 + e, a - P, bb - 1, e - 1


def _shift(x, dt, dh, dw):
    """y[t,h,w] = x[t+dt, h+dh, w+dw] with zeros outside; x [..., gt, gh, gw, C]."""
    y = np.zeros_like(x)
    gt, gh, gw = x.shape[-4:-1]
    ts, hs, ws = slice(max(0, -dt), min(gt, gt - dt)), slice(max(0, -dh), min(gh, gh - dh)), \
        slice(max(0, -dw), min(gw, gw - dw))
    tsrc, hsrc, wsrc = slice(ts.start + dt, ts.stop + dt), slice(hs.start + dh, hs.stop + dh), \
        slice(ws.start + dw, ws.stop + dw)
    if ts.start < ts.stop and hs.start < hs.stop and ws.start < ws.stop:
        y[..., ts, hs, ws, :] = x[..., tsrc, hsrc, wsrc, :]
    return y


def short_conv_backward(x, w_text, w_vis, dy, n_text: int, grid, causal_t: int = 0):
    """Adjoint of the modality-aware conv: x, dy [B,T,C]; w_text [C,4]; w_vis [C,27].

    Returns dx [B,T,C], dw_text [C,4], dw_vis [C,27] (fp64).
    """
    x, dy, wt, wv = (_f64(a) for a in (x, dy, w_text, w_vis))
    B, T, Cc = x.shape
    gt, gh, gw = (int(g) for g in grid)
    dx = np.zeros_like(x)
    dwt = np.zeros_like(wt)
    dwv = np.zeros_like(wv)
    # text: y[i] = sum_j w[j] x[i - 3 + j]  (x[<0] = 0)
    xt, dyt = x[:, :n_text], dy[:, :n_text]
    for j in range(4):
        s = 3 - j                                   # y[i] uses x[i - s]
        if s < n_text:
            dx[:, :n_text - s] += wt[:, j] * dyt[:, s:]
            dwt[:, j] = np.einsum("bic,bic->c", dyt[:, s:], xt[:, :n_text - s])
    # visual: y[t,h,w] = sum_taps W x[t+dt, h+dh, w+dw]
    if gt * gh * gw:
        xv = x[:, n_text:].reshape(B, gt, gh, gw, Cc)
        dyv = dy[:, n_text:].reshape(B, gt, gh, gw, Cc)
        dxv = np.zeros_like(xv)
        for tap, ddt, ddh, ddw in _vis_taps(causal_t):
            # x[p] feeds y[p - off]: dx[p] += W dy[p - off]
            dxv += wv[:, tap] * _shift(dyv, -ddt, -ddh, -ddw)
            dwv[:, tap] = np.einsum("bthwc,bthwc->c", dyv, _shift(xv, ddt, ddh, ddw))
        dx[:, n_text:] = dxv.reshape(B, gt * gh * gw, Cc)
    return dx, dwt, dwv


def conv_kda_backward(inp: dict, n_text: int, grid, dO, causal_t: int = 0, S0=None, dST=None):
    """Gradients of L = sum(dO * o) + sum(dST * S_T) through conv + KDA.

    Returns dict: dq, dk, dv (of the conv inputs), dalpha, dbeta, dS0, and
    dw_text_{q,k,v}, dw_vis_{q,k,v}; also the conv outputs qc, kc, vc.
    """
    from . import short_conv_heads
    qc = short_conv_heads(inp["q"], inp["w_text_q"], inp["w_vis_q"], n_text, grid, causal_t)
    kc = short_conv_heads(inp["k"], inp["w_text_k"], inp["w_vis_k"], n_text, grid, causal_t)
    vc = short_conv_heads(inp["v"], inp["w_text_v"], inp["w_vis_v"], n_text, grid, causal_t)
    g = kda_recurrence_backward(qc, kc, vc, inp["alpha"], inp["beta"], dO, S0, dST)
    out = {"dalpha": g["dalpha"], "dbeta": g["dbeta"], "dS0": g["dS0"], "qc": qc, "kc": kc, "vc": vc}
    for s, dsc in (("q", g["dq"]), ("k", g["dk"]), ("v", g["dv"])):
        x = _f64(inp[s])
        B, T, H, d = x.shape
        dx, dwt, dwv = short_conv_backward(x.reshape(B, T, H * d), inp["w_text_" + s], inp["w_vis_" + s],
                                           dsc.reshape(B, T, H * d), n_text, grid, causal_t)
        out["d" + s] = dx.reshape(B, T, H, d)
        out["dw_text_" + s] = dwt
        out["dw_vis_" + s] = dwv
    return out


def kda_chunked_backward(q, k, v, alpha, beta, dO, S0=None, dST=None, C: int = 64):
    """The gradients of kda_recurrence_backward, computed chunk by chunk.

    Per chunk (rows r of the chunk, G_r = sum_{u<=r} log alpha_u, Gam = exp(G),
    gC = G of the last row):
      forward:  Kt = Gam*K, Kd = K/Gam, Qt = Gam*Q, Kh = exp(gC - G)*K,
                A = strict_lower(Kt Kd^T), Bq = lower(Qt Kd^T), Tm = (I + Diag(beta) A)^-1,
                X = Diag(beta) V, Y = Diag(beta) Kt, W = Tm Y, Ut = Tm X,
                U = Ut - W S, O = Qt S + Bq U, S' = Diag(exp(gC)) S + Kh^T U
      reverse (given dO, dS'):
                dU = Bq^T dO + Kh dS';  dS = Qt^T dO + Diag(exp(gC)) dS' - W^T dU
                dQt = dO S^T + dBq Kd,  dBq = lower(dO U^T),  dKh = U dS'^T,
                dW = -dU S^T,  dTm = dU X^T + dW Y^T,  dM = -Tm^T dTm Tm^T,
                dA = strict_lower(Diag(beta) dM),  dX = Tm^T dU,  dY = Tm^T dW,
                dKt = Diag(beta) dY + dA Kd,  dKd = dA^T Kt + dBq^T Qt,
                dbeta = rowsum(dM * A) + rowsum(dX * V) + rowsum(dY * Kt),  dV = Diag(beta) dX,
                dQ = Gam*dQt,  dK = Gam*dKt + dKd/Gam + exp(gC - G)*dKh,
                dG = dQt*Qt + dKt*Kt - dKd*Kd - dKh*Kh (+ on the last row: sum_r dKh*Kh + exp(gC)*rowsum(dS'*S)),
                dlog alpha = reverse cumsum of dG;  dalpha = dlog alpha / alpha.
    """
    q, k, v, alpha, beta, dO = (_f64(a) for a in (q, k, v, alpha, beta, dO))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    out = {"dq": np.zeros_like(q), "dk": np.zeros_like(k), "dv": np.zeros_like(v),
           "dalpha": np.zeros_like(alpha), "dbeta": np.zeros_like(beta), "dS0": np.zeros((B, H, dk, dv))}
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else _f64(S0)[b, h].copy()
            chunks = []
            for n0 in range(0, T, C):
                sl = slice(n0, min(T, n0 + C))
                Q, K, V, be = q[b, sl, h], k[b, sl, h], v[b, sl, h], beta[b, sl, h]
                L = Q.shape[0]
                G = np.cumsum(np.log(alpha[b, sl, h]), axis=0)
                gam, gC = np.exp(G), G[-1]
                Kt, Kd, Qt, Kh = gam * K, K / gam, gam * Q, np.exp(gC - G) * K
                A = np.tril(Kt @ Kd.T, -1)
                Bq = np.tril(Qt @ Kd.T)
                Tm = np.linalg.inv(np.eye(L) + be[:, None] * A)
                X, Y = be[:, None] * V, be[:, None] * Kt
                W, Ut = Tm @ Y, Tm @ X
                U = Ut - W @ S
                chunks.append((sl, Q, K, V, be, G, gam, gC, Kt, Kd, Qt, Kh, A, Bq, Tm, X, Y, W, U, S.copy()))
                S = np.exp(gC)[:, None] * S + Kh.T @ U
            dS = np.zeros((dk, dv)) if dST is None else _f64(dST)[b, h].copy()
            for (sl, Q, K, V, be, G, gam, gC, Kt, Kd, Qt, Kh, A, Bq, Tm, X, Y, W, U, Sn) in reversed(chunks):
                dOc = dO[b, sl, h]
                dU = Bq.T @ dOc + Kh @ dS
                dBq = np.tril(dOc @ U.T)
                dQt = dOc @ Sn.T + dBq @ Kd
                dKh = U @ dS.T
                dW = -dU @ Sn.T
                dTm = dU @ X.T + dW @ Y.T
                dM = -Tm.T @ dTm @ Tm.T
                dA = np.tril(be[:, None] * dM, -1)
                dX, dY = Tm.T @ dU, Tm.T @ dW
                dKt = be[:, None] * dY + dA @ Kd
                dKd = dA.T @ Kt + dBq.T @ Qt
                out["dbeta"][b, sl, h] = np.sum(np.tril(dM, -1) * A, axis=1) + np.sum(dX * V, axis=1) + \
                    np.sum(dY * Kt, axis=1)
                out["dv"][b, sl, h] = be[:, None] * dX
                out["dq"][b, sl, h] = gam * dQt
                out["dk"][b, sl, h] = gam * dKt + dKd / gam + np.exp(gC - G) * dKh
                dG = dQt * Qt + dKt * Kt - dKd * Kd - dKh * Kh
                dG[-1] += np.sum(dKh * Kh, axis=0) + np.exp(gC) * np.sum(dS * Sn, axis=1)
                dlog = np.cumsum(dG[::-1], axis=0)[::-1]
                out["dalpha"][b, sl, h] = dlog / alpha[b, sl, h]
                dS = Qt.T @ dOc + np.exp(gC)[:, None] * dS - W.T @ dU
            out["dS0"][b, h] = dS
    return out

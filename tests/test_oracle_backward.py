"""Pins for the fp64 gradient oracle (CPU only).

The adjoint is checked against central finite differences of the forward
oracle (a route that shares nothing with the hand-written reverse pass), on
tiny streams with both modalities, both temporal paddings, an initial state
and a final-state gradient; against closed forms for one token; and the
chunk-by-chunk restatement against the token-level adjoint.
"""
import numpy as np
import pytest

import oracle
from oracle import backward as ob


def _tiny(seed, n_text=3, grid=(2, 2, 3), B=1, H=1, dk=3, dv=2):
    r = np.random.default_rng(seed)
    T = n_text + grid[0] * grid[1] * grid[2]
    inp = {"q": r.standard_normal((B, T, H, dk)), "k": r.standard_normal((B, T, H, dk)) * 0.5,
           "v": r.standard_normal((B, T, H, dv)),
           "alpha": 1 / (1 + np.exp(-(r.standard_normal((B, T, H, dk)) + 2))),
           "beta": 1 / (1 + np.exp(-r.standard_normal((B, T, H))))}
    for s, d in (("q", dk), ("k", dk), ("v", dv)):
        inp["w_text_" + s] = r.standard_normal((H * d, 4)) * 0.5
        inp["w_vis_" + s] = r.standard_normal((H * d, 27)) * 0.2
    S0 = r.standard_normal((B, H, dk, dv)) * 0.3
    dO = r.standard_normal((B, T, H, dv))
    dST = r.standard_normal((B, H, dk, dv))
    return inp, S0, dO, dST, n_text, grid


def _loss(inp, S0, dO, dST, n_text, grid, causal_t):
    _, _, _, o, st = oracle.conv_kda_forward(inp, n_text, grid, causal_t, S0)
    return float(np.sum(dO * o) + np.sum(dST * st))


@pytest.mark.parametrize("causal_t", [0, 1])
def test_gradients_match_finite_differences(causal_t):
    inp, S0, dO, dST, n_text, grid = _tiny(3 + causal_t)
    g = ob.conv_kda_backward(inp, n_text, grid, dO, causal_t, S0, dST)
    eps = 1e-6
    names = ["q", "k", "v", "alpha", "beta", "w_text_q", "w_text_k", "w_text_v", "w_vis_q", "w_vis_k", "w_vis_v"]
    for name in names + ["S0"]:
        base = S0 if name == "S0" else inp[name]
        grad = g["dS0"] if name == "S0" else g["d" + name]
        num = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            old = base[idx]
            base[idx] = old + eps
            lp = _loss(inp, S0, dO, dST, n_text, grid, causal_t)
            base[idx] = old - eps
            lm = _loss(inp, S0, dO, dST, n_text, grid, causal_t)
            base[idx] = old
            num[idx] = (lp - lm) / (2 * eps)
        scale = max(1.0, np.abs(num).max())
        assert np.abs(grad - num).max() <= 1e-6 * scale, name


def test_one_token_closed_form():
    """T = 1 from S_0 = 0: o = beta (q.k) v, so dq = beta (v.dO) k, dk = beta (v.dO) q,
    dv = beta (q.k) dO, dbeta = (q.k)(v.dO), dalpha = 0."""
    r = np.random.default_rng(7)
    q, k = r.standard_normal((1, 1, 1, 5)), r.standard_normal((1, 1, 1, 5))
    v, dO = r.standard_normal((1, 1, 1, 4)), r.standard_normal((1, 1, 1, 4))
    alpha, beta = np.full((1, 1, 1, 5), 0.7), np.full((1, 1, 1), 0.4)
    g = ob.kda_recurrence_backward(q, k, v, alpha, beta, dO)
    qk, vd = float(q.ravel() @ k.ravel()), float(v.ravel() @ dO.ravel())
    assert np.allclose(g["dq"].ravel(), 0.4 * vd * k.ravel(), atol=1e-14)
    assert np.allclose(g["dk"].ravel(), 0.4 * vd * q.ravel(), atol=1e-14)
    assert np.allclose(g["dv"].ravel(), 0.4 * qk * dO.ravel(), atol=1e-14)
    assert np.allclose(g["dbeta"].ravel(), qk * vd, atol=1e-14)
    assert np.all(g["dalpha"] == 0)


@pytest.mark.parametrize("C,T", [(1, 9), (3, 10), (16, 45), (64, 130)])
def test_chunked_gradients_equal_the_token_level_adjoint(C, T):
    r = np.random.default_rng(C + T)
    B, H, dk, dv = 2, 2, 6, 5
    q = r.standard_normal((B, T, H, dk))
    k = r.standard_normal((B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((B, T, H, dv))
    alpha = 1 / (1 + np.exp(-(r.standard_normal((B, T, H, dk)) + 3)))
    beta = 1 / (1 + np.exp(-r.standard_normal((B, T, H))))
    S0, dST = r.standard_normal((B, H, dk, dv)), r.standard_normal((B, H, dk, dv))
    dO = r.standard_normal((B, T, H, dv))
    a = ob.kda_recurrence_backward(q, k, v, alpha, beta, dO, S0, dST, ckpt=7)
    b = ob.kda_chunked_backward(q, k, v, alpha, beta, dO, S0, dST, C=C)
    for name in a:
        assert np.allclose(a[name], b[name], rtol=0, atol=1e-9 * max(1.0, np.abs(a[name]).max())), name


def test_checkpoint_interval_does_not_matter():
    r = np.random.default_rng(11)
    args = [r.standard_normal((1, 20, 1, 4)), r.standard_normal((1, 20, 1, 4)) * 0.5, r.standard_normal((1, 20, 1, 3)),
            np.full((1, 20, 1, 4), 0.9), np.full((1, 20, 1), 0.5), r.standard_normal((1, 20, 1, 3))]
    a = ob.kda_recurrence_backward(*args, ckpt=1)
    b = ob.kda_recurrence_backward(*args, ckpt=64)
    for name in a:
        assert np.array_equal(a[name], b[name]), name


def test_planted_sign_error_fails_the_finite_difference_pin():
    """A plausible mistake (the sign of the r term) planted in a copy of the adjoint."""
    inp, S0, dO, dST, n_text, grid = _tiny(5)
    qc = oracle.short_conv_heads(inp["q"], inp["w_text_q"], inp["w_vis_q"], n_text, grid)
    kc = oracle.short_conv_heads(inp["k"], inp["w_text_k"], inp["w_vis_k"], n_text, grid)
    vc = oracle.short_conv_heads(inp["v"], inp["w_text_v"], inp["w_vis_v"], n_text, grid)
    good = ob.kda_recurrence_backward(qc, kc, vc, inp["alpha"], inp["beta"], dO, S0, dST)
    # dv from a planted variant: u = beta (v + r) instead of beta (v - r) changes dbeta
    T = qc.shape[1]
    S = S0[0, 0].copy()
    bad_dbeta = np.zeros(T)
    states = []
    for t in range(T):
        states.append(S.copy())
        Sp = inp["alpha"][0, t, 0][:, None] * S
        u = inp["beta"][0, t, 0] * (vc[0, t, 0] - Sp.T @ kc[0, t, 0])
        S = Sp + np.outer(kc[0, t, 0], u)
    dS = dST[0, 0].copy()
    for t in range(T - 1, -1, -1):
        Sp = inp["alpha"][0, t, 0][:, None] * states[t]
        r = Sp.T @ kc[0, t, 0]
        u = inp["beta"][0, t, 0] * (vc[0, t, 0] - r)
        St = Sp + np.outer(kc[0, t, 0], u)
        dS = dS + np.outer(qc[0, t, 0], dO[0, t, 0])
        du = dS.T @ kc[0, t, 0]
        bad_dbeta[t] = du @ (vc[0, t, 0] + r)           # planted
        dSp = dS + np.outer(kc[0, t, 0], -inp["beta"][0, t, 0] * du)
        dS = inp["alpha"][0, t, 0][:, None] * dSp
        del St
    assert not np.allclose(bad_dbeta, good["dbeta"][0, :, 0], atol=1e-6)

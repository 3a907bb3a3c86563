"""Pins of the oracle's KDA recurrence (CPU only).

The state update is the one printed in the Chimera paper's method step (5)
(paper.rainbus.top page, "method step details"):
    S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
with the readout o_t = S_t^T q_t.  The oracle evaluates it as a delta rule
(S' = Diag(alpha) S; u = beta (v - S'^T k); S = S' + k u^T).  It is pinned by:

* brute force: the printed matrix form with explicit dk x dk transition
  matrices, unrolled into products (fp64 numpy) and in exact rational
  arithmetic (fractions) on tiny inputs;
* invariants the pages' description of alpha and beta fixes (pages' KDA
  prerequisite: alpha decays the state per channel, beta scales the write):
  beta = 0 is pure per-channel decay; alpha = 1, beta = 1 with orthonormal keys
  recalls the stored values exactly; a repeated key is overwritten;
* closed forms (T = 1), linearity, causality, equivariance, split/resume;
* the chunked regrouping (second path) for many chunk sizes and ragged tails.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle.chunked import kda_chunked


def _rand(rng, B, T, H, dk, dv, alpha_lo=0.3):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    alpha = rng.uniform(alpha_lo, 1.0, (B, T, H, dk))
    beta = rng.uniform(0.0, 1.0, (B, T, H))
    return q, k, v, alpha, beta


def _brute_force(q, k, v, alpha, beta, S0):
    """Matrix form: S_t = (prod_{r=t..1} M_r) S_0 + sum_s (prod_{r=t..s+1} M_r) beta_s k_s v_s^T."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    ST = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            M = [(np.eye(dk) - beta[b, t, h] * np.outer(k[b, t, h], k[b, t, h]))
                 @ np.diag(alpha[b, t, h]) for t in range(T)]
            for t in range(T):
                P = np.eye(dk)
                for r in range(t, -1, -1):
                    P = P @ M[r]
                S = P @ S0[b, h]
                for s in range(t + 1):
                    P = np.eye(dk)
                    for r in range(t, s, -1):
                        P = P @ M[r]
                    S = S + P @ (beta[b, s, h] * np.outer(k[b, s, h], v[b, s, h]))
                o[b, t, h] = S.T @ q[b, t, h]
                if t == T - 1:
                    ST[b, h] = S
    return o, ST


def test_recurrence_matches_unrolled_matrix_products():
    rng = np.random.default_rng(0)
    B, T, H, dk, dv = 2, 9, 2, 5, 4
    q, k, v, alpha, beta = _rand(rng, B, T, H, dk, dv)
    S0 = rng.standard_normal((B, H, dk, dv))
    o, st = oracle.kda_recurrence(q, k, v, alpha, beta, S0)
    ob, sb = _brute_force(q, k, v, alpha, beta, S0)
    np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(st, sb, rtol=1e-12, atol=1e-12)


def test_recurrence_matches_exact_rational_arithmetic():
    """dk = dv = 2, T = 3 evaluated exactly with fractions in the printed matrix form."""
    fr = Fraction
    q = [[fr(1), fr(2)], [fr(-1, 2), fr(3)], [fr(2), fr(-1)]]
    k = [[fr(1, 2), fr(1, 3)], [fr(-1, 4), fr(1)], [fr(2, 3), fr(-1, 5)]]
    v = [[fr(3), fr(-1)], [fr(1, 7), fr(2)], [fr(-2), fr(5, 3)]]
    a = [[fr(1, 2), fr(3, 4)], [fr(9, 10), fr(1, 3)], [fr(2, 5), fr(1)]]
    be = [fr(1, 2), fr(3, 4), fr(1, 5)]
    S0 = [[fr(1, 3), fr(-2)], [fr(1, 2), fr(1, 9)]]

    def matmul(A, Bm):
        return [[sum(A[i][l] * Bm[l][j] for l in range(len(Bm))) for j in range(len(Bm[0]))]
                for i in range(len(A))]

    S = [row[:] for row in S0]
    outs = []
    for t in range(3):
        kkT = [[k[t][i] * k[t][j] for j in range(2)] for i in range(2)]
        Mt = [[(1 if i == j else 0) - be[t] * kkT[i][j] for j in range(2)] for i in range(2)]
        Da = [[a[t][i] if i == j else 0 for j in range(2)] for i in range(2)]
        S = matmul(matmul(Mt, Da), S)
        S = [[S[i][j] + be[t] * k[t][i] * v[t][j] for j in range(2)] for i in range(2)]
        outs.append([sum(S[i][j] * q[t][i] for i in range(2)) for j in range(2)])

    def arr(x):
        return np.array([[float(e) for e in row] for row in x])

    o, st = oracle.kda_recurrence(arr(q)[None, :, None], arr(k)[None, :, None],
                                  arr(v)[None, :, None], arr(a)[None, :, None],
                                  np.array(be, dtype=float)[None, :, None], arr(S0)[None, None])
    np.testing.assert_allclose(o[0, :, 0], arr(outs), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(st[0, 0], arr(S), rtol=1e-14, atol=1e-15)


def test_beta_zero_is_pure_channel_decay():
    rng = np.random.default_rng(1)
    B, T, H, dk, dv = 1, 12, 2, 6, 5
    q, k, v, alpha, beta = _rand(rng, B, T, H, dk, dv)
    beta[:] = 0.0
    S0 = rng.standard_normal((B, H, dk, dv))
    o, st = oracle.kda_recurrence(q, k, v, alpha, beta, S0)
    G = np.cumprod(alpha, axis=1)                               # prod_{u<=t} alpha_u
    expect_o = np.einsum("bthi,bhij->bthj", G * q, S0)          # o_t = S_0^T (decay_t * q_t)
    np.testing.assert_allclose(o, expect_o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(st, G[:, -1][:, :, :, None] * S0, rtol=1e-12, atol=1e-13)


def test_alpha_one_beta_one_orthonormal_keys_recall_exactly():
    rng = np.random.default_rng(2)
    dk, dv, n = 8, 5, 6
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Qm[:, :n].T                                          # n orthonormal keys
    vals = rng.standard_normal((n, dv))
    T = 2 * n
    q = np.zeros((1, T, 1, dk))
    k = np.zeros((1, T, 1, dk))
    v = np.zeros((1, T, 1, dv))
    beta = np.zeros((1, T, 1))
    k[0, :n, 0], v[0, :n, 0], beta[0, :n, 0] = keys, vals, 1.0   # writes
    q[0, n:, 0] = keys[::-1]                                     # reads, beta = 0
    alpha = np.ones((1, T, 1, dk))
    o, st = oracle.kda_recurrence(q, k, v, alpha, beta)
    np.testing.assert_allclose(o[0, n:, 0], vals[::-1], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(st[0, 0], keys.T @ vals, rtol=1e-12, atol=1e-12)


def test_repeated_key_with_beta_one_overwrites_value():
    rng = np.random.default_rng(3)
    dk, dv = 4, 3
    key = rng.standard_normal(dk)
    key /= np.linalg.norm(key)
    v1, v2 = rng.standard_normal(dv), rng.standard_normal(dv)
    q = np.zeros((1, 3, 1, dk))
    q[0, 2, 0] = key
    k = np.stack([key, key, np.zeros(dk)])[None, :, None]
    v = np.stack([v1, v2, np.zeros(dv)])[None, :, None]
    beta = np.array([1.0, 1.0, 0.0])[None, :, None]
    o, _ = oracle.kda_recurrence(q, k, v, np.ones((1, 3, 1, dk)), beta)
    np.testing.assert_allclose(o[0, 2, 0], v2, rtol=1e-13, atol=1e-14)


def test_single_token_closed_form():
    rng = np.random.default_rng(4)
    q, k, v, alpha, beta = _rand(rng, 2, 1, 3, 7, 5)
    o, st = oracle.kda_recurrence(q, k, v, alpha, beta)
    expect = beta[:, 0, :, None] * np.einsum("bhi,bhi->bh", q[:, 0], k[:, 0])[..., None] * v[:, 0]
    np.testing.assert_allclose(o[:, 0], expect, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(st, beta[:, 0, :, None, None] *
                               np.einsum("bhi,bhj->bhij", k[:, 0], v[:, 0]), rtol=1e-13)


def test_linearity_in_v_and_initial_state_and_in_q():
    rng = np.random.default_rng(5)
    q, k, v, alpha, beta = _rand(rng, 1, 10, 2, 6, 4)
    _, _, v2, _, _ = _rand(rng, 1, 10, 2, 6, 4)
    S0a, S0b = rng.standard_normal((2, 1, 2, 6, 4))
    c = -1.75
    o1, s1 = oracle.kda_recurrence(q, k, v, alpha, beta, S0a)
    o2, s2 = oracle.kda_recurrence(q, k, v2, alpha, beta, S0b)
    o3, s3 = oracle.kda_recurrence(q, k, v + c * v2, alpha, beta, S0a + c * S0b)
    np.testing.assert_allclose(o3, o1 + c * o2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(s3, s1 + c * s2, rtol=1e-11, atol=1e-12)
    q2 = rng.standard_normal(q.shape)
    o4, _ = oracle.kda_recurrence(q2, k, v, alpha, beta, S0a)
    o5, _ = oracle.kda_recurrence(q + c * q2, k, v, alpha, beta, S0a)
    np.testing.assert_allclose(o5, o1 + c * o4, rtol=1e-11, atol=1e-12)


def test_causality():
    rng = np.random.default_rng(6)
    q, k, v, alpha, beta = _rand(rng, 1, 14, 1, 5, 3)
    o, _ = oracle.kda_recurrence(q, k, v, alpha, beta)
    for t in (0, 5, 12):
        q2, k2, v2, a2, b2 = (x.copy() for x in (q, k, v, alpha, beta))
        n = 14 - t - 1
        q2[:, t + 1:] = rng.standard_normal((1, n, 1, 5))
        k2[:, t + 1:] = rng.standard_normal((1, n, 1, 5))
        v2[:, t + 1:] = rng.standard_normal((1, n, 1, 3))
        a2[:, t + 1:] = rng.uniform(0.3, 1, (1, n, 1, 5))
        b2[:, t + 1:] = rng.uniform(0, 1, (1, n, 1))
        o2, _ = oracle.kda_recurrence(q2, k2, v2, a2, b2)
        assert np.array_equal(o[:, :t + 1], o2[:, :t + 1])


def test_head_and_batch_permutation_equivariance():
    rng = np.random.default_rng(7)
    q, k, v, alpha, beta = _rand(rng, 3, 8, 4, 5, 3)
    S0 = rng.standard_normal((3, 4, 5, 3))
    o, st = oracle.kda_recurrence(q, k, v, alpha, beta, S0)
    pb, ph = np.array([2, 0, 1]), np.array([3, 1, 0, 2])
    perm = lambda x: x[pb][:, :, ph]                              # noqa: E731
    o2, st2 = oracle.kda_recurrence(perm(q), perm(k), perm(v), perm(alpha), perm(beta),
                                    S0[pb][:, ph])
    np.testing.assert_allclose(o2, perm(o), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(st2, st[pb][:, ph], rtol=1e-13, atol=1e-14)


def test_split_and_resume_with_carried_state():
    rng = np.random.default_rng(8)
    q, k, v, alpha, beta = _rand(rng, 2, 21, 2, 6, 5)
    o, st = oracle.kda_recurrence(q, k, v, alpha, beta)
    T1 = 8
    oa, sa = oracle.kda_recurrence(q[:, :T1], k[:, :T1], v[:, :T1], alpha[:, :T1], beta[:, :T1])
    ob, sb = oracle.kda_recurrence(q[:, T1:], k[:, T1:], v[:, T1:], alpha[:, T1:], beta[:, T1:], sa)
    np.testing.assert_allclose(np.concatenate([oa, ob], axis=1), o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(sb, st, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("C", [1, 2, 3, 5, 16, 64])
@pytest.mark.parametrize("T", [23, 64, 130])
def test_chunked_regrouping_equals_recurrence(C, T):
    rng = np.random.default_rng(100 + C + T)
    q, k, v, alpha, beta = _rand(rng, 1, T, 2, 6, 5)
    S0 = rng.standard_normal((1, 2, 6, 5))
    o, st = oracle.kda_recurrence(q, k, v, alpha, beta, S0)
    oc, sc = kda_chunked(q, k, v, alpha, beta, S0, C=C)
    np.testing.assert_allclose(oc, o, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(sc, st, rtol=1e-11, atol=1e-12)


def test_alpha_one_reduces_to_delta_rule():
    """alpha = 1: S_t = S_{t-1} + beta k (v - S_{t-1}^T k)^T, the DeltaNet update."""
    rng = np.random.default_rng(9)
    q, k, v, _, beta = _rand(rng, 1, 15, 1, 4, 3)
    o, st = oracle.kda_recurrence(q, k, v, np.ones_like(q), beta)
    S = np.zeros((4, 3))
    for t in range(15):
        kt = k[0, t, 0]
        S = S + beta[0, t, 0] * np.outer(kt, v[0, t, 0] - S.T @ kt)
        np.testing.assert_allclose(o[0, t, 0], S.T @ q[0, t, 0], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(st[0, 0], S, rtol=1e-12, atol=1e-13)


def test_bad_shapes_raise():
    with pytest.raises(ValueError):
        oracle.kda_recurrence(np.zeros((1, 2, 1, 3)), np.zeros((1, 2, 1, 4)), np.zeros((1, 2, 1, 3)),
                              np.ones((1, 2, 1, 3)), np.zeros((1, 2, 1)))

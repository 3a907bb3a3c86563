"""Pins for the fp64 MLA attention oracle (CPU only).

Each test fixes the oracle against something other than itself: a pure-Python
loop over single elements (index conventions, which head sees which key
part), closed forms of softmax attention (one key, uniform weights, a
dominant key), and invariances that hold exactly (key-value permutation, a
shift of the shared key part, per-head independence).
"""
import math

import numpy as np
import pytest

from oracle import mla


def _rand(seed, B=2, T=9, H=3, dn=5, dr=3, dv=4):
    r = np.random.default_rng(seed)
    return (r.standard_normal((B, T, H, dn)), r.standard_normal((B, T, H, dr)),
            r.standard_normal((B, T, H, dn)), r.standard_normal((B, T, dr)), r.standard_normal((B, T, H, dv)))


def _loops(qn, qd, kn, kd, v, scale):
    """The definition, one element at a time, in plain Python floats."""
    B, T, H, dn = qn.shape
    dr, dv = qd.shape[-1], v.shape[-1]
    out = np.zeros((B, T, H, dv))
    for b in range(B):
        for h in range(H):
            for i in range(T):
                s = []
                for j in range(T):
                    acc = 0.0
                    for c in range(dn):
                        acc += float(qn[b, i, h, c]) * float(kn[b, j, h, c])
                    for c in range(dr):
                        acc += float(qd[b, i, h, c]) * float(kd[b, j, c])
                    s.append(scale * acc)
                m = max(s)
                w = [math.exp(x - m) for x in s]
                z = sum(w)
                for e in range(dv):
                    out[b, i, h, e] = sum(w[j] * float(v[b, j, h, e]) for j in range(T)) / z
    return out


def test_matches_elementwise_loops():
    x = _rand(1)
    sc = 0.37
    assert np.allclose(mla.mla_attention(*x, scale=sc), _loops(*x, sc), rtol=0, atol=1e-13)


def test_default_scale_is_inverse_sqrt_of_the_key_width():
    x = _rand(2, dn=6, dr=10)
    assert np.allclose(mla.mla_attention(*x), _loops(*x, 0.25), rtol=0, atol=1e-13)


def test_sampled_rows_and_heads_are_slices_of_the_full_result():
    x = _rand(3, T=11, H=4)
    full = mla.mla_attention(*x)
    part = mla.mla_attention(*x, rows=[10, 0, 5], heads=[3, 1])
    assert np.array_equal(part, full[:, [10, 0, 5]][:, :, [3, 1]])


def test_one_key_returns_its_value():
    qn, qd, kn, kd, v = _rand(4, T=1)
    assert np.allclose(mla.mla_attention(qn, qd, kn, kd, v), v, rtol=0, atol=1e-15)


def test_zero_query_or_equal_keys_average_the_values():
    qn, qd, kn, kd, v = _rand(5, T=8)
    mean = np.broadcast_to(v.mean(axis=1, keepdims=True), v.shape)
    o = mla.mla_attention(np.zeros_like(qn), np.zeros_like(qd), kn, kd, v)
    assert np.allclose(o, mean, rtol=0, atol=1e-14)
    kn_eq = np.broadcast_to(kn[:, :1], kn.shape).copy()
    kd_eq = np.broadcast_to(kd[:, :1], kd.shape).copy()
    o = mla.mla_attention(qn, qd, kn_eq, kd_eq, v)
    assert np.allclose(o, mean, rtol=0, atol=1e-14)


def test_a_dominant_key_wins():
    qn, qd, kn, kd, v = _rand(6, B=1, T=6, H=1, dn=4, dr=2)
    kn[0, 3, 0] = 40.0 * qn[0, 2, 0]           # query 2 matches key 3 far better than any other
    o = mla.mla_attention(qn, qd, kn, kd, v, scale=1.0)
    assert np.allclose(o[0, 2, 0], v[0, 3, 0], rtol=0, atol=1e-12)


def test_permuting_key_value_pairs_changes_nothing():
    qn, qd, kn, kd, v = _rand(7, T=10)
    perm = np.random.default_rng(0).permutation(10)
    a = mla.mla_attention(qn, qd, kn, kd, v)
    b = mla.mla_attention(qn, qd, kn[:, perm], kd[:, perm], v[:, perm])
    assert np.allclose(a, b, rtol=0, atol=1e-13)
    # permuting the queries permutes the outputs
    c = mla.mla_attention(qn[:, perm], qd[:, perm], kn, kd, v)
    assert np.allclose(c, a[:, perm], rtol=0, atol=1e-13)


def test_a_shift_of_the_shared_key_part_changes_nothing():
    qn, qd, kn, kd, v = _rand(8)
    shift = np.random.default_rng(1).standard_normal(kd.shape[-1]) * 3.0
    a = mla.mla_attention(qn, qd, kn, kd, v)
    b = mla.mla_attention(qn, qd, kn, kd + shift, v)       # the same offset to every key of a query
    assert np.allclose(a, b, rtol=0, atol=1e-12)


def test_shared_key_part_reaches_every_head_and_query_parts_only_their_own():
    qn, qd, kn, kd, v = _rand(9, H=3)
    a = mla.mla_attention(qn, qd, kn, kd, v)
    kd2 = kd.copy()
    kd2[:, 4] += 1.0                                        # one token's shared key part
    b = mla.mla_attention(qn, qd, kn, kd2, v)
    for h in range(3):
        assert not np.allclose(a[:, :, h], b[:, :, h])
    qd2 = qd.copy()
    qd2[:, :, 1] += 1.0                                     # head 1's direct query part
    c = mla.mla_attention(qn, qd2, kn, kd, v)
    assert np.array_equal(c[:, :, 0], a[:, :, 0]) and np.array_equal(c[:, :, 2], a[:, :, 2])
    assert not np.allclose(c[:, :, 1], a[:, :, 1])


@pytest.mark.parametrize("plant", ["drop_direct", "wrong_head_key", "no_max_shift_large"])
def test_planted_mistakes_are_caught(plant):
    """Plausible mistakes, planted in copies of the oracle's arithmetic, fail the pins."""
    qn, qd, kn, kd, v = _rand(10, T=6, H=2)
    sc = 0.5
    ref = _loops(qn, qd, kn, kd, v, sc)
    if plant == "drop_direct":
        bad = mla.mla_attention(qn, np.zeros_like(qd), kn, kd, v, scale=sc)
    elif plant == "wrong_head_key":
        bad = mla.mla_attention(qn, qd, kn[:, :, ::-1].copy(), kd, v, scale=sc)
    else:
        big = 800.0                                          # exp without the max shift overflows here
        with np.errstate(over="ignore", invalid="ignore"):
            s = big * np.einsum("btc,bsc->bts", qn[:, :, 0], qn[:, :, 0])
            p = np.exp(s)
            bad = (p @ v[:, :, 0]) / p.sum(axis=-1, keepdims=True)
        good = mla.mla_attention(qn[:, :, :1], np.zeros_like(qd[:, :, :1]), qn[:, :, :1], np.zeros_like(kd),
                                 v[:, :, :1], scale=big)
        assert np.all(np.isfinite(good))
        assert not np.allclose(bad, good[:, :, 0], equal_nan=False)
        return
    assert not np.allclose(bad, ref, rtol=0, atol=1e-6)


# ---- the latent path ------------------------------------------------------------------

def _latent_rand(seed, M=7, dm=6, dc=3, dr=2, H=2, dn=4, dv=5):
    r = np.random.default_rng(seed)
    return (r.standard_normal((M, dm)), r.standard_normal((dc, dm)), r.standard_normal((dr, dm)),
            r.standard_normal((H * dn, dc)), r.standard_normal((H * dv, dc)))


def test_latent_matches_element_loops():
    """Every output element as an explicit sum over the contracted index, in Python floats:
    c[m, i] = sum_k x[m, k] w_dkv[i, k]; k_nope[m, h, d] = sum_i c[m, i] w_uk[h d_nope + d, i]."""
    x, wd, wr, wk, wv = _latent_rand(3)
    H = 2
    c, kd, kn, v = mla.mla_latent(x, wd, wr, wk, wv, H)
    M, dm = x.shape
    dc, dr, dn, dvv = wd.shape[0], wr.shape[0], wk.shape[0] // H, wv.shape[0] // H
    for m in range(M):
        cl = [sum(float(x[m, k]) * float(wd[i, k]) for k in range(dm)) for i in range(dc)]
        for i in range(dc):
            assert c[m, i] == pytest.approx(cl[i], rel=1e-12, abs=1e-12)
        for i in range(dr):
            assert kd[m, i] == pytest.approx(sum(float(x[m, k]) * float(wr[i, k]) for k in range(dm)),
                                             rel=1e-12, abs=1e-12)
        for h in range(H):
            for d in range(dn):
                ref = sum(cl[i] * float(wk[h * dn + d, i]) for i in range(dc))
                assert kn[m, h, d] == pytest.approx(ref, rel=1e-12, abs=1e-12)
            for d in range(dvv):
                ref = sum(cl[i] * float(wv[h * dvv + d, i]) for i in range(dc))
                assert v[m, h, d] == pytest.approx(ref, rel=1e-12, abs=1e-12)


def test_keys_and_values_have_the_latent_rank():
    """Keys and values are decompressed from a d_c-wide latent, so the token-by-feature matrix
    [k_nope | v] has rank d_c < d_model; a path that projected x directly would have rank d_model."""
    r = np.random.default_rng(11)
    M, dm, dc, H, dn, dv = 40, 16, 5, 3, 6, 4
    x = r.standard_normal((M, dm))
    wd, wr = r.standard_normal((dc, dm)), r.standard_normal((2, dm))
    wk, wv = r.standard_normal((H * dn, dc)), r.standard_normal((H * dv, dc))
    _, _, kn, v = mla.mla_latent(x, wd, wr, wk, wv, H)
    kv = np.concatenate([kn.reshape(M, -1), v.reshape(M, -1)], axis=1)
    assert np.linalg.matrix_rank(kv) == dc
    # K_direct comes from x itself: full rank min(M, d_dir)
    _, kd, _, _ = mla.mla_latent(x, wd, wr, wk, wv, H)
    assert np.linalg.matrix_rank(kd) == 2


def test_absorbed_queries_score_against_the_latent():
    """q_h . k_nope[j, h] = (W_uk,h^T q_h) . c_j: scoring the latent with the head's absorbed
    query gives the same logits, which fixes the head split and the orientation of W_uk."""
    x, wd, wr, wk, wv = _latent_rand(5, M=9, dm=8, dc=4, H=3, dn=5)
    H, dn = 3, 5
    c, _, kn, _ = mla.mla_latent(x, wd, wr, wk, wv, H)
    q = np.random.default_rng(6).standard_normal((H, dn))
    for h in range(H):
        wkh = wk[h * dn:(h + 1) * dn]             # [d_nope, d_c]: head h's rows
        direct = kn[:, h] @ q[h]
        absorbed = c @ (wkh.T @ q[h])
        np.testing.assert_allclose(direct, absorbed, rtol=1e-12, atol=1e-12)


def test_identity_compression_reduces_to_one_projection():
    """d_c = d_model with W_dkv = I: the latent is x itself, and k_nope, v are single
    projections of x."""
    r = np.random.default_rng(8)
    M, dm, H, dn, dv = 5, 6, 2, 3, 2
    x = r.standard_normal((M, dm))
    wk, wv, wr = r.standard_normal((H * dn, dm)), r.standard_normal((H * dv, dm)), r.standard_normal((2, dm))
    c, kd, kn, v = mla.mla_latent(x, np.eye(dm), wr, wk, wv, H)
    np.testing.assert_array_equal(c, x)
    np.testing.assert_allclose(kn.reshape(M, -1), np.einsum("mk,nk->mn", x, wk), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(v.reshape(M, -1), np.einsum("mk,nk->mn", x, wv), rtol=1e-13, atol=1e-13)


def test_layer_is_latent_then_attention():
    """mla_layer on a tiny stream equals the element-loop attention of the latent's keys and values."""
    r = np.random.default_rng(9)
    B, T, H, dm, dc, dn, dr, dv = 1, 6, 2, 8, 4, 3, 2, 3
    x = r.standard_normal((B, T, dm))
    wd, wr = r.standard_normal((dc, dm)), r.standard_normal((dr, dm))
    wk, wv = r.standard_normal((H * dn, dc)), r.standard_normal((H * dv, dc))
    qn, qd = r.standard_normal((B, T, H, dn)), r.standard_normal((B, T, H, dr))
    o = mla.mla_layer(x, qn, qd, wd, wr, wk, wv, scale=0.4)
    _, kd, kn, v = mla.mla_latent(x, wd, wr, wk, wv, H)
    np.testing.assert_allclose(o, _loops(qn, qd, kn, kd, v, 0.4), rtol=1e-12, atol=1e-12)

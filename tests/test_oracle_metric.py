"""Pins of the parity metric itself (CPU only).

The gate metric is, per (batch, head), the largest absolute difference over
the largest absolute reference value, then the worst (batch, head); the
element-wise figure divides each difference by its own reference value,
floored at 1e-6 of the (batch, head)'s largest.  Every expected number below
was worked out by hand from those definitions; each case is built so that a
plausible slip (one global normalisation, the wrong pair of axes, a missing
floor) gives a different number.
"""
import numpy as np
import pytest

import oracle


def _tokens_case():
    """[B=2, T=3, H=2, d=2] reference and a perturbed copy.

    (b, h) = (0, 0): max |ref| 100, max |diff| 1    -> 0.01
    (b, h) = (0, 1): max |ref| 1,   max |diff| 0.5  -> 0.5   (the answer)
    (b, h) = (1, 0): max |ref| 2,   max |diff| 0    -> 0
    (b, h) = (1, 1): max |ref| 4,   max |diff| 0.4  -> 0.1
    """
    ref = np.zeros((2, 3, 2, 2))
    ref[0, 0, 0, 0] = 100.0
    ref[0, 0, 1, 0] = -1.0
    ref[1, 1, 0, 1] = 2.0
    ref[1, 2, 1, 0] = 4.0
    x = ref.copy()
    x[0, 1, 0, 0] += 1.0
    x[0, 2, 1, 1] -= 0.5
    x[1, 0, 1, 1] += 0.4
    return x, ref


def test_rel_err_per_batch_head():
    x, ref = _tokens_case()
    assert oracle.rel_err(x, ref) == pytest.approx(0.5, rel=1e-15)
    # one global normalisation would give 1 / 100, per batch only 0.1, per head
    # only 0.5 / 4: the case separates all of them from the answer
    assert oracle.rel_err(x, ref) != pytest.approx(0.01)


def test_rel_err_is_symmetric_in_sign_and_zero_for_equal():
    x, ref = _tokens_case()
    assert oracle.rel_err(ref, ref) == 0.0
    assert oracle.rel_err(-x, -ref) == pytest.approx(0.5, rel=1e-15)


def test_rel_err_reduces_tokens_and_channels_not_heads():
    """A transposed reduction (over heads and channels, per token) would divide the
    token-1 error of (b, h) = (0, 0) by a zero reference row and blow up."""
    ref = np.zeros((1, 2, 2, 1))
    ref[0, 0, 0, 0] = 10.0      # head 0: token 0 large, token 1 zero
    ref[0, 1, 1, 0] = 1.0       # head 1: token 1 only
    x = ref.copy()
    x[0, 1, 0, 0] = 0.1         # head 0 error on token 1: 0.1 / 10
    assert oracle.rel_err(x, ref) == pytest.approx(0.01, rel=1e-14)


def test_rel_err_state_per_batch_head():
    """[B=1, H=2, dk=2, dv=3]: head 0 max |ref| 8, diff 2 -> 0.25; head 1 max 0.5, diff 0.05 -> 0.1."""
    ref = np.zeros((1, 2, 2, 3))
    ref[0, 0, 1, 2] = -8.0
    ref[0, 1, 0, 0] = 0.5
    x = ref.copy()
    x[0, 0, 0, 0] = 2.0
    x[0, 1, 1, 1] = 0.05
    assert oracle.rel_err_state(x, ref) == pytest.approx(0.25, rel=1e-15)
    # the token-layout metric reduces other axes and must not be what states use
    assert oracle.rel_err(x, ref) != pytest.approx(0.25)


def test_rel_err_elementwise_with_floor():
    """[B=1, T=2, H=1, d=2], max |ref| = 1:
    element (0, 0): ref 1,    diff 0.01  -> 0.01
    element (0, 1): ref 1e-9, diff 1e-7  -> 1e-7 / max(1e-9, 1e-6) = 0.1
    element (1, 0): ref 0.2,  diff 0.004 -> 0.02
    element (1, 1): ref -0.5, diff 0     -> 0
    """
    ref = np.array([[[[1.0, 1e-9]], [[0.2, -0.5]]]])
    x = ref.copy()
    x[0, 0, 0, 0] += 0.01
    x[0, 0, 0, 1] += 1e-7
    x[0, 1, 0, 0] -= 0.004
    assert oracle.rel_err_elementwise(x, ref) == pytest.approx(0.1, rel=1e-9)
    # without the floor the tiny element would give 100
    assert oracle.rel_err_elementwise(x, ref, floor=0.0) == pytest.approx(100.0, rel=1e-9)
    # the floor scales with each (b, h)'s own maximum: a second head with max 1000
    ref2 = np.concatenate([ref, ref * 1000.0], axis=2)
    x2 = np.concatenate([x, ref * 1000.0], axis=2)
    assert oracle.rel_err_elementwise(x2, ref2) == pytest.approx(0.1, rel=1e-9)


def test_rel_err_elementwise_state_layout():
    """[B=1, H=1, dk=2, dv=2] state, max |ref| = 4: diff 0.4 on the 4 -> 0.1, diff 0.03 on 0.3 -> 0.1,
    diff 2e-6 on ref 0 -> 2e-6 / 4e-6 = 0.5."""
    ref = np.array([[[[4.0, 0.3], [0.0, -1.0]]]])
    x = ref.copy()
    x[0, 0, 0, 0] += 0.4
    x[0, 0, 0, 1] += 0.03
    x[0, 0, 1, 0] += 2e-6
    assert oracle.rel_err_elementwise(x, ref, layout="state") == pytest.approx(0.5, rel=1e-9)
    with pytest.raises(ValueError):
        oracle.rel_err_elementwise(x, ref, layout="bogus")

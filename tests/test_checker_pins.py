"""Pins of the comparison metrics every parity test uses: the relative L2 error
(``oracle.rel_l2``) and its per-(sequence, head) buckets (``tests._common``).
A slip in either (a wrong normalisation, a bucket summed over the wrong axes,
an empty sequence counted) would let every GPU test pass vacuously, so each is
held to values worked out by hand here."""
import math

import numpy as np
import pytest

import oracle
from tests._common import bucket_errors, close


def test_rel_l2_scaled_reference_gives_the_scale():
    """x = ref (1 + eps) has ||x - ref|| / ||ref|| = |eps| exactly, whatever ref is."""
    rng = np.random.default_rng(1)
    ref = rng.standard_normal((3, 5, 7))
    for eps in (1e-3, -2.5e-5, 0.5):
        assert oracle.rel_l2(ref * (1.0 + eps), ref) == pytest.approx(abs(eps), rel=1e-12)


def test_rel_l2_hand_values():
    # ||(1,2,2) - (1,2,3)|| / ||(1,2,3)|| = 1 / sqrt(14)
    assert oracle.rel_l2(np.array([1.0, 2.0, 2.0]), np.array([1.0, 2.0, 3.0])) == \
        pytest.approx(1.0 / math.sqrt(14.0), rel=1e-15)
    # one element off by 3 in a 2x2 of ones: 3 / 2
    x = np.ones((2, 2))
    x[1, 0] += 3.0
    assert oracle.rel_l2(x, np.ones((2, 2))) == pytest.approx(1.5, rel=1e-15)
    # a zero reference gives the absolute error (||(3, 4)|| = 5), and 0 for x = 0
    assert oracle.rel_l2(np.array([3.0, 4.0]), np.zeros(2)) == pytest.approx(5.0, rel=1e-15)
    assert oracle.rel_l2(np.zeros(2), np.zeros(2)) == 0.0
    # the norm is taken over the whole tensor, not per row: rows off by 0 and 4
    # against rows of norm 3 and 4 give 4 / 5 (per-row errors would be 0 and 1)
    ref = np.array([[3.0, 0.0], [0.0, 4.0]])
    x = ref.copy()
    x[1, 1] += 4.0
    assert oracle.rel_l2(x, ref) == pytest.approx(0.8, rel=1e-15)


def test_rel_l2_is_symmetric_in_scale_and_sign():
    rng = np.random.default_rng(2)
    ref = rng.standard_normal(100)
    x = ref + 1e-4 * rng.standard_normal(100)
    e = oracle.rel_l2(x, ref)
    assert oracle.rel_l2(-7.0 * x, -7.0 * ref) == pytest.approx(e, rel=1e-12)
    assert e > 0


def test_bucket_errors_dense_tokens():
    """[B, T, H, D]: one bucket per (b, h), over its T x D values."""
    B, T, H, D = 2, 3, 4, 5
    ref = np.ones((B, T, H, D))
    x = ref.copy()
    x[1, 2, 3, 0] += 6.0  # bucket (1, 3): ||6|| / sqrt(T D) = 6 / sqrt(15)
    e = bucket_errors(x, ref, "tokens").reshape(B, H)
    assert e[1, 3] == pytest.approx(6.0 / math.sqrt(15.0), rel=1e-14)
    e[1, 3] = 0.0
    assert np.all(e == 0.0)


def test_bucket_errors_packed_sequences_skip_empty():
    """Packed [1, T, H, D] with cu_seqlens: one bucket per (sequence, head); an
    empty sequence has none.  Sequences (2, 0, 1) tokens, H = 2, D = 4."""
    cu = [0, 2, 2, 3]
    ref = np.ones((1, 3, 2, 4))
    x = ref.copy()
    x[0, 2, 1, :] = 3.0   # sequence 2 (its one token), head 1: ||(2,2,2,2)|| / ||(1,1,1,1)|| = 2
    x[0, 0, 0, 0] = 0.0   # sequence 0, head 0: 1 / sqrt(8)
    e = bucket_errors(x, ref, "tokens", cu=cu)
    assert e.shape == (4,)  # 2 non-empty sequences x 2 heads
    assert e[0] == pytest.approx(1.0 / math.sqrt(8.0), rel=1e-14)
    assert e[1] == 0.0 and e[2] == 0.0
    assert e[3] == pytest.approx(2.0, rel=1e-14)


def test_bucket_errors_state_and_step_layouts():
    N, H, Dk, Dv = 2, 3, 4, 2
    ref = np.full((N, H, Dk, Dv), 2.0)
    x = ref.copy()
    x[0, 2] *= 1.01  # bucket (0, 2): 1e-2
    e = bucket_errors(x, ref, "state").reshape(N, H)
    assert e[0, 2] == pytest.approx(1e-2, rel=1e-12)
    assert np.count_nonzero(e) == 1
    ref = np.ones((2, 3, 4))  # decode output [B, H, D]
    x = ref.copy()
    x[1, 0, 1] = 1.0 + 2.0
    e = bucket_errors(x, ref, "step").reshape(2, 3)
    assert e[1, 0] == pytest.approx(1.0, rel=1e-14) and np.count_nonzero(e) == 1


def test_close_catches_one_bad_head_the_global_norm_hides():
    """One head of 96 at 3e-3 and the rest exact is 3e-3 / sqrt(96) globally:
    within 2e-3, but the bucket check fails."""
    rng = np.random.default_rng(3)
    ref = rng.standard_normal((1, 64, 96, 8))
    x = ref.copy()
    x[:, :, 17] *= 1.0 + 3e-3
    assert oracle.rel_l2(x, ref) < 2e-3
    with pytest.raises(AssertionError):
        close(x, ref, 2e-3, "tokens")
    g, worst = close(x, ref, 4e-3, "tokens")
    assert worst == pytest.approx(3e-3, rel=1e-9)

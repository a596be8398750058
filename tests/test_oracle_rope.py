"""Pins of the oracle's rotary position embedding: the two-dimensional rotation it
reduces to, textbook values at a hand-chosen angle, invariants (identity at
position 0, norm, composition, dependence on the position difference only) and
what it does to attention (no effect when every token shares a position, none
under a common shift of all positions)."""
import numpy as np
import pytest

from oracle import attention as A
from oracle import mask as M
from oracle import rope as R

# textbook values of cos(1) and sin(1)
COS1 = 0.5403023058681398
SIN1 = 0.8414709848078965


def test_position_zero_is_identity():
    r = np.random.default_rng(0)
    x = r.standard_normal((2, 5, 3, 16))
    np.testing.assert_array_equal(R.rope(x, np.zeros((2, 5), np.int64)), x)


@pytest.mark.parametrize("p", [1, 2, 7, 100, 1000])
def test_two_dims_is_a_counterclockwise_rotation(p):
    # d = 2: one pair (0, 1) with frequency base^0 = 1, so the angle is p radians
    r = np.random.default_rng(p)
    x = r.standard_normal((1, 1, 1, 2))
    rot = np.array([[np.cos(p), -np.sin(p)], [np.sin(p), np.cos(p)]])
    ref = rot @ x[0, 0, 0]
    np.testing.assert_allclose(R.rope(x, np.full((1, 1), p))[0, 0, 0], ref, rtol=0, atol=1e-12)


def test_pairing_and_frequency_at_a_known_angle():
    # d = 4, base 10000: dimension 1 pairs with 3 and turns at 10000^(-2/4) = 0.01 rad
    # per position, so at position 100 a unit vector along dimension 1 turns by 1 rad
    x = np.zeros((1, 1, 1, 4))
    x[0, 0, 0, 1] = 1.0
    y = R.rope(x, np.full((1, 1), 100))[0, 0, 0]
    np.testing.assert_allclose(y, [0.0, COS1, 0.0, SIN1], rtol=0, atol=1e-12)
    # dimension 0 pairs with 2 at frequency 1: position 1 turns it by 1 rad
    x = np.zeros((1, 1, 1, 4))
    x[0, 0, 0, 0] = 1.0
    y = R.rope(x, np.full((1, 1), 1))[0, 0, 0]
    np.testing.assert_allclose(y, [COS1, 0.0, SIN1, 0.0], rtol=0, atol=1e-12)


def test_norms_of_pairs_are_kept():
    r = np.random.default_rng(1)
    x = r.standard_normal((2, 7, 4, 32))
    pos = r.integers(0, 5000, (2, 7))
    y = R.rope(x, pos)
    pn = lambda a: a[..., :16] ** 2 + a[..., 16:] ** 2
    np.testing.assert_allclose(pn(y), pn(x), rtol=1e-12, atol=1e-12)


def test_composition_adds_positions():
    r = np.random.default_rng(2)
    x = r.standard_normal((1, 6, 2, 64))
    a = r.integers(0, 900, (1, 6))
    b = r.integers(0, 900, (1, 6))
    np.testing.assert_allclose(R.rope(R.rope(x, a), b), R.rope(x, a + b), rtol=0, atol=1e-10)


@pytest.mark.parametrize("d", [8, 64, 256])
def test_scores_depend_on_position_difference_only(d):
    r = np.random.default_rng(d)
    q = r.standard_normal((1, 1, 1, d))
    k = r.standard_normal((1, 1, 1, d))
    for m, n in [(5, 3), (300, 17), (17, 300), (1000, 999)]:
        lhs = float(np.sum(R.rope(q, np.full((1, 1), m)) * R.rope(k, np.full((1, 1), n))))
        rhs = float(np.sum(R.rope(q, np.full((1, 1), m - n)) * k))
        assert abs(lhs - rhs) <= 1e-10 * (1 + abs(rhs))


def test_attention_unchanged_when_all_tokens_share_a_position():
    r = np.random.default_rng(3)
    B, n, Hq, Hkv, d = 2, 13, 8, 1, 32
    ar = (r.random(n) < 0.3).astype(np.uint8)
    valid = (r.random((B, n)) < 0.9).astype(np.uint8)
    q = r.standard_normal((B, n, Hq, d))
    k = r.standard_normal((B, n, Hkv, d))
    v = r.standard_normal((B, n, Hkv, d))
    m = M.attn_mask(valid, ar)
    pos = np.full((B, n), 41)
    o = R.joint_attention_rope(q, k, v, m, pos)
    ref = A.masked_attention(q, k, v, m)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-10)


def test_attention_unchanged_under_a_common_shift():
    r = np.random.default_rng(4)
    B, n, Hq, Hkv, d = 2, 17, 8, 1, 64
    ar = (r.random(n) < 0.3).astype(np.uint8)
    valid = (r.random((B, n)) < 0.9).astype(np.uint8)
    q = r.standard_normal((B, n, Hq, d))
    k = r.standard_normal((B, n, Hkv, d))
    v = r.standard_normal((B, n, Hkv, d))
    m = M.attn_mask(valid, ar)
    pos = M.positions(valid)
    o = R.joint_attention_rope(q, k, v, m, pos)
    o2 = R.joint_attention_rope(q, k, v, m, pos + 250)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-10)
    # and rotation does change the result when positions differ
    assert np.abs(o - A.masked_attention(q, k, v, m)).max() > 1e-3

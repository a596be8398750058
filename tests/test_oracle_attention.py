"""Pins of the oracle's masked GQA attention: a library special case (torch's
scaled-dot-product attention in float64), closed forms, invariances and the
cache semantics of the decode."""
import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import mask as M
from prefix_lm_joint_amd import inputs as I


def _sdpa(q, k, v, m):
    """torch SDPA (float64, CPU, bool mask) with KV heads repeated for GQA."""
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    rep = Hq // Hkv
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(rep, dim=1)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(rep, dim=1)
    tm = torch.from_numpy(m)[:, None, :, :]
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=tm)
    return o.permute(0, 2, 1, 3).numpy()


@pytest.mark.parametrize("Hq,Hkv,d", [(8, 1, 32), (4, 2, 16), (3, 3, 8)])
@pytest.mark.parametrize("seed", range(3))
def test_matches_sdpa(Hq, Hkv, d, seed):
    r = np.random.default_rng(seed)
    B, n = 2, 19
    ar = (r.random(n) < 0.3).astype(np.uint8)
    valid = (r.random((B, n)) < 0.85).astype(np.uint8)
    q = r.standard_normal((B, n, Hq, d))
    k = r.standard_normal((B, n, Hkv, d))
    v = r.standard_normal((B, n, Hkv, d))
    m = M.attn_mask(valid, ar)
    o = A.masked_attention(q, k, v, m)
    ref = _sdpa(q, k, v, m)
    has = m.any(axis=2)
    np.testing.assert_allclose(o[has], ref[has], rtol=1e-12, atol=1e-12)
    assert (o[~has] == 0).all()


def test_single_visible_key_returns_its_value():
    r = np.random.default_rng(1)
    B, n, Hq, Hkv, d = 1, 9, 8, 1, 16
    q, k, v = (r.standard_normal((B, n, h, d)) for h in (Hq, Hkv, Hkv))
    m = np.zeros((B, n, n), bool)
    for i in range(n):
        m[0, i, (3 * i + 1) % n] = True
    o = A.masked_attention(q, k, v, m)
    for i in range(n):
        for h in range(Hq):
            assert np.array_equal(o[0, i, h], v[0, (3 * i + 1) % n, 0])


def test_equal_values_return_that_row():
    r = np.random.default_rng(2)
    B, n, d = 2, 13, 8
    q = r.standard_normal((B, n, 8, d))
    k = r.standard_normal((B, n, 1, d))
    row = r.standard_normal(d)
    v = np.broadcast_to(row, (B, n, 1, d)).copy()
    s = I.pi0_structure(8, 4)
    o = A.masked_attention(q, k, v, M.attn_mask(np.ones((B, n), np.uint8), s.ar))
    np.testing.assert_allclose(o, np.broadcast_to(row, o.shape), rtol=1e-14, atol=1e-14)


def test_zero_query_gives_mean_of_visible_values():
    r = np.random.default_rng(3)
    B, n, d = 1, 15, 8
    s = I.pi0_structure(10, 4)
    m = M.attn_mask(np.ones((B, n), np.uint8), s.ar)
    q = np.zeros((B, n, 8, d))
    k = r.standard_normal((B, n, 1, d))
    v = r.standard_normal((B, n, 1, d))
    o = A.masked_attention(q, k, v, m)
    for i in range(n):
        want = v[0, m[0, i], 0].mean(axis=0)
        np.testing.assert_allclose(o[0, i, 0], want, rtol=1e-13, atol=1e-13)


def test_masked_keys_cannot_leak_even_nan():
    """Prefix rows are unchanged when the suffix K/V (which the prefix may not
    read) is replaced by anything, NaN included (exclusion by selection)."""
    r = np.random.default_rng(4)
    B, P, S, d = 2, 10, 6, 16
    s = I.pi0_structure(P, S - 1)
    n = P + S
    valid = np.ones((B, n), np.uint8)
    valid[1, 7:P] = 0
    q = r.standard_normal((B, n, 8, d))
    k = r.standard_normal((B, n, 1, d))
    v = r.standard_normal((B, n, 1, d))
    o1 = A.joint_attention(q, k, v, valid, s.ar)
    k2, v2 = k.copy(), v.copy()
    k2[:, P:] = np.nan
    v2[:, P:] = np.inf
    k2[1, 7:P] = np.nan   # padded prefix keys, too
    o2 = A.joint_attention(q, k2, v2, valid, s.ar)
    assert np.array_equal(o1[:, :P], o2[:, :P])
    assert (o1[1, 7:P] == 0).all()


def test_permutation_inside_bidirectional_block_is_equivariant():
    r = np.random.default_rng(5)
    B, P, S, d = 1, 12, 6, 16
    s = I.pi0_structure(P, S - 1)
    n = P + S
    q = r.standard_normal((B, n, 8, d))
    k = r.standard_normal((B, n, 1, d))
    v = r.standard_normal((B, n, 1, d))
    ones = np.ones((B, n), np.uint8)
    o = A.joint_attention(q, k, v, ones, s.ar)
    perm = np.arange(n)
    perm[:P] = r.permutation(P)          # shuffle the bidirectional prefix block
    perm[P + 1:] = P + 1 + r.permutation(S - 1)   # and the action block
    op = A.joint_attention(q[:, perm], k[:, perm], v[:, perm], ones, s.ar)
    np.testing.assert_allclose(op, o[:, perm], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", range(3))
def test_cached_decode_equals_joint_suffix_rows(seed):
    """The KV-cache path gives the suffix rows of the full joint pass."""
    r = np.random.default_rng(seed)
    B, P, S, d = 2, 14, 7, 16
    s = I.pi0_structure(P, S - 1)
    pre = np.ones((B, P), np.uint8)
    pre[0, 10:] = 0
    valid = np.concatenate([pre, np.ones((B, S), np.uint8)], axis=1)
    q = r.standard_normal((B, P + S, 8, d))
    k = r.standard_normal((B, P + S, 1, d))
    v = r.standard_normal((B, P + S, 1, d))
    full = A.joint_attention(q, k, v, valid, s.ar)
    dec = A.cached_decode(q[:, P:], k[:, P:], v[:, P:], k[:, :P], v[:, :P], pre, s.ar[P:])
    np.testing.assert_allclose(dec, full[:, P:], rtol=1e-12, atol=1e-12)

"""Masked grouped-query attention over one shared KV pool (oracle, float64).

Definitions followed:
  * "π0.5 vs MM-DiT joint attention", first section: each stream computes its
    own Q/K/V; they are concatenated along the token axis into one pool and a
    single softmax (one shared denominator) runs over it.  Both experts use
    8 query heads, 1 KV head and head_dim 256.
  * "VLA 代码精读 — OpenPI & StarVLA", §1.6: the prefix is run once and its
    K/V kept; each denoising step runs only the suffix queries against the
    cached prefix K/V plus the suffix's own K/V.

Readings (the pages are silent on these):
  * scale = 1/sqrt(head_dim).
  * a masked key is excluded from the softmax by selection: it never enters
    the maximum or the sum, so its K/V values cannot affect any output.
  * a query with no visible key (a padded query) outputs zeros.
  * query head h reads KV head floor(h * Hkv / Hq).
"""
import numpy as np

from . import mask as _mask


def attention_row(q_row, k, v, visible, scale):
    """Output [Hq, d] of one query token.

    q_row [Hq, d]; k, v [Nk, Hkv, d]; visible bool [Nk].  Only the visible
    keys are gathered, so masked K/V never enter a product or a sum.
    """
    Hq, d = q_row.shape
    Hkv = k.shape[1]
    out = np.zeros((Hq, d), np.float64)
    idx = np.nonzero(visible)[0]
    if idx.size == 0:
        return out
    rep = Hq // Hkv
    for g in range(Hkv):
        heads = slice(g * rep, (g + 1) * rep)           # query heads reading KV head g
        kk = k[idx, g, :]                               # [n, d]
        vv = v[idx, g, :]
        s = scale * (q_row[heads] @ kk.T)               # [rep, n]
        w = np.exp(s - s.max(axis=1, keepdims=True))
        out[heads] = (w @ vv) / w.sum(axis=1, keepdims=True)
    return out


def masked_attention(q, k, v, m, scale=None, rows=None) -> np.ndarray:
    """q [B,Nq,Hq,d], k/v [B,Nk,Hkv,d], m bool [B,Nq,Nk] -> O [B,Nq,Hq,d] (float64).

    ``rows`` optionally restricts the work to a list of (b, i) query tokens;
    other rows of the result are left as NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    m = np.asarray(m, dtype=bool)
    B, Nq, Hq, d = q.shape
    _, Nk, Hkv, dk = k.shape
    assert dk == d and v.shape == k.shape and m.shape == (B, Nq, Nk)
    assert Hq % Hkv == 0
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    if rows is None:
        out = np.zeros((B, Nq, Hq, d), np.float64)
        rows = [(b, i) for b in range(B) for i in range(Nq)]
    else:
        out = np.full((B, Nq, Hq, d), np.nan)
    for b, i in rows:
        out[b, i] = attention_row(q[b, i], k[b], v[b], m[b, i], scale)
    return out


def joint_attention(q, k, v, input_mask, ar, seg=None, forbid=(), scale=None, rows=None) -> np.ndarray:
    """Joint attention of every token of the pool under the block prefix-LM mask."""
    m = _mask.attn_mask(input_mask, ar, seg, forbid)
    return masked_attention(q, k, v, m, scale, rows)


def cached_decode(q_s, k_s, v_s, cache_k, cache_v, prefix_mask, suffix_ar, suffix_mask=None,
                  scale=None, rows=None) -> np.ndarray:
    """Suffix queries q_s [B,S,Hq,d] over cache_k/v [B,P,Hkv,d] ++ k_s/v_s [B,S,Hkv,d].

    The mask is the decode mask of §1.6: prefix padding repeated over the
    suffix rows, then the suffix block mask.
    """
    q_s = np.asarray(q_s, dtype=np.float64)
    B, S = q_s.shape[:2]
    if suffix_mask is None:
        suffix_mask = np.ones((B, S), np.uint8)
    m = _mask.decode_mask(prefix_mask, suffix_mask, suffix_ar)
    kk = np.concatenate([np.asarray(cache_k, np.float64), np.asarray(k_s, np.float64)], axis=1)
    vv = np.concatenate([np.asarray(cache_v, np.float64), np.asarray(v_s, np.float64)], axis=1)
    return masked_attention(q_s, kk, vv, m, scale, rows)


def allowed_pairs(m) -> int:
    """Number of visible (query token, key token) entries of a mask."""
    return int(np.asarray(m, dtype=bool).sum())

"""Explicit attention masks and positions (oracle).

Definitions followed:
  * "VLA 代码精读 — OpenPI & StarVLA", §1.2 (prefix-suffix attention mask):
    a token whose ar flag is True cannot be seen by any earlier token; a token
    whose flag is False shares attention with the tokens before it.  §1.5 and
    "π0.5 vs MM-DiT joint attention" (three-block section) state the rule as:
    key j is visible from query i iff cumsum(ar)[j] <= cumsum(ar)[i].
  * §1.5: the mask is AND-ed with padding (both tokens valid); positions are
    cumsum(input_mask) - 1.  "Pi0-FAST 模型架构" §2.3 step 5 does the same AND.
  * §1.6: the decode mask for the suffix queries is the prefix padding mask
    repeated over the suffix rows, concatenated with the suffix's own block
    mask; suffix positions continue from the number of valid prefix tokens.
  * "π0.5 vs MM-DiT joint attention", three-block permission table: the expert
    block may not read the FAST block.  The cumsum rule alone lets it (the FAST
    block precedes the expert block), so forbidden (query segment, key segment)
    pairs are removed explicitly.

Readings: ar is one flag per token shared by the batch (it is concatenated
along the token axis while input_mask is per sample); cumsum is inclusive.
"""
import numpy as np


def block_ids(ar) -> np.ndarray:
    """Inclusive running count of block-opening tokens: c[i] = sum_{t<=i} ar[t]."""
    ar = np.asarray(ar).astype(np.int64)
    return np.cumsum(ar)


def attn_mask(input_mask, ar, seg=None, forbid=()) -> np.ndarray:
    """bool [B, N, N]: M[b,i,j] = c[j] <= c[i] and valid[b,i] and valid[b,j]
    and (seg[i], seg[j]) not in ``forbid``."""
    valid = np.asarray(input_mask).astype(bool)
    B, N = valid.shape
    c = block_ids(ar)
    assert c.shape == (N,)
    causal_blocks = c[None, :] <= c[:, None]                  # [N(i), N(j)]
    pad = valid[:, :, None] & valid[:, None, :]               # [B, i, j]
    m = causal_blocks[None, :, :] & pad
    if seg is not None and len(forbid) > 0:
        seg = np.asarray(seg).astype(np.int64)
        banned = np.zeros((N, N), bool)
        for qs, ks in forbid:
            banned |= (seg[:, None] == qs) & (seg[None, :] == ks)
        m &= ~banned[None, :, :]
    return m


def positions(input_mask) -> np.ndarray:
    """int64 [B, N]: running count of valid tokens minus one."""
    return np.cumsum(np.asarray(input_mask).astype(np.int64), axis=1) - 1


def decode_mask(prefix_mask, suffix_mask, suffix_ar) -> np.ndarray:
    """bool [B, S, P+S]: repeat(prefix_mask over the S suffix rows) ++ the
    suffix's own block mask (padding-AND-ed among suffix tokens)."""
    prefix_mask = np.asarray(prefix_mask).astype(bool)
    suffix_mask = np.asarray(suffix_mask).astype(bool)
    B, P = prefix_mask.shape
    S = suffix_mask.shape[1]
    pre = np.broadcast_to(prefix_mask[:, None, :], (B, S, P))
    suf = attn_mask(suffix_mask, suffix_ar)
    return np.concatenate([pre, suf], axis=-1)


def decode_positions(prefix_mask, suffix_mask) -> np.ndarray:
    """int64 [B, S]: number of valid prefix tokens + cumsum(suffix_mask) - 1."""
    npre = np.asarray(prefix_mask).astype(np.int64).sum(axis=-1)
    return npre[:, None] + np.cumsum(np.asarray(suffix_mask).astype(np.int64), axis=-1) - 1

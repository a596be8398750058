"""Rotary position embedding of Q and K at the mask's token positions (oracle, float64).

Definitions followed:
  * "VLA 代码精读 — OpenPI & StarVLA", §3.2 (design-decision table, position
    encoding row): π0 uses the rotary embedding built into its LLM, on both the
    prefix and the suffix expert.
  * §1.5: in the joint forward the token positions are cumsum(input_mask) - 1.
    §1.6: in the cached decode the suffix positions continue from the number of
    valid prefix tokens: sum(prefix_mask) + cumsum(suffix_mask) - 1.  The
    positions themselves come from oracle.mask.positions / decode_positions.

Reading (the pages give no formula): the standard rotary embedding in its
"rotate half" arrangement.  For head dimension d (even) and base b (10000),
dimension i < d/2 is paired with i + d/2 and rotated by the angle p * b^(-2i/d)
for a token at position p:

    x'[i]       = x[i] cos(a_i) - x[i + d/2] sin(a_i)
    x'[i + d/2] = x[i + d/2] cos(a_i) + x[i] sin(a_i),   a_i = p * b^(-2i/d).

Every head of a token is rotated by the same angles; Q and K are rotated before
the scores, V is not.
"""
import numpy as np

from . import attention as _attn


def rope_angles(pos, d: int, base: float = 10000.0) -> np.ndarray:
    """Angles a[..., i] = pos * base^(-2i/d), i < d/2, for integer positions ``pos``."""
    assert d % 2 == 0
    inv_freq = base ** (-(2.0 * np.arange(d // 2, dtype=np.float64)) / d)
    return np.asarray(pos, dtype=np.float64)[..., None] * inv_freq


def rope(x, pos, base: float = 10000.0) -> np.ndarray:
    """Rotate x [B, N, H, d] at positions pos [B, N] (float64 result)."""
    x = np.asarray(x, dtype=np.float64)
    B, N, H, d = x.shape
    a = rope_angles(pos, d, base)                     # [B, N, d/2]
    assert a.shape == (B, N, d // 2)
    c = np.cos(a)[:, :, None, :]
    s = np.sin(a)[:, :, None, :]
    lo, hi = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def joint_attention_rope(q, k, v, m, pos, base: float = 10000.0, scale=None) -> np.ndarray:
    """Joint attention with Q and K rotated at the joint positions (§1.5)."""
    return _attn.masked_attention(rope(q, pos, base), rope(k, pos, base), v, m, scale=scale)

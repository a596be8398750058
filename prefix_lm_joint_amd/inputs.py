"""Seeded synthetic inputs for the block prefix-LM joint-attention path.

This module is the only code shared by the HIP path's callers and the fp64
oracle: it draws random numbers and lays out token structure (which tokens
open a new block, which are padding, which segment a token belongs to). It
contains none of the method's arithmetic -- no cumulative sums, no masks, no
softmax, no Euler steps. Every tensor is produced as bf16 bit patterns
(uint16, round-to-nearest-even from float32) so that both sides read the very
same values; ``bf16_bits_to_f64`` upcasts them exactly for the oracle.

Workload shapes follow the pages:
  * "VLA 代码精读 — OpenPI & StarVLA", §1.1/§1.4: 256 image tokens per camera,
    a suffix of one state token plus a 50-step action chunk, action dim 32.
  * "π0.5 vs MM-DiT joint attention" (hebangwen), section on the three-block
    π0.5 sequence and the cost table: 3×256 patches + instruction + discrete
    state as prefix, a FAST block and a 50×32 expert chunk; 10 Euler steps;
    MM-DiT with 4096 patches + 154 text tokens over 28 steps.
  * "Pi0-FAST 模型架构", §6: 8 query heads, 1 KV head, head_dim 256, 18 layers.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

SEG_PREFIX = 0
SEG_FAST = 1
SEG_EXPERT = 2


def rng(seed: int) -> np.random.Generator:
    """PCG64 generator for ``seed``."""
    return np.random.Generator(np.random.PCG64(seed))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact upcast of bf16 bit patterns to float64."""
    u = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def bf16_normal(seed: int, shape, std: float = 1.0) -> np.ndarray:
    """N(0, std^2) samples rounded to bf16; returns uint16 bits."""
    x = rng(seed).standard_normal(shape, dtype=np.float32) * np.float32(std)
    return f32_to_bf16_bits(x)


def f32_normal(seed: int, shape, std: float = 1.0) -> np.ndarray:
    x = rng(seed).standard_normal(shape, dtype=np.float32) * np.float32(std)
    return x.astype(np.float32)


def valid_lengths(seed: int, batch: int, lo: int, hi: int) -> np.ndarray:
    """Per-sample valid prefix lengths, uniform on the integers [lo, hi]."""
    return rng(seed).integers(lo, hi + 1, size=batch).astype(np.int32)


def tail_padding_mask(lengths: np.ndarray, n: int) -> np.ndarray:
    """uint8 [B, n] with ones on slots [0, len_b) and zeros after (right padding)."""
    idx = np.arange(n)[None, :]
    return (idx < np.asarray(lengths)[:, None]).astype(np.uint8)


# ---------------------------------------------------------------------------
# Token structure of each workload.  ``ar`` marks the tokens that open a new
# block (True) or join the current one (False); ``seg`` tags the segment.
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class Structure:
    ar: np.ndarray            # uint8 [N]
    seg: np.ndarray           # uint8 [N]
    forbid: tuple             # ((query_seg, key_seg), ...) pairs that may never attend
    n_prefix: int

    @property
    def n(self) -> int:
        return int(self.ar.shape[0])


def pi0_structure(n_prefix: int, n_actions: int) -> Structure:
    """Prefix (all join one block), then a state token and an action chunk.

    State opens a block; the first action opens a block; the remaining actions
    join it ("VLA 代码精读", §1.2, prefix-suffix mask).
    """
    ar = np.concatenate([np.zeros(n_prefix), [1, 1], np.zeros(n_actions - 1)]).astype(np.uint8)
    seg = np.concatenate([np.zeros(n_prefix), np.full(n_actions + 1, SEG_EXPERT)]).astype(np.uint8)
    return Structure(ar=ar, seg=seg, forbid=(), n_prefix=n_prefix)


def pi05_structure(n_prefix: int, n_fast: int, n_expert: int) -> Structure:
    """π0.5 three-block sequence: prefix, FAST tokens (each opens a block),
    expert chunk (first opens a block); the expert may not read FAST
    ("π0.5 vs MM-DiT joint attention", three-block permission table)."""
    ar = np.concatenate([np.zeros(n_prefix), np.ones(n_fast), [1], np.zeros(n_expert - 1)]).astype(np.uint8)
    seg = np.concatenate([np.full(n_prefix, SEG_PREFIX), np.full(n_fast, SEG_FAST),
                          np.full(n_expert, SEG_EXPERT)]).astype(np.uint8)
    return Structure(ar=ar, seg=seg, forbid=((SEG_EXPERT, SEG_FAST),), n_prefix=n_prefix)


def fast_structure(n_obs: int, n_actions: int) -> Structure:
    """π0-FAST: observation tokens bidirectional, every action token opens a
    block (causal among actions) ("Pi0-FAST 模型架构", §2.3)."""
    ar = np.concatenate([np.zeros(n_obs), np.ones(n_actions)]).astype(np.uint8)
    seg = np.concatenate([np.zeros(n_obs), np.full(n_actions, SEG_FAST)]).astype(np.uint8)
    return Structure(ar=ar, seg=seg, forbid=(), n_prefix=n_obs)


def bidirectional_structure(n: int) -> Structure:
    """All tokens in one block (MM-DiT joint attention)."""
    return Structure(ar=np.zeros(n, np.uint8), seg=np.zeros(n, np.uint8), forbid=(), n_prefix=n)


def forbid_bits(pairs) -> int:
    """Bit (4*query_seg + key_seg) set for every forbidden (query, key) segment pair."""
    bits = 0
    for qs, ks in pairs:
        bits |= 1 << (4 * int(qs) + int(ks))
    return bits


# ---------------------------------------------------------------------------
# Workload presets
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class Workload:
    name: str
    B: int
    structure: Structure
    Hq: int = 8
    Hkv: int = 1
    d: int = 256
    pad_lo: Optional[int] = None     # prefix valid length range (None: no padding)
    pad_hi: Optional[int] = None
    layers: int = 1
    steps: int = 10
    horizon: int = 50
    action_dim: int = 32
    width: int = 1024
    seed_base: int = 0

    @property
    def N(self) -> int:
        return self.structure.n

    def input_mask(self) -> np.ndarray:
        """uint8 [B, N]; prefix tail padding when a length range is set, suffix always valid."""
        n, p = self.N, self.structure.n_prefix
        if self.pad_lo is None:
            return np.ones((self.B, n), np.uint8)
        lens = valid_lengths(self.seed_base + 99, self.B, self.pad_lo, self.pad_hi)
        m = np.ones((self.B, n), np.uint8)
        m[:, :p] = tail_padding_mask(lens, p)
        return m

    def qkv(self, layer: int = 0, n: Optional[int] = None):
        """bf16 bits for Q [B,n,Hq,d], K and V [B,n,Hkv,d], unit variance."""
        n = self.N if n is None else n
        s = self.seed_base + 16 * layer
        q = bf16_normal(s + 1, (self.B, n, self.Hq, self.d))
        k = bf16_normal(s + 2, (self.B, n, self.Hkv, self.d))
        v = bf16_normal(s + 3, (self.B, n, self.Hkv, self.d))
        return q, k, v


def tiny() -> Workload:
    return Workload("tiny", B=1, structure=pi0_structure(32, 8), horizon=8, action_dim=4,
                    seed_base=1000)


def pi0_step() -> Workload:
    return Workload("pi0_control_step", B=1, structure=pi0_structure(3 * 256 + 48, 50),
                    layers=18, seed_base=2000)


def pi05_train() -> Workload:
    return Workload("pi05_three_block_prefill", B=32, structure=pi05_structure(3 * 256 + 48 + 32, 64, 50),
                    pad_lo=600, pad_hi=3 * 256 + 48 + 32, seed_base=3000)


def serving_decode() -> Workload:
    return Workload("batched_cached_decode", B=64, structure=pi0_structure(3 * 256 + 48, 50),
                    pad_lo=600, pad_hi=3 * 256 + 48, layers=18, seed_base=4000)


def mmdit() -> Workload:
    return Workload("mmdit_full_bidirectional", B=2, structure=bidirectional_structure(4096 + 154),
                    Hq=24, Hkv=24, d=64, steps=28, seed_base=5000)


WORKLOADS = {w().name: w for w in (tiny, pi0_step, pi05_train, serving_decode, mmdit)}


# ---------------------------------------------------------------------------
# Velocity-net weights (random init; no trained weights exist here)
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class NetWeights:
    """Random weights of the stand-in velocity net, nn.Linear layout [out, in].

    Matrices are bf16 bits with N(0, 1/fan_in) entries; vectors are float32.
    """
    w_state: np.ndarray   # [W, A]
    b_state: np.ndarray   # [W]
    w_in: np.ndarray      # [W, A]
    b_in: np.ndarray      # [W]
    w_time: np.ndarray    # [W]
    w_q: np.ndarray       # [Hq*d, W]
    w_k: np.ndarray       # [Hkv*d, W]
    w_v: np.ndarray       # [Hkv*d, W]
    w_o: np.ndarray       # [W, Hq*d]
    w_out: np.ndarray     # [A, W]
    b_out: np.ndarray     # [A]


def net_weights(seed: int, width: int = 1024, action_dim: int = 32, Hq: int = 8, Hkv: int = 1,
                d: int = 256, bias_std: float = 0.1) -> NetWeights:
    W, A = width, action_dim
    return NetWeights(
        w_state=bf16_normal(seed + 1, (W, A), A ** -0.5),
        b_state=f32_normal(seed + 2, (W,), bias_std),
        w_in=bf16_normal(seed + 3, (W, A), A ** -0.5),
        b_in=f32_normal(seed + 4, (W,), bias_std),
        w_time=f32_normal(seed + 5, (W,), 1.0),
        w_q=bf16_normal(seed + 6, (Hq * d, W), W ** -0.5),
        w_k=bf16_normal(seed + 7, (Hkv * d, W), W ** -0.5),
        w_v=bf16_normal(seed + 8, (Hkv * d, W), W ** -0.5),
        w_o=bf16_normal(seed + 9, (W, Hq * d), (Hq * d) ** -0.5),
        w_out=bf16_normal(seed + 10, (A, W), W ** -0.5),
        b_out=f32_normal(seed + 11, (A,), bias_std),
    )


def layer_weights(seed: int, width: int, adaptive: bool, Hq: int = 8, Hkv: int = 1, d: int = 256,
                  ffn_mult: int = 4) -> dict:
    """Random weights of one stream of a joint transformer layer: fused QKV
    [Hq*d + 2*Hkv*d, W], output projection [W, Hq*d], FFN up [ffn_mult*W, W] and
    down [W, ffn_mult*W] (bf16 bits, N(0, 1/fan_in)); per-channel norm scales
    norm1 / norm2 (fp32, N(1, 0.1^2)) for a plain-norm stream, or modulation
    matrices mod1 / mod2 [2W, W] (bf16 bits, N(0, 0.25/W)) for an adaptive one."""
    W, F = width, ffn_mult * width
    w = {
        "w_qkv": bf16_normal(seed + 1, ((Hq + 2 * Hkv) * d, W), W ** -0.5),
        "w_o": bf16_normal(seed + 2, (W, Hq * d), (Hq * d) ** -0.5),
        "w_up": bf16_normal(seed + 3, (F, W), W ** -0.5),
        "w_down": bf16_normal(seed + 4, (W, F), F ** -0.5),
    }
    if adaptive:
        w["mod1"] = bf16_normal(seed + 5, (2 * W, W), 0.5 * W ** -0.5)
        w["mod2"] = bf16_normal(seed + 6, (2 * W, W), 0.5 * W ** -0.5)
    else:
        w["norm1"] = (np.float32(1.0) + f32_normal(seed + 5, (W,), 0.1)).astype(np.float32)
        w["norm2"] = (np.float32(1.0) + f32_normal(seed + 6, (W,), 0.1)).astype(np.float32)
    return w


def expert_net_weights(seed: int, width: int = 1024, action_dim: int = 32, layers: int = 18, Hq: int = 8,
                       Hkv: int = 1, d: int = 256, ffn_mult: int = 4, bias_std: float = 0.1) -> dict:
    """Random weights of π0.5's action expert at its true shape: action in-projection
    w_in [W, A] with bias b_in [W], time MLP w_t1 / w_t2 [W, W] with biases b_t1 /
    b_t2 [W], `layers` adaptive-norm expert layers (layer_weights), the final
    norm's modulation mod_f [2W, W] and the action out-projection w_out [A, W]
    with bias b_out [A].  Matrices are bf16 bits N(0, 1/fan_in) (mod_f
    N(0, 0.25/W)); biases fp32 N(0, bias_std^2)."""
    W, A = width, action_dim
    return {
        "w_in": bf16_normal(seed + 1, (W, A), A ** -0.5),
        "b_in": f32_normal(seed + 2, (W,), bias_std),
        "w_t1": bf16_normal(seed + 3, (W, W), W ** -0.5),
        "b_t1": f32_normal(seed + 4, (W,), bias_std),
        "w_t2": bf16_normal(seed + 5, (W, W), W ** -0.5),
        "b_t2": f32_normal(seed + 6, (W,), bias_std),
        "layers": [layer_weights(seed + 100 * (l + 1), W, True, Hq, Hkv, d, ffn_mult) for l in range(layers)],
        "mod_f": bf16_normal(seed + 7, (2 * W, W), 0.5 * W ** -0.5),
        "w_out": bf16_normal(seed + 8, (A, W), W ** -0.5),
        "b_out": f32_normal(seed + 9, (A,), bias_std),
    }

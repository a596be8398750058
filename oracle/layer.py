"""One π0.5 joint transformer layer around the joint attention (oracle, float64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definitions followed:
  * "π0.5 vs MM-DiT joint attention", first section: in a block the two streams
    each have their own norm, QKV projection, output projection and FFN; each
    stream computes its own Q/K/V, the token axes are concatenated into one KV
    pool, one softmax runs over it under the mask, and the output is split back
    to the streams.  The prefix (VLM) stream is 2048 wide, the action expert
    1024 wide; both have 8 query heads, 1 KV head, head_dim 256.
  * "VLA 代码精读 — OpenPI & StarVLA" §1.4: in π0.5 the expert stream normalises
    with adaRMSNorm conditioned on the flow time (a time MLP feeds it); the
    prefix stream uses a plain RMS norm.  §2.7 prints the adaptive norm's form:
    shift and scale from a linear map of silu(time embedding), then
    norm(h) * (1 + scale) + shift.

Readings (the pages leave these open):
  L1  RMS norm n(h) = h / sqrt(mean(h^2) + 1e-6) over the width; the plain
      stream scales it per channel: a = n(h) * gamma.
  L2  adaptive RMS norm: [shift | scale] = silu(c) W_mod^T (W_mod [2W, W], no
      bias), a = n(h) * (1 + scale) + shift, with c the sample's conditioning
      vector.  Each of the layer's two norms has its own parameters.
  L3  pre-norm residual block: h += Attn(norm1(h)); h += FFN(norm2(h)).
  L4  FFN(x) = gelu(x W_up^T) W_down^T, hidden width 4W, exact gelu x*Phi(x).
  L5  q, k, v = a W_qkv^T split Hq*d | Hkv*d | Hkv*d (one fused projection); no
      biases; no rotary embedding.
  L6  bf16 rounding points (every matrix product takes bf16 operands): the
      norm outputs a, silu(c), q / k / v, the attention output and the FFN's
      gelu output are rounded to bf16 (r below); products accumulate exactly;
      the residual stream h is kept unrounded.
"""
import numpy as np
from scipy.special import erf

from . import attention as _attn
from .bf16 import round_bf16

RMS_EPS = 1e-6


def rms_norm(h) -> np.ndarray:
    """h / sqrt(mean(h^2) + eps) over the last axis (L1)."""
    h = np.asarray(h, np.float64)
    return h / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + RMS_EPS)


def silu(x) -> np.ndarray:
    x = np.asarray(x, np.float64)
    return x / (1.0 + np.exp(-x))


def gelu(x) -> np.ndarray:
    """x * Phi(x), Phi the standard normal CDF (L4)."""
    x = np.asarray(x, np.float64)
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def _lin(a, w):
    """a [..., in] @ w[out, in]^T."""
    return np.asarray(a, np.float64) @ np.asarray(w, np.float64).T


def modulation(c, w_mod, r=round_bf16):
    """(shift, scale), each [B, W], from the conditioning c [B, W] (L2)."""
    ss = _lin(r(silu(c)), w_mod)
    W = ss.shape[-1] // 2
    return ss[:, :W], ss[:, W:]


def stream_norm(h, p, which: int, c=None, r=round_bf16):
    """The stream's norm `which` (1 before attention, 2 before the FFN) of h [B, T, W],
    rounded to bf16: plain (L1) when p has 'norm{which}', adaptive (L2) otherwise."""
    n = rms_norm(h)
    if p.get(f"norm{which}") is not None:
        return r(n * np.asarray(p[f"norm{which}"], np.float64))
    shift, scale = modulation(c, p[f"mod{which}"], r)
    return r(n * (1.0 + scale[:, None, :]) + shift[:, None, :])


def _round_fn(rounding):
    return round_bf16 if rounding else (lambda x: np.asarray(x, np.float64))


def stream_qkv(h, p, c=None, Hq=8, Hkv=1, d=256, rounding=True):
    """The stream's pooled inputs (q [B,T,Hq,d], k / v [B,T,Hkv,d]) = r(norm1(h) W_qkv^T), split (L5)."""
    r = _round_fn(rounding)
    h = np.asarray(h, np.float64)
    B, T = h.shape[:2]
    y = r(_lin(stream_norm(h, p, 1, c, r), p["w_qkv"]))
    return (y[..., :Hq * d].reshape(B, T, Hq, d), y[..., Hq * d:(Hq + Hkv) * d].reshape(B, T, Hkv, d),
            y[..., (Hq + Hkv) * d:].reshape(B, T, Hkv, d))


def stream_out(h, o, p, c=None, rounding=True):
    """The stream's half after the attention: h += o W_o^T; h += r(gelu(norm2(h) W_up^T)) W_down^T
    (o [B, T, Hq*d] already rounded)."""
    r = _round_fn(rounding)
    h = np.asarray(h, np.float64) + _lin(o, p["w_o"])
    u = r(gelu(_lin(stream_norm(h, p, 2, c, r), p["w_up"])))
    return h + _lin(u, p["w_down"])


def joint_layer(h_p, h_e, c, wp, we, m, Hq=8, Hkv=1, d=256, scale=None, rounding=True):
    """One layer over the prefix stream h_p [B, Np, Wp] and the expert stream
    h_e [B, Ne, We] (conditioning c [B, We] for an adaptive norm) under the joint
    mask m [B, Np+Ne, Np+Ne]; returns the updated (h_p, h_e).

    wp / we map names to arrays: w_qkv [Hq*d + 2*Hkv*d, W], w_o [W, Hq*d],
    w_up [4W, W], w_down [W, 4W], and either norm1 / norm2 [W] (plain norm) or
    mod1 / mod2 [2W, W] (adaptive norm)."""
    r = _round_fn(rounding)
    B, Np, _ = np.shape(h_p)
    Ne = np.shape(h_e)[1]
    parts = [stream_qkv(h, p, c, Hq, Hkv, d, rounding) for h, p in ((h_p, wp), (h_e, we))]
    q, k, v = (np.concatenate([pt[j] for pt in parts], axis=1) for j in range(3))
    o = r(_attn.masked_attention(q, k, v, m, scale=scale)).reshape(B, Np + Ne, Hq * d)
    return (stream_out(h_p, o[:, :Np], wp, c, rounding), stream_out(h_e, o[:, Np:], we, c, rounding))


def expert_layer_decode(h_e, c, we, cache_k, cache_v, prefix_mask, suffix_ar, Hq=8, Hkv=1, d=256, scale=None,
                        rounding=True):
    """The expert stream's half of one layer in the cached form ("VLA 代码精读"
    §1.6): its S tokens h_e [B, S, W] attend to the valid slots of the cached
    prefix K/V cache_k / cache_v [B, P, Hkv, d] plus their own K/V under the
    suffix block rule (suffix_ar [S]); norms, projections and FFN as joint_layer."""
    r = _round_fn(rounding)
    B, S = np.shape(h_e)[:2]
    q, k, v = stream_qkv(h_e, we, c, Hq, Hkv, d, rounding)
    o = r(_attn.cached_decode(q, k, v, cache_k, cache_v, prefix_mask, suffix_ar, scale=scale))
    return stream_out(h_e, o.reshape(B, S, Hq * d), we, c, rounding)

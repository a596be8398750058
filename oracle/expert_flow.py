"""π0.5 action-expert velocity net at its true shape, and the Euler sampler around it (oracle, float64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definitions followed:
  * "VLA 代码精读 — OpenPI & StarVLA" §1.4: in π0.5 the noisy actions are
    projected to the expert's width (action_in_proj), the flow time goes
    through the expert's own two-layer MLP (time_mlp_in and time_mlp_out, both
    width -> width) whose output conditions the expert's adaptive RMS norms,
    and the expert's outputs of the last H tokens are projected back to the
    action dim (action_out_proj).  §1.6: the prefix K/V are cached once and every
    Euler step runs only the expert tokens against them, layer by layer.  §1.2:
    x starts at the noise, dt = -1/N, the net is evaluated at t_k = 1 + k*dt and
    x <- x + dt*v.
  * "π0.5 vs MM-DiT joint attention", first section: each expert layer (norm,
    fused QKV, attention over the cached prefix plus the expert tokens, output
    projection, FFN) -- oracle.layer.expert_layer_decode.

Readings (the pages leave these open):
  E1  time embedding of a scalar t into the width W: for j < W/2 the period
      p_j = 4e-3 * 1000^(j / (W/2 - 1)) (geometric from 4e-3 to 4), and
      emb = [sin(2 pi t / p_j) for j] followed by [cos(2 pi t / p_j) for j].
  E2  time MLP: c = r(silu(r(emb) W_t1^T + b_t1)) W_t2^T + b_t2; no activation
      after the second layer because the adaptive norm applies silu to c
      itself (layer reading L2).  c is the same for every sample of a step.
  E3  the expert's tokens are the H action tokens (π0.5 keeps the robot state
      in the prefix as discrete tokens): h = r(x) W_in^T + b_in.
  E4  after the last layer one more adaptive RMS norm with its own modulation
      matrix mod_f [2W, W] (as the layers' norms, layer reading L2), then
      v = r(that norm) W_out^T + b_out.
  E5  layer l of the net attends to layer l of the cache.
r() rounds to bf16 (every matrix product takes bf16 operands); the residual
stream h stays unrounded.
"""
import numpy as np

from . import flow as _flow
from . import layer as _layer
from .bf16 import round_bf16

P_MIN, P_MAX = 4e-3, 4.0


def time_embedding(t: float, width: int) -> np.ndarray:
    """emb(t) [width] (E1)."""
    half = width // 2
    frac = np.arange(half, dtype=np.float64) / (half - 1)
    period = P_MIN * (P_MAX / P_MIN) ** frac
    ang = 2.0 * np.pi * float(t) / period
    return np.concatenate([np.sin(ang), np.cos(ang)])


def _round_fn(rounding):
    return round_bf16 if rounding else (lambda x: np.asarray(x, np.float64))


def _lin(a, w):
    return np.asarray(a, np.float64) @ np.asarray(w, np.float64).T


def time_cond(t: float, net: dict, rounding=True) -> np.ndarray:
    """The adaptive norms' conditioning c [W] at time t (E2)."""
    r = _round_fn(rounding)
    emb = r(time_embedding(t, net["w_t1"].shape[1]))
    u = r(_layer.silu(_lin(emb, net["w_t1"]) + np.asarray(net["b_t1"], np.float64)))
    return _lin(u, net["w_t2"]) + np.asarray(net["b_t2"], np.float64)


def final_norm(h, c, mod_f, rounding=True) -> np.ndarray:
    """r(n(h) * (1 + scale) + shift), [shift | scale] = r(silu(c)) mod_f^T (E4)."""
    r = _round_fn(rounding)
    return _layer.stream_norm(h, {"mod2": mod_f}, 2, c, r)


def expert_velocity(x, t, net, cache_k, cache_v, prefix_mask, suffix_ar, rounding=True, scale=None, Hq=8, Hkv=1,
                    d=256) -> np.ndarray:
    """v [B, H, A] of the expert net at time t for noisy actions x [B, H, A].

    net: w_in [W, A], b_in [W], w_t1 / w_t2 [W, W], b_t1 / b_t2 [W], layers (a
    list of expert-layer weight dicts with mod1 / mod2, see oracle.layer),
    mod_f [2W, W], w_out [A, W], b_out [A].  cache_k / cache_v [layers, B, P,
    Hkv, d]; prefix_mask [B, P]; suffix_ar [H]."""
    r = _round_fn(rounding)
    x = np.asarray(x, np.float64)
    B = x.shape[0]
    h = _lin(r(x), net["w_in"]) + np.asarray(net["b_in"], np.float64)
    c = np.broadcast_to(time_cond(t, net, rounding), (B, h.shape[-1]))
    for l, wl in enumerate(net["layers"]):
        h = _layer.expert_layer_decode(h, c, wl, cache_k[l], cache_v[l], prefix_mask, suffix_ar, Hq, Hkv, d,
                                       scale=scale, rounding=rounding)
    a = final_norm(h, c, net["mod_f"], rounding)
    return _lin(a, net["w_out"]) + np.asarray(net["b_out"], np.float64)


def expert_flow_sample(noise, net, cache_k, cache_v, prefix_mask, suffix_ar, num_steps=10, rounding=True, Hq=8,
                       Hkv=1, d=256):
    """The Euler sampler (oracle.flow.euler_sample) driving expert_velocity."""
    return _flow.euler_sample(
        noise, lambda x, t: expert_velocity(x, t, net, cache_k, cache_v, prefix_mask, suffix_ar, rounding, None, Hq,
                                            Hkv, d),
        num_steps)

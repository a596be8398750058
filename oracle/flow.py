"""Euler flow-matching sampler and the stand-in velocity net (oracle, float64).

Definitions followed ("VLA 代码精读 — OpenPI & StarVLA"):
  * §1.2 (flow matching, Euler sampling): in openpi's convention t = 1 is pure
    noise and t = 0 the action; dt = -1/N; x starts at the noise; each of the
    N steps evaluates v at time 1 + step*dt and sets x <- x + dt*v.
  * §1.2: the regression target velocity is noise - action.
  * §1.6: the loop runs while t >= -dt/2, which for every N >= 1 gives
    exactly N steps.

Readings: the step count is fixed at N and the time fed to the net is
t_k = 1 + k*dt evaluated in float64 (the two formulations on the page agree
on the count).
"""
import numpy as np

from . import attention as _attn
from .bf16 import round_bf16


def euler_update(x, v, dt) -> np.ndarray:
    """One Euler step x + dt*v."""
    return np.asarray(x, np.float64) + float(dt) * np.asarray(v, np.float64)


def time_grid(num_steps: int) -> np.ndarray:
    """Times t_k = 1 + k*dt, k = 0..N-1, dt = -1/N."""
    dt = -1.0 / num_steps
    return np.array([1.0 + k * dt for k in range(num_steps)], np.float64)


def euler_sample(noise, velocity, num_steps: int = 10) -> np.ndarray:
    """x_0 = noise; for k < N: x <- x + dt * velocity(x, t_k)."""
    dt = -1.0 / num_steps
    x = np.array(noise, dtype=np.float64, copy=True)
    for t in time_grid(num_steps):
        x = euler_update(x, velocity(x, t), dt)
    return x


# ---------------------------------------------------------------------------
# Stand-in velocity net.  The pages give neither the weights nor the exact
# layer of the action expert; this is a random-weight stand-in with the
# expert's head geometry, so its definition is a reading.  It is pinned to
# that reading, not to the pages' numbers: a float64 composition of library
# calls (F.linear, scaled_dot_product_attention with a hand-built mask,
# vector_norm), a closed form with the attention path zeroed, and the state
# token at row 0.  Its definition:
#
#   tokens      h[:,0]   = r(state) W_state^T + b_state            (state token)
#               h[:,1+i] = r(x_i) W_in^T + b_in + t * w_time        (action tokens)
#   18 layers   a = r(h); q = r(a W_q^T / rms(a)); k, v likewise
#               o = r(cached_decode(q, k, v, cache layer l));  h += o W_o^T
#   output      a = r(h); v_out = a[:,1:] W_out^T / rms(a[:,1:]) + b_out
#
# r(.) rounds to bf16: every matrix product takes bf16 operands and
# accumulates exactly; the attention reads and writes bf16.  rms(a) =
# sqrt(mean(a^2) + 1e-6) over the width, taken on the same bf16 activations the
# projection reads: an RMS norm before the projections ("π0.5 vs MM-DiT joint
# attention", first section: each stream has its own norm ahead of its QKV and
# output projections).  The norm is a per-row scalar, so it is applied to the product (exactly equal in real
# arithmetic to normalising first).  Without it the residual stream of a
# random-weight stack grows geometrically with depth.  One weight set is shared
# by all layers; layer l attends to cache layer l.
# ---------------------------------------------------------------------------

RMS_EPS = 1e-6


def rms(h) -> np.ndarray:
    """sqrt(mean(h^2) + eps) over the last axis, keeping it as a size-1 axis."""
    h = np.asarray(h, np.float64)
    return np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + RMS_EPS)


def _lin(a, w):
    """a [..., in] @ w[out, in]^T in float64."""
    return np.asarray(a, np.float64) @ np.asarray(w, np.float64).T


def embed_suffix(x, t, state, w) -> np.ndarray:
    """Suffix tokens h [B, 1+H, W]: state token then the action tokens at time t."""
    st = _lin(round_bf16(state), w["w_state"]) + w["b_state"]           # [B, W]
    act = _lin(round_bf16(x), w["w_in"]) + w["b_in"] + float(t) * w["w_time"]  # [B, H, W]
    return np.concatenate([st[:, None, :], act], axis=1)


def velocity_net(x, t, state, w, cache_k, cache_v, prefix_mask, suffix_ar, Hq, Hkv, d,
                 layers=None, return_trace=False):
    """Velocity [B, H, A] for actions x [B, H, A] at time t.

    ``w`` maps names to float64 arrays (bf16 values upcast); cache_k/v are
    [layers, B, P, Hkv, d].
    """
    h = embed_suffix(x, t, state, w)
    B, S, W = h.shape
    L = cache_k.shape[0] if layers is None else layers
    trace = []
    for layer in range(L):
        a = round_bf16(h)
        r_h = rms(a)
        q = round_bf16(_lin(a, w["w_q"]) / r_h).reshape(B, S, Hq, d)
        k = round_bf16(_lin(a, w["w_k"]) / r_h).reshape(B, S, Hkv, d)
        v = round_bf16(_lin(a, w["w_v"]) / r_h).reshape(B, S, Hkv, d)
        o = round_bf16(_attn.cached_decode(q, k, v, cache_k[layer], cache_v[layer], prefix_mask, suffix_ar))
        h = h + _lin(o.reshape(B, S, Hq * d), w["w_o"])
        if return_trace:
            trace.append(dict(q=q, k=k, v=v, o=o, h=h.copy()))
    a = round_bf16(h[:, 1:, :])
    vel = _lin(a, w["w_out"]) / rms(a) + w["b_out"]
    if return_trace:
        return vel, trace
    return vel

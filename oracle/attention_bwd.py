"""Gradients of the masked grouped-query attention (oracle, float64).

Training runs the same joint forward ("VLA 代码精读 — OpenPI & StarVLA", §1.5:
compute_loss calls the joint forward over [prefix, suffix] under the block mask,
and the loss is differentiated through it); this module gives the backward of
oracle.attention.masked_attention.

For one query row (sample b, token i, head h) with visible keys J, KV head
g = floor(h * Hkv / Hq), scores s_j = scale * q . k_j (j in J), weights
p = softmax(s) and output o = sum_j p_j v_j.  With the upstream gradient
u = dL/do of that row (the definitions of the derivative, written out):

    dv_j += p_j u                     (j in J; summed over the rows reading head g)
    dp_j  = u . v_j
    ds_j  = p_j (dp_j - sum_l p_l dp_l),   and sum_l p_l dp_l = u . o
    dq    = scale * sum_j ds_j k_j
    dk_j += scale * ds_j q

A row with no visible key has o = 0 by definition and contributes nothing.
Keys outside J receive nothing from that row.

Also: the natural-log log-sum-exp of each row's visible scaled scores (the
statistic a forward pass keeps for its backward), -inf for a row with none.

With the rotary embedding (oracle.rope: q and k rotated at their positions
before the scores, each pair (i, i + d/2) by an orthogonal 2x2 rotation R(p)),
the chain rule gives the gradients of the unrotated inputs as the transposed
rotation of the rotated inputs' gradients, and R(p)^T = R(-p).
"""
import numpy as np

from . import rope as _rope


def lse_rows(q, k, m, scale=None) -> np.ndarray:
    """[B, N, Hq]: log sum_j exp(scale q_i . k_j) over the visible keys j (or -inf)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    m = np.asarray(m, dtype=bool)
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    rep = Hq // Hkv
    out = np.full((B, N, Hq), -np.inf)
    for b in range(B):
        for i in range(N):
            idx = np.nonzero(m[b, i])[0]
            if idx.size == 0:
                continue
            for h in range(Hq):
                s = scale * (k[b, idx, h // rep, :] @ q[b, i, h])
                mx = s.max()
                out[b, i, h] = mx + np.log(np.exp(s - mx).sum())
    return out


def masked_attention_grads(q, k, v, m, u, scale=None):
    """(dq [B,N,Hq,d], dk [B,Nk,Hkv,d], dv [B,Nk,Hkv,d]) for upstream gradient u = dL/dO."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    m = np.asarray(m, dtype=bool)
    B, N, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    assert m.shape == (B, N, Nk) and u.shape == q.shape and Hq % Hkv == 0
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    rep = Hq // Hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for i in range(N):
            idx = np.nonzero(m[b, i])[0]
            if idx.size == 0:
                continue
            for h in range(Hq):
                g = h // rep
                kk, vv = k[b, idx, g, :], v[b, idx, g, :]
                s = scale * (kk @ q[b, i, h])
                p = np.exp(s - s.max())
                p /= p.sum()
                o = p @ vv
                dp = vv @ u[b, i, h]
                ds = p * (dp - u[b, i, h] @ o)
                dv[b, idx, g, :] += p[:, None] * u[b, i, h][None, :]
                dq[b, i, h] = scale * (ds @ kk)
                dk[b, idx, g, :] += scale * ds[:, None] * q[b, i, h][None, :]
    return dq, dk, dv


def masked_attention_grads_rope(q, k, v, m, u, pos, base=10000.0, scale=None):
    """(dq, dk, dv) of the attention with q and k rotated at positions pos [B, N]
    (oracle.rope.joint_attention_rope), for upstream gradient u."""
    pos = np.asarray(pos)
    dq, dk, dv = masked_attention_grads(_rope.rope(q, pos, base), _rope.rope(k, pos, base), v, m, u, scale)
    return _rope.rope(dq, -pos, base), _rope.rope(dk, -pos, base), dv

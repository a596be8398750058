"""Pins of the oracle's attention gradients: central finite differences of the
forward (brute force on tiny inputs), torch autograd through torch's own scaled
dot-product attention in float64 (a library special case), and the structural
facts (masked keys and key-less rows get nothing, GQA sums the heads of a KV
head, the log-sum-exp against scipy)."""
import numpy as np
import pytest
import scipy.special
import torch

from oracle import attention as A
from oracle import attention_bwd as G
from oracle import mask as M


def _case(seed, B, n, Hq, Hkv, d, p_ar=0.3, p_valid=0.85):
    r = np.random.default_rng(seed)
    ar = (r.random(n) < p_ar).astype(np.uint8)
    valid = (r.random((B, n)) < p_valid).astype(np.uint8)
    q = r.standard_normal((B, n, Hq, d))
    k = r.standard_normal((B, n, Hkv, d))
    v = r.standard_normal((B, n, Hkv, d))
    u = r.standard_normal((B, n, Hq, d))
    return q, k, v, u, M.attn_mask(valid, ar)


@pytest.mark.parametrize("Hq,Hkv", [(2, 1), (2, 2)])
def test_matches_finite_differences(Hq, Hkv):
    q, k, v, u, m = _case(0, 1, 7, Hq, Hkv, 4)
    dq, dk, dv = G.masked_attention_grads(q, k, v, m, u)
    loss = lambda q_, k_, v_: float(np.sum(u * A.masked_attention(q_, k_, v_, m)))
    h = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": (q, k, v), "k": (q, k, v), "v": (q, k, v)}[name]
            a_p = [xp if nm == name else a for nm, a in zip("qkv", args)]
            a_m = [xm if nm == name else a for nm, a in zip("qkv", args)]
            fd[idx] = (loss(*a_p) - loss(*a_m)) / (2 * h)
        np.testing.assert_allclose(grad, fd, rtol=1e-6, atol=1e-8, err_msg=name)


def _torch_grads(q, k, v, m, u):
    B, N, Hq, d = q.shape
    rep = Hq // k.shape[2]
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    kk = tk.permute(0, 2, 1, 3).repeat_interleave(rep, dim=1)
    vv = tv.permute(0, 2, 1, 3).repeat_interleave(rep, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(tq.permute(0, 2, 1, 3), kk, vv,
                                                         attn_mask=torch.from_numpy(m)[:, None])
    (o.permute(0, 2, 1, 3) * torch.from_numpy(u)).sum().backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("Hq,Hkv,d", [(8, 1, 32), (4, 2, 16)])
def test_matches_torch_autograd(Hq, Hkv, d):
    # every row sees at least itself here (all tokens valid), so torch has no empty rows
    q, k, v, u, m = _case(1, 2, 23, Hq, Hkv, d, p_valid=1.1)
    assert m.any(axis=2).all()
    got = G.masked_attention_grads(q, k, v, m, u)
    want = _torch_grads(q, k, v, m, u)
    for g_, w_, nm in zip(got, want, "qkv"):
        np.testing.assert_allclose(g_, w_, rtol=1e-10, atol=1e-12, err_msg=nm)


def test_masked_keys_and_keyless_rows_get_nothing():
    q, k, v, u, m = _case(2, 2, 19, 8, 1, 8)
    m = m.copy()
    m[:, :, 3] = False            # key 3 seen by no row
    m[0, 5, :] = False            # row 5 of sample 0 sees nothing
    dq, dk, dv = G.masked_attention_grads(q, k, v, m, u)
    assert (dk[:, 3] == 0).all() and (dv[:, 3] == 0).all()
    assert (dq[0, 5] == 0).all()


def test_gqa_sums_the_heads_of_a_kv_head():
    q, k, v, u, m = _case(3, 1, 17, 8, 1, 8)
    dq, dk, dv = G.masked_attention_grads(q, k, v, m, u)
    # the same problem with the KV head repeated per query head (MHA)
    dq8, dk8, dv8 = G.masked_attention_grads(q, np.repeat(k, 8, axis=2), np.repeat(v, 8, axis=2), m, u)
    np.testing.assert_allclose(dq, dq8, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dk[:, :, 0], dk8.sum(axis=2), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dv[:, :, 0], dv8.sum(axis=2), rtol=1e-12, atol=1e-12)


def test_lse_rows_against_scipy():
    q, k, v, u, m = _case(4, 2, 21, 4, 2, 8)
    lse = G.lse_rows(q, k, m)
    d = q.shape[-1]
    for b in range(2):
        for i in range(21):
            for h in range(4):
                s = (k[b, :, h // 2] @ q[b, i, h]) / np.sqrt(d)
                if m[b, i].any():
                    assert abs(lse[b, i, h] - scipy.special.logsumexp(s[m[b, i]])) < 1e-12
                else:
                    assert lse[b, i, h] == -np.inf


def test_rope_gradients_match_finite_differences():
    """Gradients through the rotary embedding: the transposed rotation of the
    rotated inputs' gradients equals central differences of the rotated forward."""
    from oracle import rope as R
    q, k, v, u, m = _case(5, 1, 6, 2, 1, 4)
    pos = np.array([[0, 3, 4, 9, 11, 17]])
    dq, dk, dv = G.masked_attention_grads_rope(q, k, v, m, u, pos, base=100.0)
    loss = lambda q_, k_, v_: float(np.sum(u * R.joint_attention_rope(q_, k_, v_, m, pos, 100.0)))
    h = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            a_p = [xp if nm == name else a for nm, a in zip("qkv", (q, k, v))]
            a_m = [xm if nm == name else a for nm, a in zip("qkv", (q, k, v))]
            fd[idx] = (loss(*a_p) - loss(*a_m)) / (2 * h)
        np.testing.assert_allclose(grad, fd, rtol=1e-6, atol=1e-8, err_msg=name)

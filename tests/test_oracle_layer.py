"""Pins of the joint-layer oracle (oracle/layer.py): its norm and activation
against torch's library routines, the adaptive norm's shift/scale order and its
reduction to the plain norm, the whole layer against a float64 composition of
torch's rms_norm / linear / scaled_dot_product_attention / gelu, the residual
identity, and the stream routing through the mask (a stream that cannot see the
other is bit-independent of it)."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import layer as Y
from oracle import mask as M
from prefix_lm_joint_amd import inputs as I

Hq, Hkv, d = 2, 1, 16


def _weights(seed, W, adaptive):
    w = I.layer_weights(seed, W, adaptive, Hq=Hq, Hkv=Hkv, d=d)
    return {k: (I.bf16_bits_to_f64(v) if v.dtype == np.uint16 else v.astype(np.float64)) for k, v in w.items()}


def _case(seed=0, B=2, Np=9, Ne=5, Wp=32, We=24):
    r = np.random.default_rng(seed)
    h_p = r.standard_normal((B, Np, Wp))
    h_e = r.standard_normal((B, Ne, We))
    c = r.standard_normal((B, We))
    s = I.pi05_structure(Np - 3, 3, Ne)
    valid = np.ones((B, Np + Ne), np.uint8)
    valid[0, Np - 4] = 0                  # one padded prefix token
    m = M.attn_mask(valid, s.ar, s.seg, s.forbid)
    return h_p, h_e, c, _weights(10, Wp, False), _weights(20, We, True), m


def test_rms_norm_and_gelu_match_torch():
    x = np.random.default_rng(1).standard_normal((5, 7, 48)) * 3
    want = F.rms_norm(torch.from_numpy(x), (48,), eps=Y.RMS_EPS).numpy()
    np.testing.assert_allclose(Y.rms_norm(x), want, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(Y.gelu(x), F.gelu(torch.from_numpy(x)).numpy(), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(Y.gelu(x) - Y.gelu(-x), x, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(Y.silu(x), F.silu(torch.from_numpy(x)).numpy(), rtol=1e-13, atol=1e-13)


def test_adaptive_norm_shift_then_scale():
    """[shift | scale] = silu(c) W_mod^T: a one-hot conditioning picks one column of
    W_mod, whose first half shifts and second half scales."""
    W = 6
    r = np.random.default_rng(2)
    h = r.standard_normal((1, 3, W))
    c = np.zeros((1, W))
    c[0, 0] = 1.3
    s_shift, s_scale = r.standard_normal(W), r.standard_normal(W)
    w_mod = np.zeros((2 * W, W))
    w_mod[:W, 0], w_mod[W:, 0] = s_shift, s_scale
    g = 1.3 / (1.0 + np.exp(-1.3))
    ident = lambda x: np.asarray(x, np.float64)
    got = Y.stream_norm(h, {"mod1": w_mod}, 1, c, ident)
    want = Y.rms_norm(h) * (1.0 + g * s_scale) + g * s_shift
    np.testing.assert_allclose(got, want, rtol=1e-14, atol=1e-14)
    # zero modulation is the plain RMS norm
    np.testing.assert_allclose(Y.stream_norm(h, {"mod1": np.zeros((2 * W, W))}, 1, c, ident), Y.rms_norm(h),
                               rtol=0, atol=0)


def _torch_layer(h_p, h_e, c, wp, we, m):
    """The same layer as a float64 composition of torch library calls."""
    T = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    B, Np, _ = h_p.shape
    qs, ks, vs = [], [], []

    def norm(h, p, which):
        n = F.rms_norm(h, (h.shape[-1],), eps=Y.RMS_EPS)
        if f"norm{which}" in p:
            return n * T(p[f"norm{which}"])
        ss = F.linear(F.silu(T(c)), T(p[f"mod{which}"]))
        shift, scale = ss.chunk(2, dim=-1)
        return n * (1 + scale[:, None]) + shift[:, None]

    for h, p in ((T(h_p), wp), (T(h_e), we)):
        y = F.linear(norm(h, p, 1), T(p["w_qkv"]))
        q, k, v = y.split([Hq * d, Hkv * d, Hkv * d], dim=-1)
        qs.append(q.reshape(B, -1, Hq, d))
        ks.append(k.reshape(B, -1, Hkv, d))
        vs.append(v.reshape(B, -1, Hkv, d))
    q, k, v = (torch.cat(t, dim=1).transpose(1, 2) for t in (qs, ks, vs))
    k = k.repeat_interleave(Hq // Hkv, dim=1)
    v = v.repeat_interleave(Hq // Hkv, dim=1)
    mm = T(m).bool()[:, None]
    o = F.scaled_dot_product_attention(q, k, v, attn_mask=mm)
    o = torch.where(mm.any(-1, keepdim=True), o, torch.zeros_like(o))      # key-less rows: 0
    o = o.transpose(1, 2).reshape(B, -1, Hq * d)
    out = []
    for h, p, sl in ((T(h_p), wp, slice(0, Np)), (T(h_e), we, slice(Np, None))):
        h = h + F.linear(o[:, sl], T(p["w_o"]))
        h = h + F.linear(F.gelu(F.linear(norm(h, p, 2), T(p["w_up"]))), T(p["w_down"]))
        out.append(h.numpy())
    return out


def test_layer_matches_torch_composition():
    h_p, h_e, c, wp, we, m = _case()
    got = Y.joint_layer(h_p, h_e, c, wp, we, m, Hq, Hkv, d, rounding=False)
    want = _torch_layer(h_p, h_e, c, wp, we, m)
    for g, w_ in zip(got, want):
        np.testing.assert_allclose(g, w_, rtol=1e-11, atol=1e-11)


def test_zero_output_projections_leave_the_residual_stream():
    h_p, h_e, c, wp, we, m = _case(3)
    for p in (wp, we):
        p["w_o"] = np.zeros_like(p["w_o"])
        p["w_down"] = np.zeros_like(p["w_down"])
    got = Y.joint_layer(h_p, h_e, c, wp, we, m, Hq, Hkv, d)
    assert np.array_equal(got[0], h_p) and np.array_equal(got[1], h_e)


def test_prefix_stream_cannot_see_the_expert():
    """Under the π0.5 mask no prefix or FAST row sees an expert key: the prefix
    stream's output is bit-independent of the expert's tokens, weights and time."""
    h_p, h_e, c, wp, we, m = _case(4)
    a = Y.joint_layer(h_p, h_e, c, wp, we, m, Hq, Hkv, d)[0]
    we2 = _weights(99, h_e.shape[-1], True)
    b = Y.joint_layer(h_p, h_e * -2.0 + 1.0, c + 5.0, wp, we2, m, Hq, Hkv, d)[0]
    assert np.array_equal(a, b)


def test_expert_reads_the_prefix_through_the_pool():
    """The expert's output does depend on the prefix stream (it sees the prefix
    keys), and with the expert-to-prefix pairs removed from the mask it no longer
    does."""
    h_p, h_e, c, wp, we, m = _case(5)
    Np = h_p.shape[1]
    a = Y.joint_layer(h_p, h_e, c, wp, we, m, Hq, Hkv, d)[1]
    b = Y.joint_layer(h_p + 1.0, h_e, c, wp, we, m, Hq, Hkv, d)[1]
    assert np.abs(a - b).max() > 1e-3
    m2 = m.copy()
    m2[:, Np:, :Np] = False
    a2 = Y.joint_layer(h_p, h_e, c, wp, we, m2, Hq, Hkv, d)[1]
    b2 = Y.joint_layer(h_p + 1.0, h_e, c, wp, we, m2, Hq, Hkv, d)[1]
    assert np.array_equal(a2, b2)


@pytest.mark.parametrize("seed", [6, 7])
def test_rounding_points_move_the_result_by_bf16_amounts(seed):
    h_p, h_e, c, wp, we, m = _case(seed)
    a = Y.joint_layer(h_p, h_e, c, wp, we, m, Hq, Hkv, d, rounding=True)
    b = Y.joint_layer(h_p, h_e, c, wp, we, m, Hq, Hkv, d, rounding=False)
    for x, y in zip(a, b):
        rel = np.abs(x - y).max() / np.abs(y).max()
        assert 0 < rel < 2e-2


def _layer_fp32(h_p, h_e, c, wp, we, m, bf16_p=True):
    """The layer's definition in float32 with the same bf16 rounding points (torch
    CPU), and the attention's weights rounded to bf16 before they meet V (as a
    matrix-core PV takes them): what an fp32-accumulating implementation with
    bf16 matrix-core operands gets."""
    def r(a):
        return a.to(torch.bfloat16).to(torch.float32)
    T = lambda a: torch.from_numpy(np.asarray(a, np.float32))
    B, Np, _ = h_p.shape
    mm = torch.from_numpy(np.asarray(m, bool))

    def norm(h, p, which):
        n = h / torch.sqrt((h * h).mean(-1, keepdim=True) + 1e-6)
        if f"norm{which}" in p:
            return r(n * T(p[f"norm{which}"]))
        ss = r(F.silu(T(c))) @ T(p[f"mod{which}"]).T
        W = ss.shape[-1] // 2
        return r(n * (1 + ss[:, None, W:]) + ss[:, None, :W])

    qs, ks, vs = [], [], []
    for h, p in ((T(h_p), wp), (T(h_e), we)):
        y = r(norm(h, p, 1) @ T(p["w_qkv"]).T)
        qs.append(y[..., :2048].reshape(B, -1, 8, 256))
        ks.append(y[..., 2048:2304])
        vs.append(y[..., 2304:])
    q, k, v = torch.cat(qs, 1), torch.cat(ks, 1), torch.cat(vs, 1)
    s = torch.einsum("bqhd,bkd->bqhk", q, k) / 16.0
    s = s.masked_fill(~mm[:, :, None, :], float("-inf"))
    mx = s.amax(-1, keepdim=True).clamp_min(-1e30)
    e = torch.exp(s - mx)
    if bf16_p:
        e = r(e)
    den = e.sum(-1, keepdim=True)
    o = r(torch.where(den > 0, torch.einsum("bqhk,bkd->bqhd", e, v) / den.clamp_min(1e-30), torch.zeros(())))
    o = o.reshape(B, -1, 2048)
    out = []
    for h, p, sl in ((T(h_p), wp, slice(0, Np)), (T(h_e), we, slice(Np, None))):
        h = h + o[:, sl] @ T(p["w_o"]).T
        u = r(F.gelu(norm(h, p, 2) @ T(p["w_up"]).T))
        out.append((h + u @ T(p["w_down"]).T).numpy().astype(np.float64))
    return out


def _real_case(seed, B, P, F_, E, Wp, We):
    s = I.pi05_structure(P, F_, E)
    Np = P + F_
    r = np.random.default_rng(seed + 700)
    valid = np.ones((B, s.n), np.uint8)
    valid[:, :P] = I.tail_padding_mask(r.integers(P // 2, P + 1, B), P)
    h_p = I.f32_normal(seed * 10 + 701, (B, Np, Wp)).astype(np.float64)
    h_e = I.f32_normal(seed * 10 + 702, (B, s.n - Np, We)).astype(np.float64)
    c = I.f32_normal(seed * 10 + 703, (B, We)).astype(np.float64)
    wp = {k: (I.bf16_bits_to_f64(v) if v.dtype == np.uint16 else v.astype(np.float64))
          for k, v in I.layer_weights(seed * 100 + 10, Wp, False).items()}
    we = {k: (I.bf16_bits_to_f64(v) if v.dtype == np.uint16 else v.astype(np.float64))
          for k, v in I.layer_weights(seed * 100 + 20, We, True).items()}
    return h_p, h_e, c, wp, we, M.attn_mask(valid, s.ar, s.seg, s.forbid)


def test_layer_tolerance_is_twice_the_fp32_floor():
    """Derives the layer bound the GPU tests use: an fp32 evaluation of the same
    definition (bf16 rounding points, bf16 attention weights into PV) sits this
    far from the fp64 oracle, because accumulation-order differences move values
    across bf16 rounding points (one ulp of an intermediate each).  The GPU bound
    is about twice that floor."""
    from tests.gpu_util import LAYER_MAX_ABS, LAYER_MEAN_ABS
    worst_mean = worst_max = 0.0
    for args in ((0, 2, 30, 10, 13, 512, 256), (3, 1, 120, 16, 50, 2048, 1024)):
        h_p, h_e, c, wp, we, m = _real_case(*args)
        want = Y.joint_layer(h_p, h_e, c, wp, we, m)
        got = _layer_fp32(h_p, h_e, c, wp, we, m)
        for g, w_ in zip(got, want):
            err = np.abs(g - w_)
            worst_mean, worst_max = max(worst_mean, float(err.mean())), max(worst_max, float(err.max()))
    assert 2e-4 < worst_mean < 2e-3 and worst_max < 2e-2
    assert 1.5 * worst_mean <= LAYER_MEAN_ABS <= 3.0 * worst_mean
    assert 1.5 * worst_max <= LAYER_MAX_ABS


def test_expert_decode_equals_the_joint_layers_expert_rows():
    """With the cache holding the prefix stream's K/V of the same layer, the cached
    form of the expert's layer is bit-identical to the expert rows of the joint
    layer (the prefix rows cannot see the expert, so the prefix is computed once)."""
    B, P, S, Wp, We = 2, 11, 6, 32, 24
    r = np.random.default_rng(8)
    h_p, h_e, c = r.standard_normal((B, P, Wp)), r.standard_normal((B, S, We)), r.standard_normal((B, We))
    wp, we = _weights(30, Wp, False), _weights(40, We, True)
    s = I.pi0_structure(P, S - 1)
    valid = np.ones((B, P + S), np.uint8)
    valid[1, P - 3:P] = 0
    m = M.attn_mask(valid, s.ar, s.seg, s.forbid)
    want = Y.joint_layer(h_p, h_e, c, wp, we, m, Hq, Hkv, d)[1]
    _, ck, cv = Y.stream_qkv(h_p, wp, None, Hq, Hkv, d)
    got = Y.expert_layer_decode(h_e, c, we, ck, cv, valid[:, :P], s.ar[P:], Hq, Hkv, d)
    assert np.array_equal(got, want)
    # and the cache's padded slots do not matter
    ck2, cv2 = ck.copy(), cv.copy()
    ck2[1, P - 3:] = 1e3
    cv2[1, P - 3:] = -1e3
    assert np.array_equal(Y.expert_layer_decode(h_e, c, we, ck2, cv2, valid[:, :P], s.ar[P:], Hq, Hkv, d), got)

"""Pins of the π0.5 expert-sampler oracle (oracle/expert_flow.py): the time
embedding's special values, the time MLP and the layer-free net against torch
library compositions, the wiring of the time conditioning into the (separately
pinned) expert layers, each layer's own cache layer, the zero-out-projection
closed forms of the velocity and of the sampler, and the fp32 floor the GPU
bound is derived from."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import expert_flow as X
from oracle import layer as Y
from oracle import mask as M
from prefix_lm_joint_amd import inputs as I

Hq, Hkv, d = 2, 1, 16


def _f64(w):
    if isinstance(w, list):
        return [_f64(x) for x in w]
    if isinstance(w, dict):
        return {k: _f64(v) for k, v in w.items()}
    return I.bf16_bits_to_f64(w) if w.dtype == np.uint16 else np.asarray(w, np.float64)


def _case(seed=0, B=2, P=9, H=5, W=32, A=6, layers=2):
    net = _f64(I.expert_net_weights(seed, W, A, layers, Hq, Hkv, d))
    r = np.random.default_rng(seed + 1)
    ck = r.standard_normal((max(layers, 1), B, P, Hkv, d))
    cv = r.standard_normal((max(layers, 1), B, P, Hkv, d))
    pm = np.ones((B, P), np.uint8)
    pm[1, P - 3:] = 0
    ar = np.zeros(H, np.uint8)
    ar[0] = 1
    x = r.standard_normal((B, H, A))
    return net, ck, cv, pm, ar, x


def _vel(x, t, net, ck, cv, pm, ar, rounding=True):
    return X.expert_velocity(x, t, net, ck, cv, pm, ar, rounding, None, Hq, Hkv, d)


def test_time_embedding_special_values():
    """t = 0 gives sin 0 and cos 1 exactly; a quarter of frequency j's period puts
    sin at 1 and cos at 0, at both ends and the middle of the geometric range."""
    W = 64
    half = W // 2
    e0 = X.time_embedding(0.0, W)
    assert np.array_equal(e0[:half], np.zeros(half)) and np.array_equal(e0[half:], np.ones(half))
    for j in (0, half // 2, half - 1):
        period = 4e-3 * 1000.0 ** (j / (half - 1))
        e = X.time_embedding(period / 4.0, W)
        assert abs(e[j] - 1.0) < 1e-12 and abs(e[half + j]) < 1e-12
    # the longest period is 4: on [0, 1] its sine rises monotonically
    ts = np.linspace(0.0, 1.0, 11)
    assert np.all(np.diff([X.time_embedding(t, W)[half - 1] for t in ts]) > 0)


def test_time_mlp_matches_torch_composition():
    net = _case(3)[0]
    T = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    for t in (1.0, 0.35, 0.0):
        emb = T(X.time_embedding(t, net["w_t1"].shape[1]))
        want = F.linear(F.silu(F.linear(emb, T(net["w_t1"]), T(net["b_t1"]))), T(net["w_t2"]), T(net["b_t2"]))
        np.testing.assert_allclose(X.time_cond(t, net, rounding=False), want.numpy(), rtol=1e-12, atol=1e-12)


def test_layer_free_net_matches_torch_composition():
    """No layers: in-projection, time MLP, final adaptive norm and out-projection
    as torch library calls (rms_norm, linear, silu) in float64."""
    net, ck, cv, pm, ar, x = _case(4, layers=0)
    T = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    t = 0.7
    h = F.linear(T(x), T(net["w_in"]), T(net["b_in"]))
    emb = T(X.time_embedding(t, h.shape[-1]))
    c = F.linear(F.silu(F.linear(emb, T(net["w_t1"]), T(net["b_t1"]))), T(net["w_t2"]), T(net["b_t2"]))
    shift, scale = F.linear(F.silu(c), T(net["mod_f"])).chunk(2)
    a = F.rms_norm(h, (h.shape[-1],), eps=Y.RMS_EPS) * (1 + scale) + shift
    want = F.linear(a, T(net["w_out"]), T(net["b_out"]))
    np.testing.assert_allclose(_vel(x, t, net, ck, cv, pm, ar, rounding=False), want.numpy(), rtol=1e-11,
                               atol=1e-11)


def test_layers_take_the_time_conditioning():
    """One layer: the net equals in-projection, the pinned expert layer fed the time
    MLP's c (not the embedding, not silu(c)), then the final norm and out-projection."""
    net, ck, cv, pm, ar, x = _case(5, layers=1)
    t = 0.4
    h = X._lin(x, net["w_in"]) + net["b_in"]
    c = np.broadcast_to(X.time_cond(t, net, rounding=False), h.shape[::2])
    h = Y.expert_layer_decode(h, c, net["layers"][0], ck[0], cv[0], pm, ar, Hq, Hkv, d, rounding=False)
    want = X._lin(X.final_norm(h, c, net["mod_f"], rounding=False), net["w_out"]) + net["b_out"]
    np.testing.assert_allclose(_vel(x, t, net, ck, cv, pm, ar, rounding=False), want, rtol=1e-12, atol=1e-12)


def test_each_layer_reads_its_own_cache_layer():
    """A layer with zero output and down projections leaves h unchanged, so a
    two-layer net with one such layer equals the one-layer net of the other layer
    reading that layer's cache slice (and differs if it read the other slice)."""
    net, ck, cv, pm, ar, x = _case(6, layers=2)
    for keep in (0, 1):
        drop = 1 - keep
        n2 = dict(net, layers=[dict(w) for w in net["layers"]])
        n2["layers"][drop]["w_o"] = np.zeros_like(n2["layers"][drop]["w_o"])
        n2["layers"][drop]["w_down"] = np.zeros_like(n2["layers"][drop]["w_down"])
        got = _vel(x, 0.6, n2, ck, cv, pm, ar)
        n1 = dict(net, layers=[net["layers"][keep]])
        assert np.array_equal(got, _vel(x, 0.6, n1, ck[keep:keep + 1], cv[keep:keep + 1], pm, ar))
        assert not np.array_equal(got, _vel(x, 0.6, n1, ck[drop:drop + 1], cv[drop:drop + 1], pm, ar))


def test_time_enters_only_through_the_conditioning():
    net, ck, cv, pm, ar, x = _case(7)
    assert not np.array_equal(_vel(x, 1.0, net, ck, cv, pm, ar), _vel(x, 0.5, net, ck, cv, pm, ar))
    n2 = dict(net, w_t1=np.zeros_like(net["w_t1"]), w_t2=np.zeros_like(net["w_t2"]))
    assert np.array_equal(_vel(x, 1.0, n2, ck, cv, pm, ar), _vel(x, 0.5, n2, ck, cv, pm, ar))


def test_zero_out_projection_velocity_is_the_bias():
    net, ck, cv, pm, ar, x = _case(8)
    net["w_out"] = np.zeros_like(net["w_out"])
    v = _vel(x, 0.3, net, ck, cv, pm, ar)
    assert np.array_equal(v, np.broadcast_to(net["b_out"], v.shape))


@pytest.mark.parametrize("N", [1, 3, 10])
def test_zero_out_projection_sampler_returns_noise_minus_bias(N):
    """Euler with the constant velocity b_out from t = 1 to 0 ends at noise - b_out
    ("VLA 代码精读" §1.2)."""
    net, ck, cv, pm, ar, x = _case(9, layers=1)
    net["w_out"] = np.zeros_like(net["w_out"])
    got = X.expert_flow_sample(x, net, ck, cv, pm, ar, N, True, Hq, Hkv, d)
    np.testing.assert_allclose(got, x - net["b_out"], rtol=0, atol=1e-12)


def test_padded_cache_slots_do_not_matter():
    net, ck, cv, pm, ar, x = _case(10)
    a = _vel(x, 0.8, net, ck, cv, pm, ar)
    ck2, cv2 = ck.copy(), cv.copy()
    ck2[:, 1, -3:] = 1e3
    cv2[:, 1, -3:] = -1e3
    assert np.array_equal(a, _vel(x, 0.8, net, ck2, cv2, pm, ar))


# --------------------------------------------------------------------------
# fp32 floor of the chain at the real heads (Hq = 8, Hkv = 1, d = 256)
# --------------------------------------------------------------------------

def _chain_fp32(x, t, net, ck, cv, pm, ar):
    """The expert velocity's definition in float32 with the same bf16 rounding points
    (torch CPU), attention weights rounded to bf16 before they meet V: what an
    fp32-accumulating implementation with bf16 matrix-core operands gets."""
    def r(a):
        return a.to(torch.bfloat16).to(torch.float32)
    T = lambda a: torch.from_numpy(np.asarray(a, np.float32))
    B, H, _ = x.shape
    W = net["w_in"].shape[0]

    def norm(h, mod, c):
        n = h / torch.sqrt((h * h).mean(-1, keepdim=True) + 1e-6)
        ss = r(F.silu(c)) @ T(mod).T
        return r(n * (1 + ss[:, None, W:]) + ss[:, None, :W])

    h = r(T(x)) @ T(net["w_in"]).T + T(net["b_in"])
    emb = r(T(X.time_embedding(t, W)))
    u = r(F.silu(emb @ T(net["w_t1"]).T + T(net["b_t1"])))
    c = (u @ T(net["w_t2"]).T + T(net["b_t2"]))[None].expand(B, W)
    m = torch.from_numpy(M.decode_mask(pm, np.ones((B, H), np.uint8), ar).astype(bool))
    for l, wl in enumerate(net["layers"]):
        y = r(norm(h, wl["mod1"], c) @ T(wl["w_qkv"]).T)
        q = y[..., :2048].reshape(B, H, 8, 256)
        k = torch.cat([T(ck[l][:, :, 0]), y[..., 2048:2304]], 1)
        v = torch.cat([T(cv[l][:, :, 0]), y[..., 2304:]], 1)
        s = torch.einsum("bqhd,bkd->bqhk", q, k) / 16.0
        s = s.masked_fill(~m[:, :, None, :], float("-inf"))
        e = r(torch.exp(s - s.amax(-1, keepdim=True)))
        o = r(torch.einsum("bqhk,bkd->bqhd", e, v) / e.sum(-1, keepdim=True)).reshape(B, H, 2048)
        h = h + o @ T(wl["w_o"]).T
        g = r(F.gelu(norm(h, wl["mod2"], c) @ T(wl["w_up"]).T))
        h = h + g @ T(wl["w_down"]).T
    v = norm(h, net["mod_f"], c) @ T(net["w_out"]).T + T(net["b_out"])
    return v.numpy().astype(np.float64)


def real_case(seed, B, P, H, layers, W=1024, A=32):
    """A real-width expert net, cache and noisy actions (also the GPU tests' case)."""
    net = I.expert_net_weights(seed, W, A, layers)
    ck = np.stack([I.bf16_normal(seed + 900 + l, (B, P, 1, 256)) for l in range(layers)])
    cv = np.stack([I.bf16_normal(seed + 950 + l, (B, P, 1, 256)) for l in range(layers)])
    r = np.random.default_rng(seed + 990)
    pm = I.tail_padding_mask(r.integers(P // 2, P + 1, B), P)
    ar = np.zeros(H, np.uint8)
    ar[0] = 1
    x = I.f32_normal(seed + 991, (B, H, A))
    return net, ck, cv, pm, ar, x


def test_expert_velocity_tolerance_is_twice_the_fp32_floor():
    """Derives the bound the GPU tests use for one velocity evaluation through two
    real-width expert layers: an fp32 evaluation of the same definition sits this
    far from the fp64 oracle (accumulation order moves values across bf16
    rounding points); the GPU bound is about twice that floor."""
    from tests.gpu_util import EXPERT_VEL_MAX_ABS, EXPERT_VEL_MEAN_ABS
    worst_mean = worst_max = 0.0
    for seed, t in ((11, 1.0), (12, 0.3)):
        net, ck, cv, pm, ar, x = real_case(seed, 2, 40, 50, 2)
        n64 = _f64(net)
        want = X.expert_velocity(x, t, n64, _f64(ck), _f64(cv), pm, ar)
        got = _chain_fp32(x, t, n64, _f64(ck), _f64(cv), pm, ar)
        err = np.abs(got - want)
        worst_mean, worst_max = max(worst_mean, float(err.mean())), max(worst_max, float(err.max()))
    assert 0 < worst_mean < 1e-2 and worst_max < 5e-2
    assert 1.5 * worst_mean <= EXPERT_VEL_MEAN_ABS <= 3.0 * worst_mean
    assert 1.5 * worst_max <= EXPERT_VEL_MAX_ABS

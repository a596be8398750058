"""π0.5 inference at the true layer shapes on the GPU: the prefix stream's layers
alone fill the KV cache (pi_prefix_layer_forward), then the expert sampler runs
against that cache (pi_expert_flow_sample).  Checked against the fp64 oracle:
the prefix pass equals the joint layer with no expert tokens (bit-identical), the
cached K/V equal the oracle's rounded K/V up to one bf16 rounding flip, the
residual stream stays within the layer bound, and the sampler consuming the
GPU-written cache matches the oracle sampler on the same cache."""
import numpy as np
import pytest
import torch

from oracle import expert_flow as X
from oracle import layer as Y
from oracle import mask as M
from prefix_lm_joint_amd import binding as Bd
from prefix_lm_joint_amd import inputs as I
from tests import gpu_util as G
from tests.test_gpu_layer import _dev_stream, _host_stream
from tests.test_oracle_expert_flow import _f64

pytestmark = pytest.mark.gpu


def _prefix_case(seed, B, P, Wp, layers):
    r = np.random.default_rng(seed)
    valid = I.tail_padding_mask(r.integers(P // 2, P + 1, B), P)
    ar = np.zeros(P, np.uint8)
    seg = np.zeros(P, np.uint8)
    h_p = I.f32_normal(seed + 1, (B, P, Wp))
    wps = [I.layer_weights(seed + 100 * (l + 1), Wp, False) for l in range(layers)]
    return valid, ar, seg, h_p, wps


def _run_prefix(valid, ar, seg, h_p, wps):
    B, P, _ = h_p.shape
    L = len(wps)
    m = Bd.pi_mask_build(G.u8_dev(valid), G.u8_dev(ar), G.u8_dev(seg), 0)
    ck = torch.zeros((L, B, P, 1, 256), dtype=torch.bfloat16, device=G.dev())
    cv = torch.zeros_like(ck)
    cache = Bd.KVCache(ck, cv, G.u8_dev(valid), P)
    streams = [_dev_stream(w) for w in wps]
    ws = Bd.prefix_layer_workspace(streams[0], B, P, G.dev())
    hd = G.f32_dev(h_p)
    for l, sp in enumerate(streams):
        Bd.pi_prefix_layer_forward(sp, hd, m, cache, l, ws)
    torch.cuda.synchronize()
    return hd, cache, streams, m


def _bits(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def test_prefix_layer_equals_joint_layer_and_fills_the_cache():
    G.note("pi05 prefix pass: B=2 P=45 Wp=512, 1 layer")
    valid, ar, seg, h_p, wps = _prefix_case(41, 2, 45, 512, 1)
    hd, cache, streams, m = _run_prefix(valid, ar, seg, h_p, wps)
    # the same layer through pi_joint_layer_forward with no expert tokens
    h2 = G.f32_dev(h_p)
    he = torch.zeros((2, 0, 512), dtype=torch.float32, device=G.dev())
    ws = Bd.layer_workspace(streams[0], streams[0], 2, 45, 0, G.dev())
    Bd.pi_joint_layer_forward(streams[0], streams[0], h2, he, None, m, ws)
    torch.cuda.synchronize()
    assert torch.equal(hd, h2)
    wh = _host_stream(wps[0])
    for b in range(2):
        mm = M.attn_mask(valid[b:b + 1], ar, seg, ())
        want = Y.joint_layer(h_p[b:b + 1], np.zeros((1, 0, 512)), None, wh, wh, mm)[0]
        G.assert_close(G.host64(hd)[b:b + 1], want, f"prefix pass b={b}", G.LAYER_MAX_ABS, G.LAYER_MEAN_ABS)
        _, k, v = Y.stream_qkv(h_p[b:b + 1], wh)
        for name, got, ref in (("k", cache.k[0, b:b + 1], k), ("v", cache.v[0, b:b + 1], v)):
            g = I.bf16_bits_to_f64(_bits(got.contiguous()))
            diff = np.abs(g - ref)
            flips = float((diff > 0).mean())
            G.note(f"cache {name} b={b}: rounding flips {100 * flips:.2f} %, worst {float((diff / (np.abs(ref) + 1e-2)).max()):.2e}")
            assert flips < 0.05 and np.all(diff <= 2.0 ** -7 * (np.abs(ref) + 1e-2))


def test_prefix_pass_then_expert_sampler():
    G.note("pi05 pipeline: B=2 P=40, 2 prefix layers (2048), expert sampler 2 layers (1024), 3 steps")
    valid, ar, seg, h_p, wps = _prefix_case(43, 2, 40, 2048, 2)
    hd, cache, _, _ = _run_prefix(valid, ar, seg, h_p, wps)
    net = I.expert_net_weights(45, 1024, 32, 2)
    dnet = Bd.ExpertNet.from_numpy(net, G.dev())
    sar = np.zeros(50, np.uint8)
    sar[0] = 1
    x = I.f32_normal(46, (2, 50, 32))
    xd = G.f32_dev(x)
    Bd.pi_expert_flow_sample(dnet, cache, G.u8_dev(sar), xd, num_steps=3)
    torch.cuda.synchronize()
    ck = I.bf16_bits_to_f64(_bits(cache.k.contiguous()))
    cv = I.bf16_bits_to_f64(_bits(cache.v.contiguous()))
    want = X.expert_flow_sample(x, _f64(net), ck, cv, valid, sar, num_steps=3)
    err = np.abs(G.host64(xd) - want)
    G.note(f"pipeline x: max {err.max():.3e} mean {err.mean():.3e}")
    assert err.max() <= G.EXPERT_VEL_MAX_ABS and err.mean() <= G.EXPERT_VEL_MEAN_ABS
    # and the prefix residual stream after two layers stays within twice the layer bound
    wh = [_host_stream(w) for w in wps]
    mm = M.attn_mask(valid[:1], ar, seg, ())
    hp = h_p[:1].astype(np.float64)
    for w in wh:
        hp = Y.joint_layer(hp, np.zeros((1, 0, 2048)), None, w, w, mm)[0]
    G.assert_close(G.host64(hd)[:1], hp, "prefix pass after 2 layers", 2 * G.LAYER_MAX_ABS, 2 * G.LAYER_MEAN_ABS)

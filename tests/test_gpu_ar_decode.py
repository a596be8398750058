"""Single-token autoregressive decode over the cache ("Pi0-FAST 模型架构" §4.1): each
step decodes one new token against every valid cache slot plus itself, then
appends its K/V to the cache.  Token by token, the outputs must equal the rows
of the joint attention over the whole sequence with the FAST mask (prefix
bidirectional, every generated token opening its own block), with and without
the rotary embedding."""
import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import mask as M
from oracle import rope as R
from prefix_lm_joint_amd import inputs as I
from tests.gpu_util import assert_close, bf16_dev, f64, host64, note, u8_dev

pytestmark = pytest.mark.gpu

BASE = 10000.0


def _bd():
    from prefix_lm_joint_amd import binding as Bd
    return Bd


def _i32_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(torch.device("cuda:0"))


@pytest.mark.parametrize("rope", [0.0, BASE])
@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("seed,B,P,T", [(0, 3, 100, 12), (1, 1, 300, 6)])
def test_ar_decode_matches_joint(seed, B, P, T, split, rope):
    Bd = _bd()
    dev = torch.device("cuda:0")
    s = I.fast_structure(P, T)
    N = s.n
    note(f"ar decode seed={seed} B={B} P={P} T={T} split={split} rope={rope}")
    r = np.random.default_rng(seed + 80)
    valid = np.ones((B, N), np.uint8)
    valid[:, :P] = I.tail_padding_mask(r.integers(P // 2, P + 1, B), P)
    q = I.bf16_normal(seed * 10 + 81, (B, N, 8, 256))
    k = I.bf16_normal(seed * 10 + 82, (B, N, 1, 256))
    v = I.bf16_normal(seed * 10 + 83, (B, N, 1, 256))
    # prefill of the prefix into cache layer 0 (room for the T generated tokens)
    cache = Bd.KVCache.empty(1, B, P + T, 1, 256, dev, length=P)
    cache.prefix_mask.zero_()
    cache.prefix_mask[:, :P].copy_(u8_dev(valid[:, :P]))
    sp = I.Structure(ar=s.ar[:P], seg=s.seg[:P], forbid=s.forbid, n_prefix=P)
    mp = Bd.pi_mask_build(u8_dev(valid[:, :P]), u8_dev(sp.ar), u8_dev(sp.seg), 0)
    wsp = Bd.prefill_workspace(B, P, 8, 1, 256, dev)
    Bd.pi_joint_attn_prefill(bf16_dev(q[:, :P]), bf16_dev(k[:, :P]), bf16_dev(v[:, :P]), mp, cache=cache, layer=0,
                             workspace=wsp, rope_base=rope)
    # the oracle: rows of the joint attention over the whole sequence
    mm = M.attn_mask(valid, s.ar)
    if rope:
        want = R.joint_attention_rope(f64(q), f64(k), f64(v), mm, M.positions(valid), BASE)
    else:
        want = A.masked_attention(f64(q), f64(k), f64(v), mm)
    sar = u8_dev(np.array([1], np.uint8))
    for t in range(T):
        i = P + t
        ws = Bd.decode_workspace(cache, 1)
        if not split:
            ws = ws[: (B * 256 * 2 + 255) // 256 * 256]
        o = Bd.pi_suffix_decode_step(cache, 0, bf16_dev(q[:, i:i + 1]), bf16_dev(k[:, i:i + 1]),
                                     bf16_dev(v[:, i:i + 1]), sar, workspace=ws, rope_base=rope)
        Bd.pi_kv_cache_append(cache, 0, bf16_dev(k[:, i:i + 1]), bf16_dev(v[:, i:i + 1]), rope_base=rope)
        cache.advance(1)
        torch.cuda.synchronize()
        assert_close(host64(o), want[:, i:i + 1], f"ar step {t} seed={seed} split={split} rope={rope}")
    # the appended slots are valid, and hold the (rotated) keys and the values
    assert (cache.prefix_mask[:, P:].cpu().numpy() == 1).all()
    assert torch.equal(cache.v[0, :, P:].cpu().view(torch.int16), torch.from_numpy(v[:, P:].view(np.int16)))
    if rope:
        rot = Bd.pi_rope_apply(bf16_dev(k[:, P:]), _i32_dev(M.positions(valid)[:, P:]), BASE)
        torch.cuda.synchronize()
        assert torch.equal(cache.k[0, :, P:].view(torch.int16), rot.view(torch.int16))
    else:
        assert torch.equal(cache.k[0, :, P:].cpu().view(torch.int16), torch.from_numpy(k[:, P:].view(np.int16)))


def test_ar_decode_serving_shape_sampled():
    """B=64 robots, 816 slots with valid length U[600,816], one new token per sample:
    every row of four samples against the oracle."""
    Bd = _bd()
    w = I.serving_decode()
    s = w.structure
    P, B = s.n_prefix, w.B
    note("ar decode B=64 P=816 sampled")
    pm = w.input_mask()[:, :P]
    ck = I.bf16_normal(5101, (1, B, P, 1, 256))
    cv = I.bf16_normal(5102, (1, B, P, 1, 256))
    qs = I.bf16_normal(5103, (B, 1, 8, 256))
    ks = I.bf16_normal(5104, (B, 1, 1, 256))
    vs = I.bf16_normal(5105, (B, 1, 1, 256))
    cache = Bd.KVCache(bf16_dev(ck), bf16_dev(cv), u8_dev(pm))
    sar = np.array([1], np.uint8)
    ws = Bd.decode_workspace(cache, 1)
    o = host64(Bd.pi_suffix_decode_step(cache, 0, bf16_dev(qs), bf16_dev(ks), bf16_dev(vs), u8_dev(sar),
                                        workspace=ws))
    for b in (0, 21, 42, 63):
        want = A.cached_decode(f64(qs[b:b + 1]), f64(ks[b:b + 1]), f64(vs[b:b + 1]), f64(ck[0, b:b + 1]),
                               f64(cv[0, b:b + 1]), pm[b:b + 1], sar)
        assert_close(o[b:b + 1], want, f"ar decode B=64 sample {b}")

"""Rotary position embedding on the GPU against the fp64 oracle: the standalone
rotation, the prefill with rotated Q/K at the mask's positions (GQA 8:1 and MHA
d=64, unsplit and key-split), the rotated keys it leaves in the cache, and the
cached decode with rotated suffix Q/K equal to the suffix rows of the rotated
joint attention."""
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
# One bf16 ulp of the result plus the fp32 arithmetic: the rotation is computed in
# fp32 from exact bf16 inputs with the angle reduced in fp64, so before the final
# rounding it is within a few 1e-6 of |x| of the exact value; rounding to bf16
# adds at most half an ulp, and a value that close to a rounding boundary can
# land one ulp away.
ROPE_RTOL = 2.0 ** -7
ROPE_ATOL = 1e-4


def _bd():
    from prefix_lm_joint_amd import binding as Bd
    return Bd


def _i32_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(torch.device("cuda:0"))


@pytest.mark.parametrize("B,L,H,d,max_pos,seed", [(2, 37, 8, 256, 900, 0), (1, 50, 24, 64, 5000, 1),
                                                  (3, 5, 2, 16, 100, 2), (1, 962, 1, 256, 962, 3)])
def test_rope_apply_matches_oracle(B, L, H, d, max_pos, seed):
    Bd = _bd()
    note(f"rope apply B={B} L={L} H={H} d={d}")
    r = np.random.default_rng(seed)
    x = I.bf16_normal(seed * 5 + 1, (B, L, H, d))
    pos = r.integers(0, max_pos, (B, L)).astype(np.int32)
    pos[0, 0] = 0
    xd = bf16_dev(x)
    y = host64(Bd.pi_rope_apply(xd, _i32_dev(pos), BASE))
    torch.cuda.synchronize()
    want = R.rope(f64(x), pos, BASE)
    err = np.abs(y - want)
    bound = ROPE_RTOL * np.abs(want) + ROPE_ATOL
    note(f"rope apply: max_abs={err.max():.3e} worst ratio={np.max(err / bound):.3f}")
    assert (err <= bound).all()
    np.testing.assert_array_equal(y[0, 0], f64(x)[0, 0])   # position 0 is the identity
    # in place gives the same bits
    y2 = Bd.pi_rope_apply(xd, _i32_dev(pos), BASE, y=xd)
    torch.cuda.synchronize()
    assert np.array_equal(host64(y2), y)


def _mask(valid, s):
    Bd = _bd()
    return Bd.pi_mask_build(u8_dev(valid), u8_dev(s.ar), u8_dev(s.seg), I.forbid_bits(s.forbid))


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("seed,B,P,F,E", [(0, 2, 150, 20, 13), (1, 3, 97, 0, 50), (2, 1, 300, 64, 50)])
def test_prefill_rope_matches_oracle(seed, B, P, F, E, split):
    Bd = _bd()
    s = I.pi05_structure(P, F, E) if F else I.pi0_structure(P, E - 1)
    N = s.n
    note(f"prefill rope seed={seed} B={B} N={N} split={split}")
    r = np.random.default_rng(seed + 40)
    valid = np.ones((B, N), np.uint8)
    valid[:, :P] = I.tail_padding_mask(r.integers(P // 2, P + 1, B), P)
    q = I.bf16_normal(seed * 10 + 41, (B, N, 8, 256))
    k = I.bf16_normal(seed * 10 + 42, (B, N, 1, 256))
    v = I.bf16_normal(seed * 10 + 43, (B, N, 1, 256))
    m = _mask(valid, s)
    ws = Bd.prefill_workspace(B, N, 8, 1, 256, torch.device("cuda:0"))
    if not split:   # room for the rotated K only: the call runs unsplit
        ws = ws[: (B * N * 256 * 2 + 255) // 256 * 256]
    qd, kd = bf16_dev(q), bf16_dev(k)
    o = Bd.pi_joint_attn_prefill(qd, kd, bf16_dev(v), m, workspace=ws, rope_base=BASE)
    torch.cuda.synchronize()
    pos = M.positions(valid)
    mm = M.attn_mask(valid, s.ar, s.seg, s.forbid)
    want = R.joint_attention_rope(f64(q), f64(k), f64(v), mm, pos, BASE)
    got = host64(o)
    assert_close(got, want, f"prefill rope {seed} split={split}")
    assert (got[valid == 0] == 0).all()
    # the inputs are left as they were
    assert torch.equal(qd.cpu().view(torch.int16), torch.from_numpy(q.view(np.int16)))
    assert torch.equal(kd.cpu().view(torch.int16), torch.from_numpy(k.view(np.int16)))
    # and the rotation matters at these positions
    assert np.abs(want - A.masked_attention(f64(q), f64(k), f64(v), mm)).max() > 0.05


def test_prefill_rope_mha_d64():
    Bd = _bd()
    s = I.bidirectional_structure(333)
    B, N, H = 2, s.n, 3
    note("prefill rope MHA d=64")
    valid = np.ones((B, N), np.uint8)
    valid[1, 300:] = 0
    q = I.bf16_normal(51, (B, N, H, 64))
    k = I.bf16_normal(52, (B, N, H, 64))
    v = I.bf16_normal(53, (B, N, H, 64))
    m = _mask(valid, s)
    ws = Bd.prefill_workspace(B, N, H, H, 64, torch.device("cuda:0"))
    o = Bd.pi_joint_attn_prefill(bf16_dev(q), bf16_dev(k), bf16_dev(v), m, workspace=ws, rope_base=BASE)
    torch.cuda.synchronize()
    mm = M.attn_mask(valid, s.ar)
    want = R.joint_attention_rope(f64(q), f64(k), f64(v), mm, M.positions(valid), BASE)
    assert_close(host64(o), want, "prefill rope MHA d=64")


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("seed,B,P", [(0, 3, 100), (1, 1, 816)])
def test_rope_cache_then_decode_matches_joint(seed, B, P, split):
    """Prefix-only prefill with the rotary embedding writes rotated keys into the
    cache; the cached decode then rotates its suffix Q/K at (valid prefix slots) + t
    and equals the suffix rows of the rotated joint attention."""
    Bd = _bd()
    S = 51
    s = I.pi0_structure(P, S - 1)
    N = s.n
    note(f"rope cache+decode seed={seed} B={B} P={P} split={split}")
    r = np.random.default_rng(seed + 60)
    valid = np.ones((B, N), np.uint8)
    valid[:, :P] = I.tail_padding_mask(r.integers(P // 2, P + 1, B), P)
    q = I.bf16_normal(seed * 10 + 61, (B, N, 8, 256))
    k = I.bf16_normal(seed * 10 + 62, (B, N, 1, 256))
    v = I.bf16_normal(seed * 10 + 63, (B, N, 1, 256))
    dev = torch.device("cuda:0")
    # prefix-only prefill into cache layer 1
    sp = I.Structure(ar=s.ar[:P], seg=s.seg[:P], forbid=s.forbid, n_prefix=P)
    cache = Bd.KVCache.empty(2, B, P, 1, 256, dev, length=P)
    cache.prefix_mask.copy_(u8_dev(valid[:, :P]))
    mp = _mask(valid[:, :P], sp)
    wsp = Bd.prefill_workspace(B, P, 8, 1, 256, dev)
    Bd.pi_joint_attn_prefill(bf16_dev(q[:, :P]), bf16_dev(k[:, :P]), bf16_dev(v[:, :P]), mp, cache=cache, layer=1,
                             workspace=wsp, rope_base=BASE)
    torch.cuda.synchronize()
    # the cache holds the rotated keys of the prefix (the standalone rotation's bits)
    pos_p = M.positions(valid[:, :P])
    rot = Bd.pi_rope_apply(bf16_dev(k[:, :P]), _i32_dev(pos_p), BASE)
    torch.cuda.synchronize()
    assert torch.equal(cache.k[1].view(torch.int16), rot.view(torch.int16))
    assert torch.equal(cache.v[1].cpu().view(torch.int16), torch.from_numpy(v[:, :P].view(np.int16)))
    # cached decode with rotated suffix Q/K
    ws = Bd.decode_workspace(cache, S)
    if not split:
        ws = ws[: (B * S * 256 * 2 + 255) // 256 * 256]
    o = Bd.pi_suffix_decode_step(cache, 1, bf16_dev(q[:, P:]), bf16_dev(k[:, P:]), bf16_dev(v[:, P:]),
                                 u8_dev(s.ar[P:]), workspace=ws, rope_base=BASE)
    torch.cuda.synchronize()
    mm = M.attn_mask(valid, s.ar)
    pos = M.positions(valid)
    want = R.joint_attention_rope(f64(q), f64(k), f64(v), mm, pos, BASE)[:, P:]
    assert_close(host64(o), want, f"rope decode vs rotated joint seed={seed} split={split}")

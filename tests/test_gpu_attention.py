"""Prefill and cached-decode parity of the HIP kernels against the fp64 oracle,
and the bit-exact invariances of the masked attention."""
import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import mask as M
from prefix_lm_joint_amd import inputs as I
from tests.gpu_util import assert_close, bf16_dev, f64, host64, note, u8_dev

pytestmark = pytest.mark.gpu


def _bd():
    from prefix_lm_joint_amd import binding as Bd
    return Bd


def _prefill(q, k, v, valid, s, cache=None, layer=0, split=False):
    """split: pass the small-batch key-split workspace (asserting the shape asks for one)."""
    Bd = _bd()
    m = Bd.pi_mask_build(u8_dev(valid), u8_dev(s.ar), u8_dev(s.seg), I.forbid_bits(s.forbid))
    ws = None
    if split:
        B, L, Hq, d = q.shape
        ws = Bd.prefill_workspace(B, L, Hq, k.shape[2], d, torch.device("cuda:0"))
        assert ws is not None, "shape too small to split its keys"
    o = Bd.pi_joint_attn_prefill(bf16_dev(q), bf16_dev(k), bf16_dev(v), m, cache=cache, layer=layer, workspace=ws)
    torch.cuda.synchronize()
    return o


def _sample_rows(valid, n_rows, seed, must=()):
    r = np.random.default_rng(seed)
    B, N = valid.shape
    rows = set(must)
    while len(rows) < n_rows:
        rows.add((int(r.integers(B)), int(r.integers(N))))
    return sorted(rows)


# ----------------------------------------------------------------------------
# prefill, full comparison at sizes the oracle finishes in seconds
# ----------------------------------------------------------------------------

def test_prefill_tiny():
    w = I.tiny()
    note("prefill tiny")
    q, k, v = w.qkv()
    valid = w.input_mask()
    o = _prefill(q, k, v, valid, w.structure)
    want = A.joint_attention(f64(q), f64(k), f64(v), valid, w.structure.ar)
    assert_close(host64(o), want, "prefill tiny")


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("seed,B,P,F,E", [(0, 2, 150, 20, 13), (1, 3, 97, 0, 50), (2, 1, 300, 64, 50)])
def test_prefill_three_block_ragged(seed, B, P, F, E, split):
    """π0.5-style prefix / FAST / expert with tail padding, ragged tiles, forbidden
    edge; unsplit and with the small-batch key split."""
    s = I.pi05_structure(P, F, E) if F else I.pi0_structure(P, E - 1)
    N = s.n
    note(f"prefill three-block seed={seed} B={B} N={N} split={split}")
    r = np.random.default_rng(seed)
    valid = np.ones((B, N), np.uint8)
    valid[:, :P] = I.tail_padding_mask(r.integers(P // 2, P + 1, B), P)
    q = I.bf16_normal(seed * 10 + 1, (B, N, 8, 256))
    k = I.bf16_normal(seed * 10 + 2, (B, N, 1, 256))
    v = I.bf16_normal(seed * 10 + 3, (B, N, 1, 256))
    o = _prefill(q, k, v, valid, s, split=split)
    want = A.joint_attention(f64(q), f64(k), f64(v), valid, s.ar, s.seg, s.forbid)
    assert_close(host64(o), want, f"prefill three-block {seed} split={split}")
    pad_rows = valid == 0
    assert (host64(o)[pad_rows] == 0).all()


def test_prefill_mha_d64_small():
    s = I.bidirectional_structure(333)
    B, N, H = 2, s.n, 3
    note("prefill mha d64 small")
    valid = np.ones((B, N), np.uint8)
    q = I.bf16_normal(71, (B, N, H, 64))
    k = I.bf16_normal(72, (B, N, H, 64))
    v = I.bf16_normal(73, (B, N, H, 64))
    o = _prefill(q, k, v, valid, s)
    want = A.joint_attention(f64(q), f64(k), f64(v), valid, s.ar)
    assert_close(host64(o), want, "prefill mha d64")


@pytest.mark.parametrize("split", [False, True])
def test_prefill_pi0_joint_867_full(split):
    """π0 control-step joint pool: 816 prefix + state + 50 actions, every row."""
    w = I.pi0_step()
    note(f"prefill pi0 joint 867 split={split}")
    q, k, v = w.qkv()
    valid = w.input_mask()
    o = _prefill(q, k, v, valid, w.structure, split=split)
    want = A.joint_attention(f64(q), f64(k), f64(v), valid, w.structure.ar)
    assert_close(host64(o), want, f"prefill pi0 joint 867 split={split}")


# ----------------------------------------------------------------------------
# prefill at the full workload sizes: sampled rows
# ----------------------------------------------------------------------------

def test_prefill_pi05_training_shape_sampled():
    w = I.pi05_train()
    s = w.structure
    note("prefill pi05 B=32 L=962 sampled")
    q, k, v = w.qkv()
    valid = w.input_mask()
    o = host64(_prefill(q, k, v, valid, s))
    P = s.n_prefix
    must = [(0, 0), (31, P - 1), (5, P), (5, P + 63), (7, P + 64), (7, s.n - 1), (12, P + 17), (3, 599)]
    rows = _sample_rows(valid, 64, 3, must)
    want = A.joint_attention(f64(q), f64(k), f64(v), valid, s.ar, s.seg, s.forbid, rows=rows)
    got = np.stack([o[b, i] for b, i in rows])
    ref = np.stack([want[b, i] for b, i in rows])
    assert_close(got, ref, "prefill pi05 sampled")
    assert (o[valid == 0] == 0).all()


def test_prefill_mmdit_sampled():
    w = I.mmdit()
    note("prefill mmdit B=2 L=4250 H=24 d=64 sampled")
    q, k, v = w.qkv()
    valid = w.input_mask()
    o = host64(_prefill(q, k, v, valid, w.structure))
    rows = _sample_rows(valid, 24, 5, [(0, 0), (1, 4249), (1, 4095), (0, 4096)])
    want = A.joint_attention(f64(q), f64(k), f64(v), valid, w.structure.ar, rows=rows)
    got = np.stack([o[b, i] for b, i in rows])
    ref = np.stack([want[b, i] for b, i in rows])
    assert_close(got, ref, "prefill mmdit sampled")


# ----------------------------------------------------------------------------
# bit-exact invariances
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("split", [False, True])
def test_prefix_rows_invariant_to_suffix_kv_bit_exact(split):
    """Rows that may not read a key are bit-identical whatever that key holds.

    Masked scores are replaced by -inf before the running max, so NaN in masked K
    cannot leak; padded keys are zero-filled when staged, so NaN in padded K or V
    cannot leak.  Masked but valid V is multiplied by an exact zero weight inside
    the matrix-core product, so finite perturbations of it are bit-exact too."""
    s = I.pi05_structure(200, 64, 50)
    B, N, P = 2, s.n, 200
    note("invariance prefix vs suffix K/V")
    valid = np.ones((B, N), np.uint8)
    valid[1, 150:P] = 0
    q = I.bf16_normal(81, (B, N, 8, 256))
    k = I.bf16_normal(82, (B, N, 1, 256))
    v = I.bf16_normal(83, (B, N, 1, 256))
    o1 = _prefill(q, k, v, valid, s, split=split).cpu()
    big = I.bf16_normal(85, (B, N, 1, 256), std=3.0e4)
    k2, v2 = k.copy(), v.copy()
    k2[:, P:] = 0x7FC0      # NaN in every suffix key
    v2[:, P:] = big[:, P:]  # huge finite suffix values
    k2[1, 150:P] = 0x7FC0   # padded prefix slots: NaN in K and V
    v2[1, 150:P] = 0x7FC0
    o2 = _prefill(q, k2, v2, valid, s, split=split).cpu()
    assert torch.equal(o1[:, :P].view(torch.int16), o2[:, :P].view(torch.int16))
    # expert rows do not read FAST: perturb FAST K/V only
    k3, v3 = k.copy(), v.copy()
    k3[:, P:P + 64] = 0x7FC0
    v3[:, P:P + 64] = big[:, P:P + 64]
    o3 = _prefill(q, k3, v3, valid, s, split=split).cpu()
    assert torch.equal(o1[:, P + 64:].view(torch.int16), o3[:, P + 64:].view(torch.int16))
    # FAST token t does not read FAST tokens after it
    t = 20
    k4, v4 = k.copy(), v.copy()
    k4[:, P + t + 1:] = 0x7FC0
    v4[:, P + t + 1:] = big[:, P + t + 1:]
    o4 = _prefill(q, k4, v4, valid, s, split=split).cpu()
    assert torch.equal(o1[:, :P + t + 1].view(torch.int16), o4[:, :P + t + 1].view(torch.int16))


@pytest.mark.parametrize("split", [False, True])
def test_prefill_padded_keys_in_first_tiles(split):
    """Padded keys inside the first two key tiles (a hole in tile 0, all of tile 0
    padded, a hole in tile 1, tile 1 partly padded), holding NaN in K and V: the
    tile loop's first loads are issued before its steady state, and a padded key
    must land as zeros there too.  Compared with the oracle on every row, and
    padded rows are zero."""
    s = I.pi05_structure(150, 20, 13)
    B, N, P = 4, s.n, 150
    note(f"prefill padded first tiles split={split}")
    valid = np.ones((B, N), np.uint8)
    valid[0, 3:9] = 0          # hole in tile 0
    valid[1, 0:32] = 0         # tile 0 fully padded (EMPTY for every query block)
    valid[2, 40:41] = 0        # hole in tile 1
    valid[3, 50:P] = 0         # tile 1 partly padded, the rest of the prefix too
    q = I.bf16_normal(91, (B, N, 8, 256))
    k = I.bf16_normal(92, (B, N, 1, 256))
    v = I.bf16_normal(93, (B, N, 1, 256))
    k[valid == 0] = 0x7FC0
    v[valid == 0] = 0x7FC0
    o = host64(_prefill(q, k, v, valid, s, split=split))
    kz, vz = k.copy(), v.copy()
    kz[valid == 0] = 0
    vz[valid == 0] = 0
    want = A.joint_attention(f64(q), f64(kz), f64(vz), valid, s.ar, s.seg, s.forbid)
    assert np.isfinite(o).all()
    assert_close(o, want, f"prefill padded first tiles split={split}")
    assert (o[valid == 0] == 0).all()


def test_decode_ignores_garbage_in_padded_slots():
    """Padded cache slots may hold anything (uninitialised memory, NaN)."""
    Bd = _bd()
    B, P, S = 3, 130, 51
    ck = I.bf16_normal(91, (1, B, P, 1, 256))
    cv = I.bf16_normal(92, (1, B, P, 1, 256))
    pm = I.tail_padding_mask(np.array([130, 100, 71]), P)
    sar = np.array([1, 1] + [0] * (S - 2), np.uint8)
    qs, ks, vs = (I.bf16_normal(93 + i, (B, S, h, 256)) for i, h in enumerate((8, 1, 1)))
    o1 = Bd.pi_suffix_decode_step(_cache_from(ck, cv, pm), 0, bf16_dev(qs), bf16_dev(ks), bf16_dev(vs),
                                  u8_dev(sar)).cpu()
    ck2, cv2 = ck.copy(), cv.copy()
    ck2[0][pm == 0] = 0x7FC0
    cv2[0][pm == 0] = 0xFF80
    o2 = Bd.pi_suffix_decode_step(_cache_from(ck2, cv2, pm), 0, bf16_dev(qs), bf16_dev(ks), bf16_dev(vs),
                                  u8_dev(sar)).cpu()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


@pytest.mark.parametrize("split", [False, True])
def test_prefill_is_deterministic(split):
    w = I.pi0_step()
    q, k, v = w.qkv()
    valid = w.input_mask()
    o1 = _prefill(q, k, v, valid, w.structure, split=split).cpu()
    o2 = _prefill(q, k, v, valid, w.structure, split=split).cpu()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


# ----------------------------------------------------------------------------
# cached decode
# ----------------------------------------------------------------------------

def _cache_from(kl, vl, pm, length=None):
    Bd = _bd()
    return Bd.KVCache(bf16_dev(kl), bf16_dev(vl), u8_dev(pm), length)


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("seed,B,P,S", [(0, 4, 100, 51), (1, 3, 37, 9), (2, 9, 64, 33), (3, 2, 1, 1),
                                        (4, 1, 816, 51)])
def test_decode_parity_small(seed, B, P, S, split):
    """Unsplit and key-split (small-batch) decode against the oracle."""
    Bd = _bd()
    note(f"decode seed={seed} B={B} P={P} S={S} split={split}")
    r = np.random.default_rng(seed)
    layers = 2
    ck = I.bf16_normal(seed * 7 + 1, (layers, B, P, 1, 256))
    cv = I.bf16_normal(seed * 7 + 2, (layers, B, P, 1, 256))
    pm = I.tail_padding_mask(r.integers(max(1, P // 2), P + 1, B), P)
    pm[0, 0] = 0 if P > 1 else 1   # a hole at the front, too
    sar = np.array([1, 1] + [0] * (S - 2), np.uint8)[:S] if S > 1 else np.array([1], np.uint8)
    qs = I.bf16_normal(seed * 7 + 3, (B, S, 8, 256))
    ks = I.bf16_normal(seed * 7 + 4, (B, S, 1, 256))
    vs = I.bf16_normal(seed * 7 + 5, (B, S, 1, 256))
    cache = _cache_from(ck, cv, pm)
    ws = Bd.decode_workspace(cache, S) if split else None
    tiles = -(-P // 32) + -(-S // 32)
    if split and B <= 4 and tiles >= 4:
        assert ws is not None   # small batches with enough key tiles split their keys
    for layer in range(layers):
        o = Bd.pi_suffix_decode_step(cache, layer, bf16_dev(qs), bf16_dev(ks), bf16_dev(vs), u8_dev(sar),
                                     workspace=ws)
        torch.cuda.synchronize()
        want = A.cached_decode(f64(qs), f64(ks), f64(vs), f64(ck[layer]), f64(cv[layer]), pm, sar)
        assert_close(host64(o), want, f"decode seed={seed} layer={layer} split={split}")


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("seed,B,P,cap,S", [(10, 1, 816, 840, 51), (11, 2, 300, 300, 20), (12, 1, 70, 96, 51),
                                            (13, 1, 1, 32, 51), (14, 1, 0, 64, 51)])
def test_decode_few_samples_holes_nan_and_spike(seed, B, P, cap, S, split):
    """The few-sample decode (a handful of key tiles per workgroup, all loaded at
    once): padded slots scattered inside the cache length holding NaN K/V, a cache
    capacity beyond its length, a late score maximum of 90 above the rest, an
    empty cache, against the oracle."""
    Bd = _bd()
    note(f"few-sample decode seed={seed} B={B} len={P} cap={cap} S={S} split={split}")
    r = np.random.default_rng(seed)
    ck = I.bf16_normal(seed * 7 + 1, (1, B, cap, 1, 256))
    cv = I.bf16_normal(seed * 7 + 2, (1, B, cap, 1, 256))
    pm = (r.random((B, cap)) < 0.8).astype(np.uint8)
    pm[:, P:] = 0
    if P > 0:
        pm[:, 0] = 1
    pad = pm == 0
    ck_dev, cv_dev = ck.copy(), cv.copy()
    ck_dev[0][pad] = 0x7FC0      # NaN in every padded slot of what the kernel reads
    cv_dev[0][pad] = 0x7FC0
    sar = np.array([1, 1] + [0] * (S - 2), np.uint8)
    qs = I.bf16_normal(seed * 7 + 3, (B, S, 8, 256))
    ks = I.bf16_normal(seed * 7 + 4, (B, S, 1, 256))
    vs = I.bf16_normal(seed * 7 + 5, (B, S, 1, 256))
    if P > 40:
        # one late valid slot scores 90 against query row (token 3, head 2) of sample 0
        j = int(np.flatnonzero(pm[0, :P])[-1])
        qv = np.zeros(256)
        qv[:4] = 1.0
        qs[0, 3, 2] = I.f32_to_bf16_bits(qv)
        kv = np.zeros(256)
        kv[:4] = 90.0 * 16.0 / 4.0   # score 90 after the 1/16 scale
        ck[0, 0, j, 0] = ck_dev[0, 0, j, 0] = I.f32_to_bf16_bits(kv)
    cache = _cache_from(ck_dev, cv_dev, pm, length=P)
    ws = Bd.decode_workspace(cache, S) if split else None
    o = Bd.pi_suffix_decode_step(cache, 0, bf16_dev(qs), bf16_dev(ks), bf16_dev(vs), u8_dev(sar), workspace=ws)
    torch.cuda.synchronize()
    got = host64(o)
    assert np.isfinite(got).all()
    want = A.cached_decode(f64(qs), f64(ks), f64(vs), f64(ck[0, :, :P]), f64(cv[0, :, :P]), pm[:, :P], sar)
    assert_close(got, want, f"few-sample decode seed={seed} split={split}")


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("seed,B,P,S,flags", [(20, 6, 70, 128, "random"), (21, 5, 40, 100, "all"),
                                              (22, 7, 33, 37, "random"), (23, 6, 64, 65, "last")])
def test_decode_multi_block_suffix(seed, B, P, S, flags, split):
    """The batched decode with suffixes of several blocks (random block starts,
    every token its own block as in an autoregressive suffix, a lone block start
    at the last token), up to the 128-token limit: each row sees the cache's valid
    slots and the suffix up to the end of its own block.  Every row against the
    oracle."""
    Bd = _bd()
    note(f"decode multi-block suffix seed={seed} B={B} P={P} S={S} flags={flags} split={split}")
    r = np.random.default_rng(seed)
    ck = I.bf16_normal(seed * 7 + 1, (1, B, P, 1, 256))
    cv = I.bf16_normal(seed * 7 + 2, (1, B, P, 1, 256))
    pm = I.tail_padding_mask(r.integers(P // 2, P + 1, B), P)
    if flags == "random":
        sar = (r.random(S) < 0.2).astype(np.uint8)
    elif flags == "all":
        sar = np.ones(S, np.uint8)
    else:
        sar = np.zeros(S, np.uint8)
        sar[S - 1] = 1
    sar[0] = 1
    qs = I.bf16_normal(seed * 7 + 3, (B, S, 8, 256))
    ks = I.bf16_normal(seed * 7 + 4, (B, S, 1, 256))
    vs = I.bf16_normal(seed * 7 + 5, (B, S, 1, 256))
    cache = _cache_from(ck, cv, pm)
    ws = Bd.decode_workspace(cache, S) if split else None
    o = Bd.pi_suffix_decode_step(cache, 0, bf16_dev(qs), bf16_dev(ks), bf16_dev(vs), u8_dev(sar), workspace=ws)
    torch.cuda.synchronize()
    want = A.cached_decode(f64(qs), f64(ks), f64(vs), f64(ck[0]), f64(cv[0]), pm, sar)
    assert_close(host64(o), want, f"decode multi-block seed={seed} split={split}")


def test_decode_matches_full_recompute():
    """The cached path equals the suffix rows of the joint prefill (same inputs)."""
    Bd = _bd()
    w = I.pi0_step()
    s = w.structure
    P, N = s.n_prefix, s.n
    note("decode vs full recompute (pi0 867)")
    q, k, v = w.qkv()
    valid = w.input_mask()
    full = _prefill(q, k, v, valid, s)
    cache = _cache_from(k[None, :, :P], v[None, :, :P], valid[:, :P])
    for ws in (None, Bd.decode_workspace(cache, s.n - P)):
        o = Bd.pi_suffix_decode_step(cache, 0, bf16_dev(q[:, P:]), bf16_dev(k[:, P:]), bf16_dev(v[:, P:]),
                                     u8_dev(s.ar[P:]), workspace=ws)
        torch.cuda.synchronize()
        assert_close(host64(o), host64(full[:, P:]), f"decode vs joint prefill (split={ws is not None})")


def test_prefill_writes_cache_for_decode():
    Bd = _bd()
    w = I.pi0_step()
    s = w.structure
    P = s.n_prefix
    q, k, v = w.qkv()
    valid = w.input_mask()
    cache = Bd.KVCache.empty(3, 1, 900, 1, 256, torch.device("cuda:0"), length=P)
    cache.prefix_mask[:, :P] = u8_dev(valid[:, :P])
    _prefill(q, k, v, valid, s, cache=cache, layer=2)
    assert torch.equal(cache.k[2, :, :P].cpu().view(torch.int16),
                       torch.from_numpy(k[:, :P].view(np.int16)))
    assert torch.equal(cache.v[2, :, :P].cpu().view(torch.int16),
                       torch.from_numpy(v[:, :P].view(np.int16)))


def test_decode_serving_shape_sampled():
    """B=64 robots, 816 slots with valid length U[600,816], 51 suffix queries: one layer,
    every row of four samples checked against the oracle."""
    Bd = _bd()
    w = I.serving_decode()
    s = w.structure
    P, S, B = s.n_prefix, s.n - s.n_prefix, w.B
    note("decode B=64 P=816 sampled")
    pm = w.input_mask()[:, :P]
    ck = I.bf16_normal(4101, (1, B, P, 1, 256))
    cv = I.bf16_normal(4102, (1, B, P, 1, 256))
    qs = I.bf16_normal(4103, (B, S, 8, 256))
    ks = I.bf16_normal(4104, (B, S, 1, 256))
    vs = I.bf16_normal(4105, (B, S, 1, 256))
    cache = _cache_from(ck, cv, pm)
    o = host64(Bd.pi_suffix_decode_step(cache, 0, bf16_dev(qs), bf16_dev(ks), bf16_dev(vs), u8_dev(s.ar[P:])))
    for b in (0, 17, 40, 63):
        want = A.cached_decode(f64(qs[b:b + 1]), f64(ks[b:b + 1]), f64(vs[b:b + 1]), f64(ck[0, b:b + 1]),
                               f64(cv[0, b:b + 1]), pm[b:b + 1], s.ar[P:])
        assert_close(o[b:b + 1], want, f"decode serving sample {b}")

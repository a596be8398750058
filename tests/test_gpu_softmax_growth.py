"""The attention kernels' softmax against a reference maximum fixed at a row's
first visible key tile ("π0.5 vs MM-DiT joint attention", first section: one
softmax over the whole pool).  When a row's true maximum ends more than 64
(base 2) above that reference, the workgroup redoes its tiles with the true
maximum.  Unit-variance inputs never get there, so these inputs plant a key
equal to c*q for chosen rows: a scaled score of about 60 or 100 (natural log),
i.e. 87 or 144 above zero in base 2, in a key tile after the row's first (the
100 case overflows fp32 weights without the second pass).  A control row gets
its large score in its first tile.  Finite inputs throughout; prefill and
decode, unsplit and key-split, against the fp64 oracle at the parity
bound (max-abs 1e-2, mean-abs 1e-3), and the spiked rows against the value row they must select."""
import numpy as np
import pytest
import torch

from oracle import attention as A
from prefix_lm_joint_amd import inputs as I
from tests.gpu_util import assert_close, bf16_dev, f64, host64, note, u8_dev

pytestmark = pytest.mark.gpu

SCALE = 1.0 / 16.0


def _bd():
    from prefix_lm_joint_amd import binding as Bd
    return Bd


def _plant(k_bits, q_bits, kidx, qidx, score):
    """k[kidx] <- bf16(c * q[qidx]) with c set so that SCALE * q.k is about `score`."""
    qv = f64(q_bits[qidx])
    c = score / (SCALE * float(qv @ qv))
    k_bits[kidx] = I.f32_to_bf16_bits((c * qv).astype(np.float32))


@pytest.mark.parametrize("split", [False, True])
def test_prefill_late_maximum(split):
    Bd = _bd()
    P, F, E = 300, 64, 50
    s = I.pi05_structure(P, F, E)
    B, N = 2, s.n
    note(f"prefill late row maximum split={split} N={N}")
    valid = np.ones((B, N), np.uint8)
    valid[1, 250:P] = 0
    q = I.bf16_normal(9101, (B, N, 8, 256))
    k = I.bf16_normal(9102, (B, N, 1, 256))
    v = I.bf16_normal(9103, (B, N, 1, 256))
    # (sample, query token, head) -> (key token, scaled score); key tiles of 32
    spikes = {(0, 10, 3): (270, 60.0),       # tile 8: late for every key split too
              (0, 200, 5): (260, 100.0),     # tile 8, weight 2^144 without the second pass
              (0, 50, 0): (3, 60.0),         # control: the maximum sits in the first tile
              (1, N - 20, 2): (N - 5, 60.0)}  # expert row, last key tile
    for (b, i, h), (j, sc) in spikes.items():
        _plant(k, q, (b, j, 0), (b, i, h), sc)
    m = Bd.pi_mask_build(u8_dev(valid), u8_dev(s.ar), u8_dev(s.seg), I.forbid_bits(s.forbid))
    ws = Bd.prefill_workspace(B, N, 8, 1, 256, torch.device("cuda:0")) if split else None
    if split:
        assert ws is not None
    o = host64(Bd.pi_joint_attn_prefill(bf16_dev(q), bf16_dev(k), bf16_dev(v), m, workspace=ws))
    torch.cuda.synchronize()
    want = A.joint_attention(f64(q), f64(k), f64(v), valid, s.ar, s.seg, s.forbid)
    assert_close(o, want, f"prefill late maximum split={split}")
    for (b, i, h), (j, sc) in spikes.items():
        # the planted key takes all the weight: the row is that key's value, bf16-rounded
        np.testing.assert_allclose(o[b, i, h], f64(v[b, j, 0]), rtol=0, atol=1e-2)


@pytest.mark.parametrize("split", [False, True])
def test_decode_late_maximum(split):
    Bd = _bd()
    B, P, S = 3, 500, 51
    note(f"decode late row maximum split={split}")
    ck = I.bf16_normal(9201, (1, B, P, 1, 256))
    cv = I.bf16_normal(9202, (1, B, P, 1, 256))
    pm = I.tail_padding_mask(np.array([500, 450, 480]), P)
    sar = np.array([1, 1] + [0] * (S - 2), np.uint8)
    qs = I.bf16_normal(9203, (B, S, 8, 256))
    ks = I.bf16_normal(9204, (B, S, 1, 256))
    vs = I.bf16_normal(9205, (B, S, 1, 256))
    # (sample, suffix token, head) -> (("cache" | "suffix", key index), score)
    spikes = {(0, 10, 4): (("cache", 470), 60.0),     # cache tile 14
              (1, 30, 7): (("suffix", 40), 100.0),    # the suffix's own keys come last
              (2, 0, 0): (("cache", 2), 60.0),        # control: first tile
              (2, 5, 1): (("cache", 440), 80.0)}      # same query block as the control row
    for (b, t, h), ((where, j), sc) in spikes.items():
        if where == "cache":
            _plant(ck, qs, (0, b, j, 0), (b, t, h), sc)
        else:
            _plant(ks, qs, (b, j, 0), (b, t, h), sc)
    cache = Bd.KVCache(bf16_dev(ck), bf16_dev(cv), u8_dev(pm))
    ws = Bd.decode_workspace(cache, S) if split else None
    if split:
        assert ws is not None
    o = host64(Bd.pi_suffix_decode_step(cache, 0, bf16_dev(qs), bf16_dev(ks), bf16_dev(vs), u8_dev(sar),
                                        workspace=ws))
    torch.cuda.synchronize()
    want = A.cached_decode(f64(qs), f64(ks), f64(vs), f64(ck[0]), f64(cv[0]), pm, sar)
    assert_close(o, want, f"decode late maximum split={split}")
    for (b, t, h), ((where, j), sc) in spikes.items():
        vrow = f64(cv[0, b, j, 0]) if where == "cache" else f64(vs[b, j, 0])
        np.testing.assert_allclose(o[b, t, h], vrow, rtol=0, atol=1e-2)

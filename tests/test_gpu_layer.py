"""One π0.5 joint transformer layer on the GPU against the fp64 oracle
(oracle/layer.py): the prefix stream with the plain RMS norm, the expert stream
with the adaptive norm, the joint attention over the concatenated pool in
between, at small widths with ragged row counts, at the real widths (2048 and
1024, FFN 4x), and one sample of the full π0.5 training batch (B = 32, 912 + 50
tokens) in the launch configuration the benchmark times.

Tolerance: the oracle applies the same bf16 rounding points, but any
fp32-accumulating implementation that feeds the attention weights to the matrix
cores in bf16 moves values across those points (one ulp of an intermediate
each), and the norms and FFN carry that on: an fp32 evaluation of the same
definition sits up to 1.5e-3 mean-abs / 8.6e-3 max-abs from the oracle
(tests/test_oracle_layer.py derives it).  The bound is about twice that:
max-abs <= 2e-2, mean-abs <= 3e-3 on the O(1) residual stream.
"""
import numpy as np
import pytest
import torch

from oracle import layer as Y
from oracle import mask as M
from prefix_lm_joint_amd import inputs as I
from tests.gpu_util import LAYER_MAX_ABS, LAYER_MEAN_ABS, assert_close, bf16_dev, f32_dev, f64, note, u8_dev

pytestmark = pytest.mark.gpu


def _bd():
    from prefix_lm_joint_amd import binding as Bd
    return Bd


def _dev_stream(w):
    Bd = _bd()
    t = {k: (bf16_dev(v) if v.dtype == np.uint16 else f32_dev(v)) for k, v in w.items()}
    return Bd.LayerStream(t["w_qkv"], t["w_o"], t["w_up"], t["w_down"], t.get("norm1"), t.get("norm2"), t.get("mod1"),
                          t.get("mod2"))


def _host_stream(w):
    return {k: (f64(v) if v.dtype == np.uint16 else v.astype(np.float64)) for k, v in w.items()}


def _run(seed, B, s, Wp, We, pad=True, check=None):
    Bd = _bd()
    Np = s.n_prefix + (s.seg == I.SEG_FAST).sum()
    N = s.n
    Ne = N - Np
    r = np.random.default_rng(seed + 700)
    valid = np.ones((B, N), np.uint8)
    if pad:
        P = s.n_prefix
        valid[:, :P] = I.tail_padding_mask(r.integers(P // 2, P + 1, B), P)
    h_p = I.f32_normal(seed * 10 + 701, (B, Np, Wp))
    h_e = I.f32_normal(seed * 10 + 702, (B, Ne, We))
    c = I.f32_normal(seed * 10 + 703, (B, We))
    wp = I.layer_weights(seed * 100 + 10, Wp, False)
    we = I.layer_weights(seed * 100 + 20, We, True)
    m = Bd.pi_mask_build(u8_dev(valid), u8_dev(s.ar), u8_dev(s.seg), I.forbid_bits(s.forbid))
    sp, se = _dev_stream(wp), _dev_stream(we)
    ws = Bd.layer_workspace(sp, se, B, Np, Ne, torch.device("cuda:0"))
    hp_d, he_d = f32_dev(h_p), f32_dev(h_e)
    Bd.pi_joint_layer_forward(sp, se, hp_d, he_d, f32_dev(c), m, ws)
    torch.cuda.synchronize()
    got_p = hp_d.cpu().numpy().astype(np.float64)
    got_e = he_d.cpu().numpy().astype(np.float64)
    rows = range(B) if check is None else check
    for b in rows:
        mm = M.attn_mask(valid[b:b + 1], s.ar, s.seg, s.forbid)
        want_p, want_e = Y.joint_layer(h_p[b:b + 1], h_e[b:b + 1], c[b:b + 1], _host_stream(wp), _host_stream(we), mm)
        assert_close(got_p[b:b + 1], want_p, f"layer prefix stream b={b} (Wp={Wp}, Np={Np})", LAYER_MAX_ABS,
                     LAYER_MEAN_ABS)
        assert_close(got_e[b:b + 1], want_e, f"layer expert stream b={b} (We={We}, Ne={Ne})", LAYER_MAX_ABS,
                     LAYER_MEAN_ABS)
    return got_p, got_e


@pytest.mark.parametrize("seed,B,P,F,E,Wp,We", [(0, 2, 30, 10, 13, 512, 256), (1, 3, 37, 0, 11, 256, 512),
                                                (2, 1, 150, 20, 50, 768, 256)])
def test_layer_small_widths_match_oracle(seed, B, P, F, E, Wp, We):
    s = I.pi05_structure(P, F, E) if F else I.pi0_structure(P, E - 1)
    note(f"layer seed={seed} B={B} P={P} F={F} E={E} Wp={Wp} We={We}")
    _run(seed, B, s, Wp, We)


@pytest.mark.parametrize("which", ["prefix_only", "expert_only"])
def test_layer_one_empty_stream(which):
    """A stream with no tokens (Np = 0 or Ne = 0): the other stream's layer alone,
    against the oracle's joint layer with an empty stream."""
    Bd = _bd()
    B, W = 2, 512
    n = 70
    s = I.bidirectional_structure(n)
    valid = np.ones((B, n), np.uint8)
    valid[1, 60:] = 0
    note(f"layer with one empty stream: {which}")
    wp = I.layer_weights(810, W, False)
    we = I.layer_weights(820, 256, True)
    h = I.f32_normal(811, (B, n, W if which == "prefix_only" else 256))
    c = I.f32_normal(812, (B, 256))
    m = Bd.pi_mask_build(u8_dev(valid), u8_dev(s.ar), u8_dev(s.seg), 0)
    sp, se = _dev_stream(wp), _dev_stream(we)
    empty_p = torch.empty((B, 0, W), dtype=torch.float32, device="cuda:0")
    empty_e = torch.empty((B, 0, 256), dtype=torch.float32, device="cuda:0")
    hd = f32_dev(h)
    if which == "prefix_only":
        ws = Bd.layer_workspace(sp, se, B, n, 0, torch.device("cuda:0"))
        Bd.pi_joint_layer_forward(sp, se, hd, empty_e, None, m, ws)
    else:
        ws = Bd.layer_workspace(sp, se, B, 0, n, torch.device("cuda:0"))
        Bd.pi_joint_layer_forward(sp, se, empty_p, hd, f32_dev(c), m, ws)
    torch.cuda.synchronize()
    mm = M.attn_mask(valid, s.ar)
    if which == "prefix_only":
        want = Y.joint_layer(h, np.zeros((B, 0, 256)), c, _host_stream(wp), _host_stream(we), mm)[0]
    else:
        want = Y.joint_layer(np.zeros((B, 0, W)), h, c, _host_stream(wp), _host_stream(we), mm)[1]
    assert_close(hd.cpu().numpy().astype(np.float64), want, f"layer {which}", LAYER_MAX_ABS, LAYER_MEAN_ABS)


def test_layer_real_widths_match_oracle():
    s = I.pi05_structure(200, 16, 50)
    note("layer real widths 2048 / 1024, B=2")
    _run(3, 2, s, 2048, 1024)


def test_layer_training_shape_sampled():
    """B = 32, 848-token prefix (valid lengths U{600..848}) + 64 FAST + 50 expert,
    widths 2048 / 1024: sample 31 against the oracle."""
    w = I.pi05_train()
    note("layer training shape B=32 sampled")
    _run(4, w.B, w.structure, 2048, 1024, check=[31])


def _expert_decode(seed, B, P, S, W, check=None, lens=None):
    """The expert layer in the cached form against random cached prefix K/V."""
    Bd = _bd()
    dev = torch.device("cuda:0")
    r = np.random.default_rng(seed + 900)
    pm = I.tail_padding_mask(r.integers(P // 2, P + 1, B) if lens is None else lens, P)
    ck = I.bf16_normal(seed * 10 + 901, (1, B, P, 1, 256))
    cv = I.bf16_normal(seed * 10 + 902, (1, B, P, 1, 256))
    h_e = I.f32_normal(seed * 10 + 903, (B, S, W))
    c = I.f32_normal(seed * 10 + 904, (B, W))
    sar = np.zeros(S, np.uint8)
    sar[0] = 1                              # the action chunk: one bidirectional block
    we = I.layer_weights(seed * 100 + 50, W, True)
    cache = Bd.KVCache(bf16_dev(ck), bf16_dev(cv), u8_dev(pm), P)
    se = _dev_stream(we)
    ws = Bd.expert_decode_workspace(se, cache, S)
    hd = f32_dev(h_e)
    Bd.pi_expert_layer_decode(se, cache, 0, hd, f32_dev(c), u8_dev(sar), ws)
    torch.cuda.synchronize()
    got = hd.cpu().numpy().astype(np.float64)
    for b in (range(B) if check is None else check):
        want = Y.expert_layer_decode(h_e[b:b + 1], c[b:b + 1], _host_stream(we), f64(ck[0, b:b + 1]),
                                     f64(cv[0, b:b + 1]), pm[b:b + 1], sar)
        assert_close(got[b:b + 1], want, f"expert decode b={b} (W={W}, P={P}, S={S})", LAYER_MAX_ABS, LAYER_MEAN_ABS)


@pytest.mark.parametrize("seed,B,P,S,W", [(0, 2, 100, 50, 1024), (1, 3, 37, 17, 256), (3, 1, 816, 50, 1024)])
def test_expert_layer_decode_matches_oracle(seed, B, P, S, W):
    note(f"expert decode seed={seed} B={B} P={P} S={S} W={W}")
    _expert_decode(seed, B, P, S, W)


def test_expert_layer_decode_serving_shape_sampled():
    """B = 64 robots, 816 cached slots with valid lengths U[600, 816], 50 action
    tokens, width 1024: two samples against the oracle."""
    note("expert decode B=64 P=816 sampled")
    w = I.serving_decode()
    lens = w.input_mask()[:, :816].sum(axis=1)
    _expert_decode(2, 64, 816, 50, 1024, check=[0, 63], lens=lens)

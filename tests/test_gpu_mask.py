"""pi_mask_build on the GPU: block ids, positions, the dense expansion and the
tile table are bit-exact against the oracle's explicit mask."""
import numpy as np
import pytest
import torch

from oracle import mask as M
from prefix_lm_joint_amd import inputs as I
from tests.gpu_util import note, u8_dev

pytestmark = pytest.mark.gpu


def _classes_from_dense(dense, N):
    B = dense.shape[0]
    n_qt, n_kt = -(-N // 16), -(-N // 32)
    pad = np.zeros((B, n_qt * 16, n_kt * 32), bool)
    pad[:, :N, :N] = dense
    inr = np.zeros((n_qt * 16, n_kt * 32), bool)
    inr[:N, :N] = True
    vis = pad.reshape(B, n_qt, 16, n_kt, 32).sum(axis=(2, 4))
    pairs = inr.reshape(n_qt, 16, n_kt, 32).sum(axis=(1, 3))[None]
    complete_k = (np.arange(n_kt) * 32 + 32 <= N)[None, None, :]
    cls = np.full(vis.shape, 1, np.uint8)
    cls[vis == 0] = 0
    cls[(vis == pairs) & complete_k & (vis > 0)] = 2
    return cls


def _check(name, input_mask, ar, seg, forbid):
    from prefix_lm_joint_amd import binding as Bd
    note(f"mask {name}: B={input_mask.shape[0]} N={input_mask.shape[1]}")
    B, N = input_mask.shape
    m = Bd.pi_mask_build(u8_dev(input_mask), u8_dev(ar), u8_dev(seg) if seg is not None else None,
                         I.forbid_bits(forbid))
    dense = Bd.pi_mask_materialize(m)
    torch.cuda.synchronize()
    want = M.attn_mask(input_mask, ar, seg, forbid)
    assert np.array_equal(dense.cpu().numpy().astype(bool), want), name
    assert np.array_equal(m.bid().cpu().numpy(), M.block_ids(ar)), name
    assert np.array_equal(m.pos().cpu().numpy(), M.positions(input_mask)), name
    assert np.array_equal(m.tiles().cpu().numpy(), _classes_from_dense(want, N)), name


@pytest.mark.parametrize("wl", ["tiny", "pi0_control_step", "pi05_three_block_prefill", "mmdit_full_bidirectional"])
def test_workload_masks_bit_exact(wl):
    w = I.WORKLOADS[wl]()
    s = w.structure
    _check(wl, w.input_mask(), s.ar, s.seg, s.forbid)


def test_pi0fast_mask_bit_exact():
    s = I.fast_structure(300, 40)
    valid = np.ones((2, s.n), np.uint8)
    valid[1, 250:300] = 0
    _check("pi0fast", valid, s.ar, s.seg, s.forbid)


@pytest.mark.parametrize("seed,B,N", [(0, 1, 1), (1, 3, 17), (2, 2, 100), (3, 3, 333), (4, 1, 1025), (5, 2, 2100)])
def test_random_masks_bit_exact(seed, B, N):
    r = np.random.default_rng(seed)
    ar = (r.random(N) < r.random() * 0.5).astype(np.uint8)
    valid = (r.random((B, N)) < 0.9).astype(np.uint8)
    seg = r.integers(0, 4, N).astype(np.uint8)
    pairs = [(int(a), int(b)) for a in range(4) for b in range(4) if r.random() < 0.2]
    _check(f"random{seed}", valid, ar, seg, tuple(pairs))

"""Backward of the joint attention on the GPU against the fp64 oracle
(oracle.attention_bwd): the forward's log-sum-exp output, then dq, dk, dv for a
seeded upstream gradient, on the π0.5 training structure (padded prefix, FAST
block, expert block with the expert->FAST pairs forbidden), π0, FAST and
bidirectional masks, ragged lengths, and sampled rows of the full B=32 x 962
training shape; plus the exact facts: masked keys and key-less rows get exactly
zero, and the result is bitwise repeatable.

Tolerance (derived from the arithmetic).  The GPU rounds P and dS to bf16 as
matrix-core operands, takes O rounded to bf16 from the forward for Dr = dO.O,
and rounds each gradient to bf16: each rounding is at most 2^-9 relative.  An
element's error therefore scales with its own size (output rounding) plus the
size of the terms summed into it (operand roundings; an element that is small
by cancellation keeps the terms' error), and the terms scale with the
gradient's RMS.  The bound is per element, |err| <= 2e-2 (|ref| + RMS(ref)),
with mean-abs <= 3e-3 RMS(ref) (bf16 output rounding alone gives ~1e-3 RMS);
measured worst cases: 1.4e-2 and 1.8e-3.  With the rotary embedding two more
bf16 roundings (rotated Q / K, rotated-back gradients): 3.5e-2 and 4.5e-3.  The
log-sum-exp (row sums of
bf16-rounded weights, relative error <= 2^-9 worst case) within 4e-3 absolute.
"""
import numpy as np
import pytest
import torch

from oracle import attention_bwd as G
from oracle import mask as M
from prefix_lm_joint_amd import inputs as I
from tests.gpu_util import bf16_dev, f64, host64, note, u8_dev

pytestmark = pytest.mark.gpu

GRAD_REL = 2e-2
GRAD_MEAN_REL = 3e-3
# With the rotary embedding two more bf16 roundings enter (the rotated Q / K
# operands, and the gradients rounded once as rotated and again after turning
# back), each up to 2^-9 relative: the bounds grow accordingly.
GRAD_REL_ROPE = 3.5e-2
GRAD_MEAN_REL_ROPE = 4.5e-3
LSE_ABS = 4e-3


def _bd():
    from prefix_lm_joint_amd import binding as Bd
    return Bd


def _mask(valid, s):
    Bd = _bd()
    return Bd.pi_mask_build(u8_dev(valid), u8_dev(s.ar), u8_dev(s.seg), I.forbid_bits(s.forbid))


def _case(seed, B, s, pad=True):
    N = s.n
    r = np.random.default_rng(seed + 500)
    valid = np.ones((B, N), np.uint8)
    if pad and s.n_prefix > 1:
        P = s.n_prefix
        valid[:, :P] = I.tail_padding_mask(r.integers(P // 2, P + 1, B), P)
    q = I.bf16_normal(seed * 10 + 501, (B, N, 8, 256))
    k = I.bf16_normal(seed * 10 + 502, (B, N, 1, 256))
    v = I.bf16_normal(seed * 10 + 503, (B, N, 1, 256))
    u = I.bf16_normal(seed * 10 + 504, (B, N, 8, 256))
    return valid, q, k, v, u


def _forward(q, k, v, m, split):
    Bd = _bd()
    B, N = q.shape[:2]
    dev = torch.device("cuda:0")
    ws = Bd.prefill_workspace(B, N, 8, 1, 256, dev) if split else None
    lse = torch.empty((B, N, 8), dtype=torch.float32, device=dev)
    o = Bd.pi_joint_attn_prefill(bf16_dev(q), bf16_dev(k), bf16_dev(v), m, workspace=ws, lse=lse)
    return o, lse


def _backward(q, k, v, o, u, lse, m):
    Bd = _bd()
    B, N = q.shape[:2]
    ws = Bd.backward_workspace(B, N, 8, 1, 256, torch.device("cuda:0"))
    return Bd.pi_joint_attn_backward(bf16_dev(q), bf16_dev(k), bf16_dev(v), o, bf16_dev(u), lse, m, ws)


def _check_grad(got, want, what, rel_bound=None, mean_bound=None):
    err = np.abs(got - want)
    rms = float(np.sqrt(np.mean(want ** 2)))
    rel = err / (np.abs(want) + rms)
    worst = np.unravel_index(np.argmax(rel), rel.shape)
    mean = float(err.mean())
    note(f"{what}: rms(ref)={rms:.3e} max_abs={err.max():.3e} max err/(|ref|+rms)={rel[worst]:.2e} "
         f"at ref={want[worst]:.3e} mean_abs={mean:.3e} ({mean / rms:.2e} rms)")
    assert np.isfinite(got).all(), what
    rel_bound = GRAD_REL if rel_bound is None else rel_bound
    mean_bound = GRAD_MEAN_REL if mean_bound is None else mean_bound
    assert rel[worst] <= rel_bound and mean <= mean_bound * rms, what


STRUCTS = {
    "pi05": lambda: I.pi05_structure(150, 20, 13),
    "pi05_ragged": lambda: I.pi05_structure(97, 9, 7),
    "pi0": lambda: I.pi0_structure(97, 50),
    "fast": lambda: I.fast_structure(60, 17),
    "bidir": lambda: I.bidirectional_structure(70),
}


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("name,B", [("pi05", 2), ("pi0", 3), ("fast", 1)])
def test_forward_lse_matches_oracle(name, B, split):
    s = STRUCTS[name]()
    valid, q, k, v, _ = _case(1, B, s)
    note(f"lse {name} B={B} N={s.n} split={split}")
    m = _mask(valid, s)
    _, lse = _forward(q, k, v, m, split)
    torch.cuda.synchronize()
    mm = M.attn_mask(valid, s.ar, s.seg, s.forbid)
    want = G.lse_rows(f64(q), f64(k), mm)
    got = host64(lse)
    fin = np.isfinite(want)
    assert np.array_equal(np.isfinite(got), fin) and (got[~fin] == -np.inf).all()
    err = np.abs(got[fin] - want[fin]).max()
    note(f"lse {name}: max_abs={err:.3e}")
    assert err <= LSE_ABS


@pytest.mark.parametrize("name,B,seed", [("pi05", 2, 0), ("pi05_ragged", 3, 1), ("pi0", 2, 2), ("fast", 2, 3),
                                         ("bidir", 1, 4)])
def test_backward_matches_oracle(name, B, seed):
    s = STRUCTS[name]()
    valid, q, k, v, u = _case(seed, B, s)
    note(f"backward {name} B={B} N={s.n} seed={seed}")
    m = _mask(valid, s)
    o, lse = _forward(q, k, v, m, False)
    dq, dk, dv = _backward(q, k, v, o, u, lse, m)
    torch.cuda.synchronize()
    mm = M.attn_mask(valid, s.ar, s.seg, s.forbid)
    want = G.masked_attention_grads(f64(q), f64(k), f64(v), mm, f64(u))
    for got, w, nm in zip((dq, dk, dv), want, ("dq", "dk", "dv")):
        _check_grad(host64(got), w, f"backward {name} {nm}")
    # exact zeros: padded tokens' key gradients and key-less rows' query gradients
    pad = valid == 0
    assert (host64(dk)[pad] == 0).all() and (host64(dv)[pad] == 0).all()
    assert (host64(dq)[pad] == 0).all()


@pytest.mark.parametrize("name,B,seed", [("pi05", 2, 11), ("pi0", 1, 12)])
def test_backward_rope_matches_oracle(name, B, seed):
    """With the rotary embedding (base 10000 at the mask's positions): forward and
    backward with rope_base against the gradients through the rotation."""
    from oracle import rope as R
    Bd = _bd()
    s = STRUCTS[name]()
    valid, q, k, v, u = _case(seed, B, s)
    note(f"backward rope {name} B={B} N={s.n}")
    m = _mask(valid, s)
    dev = torch.device("cuda:0")
    qd, kd, vd = bf16_dev(q), bf16_dev(k), bf16_dev(v)
    lse = torch.empty((B, s.n, 8), dtype=torch.float32, device=dev)
    o = Bd.pi_joint_attn_prefill(qd, kd, vd, m, workspace=Bd.prefill_workspace(B, s.n, 8, 1, 256, dev), lse=lse,
                                 rope_base=10000.0)
    ws = Bd.backward_workspace(B, s.n, 8, 1, 256, dev, rope_base=10000.0)
    dq, dk, dv = Bd.pi_joint_attn_backward(qd, kd, vd, o, bf16_dev(u), lse, m, ws, rope_base=10000.0)
    torch.cuda.synchronize()
    mm = M.attn_mask(valid, s.ar, s.seg, s.forbid)
    want = G.masked_attention_grads_rope(f64(q), f64(k), f64(v), mm, f64(u), M.positions(valid), 10000.0)
    for got, w, nm in zip((dq, dk, dv), want, ("dq", "dk", "dv")):
        _check_grad(host64(got), w, f"backward rope {name} {nm}", GRAD_REL_ROPE, GRAD_MEAN_REL_ROPE)
    # the inputs are left as they were
    assert torch.equal(qd.cpu().view(torch.int16), torch.from_numpy(q.view(np.int16)))
    # and the rotation matters at these positions
    plain = G.masked_attention_grads(f64(q), f64(k), f64(v), mm, f64(u))
    assert np.abs(plain[0] - want[0]).max() > 0.05


def test_backward_edge_cases():
    """A 5-token sequence (one partial tile of everything), and a sample whose
    tokens are all padding (every row key-less: all its gradients exactly 0)."""
    s = I.bidirectional_structure(5)
    valid, q, k, v, u = _case(13, 2, s, pad=False)
    valid[1, :] = 0
    note("backward edge cases L=5, one fully padded sample")
    m = _mask(valid, s)
    o, lse = _forward(q, k, v, m, False)
    dq, dk, dv = _backward(q, k, v, o, u, lse, m)
    torch.cuda.synchronize()
    assert (host64(lse)[1] == -np.inf).all()
    for t in (dq, dk, dv):
        assert (host64(t)[1] == 0).all()
    mm = M.attn_mask(valid, s.ar)
    want = G.masked_attention_grads(f64(q), f64(k), f64(v), mm, f64(u))
    for got, w, nm in zip((dq, dk, dv), want, ("dq", "dk", "dv")):
        _check_grad(host64(got)[:1], w[:1], f"backward L=5 {nm}")


def test_backward_masked_inputs_do_not_reach_gradients():
    """Setting K/V at padded slots and Q/dO at padded rows to NaN leaves every
    gradient bit-identical: masked pairs enter nothing."""
    s = STRUCTS["pi05"]()
    valid, q, k, v, u = _case(7, 2, s)
    note("backward masked-input invariance")
    m = _mask(valid, s)
    o, lse = _forward(q, k, v, m, False)
    ref = [t.clone() for t in _backward(q, k, v, o, u, lse, m)]
    pad = valid == 0
    assert pad.any()
    k2, v2, q2, u2 = k.copy(), v.copy(), q.copy(), u.copy()
    nan = np.uint16(0x7FC0)
    k2[pad] = nan
    v2[pad] = nan
    q2[pad] = nan
    u2[pad] = nan
    out = _backward(q2, k2, v2, o, u2, lse, m)
    torch.cuda.synchronize()
    for a, b_, nm in zip(ref, out, ("dq", "dk", "dv")):
        assert torch.equal(a.view(torch.int16), b_.view(torch.int16)), nm


def test_backward_is_deterministic():
    s = STRUCTS["pi05_ragged"]()
    valid, q, k, v, u = _case(8, 3, s)
    note("backward determinism")
    m = _mask(valid, s)
    o, lse = _forward(q, k, v, m, False)
    a = [t.clone() for t in _backward(q, k, v, o, u, lse, m)]
    b = _backward(q, k, v, o, u, lse, m)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_backward_training_shape_sampled():
    """The π0.5 training shape (B = 32, L = 962: 848 prefix tokens with valid
    lengths U{600..848}, 64 FAST, 50 expert), in the launch configuration the
    benchmark times; every gradient of two samples against the oracle."""
    w = I.pi05_train()
    s = w.structure
    note("backward training shape B=32 L=962 sampled")
    valid = w.input_mask()
    B, N = valid.shape
    q = I.bf16_normal(9101, (B, N, 8, 256))
    k = I.bf16_normal(9102, (B, N, 1, 256))
    v = I.bf16_normal(9103, (B, N, 1, 256))
    u = I.bf16_normal(9104, (B, N, 8, 256))
    m = _mask(valid, s)
    o, lse = _forward(q, k, v, m, False)
    dq, dk, dv = _backward(q, k, v, o, u, lse, m)
    torch.cuda.synchronize()
    for b in (0, 31):
        mm = M.attn_mask(valid[b:b + 1], s.ar, s.seg, s.forbid)
        want = G.masked_attention_grads(f64(q[b:b + 1]), f64(k[b:b + 1]), f64(v[b:b + 1]), mm, f64(u[b:b + 1]))
        for got, wt, nm in zip((dq, dk, dv), want, ("dq", "dk", "dv")):
            _check_grad(host64(got[b:b + 1]), wt, f"backward B=32 sample {b} {nm}")

"""GPU parity of π0.5's action expert at its true shape and of the Euler sampler
it drives (pi_expert_velocity_eval, pi_expert_flow_sample) against the fp64
oracle (oracle/expert_flow.py), through the C ABI."""
import numpy as np
import pytest
import torch

from oracle import expert_flow as X
from prefix_lm_joint_amd import binding as Bd
from prefix_lm_joint_amd import inputs as I
from tests import gpu_util as G
from tests.test_oracle_expert_flow import _f64, real_case

pytestmark = pytest.mark.gpu


def _upload(net, ck, cv, pm, ar):
    cache = Bd.KVCache(G.bf16_dev(ck), G.bf16_dev(cv), G.u8_dev(pm))
    return Bd.ExpertNet.from_numpy(net, G.dev()), cache, G.u8_dev(ar)


def _close(got, want, what):
    err = np.abs(got - want)
    G.note(f"{what}: max {err.max():.3e} mean {err.mean():.3e} (|want| mean {np.abs(want).mean():.3f})")
    assert np.isfinite(got).all()
    assert err.max() <= G.EXPERT_VEL_MAX_ABS and err.mean() <= G.EXPERT_VEL_MEAN_ABS, what


@pytest.mark.parametrize("t", [1.0, 0.375])
def test_expert_velocity_matches_oracle(t):
    G.note(f"expert velocity B=2 P=40 H=50 layers=2 t={t}")
    net, ck, cv, pm, ar, x = real_case(11, 2, 40, 50, 2)
    dnet, cache, sar = _upload(net, ck, cv, pm, ar)
    vel = Bd.pi_expert_velocity_eval(dnet, cache, sar, G.f32_dev(x), t)
    torch.cuda.synchronize()
    want = X.expert_velocity(x, t, _f64(net), _f64(ck), _f64(cv), pm, ar)
    _close(G.host64(vel), want, f"velocity t={t}")


def test_expert_flow_sample_matches_oracle():
    G.note("expert sampler B=2 P=40 H=50 layers=2 steps=3")
    net, ck, cv, pm, ar, x = real_case(13, 2, 40, 50, 2)
    dnet, cache, sar = _upload(net, ck, cv, pm, ar)
    xd = G.f32_dev(x)
    Bd.pi_expert_flow_sample(dnet, cache, sar, xd, num_steps=3)
    torch.cuda.synchronize()
    want = X.expert_flow_sample(x, _f64(net), _f64(ck), _f64(cv), pm, ar, num_steps=3)
    _close(G.host64(xd), want, "sampler x after 3 steps")


def test_zero_out_projection_returns_noise_minus_bias():
    """w_out = 0: every step's velocity is b_out, so ten Euler steps from t = 1 to 0
    end at noise - b_out (fp32 accumulation of ten dt*b terms)."""
    G.note("expert sampler closed form B=3 layers=1 steps=10")
    net, ck, cv, pm, ar, x = real_case(15, 3, 40, 50, 1)
    net["w_out"] = np.zeros_like(net["w_out"])
    dnet, cache, sar = _upload(net, ck, cv, pm, ar)
    xd = G.f32_dev(x)
    Bd.pi_expert_flow_sample(dnet, cache, sar, xd, num_steps=10)
    torch.cuda.synchronize()
    np.testing.assert_allclose(G.host64(xd), x - net["b_out"], rtol=0, atol=2e-6)


def test_full_shape_sampler_is_deterministic_and_sample_independent():
    """18 expert layers, 10 steps, B = 4 over an 816-slot cache with padded tails:
    two runs are bit-identical, and a sample's actions do not depend on the other
    samples (sample 2 alone in a B = 1 call gives the same bits)."""
    G.note("expert sampler full shape B=4 P=816 layers=18 steps=10")
    net, ck, cv, pm, ar, x = real_case(17, 4, 816, 50, 18)
    dnet, cache, sar = _upload(net, ck, cv, pm, ar)
    ws = Bd.expert_flow_workspace(dnet, cache, 50, 10)
    outs = []
    for _ in range(2):
        xd = G.f32_dev(x)
        Bd.pi_expert_flow_sample(dnet, cache, sar, xd, num_steps=10, workspace=ws)
        outs.append(G.host64(xd))
    torch.cuda.synchronize()
    assert np.isfinite(outs[0]).all() and np.array_equal(outs[0], outs[1])
    assert np.abs(outs[0] - x).mean() > 0.1            # the net moved the noise
    one = Bd.KVCache(G.bf16_dev(ck[:, 2:3]), G.bf16_dev(cv[:, 2:3]), G.u8_dev(pm[2:3]))
    x2 = G.f32_dev(x[2:3])
    Bd.pi_expert_flow_sample(dnet, one, sar, x2, num_steps=10)
    torch.cuda.synchronize()
    G.note(f"B=1 vs row 2 of B=4: max diff {np.abs(G.host64(x2)[0] - outs[0][2]).max():.3e}")
    np.testing.assert_allclose(G.host64(x2)[0], outs[0][2], rtol=0, atol=G.EXPERT_VEL_MAX_ABS)


@pytest.mark.parametrize("seed", [31, 32])
def test_small_odd_shapes_match_oracle(seed):
    """Width 256, 7 actions of dim 7, B = 3 over a 37-slot cache with ragged valid
    lengths: a velocity evaluation and two sampler steps (the same fp32 floor as the
    real width, measured for these shapes at mean 2.2e-3 / max 1.1e-2)."""
    G.note(f"expert small odd shapes seed={seed} B=3 P=37 H=7 A=7 W=256 layers=2")
    net, ck, cv, pm, ar, x = real_case(seed, 3, 37, 7, 2, W=256, A=7)
    dnet, cache, sar = _upload(net, ck, cv, pm, ar)
    vel = Bd.pi_expert_velocity_eval(dnet, cache, sar, G.f32_dev(x), 0.625)
    xd = G.f32_dev(x)
    Bd.pi_expert_flow_sample(dnet, cache, sar, xd, num_steps=2)
    torch.cuda.synchronize()
    n64, ck64, cv64 = _f64(net), _f64(ck), _f64(cv)
    _close(G.host64(vel), X.expert_velocity(x, 0.625, n64, ck64, cv64, pm, ar), "small velocity")
    _close(G.host64(xd), X.expert_flow_sample(x, n64, ck64, cv64, pm, ar, num_steps=2), "small sampler")

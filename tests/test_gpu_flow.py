"""Euler update, flow sampler and stand-in velocity net on the GPU vs the oracle."""
import numpy as np
import pytest
import torch

from oracle import flow as F
from prefix_lm_joint_amd import inputs as I
from tests.gpu_util import NET_MAX_ABS, NET_MEAN_ABS, assert_close, bf16_dev, f32_dev, f64, host64, note, u8_dev

pytestmark = pytest.mark.gpu


def _bd():
    from prefix_lm_joint_amd import binding as Bd
    return Bd


def test_euler_update_matches_oracle():
    Bd = _bd()
    r = np.random.default_rng(0)
    for n in (1, 7, 1600, 102400 + 3):
        x = r.standard_normal(n).astype(np.float32)
        v = r.standard_normal(n).astype(np.float32)
        xd = f32_dev(x)
        Bd.pi_euler_update(xd, f32_dev(v), -0.1)
        want = F.euler_update(x, v, np.float32(-0.1))
        got = host64(xd)
        assert np.abs(got - want).max() <= 2e-7 * (np.abs(x) + np.abs(v)).max()


def test_flow_constant_velocity_tiny_closed_form():
    """Tiny: v = noise - action held fixed; 10 Euler steps return the action."""
    Bd = _bd()
    r = np.random.default_rng(11)
    noise = r.standard_normal((1, 8, 4)).astype(np.float32)
    action = r.standard_normal((1, 8, 4)).astype(np.float32)
    v = (noise - action).astype(np.float32)
    x = f32_dev(noise)
    Bd.pi_flow_sample(None, None, None, None, f32_dev(v), x, num_steps=10)
    got = host64(x)
    assert np.abs(got - (noise.astype(np.float64) - v)).max() <= 1e-5 * np.abs(v).max()
    assert np.abs(got - action).max() <= 1e-5 * np.abs(v).max() + 1e-6


def _net_case(seed, B, P, H, A, W, layers, lens=None):
    Bd = _bd()
    w = I.net_weights(seed, width=W, action_dim=A)
    net = Bd.VelocityNet.from_numpy(w, torch.device("cuda:0"))
    wf = {f: (f64(getattr(w, f)) if getattr(w, f).dtype == np.uint16 else getattr(w, f).astype(np.float64))
          for f in Bd.VelocityNet.FIELDS}
    ck = I.bf16_normal(seed + 20, (layers, B, P, 1, 256))
    cv = I.bf16_normal(seed + 21, (layers, B, P, 1, 256))
    if lens is None:
        lens = I.valid_lengths(seed + 22, B, max(1, (3 * P) // 4), P)
    pm = I.tail_padding_mask(lens, P)
    cache = Bd.KVCache(bf16_dev(ck), bf16_dev(cv), u8_dev(pm))
    sar = I.pi0_structure(P, H).ar[P:]
    state = I.f32_normal(seed + 23, (B, A))
    x0 = I.f32_normal(seed + 24, (B, H, A))
    oracle_v = lambda x, t: F.velocity_net(x, t, state.astype(np.float64), wf, f64(ck), f64(cv), pm, sar, 8, 1, 256)
    return net, cache, u8_dev(sar), state, x0, oracle_v


@pytest.mark.parametrize("seed,B,P,H,A,W,layers", [(100, 2, 100, 50, 32, 256, 3), (200, 3, 45, 8, 4, 128, 2),
                                                   (600, 7, 64, 50, 32, 256, 2), (700, 6, 40, 50, 32, 512, 1)])
def test_velocity_eval_small(seed, B, P, H, A, W, layers):
    """Against the oracle on every row; the last two cases have more than 256 token
    rows (357 and 306, a partial last 64-row tile), so their projections take the
    wide-tile product of a batch of samples."""
    Bd = _bd()
    note(f"velocity eval seed={seed}")
    net, cache, sar, state, x0, oracle_v = _net_case(seed, B, P, H, A, W, layers)
    for t in (1.0, 0.3):
        t32 = float(np.float32(t))
        vel = Bd.pi_velocity_eval(net, cache, sar, f32_dev(state), f32_dev(x0), t32)
        torch.cuda.synchronize()
        assert_close(host64(vel), oracle_v(x0.astype(np.float64), t32), f"velocity seed={seed} t={t}",
                     NET_MAX_ABS, NET_MEAN_ABS)


@pytest.mark.parametrize("seed,B,P,H,A,W,layers", [(300, 2, 100, 50, 32, 256, 3), (400, 1, 32, 8, 4, 64, 1),
                                                   (800, 6, 40, 50, 32, 256, 1)])
def test_flow_sample_end_to_end_small(seed, B, P, H, A, W, layers):
    Bd = _bd()
    note(f"flow sample seed={seed}")
    net, cache, sar, state, x0, oracle_v = _net_case(seed, B, P, H, A, W, layers)
    x = f32_dev(x0)
    Bd.pi_flow_sample(net, cache, sar, f32_dev(state), None, x, num_steps=10)
    torch.cuda.synchronize()
    want = F.euler_sample(x0.astype(np.float64), oracle_v, 10)
    assert_close(host64(x), want, f"flow sample seed={seed}", NET_MAX_ABS, NET_MEAN_ABS)


def test_flow_teacher_forced_steps_small():
    """Each GPU step, started from the GPU's own x_k, matches the oracle's step."""
    Bd = _bd()
    net, cache, sar, state, x0, oracle_v = _net_case(500, 2, 80, 50, 32, 256, 2)
    x = f32_dev(x0)
    N = 10
    for kstep in range(N):
        xk = host64(x)
        t = 1.0 + kstep * (-1.0 / N)
        vel = Bd.pi_velocity_eval(net, cache, sar, f32_dev(state), x, float(np.float32(t)))
        Bd.pi_euler_update(x, vel, -1.0 / N)
        torch.cuda.synchronize()
        want = F.euler_update(xk, oracle_v(xk, float(np.float32(t))), -1.0 / N)
        assert_close(host64(x), want, f"teacher-forced step {kstep}", NET_MAX_ABS, NET_MEAN_ABS)


def test_velocity_eval_pi0_full_size():
    """π0 control-step shape: width 1024, 18 cache layers of 816 slots, 51 suffix tokens."""
    Bd = _bd()
    w = I.pi0_step()
    note("velocity eval pi0 full size")
    P = w.structure.n_prefix
    net, cache, sar, state, x0, oracle_v = _net_case(2100, 1, P, 50, 32, 1024, 18, lens=np.array([P]))
    t = float(np.float32(0.7))
    vel = Bd.pi_velocity_eval(net, cache, sar, f32_dev(state), f32_dev(x0), t)
    torch.cuda.synchronize()
    assert_close(host64(vel), oracle_v(x0.astype(np.float64), t), "velocity pi0 full size", NET_MAX_ABS,
                 NET_MEAN_ABS)


def test_velocity_eval_serving_shape_sampled():
    """B=64 robots, 816 slots (valid U[600,816]), 18 layers: two samples vs the oracle."""
    Bd = _bd()
    note("velocity eval B=64 sampled")
    P, B = 816, 64
    net, cache, sar, state, x0, _ = _net_case(4200, B, P, 50, 32, 1024, 18,
                                             lens=I.valid_lengths(4299, B, 600, P))
    t = float(np.float32(0.5))
    vel = host64(Bd.pi_velocity_eval(net, cache, sar, f32_dev(state), f32_dev(x0), t))
    w = I.net_weights(4200, width=1024, action_dim=32)
    wf = {f: (f64(getattr(w, f)) if getattr(w, f).dtype == np.uint16 else getattr(w, f).astype(np.float64))
          for f in Bd.VelocityNet.FIELDS}
    pm = cache.prefix_mask.cpu().numpy()
    for b in (0, 63):
        ck = host64(cache.k[:, b:b + 1])
        cv = host64(cache.v[:, b:b + 1])
        want = F.velocity_net(x0[b:b + 1].astype(np.float64), t, state[b:b + 1].astype(np.float64), wf,
                              ck, cv, pm[b:b + 1], sar.cpu().numpy(), 8, 1, 256)
        assert_close(vel[b:b + 1], want, f"velocity serving sample {b}", NET_MAX_ABS, NET_MEAN_ABS)


def test_velocity_eval_without_out_projection():
    """W_o = 0: the layers leave h untouched, isolating the embedding and the
    normalised output projection (tight tolerance)."""
    Bd = _bd()
    net, cache, sar, state, x0, _ = _net_case(600, 3, 40, 50, 32, 256, 2)
    net.t["w_o"].zero_()
    wz = I.net_weights(600, width=256, action_dim=32)
    wf = {f: (f64(getattr(wz, f)) if getattr(wz, f).dtype == np.uint16 else getattr(wz, f).astype(np.float64))
          for f in Bd.VelocityNet.FIELDS}
    wf["w_o"] = np.zeros_like(wf["w_o"])
    t = float(np.float32(0.25))
    vel = Bd.pi_velocity_eval(net, cache, sar, f32_dev(state), f32_dev(x0), t)
    torch.cuda.synchronize()
    pm = cache.prefix_mask.cpu().numpy()
    want = F.velocity_net(x0.astype(np.float64), t, state.astype(np.float64), wf, host64(cache.k),
                          host64(cache.v), pm, sar.cpu().numpy(), 8, 1, 256)
    assert_close(host64(vel), want, "velocity with W_o = 0", max_abs=2e-4, mean_abs=2e-5)

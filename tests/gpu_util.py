"""Helpers for the GPU parity tests: device upload of the seeded inputs and the
parity tolerance check (max-abs <= 1e-2, mean-abs <= 1e-3 against the fp64
oracle on unit-variance bf16 inputs)."""
import os
import sys

import numpy as np
import torch

from prefix_lm_joint_amd import inputs as I

MAX_ABS = 1e-2
MEAN_ABS = 1e-3
# Stand-in velocity net (and the sampler driven by it): its definition rounds
# data-dependent activations to bf16 at 2 + 2 per layer points, so any fp32-
# accumulating implementation differs from the fp64 oracle by whole-ulp flips;
# tests/test_oracle_flow.py::test_net_tolerance_is_twice_the_fp32_floor measures
# that floor (~1.1e-3 mean-abs at the π0 shape) and pins this bound to it.
NET_MAX_ABS = 1e-2
NET_MEAN_ABS = 2.5e-3
# One joint layer (norms, projections, FFN around the attention): the same
# rounding-point floor, measured for an fp32 evaluation with bf16 attention
# weights by tests/test_oracle_layer.py::test_layer_tolerance_is_twice_the_fp32_floor
# (up to 1.5e-3 mean-abs, 8.6e-3 max-abs); the bound is about twice that.
LAYER_MAX_ABS = 2e-2
LAYER_MEAN_ABS = 3e-3
# π0.5's expert velocity at the true width through two expert layers (in- and
# out-projections, time MLP, final adaptive norm): the same floor, measured by
# tests/test_oracle_expert_flow.py::test_expert_velocity_tolerance_is_twice_the_fp32_floor
# (up to 2.3e-3 mean-abs, 1.2e-2 max-abs for velocities of mean magnitude ~0.8).
EXPERT_VEL_MAX_ABS = 3e-2
EXPERT_VEL_MEAN_ABS = 5e-3


def dev():
    return torch.device("cuda:0")


def note(msg):
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)
    path = os.environ.get("PI_GPU_LOG")
    if path:
        with open(path, "a") as f:
            f.write(msg + "\n")


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> device bfloat16 tensor (same bytes)."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev())


def u8_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(dev())


def f32_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev())


def host64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def f64(bits):
    return I.bf16_bits_to_f64(bits)


def assert_close(got: np.ndarray, want: np.ndarray, what: str, max_abs=MAX_ABS, mean_abs=MEAN_ABS):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - want)
    mx, mean = float(err.max()), float(err.mean())
    note(f"{what}: max_abs={mx:.3e} mean_abs={mean:.3e}")
    assert mx <= max_abs and mean <= mean_abs, f"{what}: max_abs {mx:.3e} mean_abs {mean:.3e}"

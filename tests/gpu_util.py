"""Helpers for the GPU parity tests: device upload of the seeded inputs and the
spec tolerance check (max-abs <= 1e-2, mean-abs <= 1e-3 against the fp64
oracle on unit-variance bf16 inputs)."""
import sys

import numpy as np
import torch

from prefix_lm_joint_amd import inputs as I

MAX_ABS = 1e-2
MEAN_ABS = 1e-3


def dev():
    return torch.device("cuda:0")


def note(msg):
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


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

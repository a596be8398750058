"""Rounding of float64 values to bfloat16, written for the oracle alone.

Used only where the stand-in velocity net defines a bf16 rounding point
(operands of its matrix products, the attention inputs and output).  Rounds
the exact float64 value once, to nearest with ties to even, keeping the
float64 container: bf16 keeps 8 significant bits, so the low 45 of float64's
52 fraction bits are rounded away.  Values are assumed inside float32's normal
range (true for every workload here); zeros stay zeros.
"""
import numpy as np

_DROP = 45  # float64 fraction bits (52) minus bf16 fraction bits (7)


def round_bf16(x) -> np.ndarray:
    a = np.ascontiguousarray(x, dtype=np.float64)
    u = a.view(np.uint64).copy()
    lsb = (u >> np.uint64(_DROP)) & np.uint64(1)
    u = u + (np.uint64((1 << (_DROP - 1)) - 1) + lsb)
    u = u & ~np.uint64((1 << _DROP) - 1)
    return u.view(np.float64).reshape(a.shape)

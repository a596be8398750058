"""Thin ctypes binding of libpi_joint.so (include/pi_joint.h).

Argument marshalling only: every step runs in the HIP library.  Tensors are torch
tensors on a ROCm device.  The C ABI sees only pointers and sizes, so every
wrapper checks the full shape and dtype of each tensor it passes against the
sizes it passes (ValueError before anything reaches the library, so a wrong or
undersized tensor can never turn into an out-of-bounds device access), plus
device placement and contiguity; the library then validates the sizes
themselves.  Workspaces a wrapper allocates for a caller-given stream are
recorded on that stream.  There is no fallback: if the library is missing or a
call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpi_joint.so")

PI_SEG_PREFIX, PI_SEG_FAST, PI_SEG_EXPERT = 0, 1, 2
PI_TILE_EMPTY, PI_TILE_PARTIAL, PI_TILE_FULL = 0, 1, 2
PI_MASK_TILE_Q, PI_MASK_TILE_K = 16, 32

_c_p = ctypes.c_void_p
_c_i = ctypes.c_int
_c_f = ctypes.c_float


class PiMask(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("N", ctypes.c_int32), ("n_qt", ctypes.c_int32), ("n_kt", ctypes.c_int32),
                ("forbid_bits", ctypes.c_uint32), ("bid", _c_p), ("pos", _c_p), ("tok", _c_p), ("tiles", _c_p)]


class PiKvCache(ctypes.Structure):
    _fields_ = [("k", _c_p), ("v", _c_p), ("prefix_mask", _c_p), ("layers", ctypes.c_int32),
                ("B", ctypes.c_int32), ("capacity", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("len", ctypes.c_int32)]


class PiVelocityNet(ctypes.Structure):
    _fields_ = [("width", ctypes.c_int32), ("action_dim", ctypes.c_int32), ("Hq", ctypes.c_int32),
                ("Hkv", ctypes.c_int32), ("d", ctypes.c_int32),
                ("w_state", _c_p), ("b_state", _c_p), ("w_in", _c_p), ("b_in", _c_p), ("w_time", _c_p),
                ("w_q", _c_p), ("w_k", _c_p), ("w_v", _c_p), ("w_o", _c_p), ("w_out", _c_p), ("b_out", _c_p)]


class PiLayerStream(ctypes.Structure):
    _fields_ = [("width", ctypes.c_int32), ("ffn", ctypes.c_int32), ("w_qkv", _c_p), ("w_o", _c_p), ("w_up", _c_p),
                ("w_down", _c_p), ("norm1", _c_p), ("norm2", _c_p), ("mod1", _c_p), ("mod2", _c_p)]


class PiExpertNet(ctypes.Structure):
    _fields_ = [("width", ctypes.c_int32), ("action_dim", ctypes.c_int32), ("layers", ctypes.c_int32),
                ("w_in", _c_p), ("b_in", _c_p), ("w_t1", _c_p), ("b_t1", _c_p), ("w_t2", _c_p), ("b_t2", _c_p),
                ("layer", ctypes.POINTER(PiLayerStream)), ("mod_f", _c_p), ("w_out", _c_p), ("b_out", _c_p)]


_SIGS = {
    "pi_mask_workspace_bytes": (ctypes.c_size_t, [_c_i, _c_i]),
    "pi_mask_build": (_c_i, [_c_p, _c_p, _c_p, ctypes.c_uint32, _c_i, _c_i, _c_p, ctypes.c_size_t,
                             ctypes.POINTER(PiMask), _c_p]),
    "pi_mask_materialize": (_c_i, [ctypes.POINTER(PiMask), _c_p, _c_p]),
    "pi_prefill_workspace_bytes": (ctypes.c_size_t, [_c_i, _c_i, _c_i, _c_i, _c_i]),
    "pi_joint_attn_prefill": (_c_i, [_c_p, _c_p, _c_p, _c_i, _c_i, _c_i, _c_i, _c_i, _c_f, _c_f,
                                     ctypes.POINTER(PiMask), _c_p, _c_p, ctypes.POINTER(PiKvCache), _c_i, _c_p,
                                     ctypes.c_size_t, _c_p]),
    "pi_attn_backward_workspace_bytes": (ctypes.c_size_t, [_c_i, _c_i, _c_i, _c_i, _c_i, _c_f]),
    "pi_joint_attn_backward": (_c_i, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i, _c_i, _c_i, _c_i, _c_i, _c_f, _c_f,
                                      ctypes.POINTER(PiMask), _c_p, _c_p, _c_p, _c_p, ctypes.c_size_t, _c_p]),
    "pi_joint_layer_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(PiLayerStream), ctypes.POINTER(PiLayerStream),
                                                         _c_i, _c_i, _c_i]),
    "pi_joint_layer_forward": (_c_i, [ctypes.POINTER(PiLayerStream), ctypes.POINTER(PiLayerStream), _c_p, _c_p, _c_p,
                                      _c_i, _c_i, _c_i, _c_f, ctypes.POINTER(PiMask), _c_p, ctypes.c_size_t, _c_p]),
    "pi_prefix_layer_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(PiLayerStream), _c_i, _c_i]),
    "pi_prefix_layer_forward": (_c_i, [ctypes.POINTER(PiLayerStream), _c_p, _c_p, _c_i, _c_i, _c_f,
                                       ctypes.POINTER(PiMask), ctypes.POINTER(PiKvCache), _c_i, _c_p, ctypes.c_size_t,
                                       _c_p]),
    "pi_expert_layer_decode_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(PiLayerStream), _c_i, _c_i, _c_i]),
    "pi_expert_layer_decode": (_c_i, [ctypes.POINTER(PiLayerStream), ctypes.POINTER(PiKvCache), _c_i, _c_p, _c_p, _c_p,
                                      _c_i, _c_i, _c_f, _c_p, ctypes.c_size_t, _c_p]),
    "pi_decode_workspace_bytes": (ctypes.c_size_t, [_c_i, _c_i, _c_i, _c_i]),
    "pi_suffix_decode_step": (_c_i, [ctypes.POINTER(PiKvCache), _c_i, _c_p, _c_p, _c_p, _c_p, _c_i, _c_i, _c_i,
                                     _c_f, _c_f, _c_p, _c_p, ctypes.c_size_t, _c_p]),
    "pi_suffix_decode_step_noalloc": (_c_i, [ctypes.POINTER(PiKvCache), _c_i, _c_p, _c_p, _c_p, _c_p, _c_i, _c_i,
                                             _c_i, _c_f, _c_f, _c_p, _c_p]),
    "pi_rope_apply": (_c_i, [_c_p, _c_p, _c_i, _c_i, _c_i, _c_i, _c_p, _c_f, _c_p]),
    "pi_kv_cache_append": (_c_i, [ctypes.POINTER(PiKvCache), _c_i, _c_p, _c_p, _c_i, _c_f, _c_p]),
    "pi_euler_update": (_c_i, [_c_p, _c_p, _c_f, ctypes.c_int64, _c_p]),
    "pi_flow_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(PiVelocityNet), _c_i, _c_i]),
    "pi_velocity_eval": (_c_i, [ctypes.POINTER(PiVelocityNet), ctypes.POINTER(PiKvCache), _c_p, _c_p, _c_p, _c_f,
                                _c_p, _c_i, _c_i, _c_i, _c_p, ctypes.c_size_t, _c_p]),
    "pi_flow_sample": (_c_i, [ctypes.POINTER(PiVelocityNet), ctypes.POINTER(PiKvCache), _c_p, _c_p, _c_p, _c_p,
                              _c_i, _c_i, _c_i, _c_i, _c_p, ctypes.c_size_t, _c_p]),
    "pi_expert_flow_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(PiExpertNet), _c_i, _c_i, _c_i, _c_i]),
    "pi_expert_velocity_eval": (_c_i, [ctypes.POINTER(PiExpertNet), ctypes.POINTER(PiKvCache), _c_p, _c_p, _c_f, _c_p,
                                       _c_i, _c_i, _c_i, _c_p, ctypes.c_size_t, _c_p]),
    "pi_expert_flow_sample": (_c_i, [ctypes.POINTER(PiExpertNet), ctypes.POINTER(PiKvCache), _c_p, _c_p, _c_i, _c_i,
                                     _c_i, _c_i, _c_p, ctypes.c_size_t, _c_p]),
    "pi_status_string": (ctypes.c_char_p, [_c_i]),
    "pi_last_error": (ctypes.c_char_p, []),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libpi_joint.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m prefix_lm_joint_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


class PiError(RuntimeError):
    def __init__(self, fn: str, status: int):
        L = lib()
        super().__init__(f"{fn}: {L.pi_status_string(status).decode()} ({status}): {L.pi_last_error().decode()}")
        self.status = status


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise PiError(fn, status)


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _expect(t: Optional[torch.Tensor], shape, dtype, name: str, optional: bool = False) -> None:
    """ValueError unless t has exactly `shape` (entries None match any size) and `dtype`."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    got = tuple(t.shape)
    if len(got) != len(shape) or any(w is not None and g != w for g, w in zip(got, shape)):
        raise ValueError(f"{name} has shape {got}, expected {tuple('*' if w is None else w for w in shape)}")


def _own(workspace: Optional[torch.Tensor], stream) -> None:
    """Keep a wrapper-allocated workspace alive until the work queued on `stream` is done."""
    if workspace is not None and stream is not None:
        workspace.record_stream(stream)


def _ptr(t: Optional[torch.Tensor], dtype=None, name="tensor"):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


# ---------------------------------------------------------------------------
# Mask
# ---------------------------------------------------------------------------

class Mask:
    """Compact mask: the ctypes struct plus the device workspace it points into."""

    def __init__(self, struct: PiMask, workspace: torch.Tensor):
        self.struct = struct
        self.workspace = workspace

    @property
    def B(self):
        return self.struct.B

    @property
    def N(self):
        return self.struct.N

    def _view(self, addr, count, dtype):
        base = self.workspace.data_ptr()
        itemsize = torch.empty((), dtype=dtype).element_size()
        off = addr - base
        return self.workspace[off:off + count * itemsize].view(dtype)

    def bid(self):
        return self._view(self.struct.bid, self.N, torch.int32)

    def pos(self):
        return self._view(self.struct.pos, self.B * self.N, torch.int32).view(self.B, self.N)

    def tok(self):
        return self._view(self.struct.tok, self.B * self.N, torch.int32).view(self.B, self.N)

    def tiles(self):
        s = self.struct
        return self._view(s.tiles, s.B * s.n_qt * s.n_kt, torch.uint8).view(s.B, s.n_qt, s.n_kt)


def pi_mask_workspace_bytes(B: int, N: int) -> int:
    return int(lib().pi_mask_workspace_bytes(B, N))


def pi_mask_build(input_mask: torch.Tensor, ar: torch.Tensor, seg: Optional[torch.Tensor] = None,
                  forbid_bits: int = 0, workspace: Optional[torch.Tensor] = None, stream=None) -> Mask:
    if input_mask.dim() != 2:
        raise ValueError(f"input_mask must be [B, N], got {tuple(input_mask.shape)}")
    B, N = input_mask.shape
    _expect(input_mask, (B, N), torch.uint8, "input_mask")
    _expect(ar, (N,), torch.uint8, "ar")
    _expect(seg, (N,), torch.uint8, "seg", optional=True)
    _expect(workspace, (None,), torch.uint8, "workspace", optional=True)
    nbytes = pi_mask_workspace_bytes(B, N)
    own = workspace is None
    if own:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=input_mask.device)
        _own(workspace, stream)
    out = PiMask()
    _check("pi_mask_build", lib().pi_mask_build(
        _ptr(input_mask, torch.uint8, "input_mask"), _ptr(ar, torch.uint8, "ar"), _ptr(seg, torch.uint8, "seg"),
        forbid_bits, B, N, _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), ctypes.byref(out),
        _stream(stream)))
    return Mask(out, workspace)


def pi_mask_materialize(mask: Mask, dense: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    if dense is None:
        dense = torch.empty((mask.B, mask.N, mask.N), dtype=torch.uint8, device=mask.workspace.device)
    _expect(dense, (mask.B, mask.N, mask.N), torch.uint8, "dense")
    _check("pi_mask_materialize", lib().pi_mask_materialize(ctypes.byref(mask.struct),
                                                            _ptr(dense, torch.uint8, "dense"), _stream(stream)))
    return dense


# ---------------------------------------------------------------------------
# KV cache, attention
# ---------------------------------------------------------------------------

class KVCache:
    """Caller-owned per-layer prefix KV cache: k, v bf16 [layers, B, capacity, Hkv, d]."""

    def __init__(self, k: torch.Tensor, v: torch.Tensor, prefix_mask: torch.Tensor, length: Optional[int] = None):
        if k.dim() != 5:
            raise ValueError(f"cache k must be [layers, B, capacity, Hkv, d], got {tuple(k.shape)}")
        layers, B, cap, Hkv, d = k.shape
        _expect(k, (layers, B, cap, Hkv, d), torch.bfloat16, "cache.k")
        _expect(v, (layers, B, cap, Hkv, d), torch.bfloat16, "cache.v")
        _expect(prefix_mask, (B, cap), torch.uint8, "prefix_mask")
        if length is not None and not 0 <= length <= cap:
            raise ValueError(f"cache length {length} outside [0, {cap}]")
        self.k, self.v, self.prefix_mask = k, v, prefix_mask
        self.struct = PiKvCache(_ptr(k, torch.bfloat16, "cache.k"), _ptr(v, torch.bfloat16, "cache.v"),
                                _ptr(prefix_mask, torch.uint8, "prefix_mask"), layers, B, cap, Hkv, d,
                                cap if length is None else length)

    @classmethod
    def empty(cls, layers, B, capacity, Hkv, d, device, length=None):
        k = torch.empty((layers, B, capacity, Hkv, d), dtype=torch.bfloat16, device=device)
        v = torch.empty_like(k)
        pm = torch.ones((B, capacity), dtype=torch.uint8, device=device)
        return cls(k, v, pm, length)

    @property
    def length(self) -> int:
        return int(self.struct.len)

    def advance(self, n: int) -> None:
        """Raise the slot count after pi_kv_cache_append has written n tokens to every layer."""
        assert self.struct.len + n <= self.struct.capacity
        self.struct.len += n

    def layer_k(self, layer):
        return self.k[layer]

    def layer_v(self, layer):
        return self.v[layer]


def pi_prefill_workspace_bytes(B: int, L: int, Hq: int, Hkv: int, d: int) -> int:
    return int(lib().pi_prefill_workspace_bytes(B, L, Hq, Hkv, d))


def prefill_workspace(B: int, L: int, Hq: int, Hkv: int, d: int, device) -> Optional[torch.Tensor]:
    """Device workspace for the rotary embedding and the key split of small batches (None if not needed)."""
    n = pi_prefill_workspace_bytes(B, L, Hq, Hkv, d)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def pi_joint_attn_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mask: Mask, o: Optional[torch.Tensor] = None,
                          scale: Optional[float] = None, cache: Optional[KVCache] = None, layer: int = 0,
                          workspace: Optional[torch.Tensor] = None, stream=None,
                          rope_base: float = 0.0, lse: Optional[torch.Tensor] = None) -> torch.Tensor:
    """``lse`` (fp32 [B, L, Hq]), when given, receives each row's log-sum-exp for a backward pass."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError(f"q, k must be [B, L, H, d], got {tuple(q.shape)}, {tuple(k.shape)}")
    B, L, Hq, d = q.shape
    Hkv = k.shape[2]
    _expect(q, (B, L, Hq, d), torch.bfloat16, "q")
    _expect(k, (B, L, Hkv, d), torch.bfloat16, "k")
    _expect(v, (B, L, Hkv, d), torch.bfloat16, "v")
    _expect(o, (B, L, Hq, d), torch.bfloat16, "o", optional=True)
    _expect(lse, (B, L, Hq), torch.float32, "lse", optional=True)
    _expect(workspace, (None,), torch.uint8, "workspace", optional=True)
    if (mask.B, mask.N) != (B, L):
        raise ValueError(f"mask built for B={mask.B} N={mask.N}, q has B={B} L={L}")
    if cache is not None and (cache.struct.B, cache.struct.Hkv, cache.struct.d) != (B, Hkv, d):
        raise ValueError("cache batch / heads / head_dim do not match q, k")
    if scale is None:
        scale = d ** -0.5
    if o is None:
        o = torch.empty_like(q)
    _check("pi_joint_attn_prefill", lib().pi_joint_attn_prefill(
        _ptr(q, torch.bfloat16, "q"), _ptr(k, torch.bfloat16, "k"), _ptr(v, torch.bfloat16, "v"), B, L, Hq, Hkv, d,
        scale, rope_base, ctypes.byref(mask.struct), _ptr(o, torch.bfloat16, "o"),
        _ptr(lse, torch.float32, "lse") if lse is not None else None,
        ctypes.byref(cache.struct) if cache is not None else None, layer,
        _ptr(workspace, torch.uint8, "workspace") if workspace is not None else None,
        workspace.numel() if workspace is not None else 0, _stream(stream)))
    return o


def pi_attn_backward_workspace_bytes(B: int, L: int, Hq: int, Hkv: int, d: int, rope_base: float = 0.0) -> int:
    return int(lib().pi_attn_backward_workspace_bytes(B, L, Hq, Hkv, d, rope_base))


def backward_workspace(B: int, L: int, Hq: int, Hkv: int, d: int, device, rope_base: float = 0.0) -> torch.Tensor:
    """Device workspace of pi_joint_attn_backward (the rows' statistics; with the
    rotary embedding also the rotated Q/K)."""
    n = pi_attn_backward_workspace_bytes(B, L, Hq, Hkv, d, rope_base)
    if n == 0:
        raise ValueError(f"pi_joint_attn_backward does not support (Hq={Hq}, Hkv={Hkv}, d={d})")
    return torch.empty(n, dtype=torch.uint8, device=device)


def pi_joint_attn_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, dout: torch.Tensor,
                           lse: torch.Tensor, mask: Mask, workspace: torch.Tensor, scale: Optional[float] = None,
                           dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
                           dv: Optional[torch.Tensor] = None, stream=None, rope_base: float = 0.0):
    """Gradients (dq, dk, dv) of the prefill for upstream gradient ``dout``; ``o`` and ``lse``
    are the prefill's output and log-sum-exp (taken with the same ``rope_base``)."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError(f"q, k must be [B, L, H, d], got {tuple(q.shape)}, {tuple(k.shape)}")
    B, L, Hq, d = q.shape
    Hkv = k.shape[2]
    for t, n in ((q, "q"), (o, "o"), (dout, "dout"), (dq, "dq")):
        _expect(t, (B, L, Hq, d), torch.bfloat16, n, optional=n == "dq")
    for t, n in ((k, "k"), (v, "v"), (dk, "dk"), (dv, "dv")):
        _expect(t, (B, L, Hkv, d), torch.bfloat16, n, optional=n in ("dk", "dv"))
    _expect(lse, (B, L, Hq), torch.float32, "lse")
    _expect(workspace, (None,), torch.uint8, "workspace")
    if (mask.B, mask.N) != (B, L):
        raise ValueError(f"mask built for B={mask.B} N={mask.N}, q has B={B} L={L}")
    if scale is None:
        scale = d ** -0.5
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check("pi_joint_attn_backward", lib().pi_joint_attn_backward(
        _ptr(q, torch.bfloat16, "q"), _ptr(k, torch.bfloat16, "k"), _ptr(v, torch.bfloat16, "v"),
        _ptr(o, torch.bfloat16, "o"), _ptr(dout, torch.bfloat16, "dout"), _ptr(lse, torch.float32, "lse"),
        B, L, Hq, Hkv, d, scale, rope_base, ctypes.byref(mask.struct), _ptr(dq, torch.bfloat16, "dq"),
        _ptr(dk, torch.bfloat16, "dk"), _ptr(dv, torch.bfloat16, "dv"), _ptr(workspace, torch.uint8, "workspace"),
        workspace.numel(), _stream(stream)))
    return dq, dk, dv


class LayerStream:
    """Device weights of one stream of a joint layer (keeps the tensors alive)."""

    def __init__(self, w_qkv, w_o, w_up, w_down, norm1=None, norm2=None, mod1=None, mod2=None):
        if w_qkv.dim() != 2 or w_up.dim() != 2:
            raise ValueError("w_qkv and w_up must be matrices")
        W, F = int(w_qkv.shape[1]), int(w_up.shape[0])
        _expect(w_qkv, (None, W), torch.bfloat16, "w_qkv")
        _expect(w_o, (W, None), torch.bfloat16, "w_o")
        _expect(w_up, (F, W), torch.bfloat16, "w_up")
        _expect(w_down, (W, F), torch.bfloat16, "w_down")
        if w_qkv.shape[0] != w_o.shape[1] + 2 * 256:
            raise ValueError(f"w_qkv has {w_qkv.shape[0]} rows, expected Hq*d + 2*Hkv*d = {w_o.shape[1] + 512}")
        for t, n in ((norm1, "norm1"), (norm2, "norm2")):
            _expect(t, (W,), torch.float32, n, optional=True)
        for t, n in ((mod1, "mod1"), (mod2, "mod2")):
            _expect(t, (2 * W, W), torch.bfloat16, n, optional=True)
        self.tensors = dict(w_qkv=w_qkv, w_o=w_o, w_up=w_up, w_down=w_down, norm1=norm1, norm2=norm2, mod1=mod1,
                            mod2=mod2)
        bf = lambda t, n: _ptr(t, torch.bfloat16, n) if t is not None else None
        f32 = lambda t, n: _ptr(t, torch.float32, n) if t is not None else None
        self.struct = PiLayerStream(int(w_qkv.shape[1]), int(w_up.shape[0]), bf(w_qkv, "w_qkv"), bf(w_o, "w_o"),
                                    bf(w_up, "w_up"), bf(w_down, "w_down"), f32(norm1, "norm1"), f32(norm2, "norm2"),
                                    bf(mod1, "mod1"), bf(mod2, "mod2"))


def pi_joint_layer_workspace_bytes(prefix: LayerStream, expert: LayerStream, B: int, Np: int, Ne: int) -> int:
    return int(lib().pi_joint_layer_workspace_bytes(ctypes.byref(prefix.struct), ctypes.byref(expert.struct), B, Np,
                                                    Ne))


def layer_workspace(prefix: LayerStream, expert: LayerStream, B: int, Np: int, Ne: int, device) -> torch.Tensor:
    n = pi_joint_layer_workspace_bytes(prefix, expert, B, Np, Ne)
    if n == 0:
        raise ValueError("pi_joint_layer_forward does not support these streams")
    return torch.empty(n, dtype=torch.uint8, device=device)


def pi_joint_layer_forward(prefix: LayerStream, expert: LayerStream, h_p: torch.Tensor, h_e: torch.Tensor,
                           cond: Optional[torch.Tensor], mask: Mask, workspace: torch.Tensor,
                           scale: Optional[float] = None, stream=None) -> None:
    """One joint layer; updates h_p [B, Np, Wp] and h_e [B, Ne, We] (fp32) in place."""
    B, Np = h_p.shape[:2]
    Ne = h_e.shape[1]
    _expect(h_p, (B, Np, prefix.struct.width), torch.float32, "h_p")
    _expect(h_e, (B, Ne, expert.struct.width), torch.float32, "h_e")
    # cond conditions the adaptive stream; a stream with no tokens needs none
    adaptive = [st for st, n in ((prefix, Np), (expert, Ne)) if st.tensors["mod1"] is not None and n > 0]
    if adaptive:
        _expect(cond, (B, adaptive[0].struct.width), torch.float32, "cond")
    _expect(workspace, (None,), torch.uint8, "workspace")
    if (mask.B, mask.N) != (B, Np + Ne):
        raise ValueError(f"mask built for B={mask.B} N={mask.N}, layer has B={B} N={Np + Ne}")
    if scale is None:
        scale = 256 ** -0.5
    _check("pi_joint_layer_forward", lib().pi_joint_layer_forward(
        ctypes.byref(prefix.struct), ctypes.byref(expert.struct), _ptr(h_p, torch.float32, "h_p"),
        _ptr(h_e, torch.float32, "h_e"), _ptr(cond, torch.float32, "cond") if cond is not None else None, B, Np, Ne,
        scale, ctypes.byref(mask.struct), _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
        _stream(stream)))


def prefix_layer_workspace(prefix: LayerStream, B: int, Np: int, device) -> torch.Tensor:
    n = int(lib().pi_prefix_layer_workspace_bytes(ctypes.byref(prefix.struct), B, Np))
    if n == 0:
        raise ValueError("pi_prefix_layer_forward does not support this stream")
    return torch.empty(n, dtype=torch.uint8, device=device)


def pi_prefix_layer_forward(prefix: LayerStream, h_p: torch.Tensor, mask: Mask, cache: "KVCache", layer: int,
                            workspace: torch.Tensor, cond: Optional[torch.Tensor] = None,
                            scale: Optional[float] = None, stream=None) -> None:
    """The prefix stream's layer alone; updates h_p [B, Np, W] (fp32) in place and writes
    the layer's K/V into cache layer `layer` (slots [0, Np))."""
    B, Np = h_p.shape[:2]
    _expect(h_p, (B, Np, prefix.struct.width), torch.float32, "h_p")
    if prefix.tensors["mod1"] is not None:
        _expect(cond, (B, prefix.struct.width), torch.float32, "cond")
    _expect(workspace, (None,), torch.uint8, "workspace")
    if (mask.B, mask.N) != (B, Np):
        raise ValueError(f"mask built for B={mask.B} N={mask.N}, prefix has B={B} N={Np}")
    if scale is None:
        scale = 256 ** -0.5
    _check("pi_prefix_layer_forward", lib().pi_prefix_layer_forward(
        ctypes.byref(prefix.struct), _ptr(h_p, torch.float32, "h_p"),
        _ptr(cond, torch.float32, "cond") if cond is not None else None, B, Np, scale, ctypes.byref(mask.struct),
        ctypes.byref(cache.struct), layer, _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
        _stream(stream)))


def pi_expert_layer_decode_workspace_bytes(expert: LayerStream, B: int, S: int, length: int) -> int:
    return int(lib().pi_expert_layer_decode_workspace_bytes(ctypes.byref(expert.struct), B, S, length))


def expert_decode_workspace(expert: LayerStream, cache: "KVCache", S: int) -> torch.Tensor:
    n = pi_expert_layer_decode_workspace_bytes(expert, cache.struct.B, S, cache.struct.len)
    if n == 0:
        raise ValueError("pi_expert_layer_decode does not support this stream")
    return torch.empty(n, dtype=torch.uint8, device=cache.k.device)


def pi_expert_layer_decode(expert: LayerStream, cache: "KVCache", layer: int, h_e: torch.Tensor,
                           cond: Optional[torch.Tensor], suffix_ar: torch.Tensor, workspace: torch.Tensor,
                           scale: Optional[float] = None, stream=None) -> None:
    """The expert stream's layer against cache layer `layer`; updates h_e [B, S, W] (fp32) in place."""
    B, S = h_e.shape[:2]
    _expect(h_e, (B, S, expert.struct.width), torch.float32, "h_e")
    if expert.tensors["mod1"] is not None:
        _expect(cond, (B, expert.struct.width), torch.float32, "cond")
    _expect(suffix_ar, (S,), torch.uint8, "suffix_ar")
    _expect(workspace, (None,), torch.uint8, "workspace")
    if cache.struct.B != B:
        raise ValueError(f"cache holds B={cache.struct.B} samples, h_e has {B}")
    if scale is None:
        scale = 256 ** -0.5
    _check("pi_expert_layer_decode", lib().pi_expert_layer_decode(
        ctypes.byref(expert.struct), ctypes.byref(cache.struct), layer, _ptr(h_e, torch.float32, "h_e"),
        _ptr(cond, torch.float32, "cond") if cond is not None else None, _ptr(suffix_ar, torch.uint8, "suffix_ar"),
        B, S, scale, _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)))


def pi_decode_workspace_bytes(B: int, S: int, Hq: int, length: int) -> int:
    return int(lib().pi_decode_workspace_bytes(B, S, Hq, length))


def decode_workspace(cache: KVCache, S: int, Hq: int = 8) -> Optional[torch.Tensor]:
    """Device workspace for the rotary embedding and the key split of small batches (None if not needed)."""
    n = pi_decode_workspace_bytes(cache.struct.B, S, Hq, cache.struct.len)
    return torch.empty(n, dtype=torch.uint8, device=cache.k.device) if n else None


def pi_suffix_decode_step(cache: KVCache, layer: int, q_s: torch.Tensor, k_s: torch.Tensor, v_s: torch.Tensor,
                          suffix_ar: torch.Tensor, o_s: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                          workspace: Optional[torch.Tensor] = None, stream=None,
                          rope_base: float = 0.0) -> torch.Tensor:
    """``workspace`` from decode_workspace() enables the key split of small batches (None runs unsplit)
    and is required with ``rope_base`` > 0."""
    if q_s.dim() != 4:
        raise ValueError(f"q_s must be [B, S, Hq, d], got {tuple(q_s.shape)}")
    B, S, Hq, d = q_s.shape
    c = cache.struct
    if (c.B, c.d) != (B, d):
        raise ValueError(f"cache holds B={c.B}, d={c.d}; q_s has B={B}, d={d}")
    _expect(q_s, (B, S, Hq, d), torch.bfloat16, "q_s")
    _expect(k_s, (B, S, c.Hkv, d), torch.bfloat16, "k_s")
    _expect(v_s, (B, S, c.Hkv, d), torch.bfloat16, "v_s")
    _expect(suffix_ar, (S,), torch.uint8, "suffix_ar")
    _expect(o_s, (B, S, Hq, d), torch.bfloat16, "o_s", optional=True)
    _expect(workspace, (None,), torch.uint8, "workspace", optional=True)
    if scale is None:
        scale = d ** -0.5
    if o_s is None:
        o_s = torch.empty_like(q_s)
    _check("pi_suffix_decode_step", lib().pi_suffix_decode_step(
        ctypes.byref(cache.struct), layer, _ptr(q_s, torch.bfloat16, "q_s"), _ptr(k_s, torch.bfloat16, "k_s"),
        _ptr(v_s, torch.bfloat16, "v_s"), _ptr(suffix_ar, torch.uint8, "suffix_ar"), B, S, Hq, scale, rope_base,
        _ptr(o_s, torch.bfloat16, "o_s"), _ptr(workspace, torch.uint8, "workspace"),
        workspace.numel() if workspace is not None else 0, _stream(stream)))
    return o_s


def pi_suffix_decode_step_noalloc(cache: KVCache, layer: int, q_s: torch.Tensor, k_s: torch.Tensor,
                                  v_s: torch.Tensor, suffix_ar: torch.Tensor, o_s: torch.Tensor,
                                  scale: Optional[float] = None, stream=None, rope_base: float = 0.0) -> torch.Tensor:
    """pi_suffix_decode_step without a workspace: the library's own per-GPU scratch
    stands in for it, and neither this wrapper nor the library allocates (o_s is
    required).  Calls overlapping on one GPU race on that scratch."""
    if q_s.dim() != 4:
        raise ValueError(f"q_s must be [B, S, Hq, d], got {tuple(q_s.shape)}")
    B, S, Hq, d = q_s.shape
    c = cache.struct
    if (c.B, c.d) != (B, d):
        raise ValueError(f"cache holds B={c.B}, d={c.d}; q_s has B={B}, d={d}")
    _expect(q_s, (B, S, Hq, d), torch.bfloat16, "q_s")
    _expect(k_s, (B, S, c.Hkv, d), torch.bfloat16, "k_s")
    _expect(v_s, (B, S, c.Hkv, d), torch.bfloat16, "v_s")
    _expect(suffix_ar, (S,), torch.uint8, "suffix_ar")
    _expect(o_s, (B, S, Hq, d), torch.bfloat16, "o_s")
    if scale is None:
        scale = d ** -0.5
    _check("pi_suffix_decode_step_noalloc", lib().pi_suffix_decode_step_noalloc(
        ctypes.byref(cache.struct), layer, _ptr(q_s, torch.bfloat16, "q_s"), _ptr(k_s, torch.bfloat16, "k_s"),
        _ptr(v_s, torch.bfloat16, "v_s"), _ptr(suffix_ar, torch.uint8, "suffix_ar"), B, S, Hq, scale, rope_base,
        _ptr(o_s, torch.bfloat16, "o_s"), _stream(stream)))
    return o_s


def pi_rope_apply(x: torch.Tensor, pos: torch.Tensor, base: float = 10000.0, y: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    """Rotary embedding of x [B, L, H, d] bf16 at positions pos [B, L] int32 (y may be x)."""
    if x.dim() != 4:
        raise ValueError(f"x must be [B, L, H, d], got {tuple(x.shape)}")
    B, L, H, d = x.shape
    _expect(x, (B, L, H, d), torch.bfloat16, "x")
    _expect(pos, (B, L), torch.int32, "pos")
    _expect(y, (B, L, H, d), torch.bfloat16, "y", optional=True)
    if y is None:
        y = torch.empty_like(x)
    _check("pi_rope_apply", lib().pi_rope_apply(_ptr(x, torch.bfloat16, "x"), _ptr(y, torch.bfloat16, "y"), B, L, H,
                                                d, _ptr(pos, torch.int32, "pos"), base, _stream(stream)))
    return y


def pi_kv_cache_append(cache: KVCache, layer: int, k_new: torch.Tensor, v_new: torch.Tensor,
                       rope_base: float = 0.0, stream=None) -> None:
    """Write k_new/v_new [B, n, Hkv, d] at slots [len, len + n) of one layer and mark them valid.
    The caller advances the length (KVCache.advance) once every layer has its tokens."""
    c = cache.struct
    if k_new.dim() != 4:
        raise ValueError(f"k_new must be [B, n, Hkv, d], got {tuple(k_new.shape)}")
    n = k_new.shape[1]
    _expect(k_new, (c.B, n, c.Hkv, c.d), torch.bfloat16, "k_new")
    _expect(v_new, (c.B, n, c.Hkv, c.d), torch.bfloat16, "v_new")
    _check("pi_kv_cache_append", lib().pi_kv_cache_append(
        ctypes.byref(cache.struct), layer, _ptr(k_new, torch.bfloat16, "k_new"), _ptr(v_new, torch.bfloat16, "v_new"),
        n, rope_base, _stream(stream)))


def pi_euler_update(x: torch.Tensor, v: torch.Tensor, dt: float, stream=None) -> torch.Tensor:
    _expect(x, tuple(x.shape), torch.float32, "x")
    _expect(v, tuple(x.shape), torch.float32, "v")
    _check("pi_euler_update", lib().pi_euler_update(_ptr(x, torch.float32, "x"), _ptr(v, torch.float32, "v"), dt,
                                                    x.numel(), _stream(stream)))
    return x


# ---------------------------------------------------------------------------
# Velocity net and flow sampler
# ---------------------------------------------------------------------------

class VelocityNet:
    """Device weights of the stand-in velocity net (see pi_joint.h)."""

    FIELDS = ("w_state", "b_state", "w_in", "b_in", "w_time", "w_q", "w_k", "w_v", "w_o", "w_out", "b_out")

    def __init__(self, tensors: dict, Hq=8, Hkv=1, d=256):
        self.t = tensors
        if tensors["w_in"].dim() != 2:
            raise ValueError("w_in must be [W, A]")
        W, A = tensors["w_in"].shape
        shapes = dict(w_state=(W, A), b_state=(W,), w_in=(W, A), b_in=(W,), w_time=(W,), w_q=(Hq * d, W),
                      w_k=(Hkv * d, W), w_v=(Hkv * d, W), w_o=(W, Hq * d), w_out=(A, W), b_out=(A,))
        for f in self.FIELDS:
            want = torch.bfloat16 if f.startswith("w_") and f != "w_time" else torch.float32
            _expect(tensors[f], shapes[f], want, f)
        ptrs = []
        for f in self.FIELDS:
            want = torch.bfloat16 if f.startswith("w_") and f != "w_time" else torch.float32
            ptrs.append(_ptr(tensors[f], want, f))
        self.struct = PiVelocityNet(W, A, Hq, Hkv, d, *ptrs)
        self.width, self.action_dim = W, A

    @classmethod
    def from_numpy(cls, weights, device, Hq=8, Hkv=1, d=256):
        """``weights``: an inputs.NetWeights (bf16 bits as uint16, vectors float32)."""
        import numpy as np
        t = {}
        for f in cls.FIELDS:
            a = getattr(weights, f)
            if a.dtype == np.uint16:
                t[f] = torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(device)
            else:
                t[f] = torch.from_numpy(a.astype(np.float32)).to(device)
        return cls(t, Hq, Hkv, d)


def pi_flow_workspace_bytes(net: VelocityNet, B: int, H: int) -> int:
    return int(lib().pi_flow_workspace_bytes(ctypes.byref(net.struct), B, H))


def flow_workspace(net: VelocityNet, B: int, H: int, device) -> torch.Tensor:
    return torch.empty(pi_flow_workspace_bytes(net, B, H), dtype=torch.uint8, device=device)


def pi_velocity_eval(net: VelocityNet, cache: KVCache, suffix_ar: torch.Tensor, state: torch.Tensor, x: torch.Tensor,
                     t: float, vel: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
    if x.dim() != 3:
        raise ValueError(f"x must be [B, H, A], got {tuple(x.shape)}")
    B, H, A = x.shape
    _expect(x, (B, H, net.action_dim), torch.float32, "x")
    _expect(state, (B, A), torch.float32, "state")
    _expect(suffix_ar, (H + 1,), torch.uint8, "suffix_ar")
    _expect(vel, (B, H, A), torch.float32, "vel", optional=True)
    _expect(workspace, (None,), torch.uint8, "workspace", optional=True)
    if cache.struct.B != B:
        raise ValueError(f"cache holds B={cache.struct.B} samples, x has {B}")
    if vel is None:
        vel = torch.empty_like(x)
    if workspace is None:
        workspace = flow_workspace(net, B, H, x.device)
        _own(workspace, stream)
    _check("pi_velocity_eval", lib().pi_velocity_eval(
        ctypes.byref(net.struct), ctypes.byref(cache.struct), _ptr(suffix_ar, torch.uint8, "suffix_ar"),
        _ptr(state, torch.float32, "state"), _ptr(x, torch.float32, "x"), t, _ptr(vel, torch.float32, "vel"), B, H,
        A, _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)))
    return vel


def pi_flow_sample(net: Optional[VelocityNet], cache: Optional[KVCache], suffix_ar: Optional[torch.Tensor],
                   state: Optional[torch.Tensor], v_const: Optional[torch.Tensor], x: torch.Tensor,
                   num_steps: int = 10, workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    if x.dim() != 3:
        raise ValueError(f"x must be [B, H, A], got {tuple(x.shape)}")
    B, H, A = x.shape
    _expect(x, (B, H, A), torch.float32, "x")
    _expect(workspace, (None,), torch.uint8, "workspace", optional=True)
    if net is not None:
        if cache is None or cache.struct.B != B:
            raise ValueError("net mode needs a cache holding the batch's B samples")
        _expect(x, (B, H, net.action_dim), torch.float32, "x")
        _expect(state, (B, A), torch.float32, "state")
        _expect(suffix_ar, (H + 1,), torch.uint8, "suffix_ar")
    else:
        _expect(v_const, (B, H, A), torch.float32, "v_const")
    if net is not None and workspace is None:
        workspace = flow_workspace(net, B, H, x.device)
        _own(workspace, stream)
    _check("pi_flow_sample", lib().pi_flow_sample(
        ctypes.byref(net.struct) if net is not None else None,
        ctypes.byref(cache.struct) if cache is not None else None,
        _ptr(suffix_ar, torch.uint8, "suffix_ar"), _ptr(state, torch.float32, "state"),
        _ptr(v_const, torch.float32, "v_const"), _ptr(x, torch.float32, "x"), B, H, A, num_steps,
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel() if workspace is not None else 0,
        _stream(stream)))
    return x


# ---------------------------------------------------------------------------
# π0.5 action expert at its true shape and the sampler driven by it
# ---------------------------------------------------------------------------

class ExpertNet:
    """Device weights of π0.5's action expert (see pi_joint.h; keeps the tensors alive)."""

    FIELDS = ("w_in", "b_in", "w_t1", "b_t1", "w_t2", "b_t2", "mod_f", "w_out", "b_out")

    def __init__(self, tensors: dict, layers: list):
        self.t = tensors
        self.layers = layers
        if tensors["w_in"].dim() != 2:
            raise ValueError("w_in must be [W, A]")
        W, A = tensors["w_in"].shape
        shapes = dict(w_in=(W, A), b_in=(W,), w_t1=(W, W), b_t1=(W,), w_t2=(W, W), b_t2=(W,), mod_f=(2 * W, W),
                      w_out=(A, W), b_out=(A,))
        for f in self.FIELDS:
            _expect(tensors[f], shapes[f], torch.bfloat16 if f.startswith(("w_", "mod")) else torch.float32, f)
        for i, l in enumerate(layers):
            if l.struct.width != W or l.tensors["mod1"] is None:
                raise ValueError(f"expert layer {i} must be an adaptive stream of width {W}")
        self._arr = (PiLayerStream * len(layers))(*[l.struct for l in layers])
        p = {f: _ptr(tensors[f], torch.bfloat16 if f.startswith(("w_", "mod")) else torch.float32, f)
             for f in self.FIELDS}
        self.struct = PiExpertNet(W, A, len(layers), p["w_in"], p["b_in"], p["w_t1"], p["b_t1"], p["w_t2"],
                                  p["b_t2"], ctypes.cast(self._arr, ctypes.POINTER(PiLayerStream)), p["mod_f"],
                                  p["w_out"], p["b_out"])
        self.width, self.action_dim = W, A

    @classmethod
    def from_numpy(cls, weights: dict, device):
        """``weights``: inputs.expert_net_weights (bf16 bits as uint16, vectors float32)."""
        import numpy as np

        def up(a):
            if a.dtype == np.uint16:
                return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(device)
            return torch.from_numpy(a.astype(np.float32)).to(device)

        t = {f: up(weights[f]) for f in cls.FIELDS}
        layers = [LayerStream(**{k: up(v) for k, v in lw.items()}) for lw in weights["layers"]]
        return cls(t, layers)


def pi_expert_flow_workspace_bytes(net: ExpertNet, B: int, H: int, length: int, num_steps: int) -> int:
    return int(lib().pi_expert_flow_workspace_bytes(ctypes.byref(net.struct), B, H, length, num_steps))


def expert_flow_workspace(net: ExpertNet, cache: KVCache, H: int, num_steps: int) -> torch.Tensor:
    n = pi_expert_flow_workspace_bytes(net, cache.struct.B, H, cache.struct.len, num_steps)
    if n == 0:
        raise ValueError("pi_expert_flow_sample does not support this net / shape")
    return torch.empty(n, dtype=torch.uint8, device=cache.k.device)


def pi_expert_velocity_eval(net: ExpertNet, cache: KVCache, suffix_ar: torch.Tensor, x: torch.Tensor, t: float,
                            vel: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                            stream=None) -> torch.Tensor:
    if x.dim() != 3:
        raise ValueError(f"x must be [B, H, A], got {tuple(x.shape)}")
    B, H, A = x.shape
    _expect(x, (B, H, net.action_dim), torch.float32, "x")
    _expect(suffix_ar, (H,), torch.uint8, "suffix_ar")
    _expect(vel, (B, H, A), torch.float32, "vel", optional=True)
    _expect(workspace, (None,), torch.uint8, "workspace", optional=True)
    if cache.struct.B != B:
        raise ValueError(f"cache holds B={cache.struct.B} samples, x has {B}")
    if vel is None:
        vel = torch.empty_like(x)
    if workspace is None:
        workspace = expert_flow_workspace(net, cache, H, 1)
        _own(workspace, stream)
    _check("pi_expert_velocity_eval", lib().pi_expert_velocity_eval(
        ctypes.byref(net.struct), ctypes.byref(cache.struct), _ptr(suffix_ar, torch.uint8, "suffix_ar"),
        _ptr(x, torch.float32, "x"), t, _ptr(vel, torch.float32, "vel"), B, H, A,
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)))
    return vel


def pi_expert_flow_sample(net: ExpertNet, cache: KVCache, suffix_ar: torch.Tensor, x: torch.Tensor,
                          num_steps: int = 10, workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Euler sampler with the expert net: x [B, H, A] fp32 holds the noise and ends as the actions."""
    if x.dim() != 3:
        raise ValueError(f"x must be [B, H, A], got {tuple(x.shape)}")
    B, H, A = x.shape
    _expect(x, (B, H, net.action_dim), torch.float32, "x")
    _expect(suffix_ar, (H,), torch.uint8, "suffix_ar")
    _expect(workspace, (None,), torch.uint8, "workspace", optional=True)
    if cache.struct.B != B:
        raise ValueError(f"cache holds B={cache.struct.B} samples, x has {B}")
    if workspace is None:
        workspace = expert_flow_workspace(net, cache, H, num_steps)
        _own(workspace, stream)
    _check("pi_expert_flow_sample", lib().pi_expert_flow_sample(
        ctypes.byref(net.struct), ctypes.byref(cache.struct), _ptr(suffix_ar, torch.uint8, "suffix_ar"),
        _ptr(x, torch.float32, "x"), B, H, A, num_steps, _ptr(workspace, torch.uint8, "workspace"),
        workspace.numel(), _stream(stream)))
    return x

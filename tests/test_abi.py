"""The C-ABI library loads, exports every function include/pi_joint.h declares,
and rejects bad arguments on the host before anything is launched (no GPU is
touched by these tests)."""
import ctypes
import os
import re

import pytest

from prefix_lm_joint_amd import binding as Bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pi_joint.h")

needs_lib = pytest.mark.skipif(not os.path.exists(Bd.LIB_PATH), reason="libpi_joint.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pi_[a-z_0-9]+)\s*\(", text)) - {"PI_FORBID"})


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("pi_mask_build", "pi_joint_attn_prefill", "pi_suffix_decode_step", "pi_euler_update",
                     "pi_flow_sample"):
        assert required in names


@needs_lib
def test_library_exports_every_declared_function():
    lib = ctypes.CDLL(Bd.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    # the binding declares a signature for every exported entry point
    assert set(declared_functions()) <= set(Bd._SIGS), set(declared_functions()) - set(Bd._SIGS)


@needs_lib
def test_status_strings():
    lib = Bd.lib()
    assert lib.pi_status_string(0) == b"ok"
    assert lib.pi_status_string(-3) == b"workspace too small"


@needs_lib
def test_workspace_queries_are_host_only():
    lib = Bd.lib()
    assert lib.pi_mask_workspace_bytes(2, 100) > 0
    assert lib.pi_mask_workspace_bytes(0, 100) == 0
    assert lib.pi_mask_workspace_bytes(1, (1 << 20) + 1) == 0
    net = Bd.PiVelocityNet(1024, 32, 8, 1, 256)
    n1 = lib.pi_flow_workspace_bytes(ctypes.byref(net), 1, 50)
    n64 = lib.pi_flow_workspace_bytes(ctypes.byref(net), 64, 50)
    assert 0 < n1 < n64


P = ctypes.c_void_p
FAKE = P(0x10000)  # a non-null, 16-byte aligned address that is never dereferenced


@needs_lib
def test_prefill_rejects_bad_arguments_before_launch():
    lib = Bd.lib()
    m = Bd.PiMask(B=1, N=64, n_qt=4, n_kt=2, forbid_bits=0, bid=FAKE, pos=FAKE, tok=FAKE, tiles=FAKE)
    call = lambda **kw: lib.pi_joint_attn_prefill(
        kw.get("q", FAKE), FAKE, FAKE, kw.get("B", 1), kw.get("L", 64), kw.get("Hq", 8), kw.get("Hkv", 1),
        kw.get("d", 256), kw.get("scale", 0.0625), kw.get("rope", 0.0), ctypes.byref(m), FAKE, None, None, 0,
        kw.get("ws", None), kw.get("ws_bytes", 0), None)
    assert call(d=128) == -2                 # unsupported head dim
    assert call(Hq=6, Hkv=4) == -1           # Hq not a multiple of Hkv
    assert call(L=65) == -1                  # mask built for another length
    assert call(scale=0.0) == -1
    assert call(rope=0.5) == -1              # rope_base must be 0 or > 1
    assert call(q=P(0x10008)) == -1          # misaligned
    assert call(q=None) == -1
    assert b"pi_joint_attn_prefill" in lib.pi_last_error()
    # the rotary embedding needs the workspace (rotated K)
    assert call(rope=10000.0) == -3
    assert call(rope=10000.0, ws=P(0x100000), ws_bytes=64 * 256 * 2 - 1) == -3
    # the workspace holds the rotated K, plus the key split's partials for a small GQA batch
    need = lib.pi_prefill_workspace_bytes(1, 816, 8, 1, 256)
    assert need > 816 * 256 * 2
    assert lib.pi_prefill_workspace_bytes(1, 816, 24, 24, 64) == 816 * 24 * 64 * 2
    assert lib.pi_prefill_workspace_bytes(1, 816, 8, 2, 256) == 0          # unsupported heads
    m816 = Bd.PiMask(B=1, N=816, n_qt=51, n_kt=26, forbid_bits=0, bid=FAKE, pos=FAKE, tok=FAKE, tiles=FAKE)
    assert lib.pi_joint_attn_prefill(FAKE, FAKE, FAKE, 1, 816, 8, 1, 256, 0.0625, 0.0, ctypes.byref(m816), FAKE,
                                     None, None, 0, P(0x100010), need, None) == -1   # misaligned workspace


@needs_lib
def test_backward_rejects_bad_arguments_before_launch():
    lib = Bd.lib()
    m = Bd.PiMask(B=2, N=64, n_qt=4, n_kt=2, forbid_bits=0, bid=FAKE, pos=FAKE, tok=FAKE, tiles=FAKE)
    need = lib.pi_attn_backward_workspace_bytes(2, 64, 8, 1, 256, 0.0)
    assert need == 2 * (2 * 64 * 8 * 4)     # lse2 and Dr, fp32 per row of 2*64*8 rows
    # with the rotary embedding also the rotated Q and K and the negated positions
    assert lib.pi_attn_backward_workspace_bytes(2, 64, 8, 1, 256, 10000.0) == need + 2 * 64 * 8 * 256 * 2 + \
        2 * 64 * 256 * 2 + 512
    assert lib.pi_attn_backward_workspace_bytes(2, 64, 24, 24, 64, 0.0) == 0     # unsupported heads
    call = lambda **kw: lib.pi_joint_attn_backward(
        kw.get("q", FAKE), FAKE, FAKE, FAKE, FAKE, kw.get("lse", FAKE), kw.get("B", 2), kw.get("L", 64),
        kw.get("Hq", 8), kw.get("Hkv", 1), kw.get("d", 256), kw.get("scale", 0.0625), kw.get("rope", 0.0),
        ctypes.byref(m),
        kw.get("dq", FAKE), FAKE, FAKE, kw.get("ws", P(0x100000)), kw.get("ws_bytes", need), None)
    assert call(d=64, Hq=1) == -2            # unsupported heads
    assert call(L=65) == -1                  # mask built for another length
    assert call(scale=0.0) == -1
    assert call(q=P(0x10008)) == -1          # misaligned
    assert call(lse=P(0x10002)) == -1        # misaligned lse
    assert call(dq=None) == -1
    assert call(ws=None) == -3
    assert call(ws_bytes=need - 1) == -3
    assert call(ws=P(0x100010)) == -1        # misaligned workspace
    assert call(rope=0.5) == -1              # rope_base must be 0 or > 1
    assert call(rope=10000.0) == -3          # the rotary embedding needs the larger workspace
    assert b"pi_joint_attn_backward" in lib.pi_last_error()


@needs_lib
def test_layer_rejects_bad_arguments_before_launch():
    lib = Bd.lib()
    m = Bd.PiMask(B=2, N=60, n_qt=4, n_kt=2, forbid_bits=0, bid=FAKE, pos=FAKE, tok=FAKE, tiles=FAKE)
    sp = Bd.PiLayerStream(2048, 8192, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None)
    se = Bd.PiLayerStream(1024, 4096, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE)
    need = lib.pi_joint_layer_workspace_bytes(ctypes.byref(sp), ctypes.byref(se), 2, 50, 10)
    assert need > 2 * 60 * 2048 * 2 * 2     # at least the pooled q and o
    call = lambda p=sp, e=se, **kw: lib.pi_joint_layer_forward(
        ctypes.byref(p), ctypes.byref(e), FAKE, FAKE, kw.get("cond", FAKE), 2, kw.get("Np", 50), 10,
        kw.get("scale", 0.0625), ctypes.byref(m), kw.get("ws", P(0x100000)), kw.get("ws_bytes", need), None)
    assert call(Np=51) == -1                                    # mask built for another length
    assert call(cond=None) == -1                                # the adaptive stream needs cond
    assert call(scale=0.0) == -1
    assert call(ws=None) == -3 and call(ws_bytes=need - 1) == -3
    assert call(ws=P(0x100010)) == -1                           # misaligned workspace
    odd = Bd.PiLayerStream(1000, 4096, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE)
    assert call(e=odd) == -1                                    # width not a multiple of 256
    both = Bd.PiLayerStream(1024, 4096, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    assert call(e=both) == -1                                   # plain and adaptive norm at once
    ada_p = Bd.PiLayerStream(2048, 8192, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE)
    assert call(p=ada_p) == -2                                  # two adaptive streams
    assert lib.pi_joint_layer_workspace_bytes(ctypes.byref(odd), ctypes.byref(se), 2, 50, 10) == 0
    assert b"pi_joint_layer_forward" in lib.pi_last_error()
    # the cached form of the expert's layer
    cache = Bd.PiKvCache(FAKE, FAKE, FAKE, 18, 2, 816, 1, 256, 816)
    need_d = lib.pi_expert_layer_decode_workspace_bytes(ctypes.byref(se), 2, 50, 816)
    assert need_d > 2 * 50 * 4096 * 2 and lib.pi_expert_layer_decode_workspace_bytes(ctypes.byref(odd), 2, 50, 816) == 0
    dec = lambda e=se, **kw: lib.pi_expert_layer_decode(
        ctypes.byref(e), ctypes.byref(cache), kw.get("layer", 0), FAKE, kw.get("cond", FAKE), FAKE, kw.get("B", 2),
        50, 0.0625, kw.get("ws", P(0x100000)), kw.get("ws_bytes", need_d), None)
    assert dec(layer=18) == -1 and dec(B=3) == -1 and dec(cond=None) == -1
    long_s = lambda: lib.pi_expert_layer_decode(ctypes.byref(se), ctypes.byref(cache), 0, FAKE, FAKE, FAKE, 2, 129,
                                                0.0625, P(0x100000), 1 << 40, None)
    assert long_s() == -1                                       # S > 128, rejected before any launch
    assert dec(ws_bytes=need_d - 1) == -3 and dec(e=odd) == -1
    assert b"pi_expert_layer_decode" in lib.pi_last_error()


@needs_lib
def test_decode_and_flow_reject_bad_arguments_before_launch():
    lib = Bd.lib()
    cache = Bd.PiKvCache(FAKE, FAKE, FAKE, 18, 4, 816, 1, 256, 816)
    dec = lambda **kw: lib.pi_suffix_decode_step(ctypes.byref(cache), kw.get("layer", 0), FAKE, FAKE, FAKE, FAKE,
                                                 kw.get("B", 4), kw.get("S", 51), kw.get("Hq", 8), 0.0625,
                                                 kw.get("rope", 0.0), FAKE, kw.get("ws", None), kw.get("ws_bytes", 0),
                                                 None)
    assert dec(layer=18) == -1
    assert dec(B=3) == -1
    assert dec(S=129) == -1
    assert dec(Hq=4) == -2
    assert dec(rope=1.0) == -1
    assert dec(rope=10000.0) == -3           # the rotary embedding needs the workspace
    # a misaligned workspace is rejected
    need = lib.pi_decode_workspace_bytes(4, 51, 8, 816)
    assert dec(ws=P(0x100010), ws_bytes=need) == -1
    # the workspace holds the rotated suffix K (every batch) plus a small batch's split partials
    rot64 = (64 * 51 * 256 * 2 + 255) // 256 * 256
    assert lib.pi_decode_workspace_bytes(64, 51, 8, 816) == rot64
    assert need > (4 * 51 * 256 * 2 + 255) // 256 * 256
    assert lib.pi_euler_update(FAKE, FAKE, -0.1, -1, None) == -1
    assert lib.pi_flow_sample(None, None, None, None, None, FAKE, 1, 50, 32, 0, None, 0, None) == -1
    assert lib.pi_flow_sample(None, None, None, None, None, FAKE, 1, 50, 32, 10, None, 0, None) == -1  # no v_const
    net = Bd.PiVelocityNet(1024, 32, 8, 1, 256, *([FAKE] * 11))
    ws_need = lib.pi_flow_workspace_bytes(ctypes.byref(net), 4, 50)
    r = lib.pi_flow_sample(ctypes.byref(net), ctypes.byref(cache), FAKE, FAKE, None, FAKE, 4, 50, 32, 10,
                           P(0x100000), ws_need - 1, None)
    assert r == -3
    net_bad = Bd.PiVelocityNet(1000, 32, 8, 1, 256, *([FAKE] * 11))
    assert lib.pi_flow_sample(ctypes.byref(net_bad), ctypes.byref(cache), FAKE, FAKE, None, FAKE, 4, 50, 32, 10,
                              P(0x100000), 1 << 30, None) == -2


@needs_lib
def test_cache_append_rejects_bad_arguments_before_launch():
    lib = Bd.lib()
    cache = Bd.PiKvCache(FAKE, FAKE, FAKE, 2, 4, 816, 1, 256, 810)
    app = lambda **kw: lib.pi_kv_cache_append(ctypes.byref(cache), kw.get("layer", 0), kw.get("k", FAKE), FAKE,
                                              kw.get("n", 1), kw.get("rope", 0.0), None)
    assert app(layer=2) == -1
    assert app(n=7) == -1                    # 810 + 7 > 816 slots
    assert app(n=0) == -1
    assert app(rope=0.5) == -1
    assert app(k=P(0x10008)) == -1
    assert b"pi_kv_cache_append" in lib.pi_last_error()


@needs_lib
def test_rope_rejects_bad_arguments_before_launch():
    lib = Bd.lib()
    call = lambda **kw: lib.pi_rope_apply(kw.get("x", FAKE), kw.get("y", FAKE), kw.get("B", 2), kw.get("L", 10),
                                          kw.get("H", 8), kw.get("d", 256), kw.get("pos", FAKE),
                                          kw.get("base", 10000.0), None)
    assert call(d=24) == -2                  # not a multiple of 16
    assert call(d=1024) == -2
    assert call(base=1.0) == -1
    assert call(pos=None) == -1
    assert call(y=P(0x10004)) == -1          # misaligned
    assert call(L=0) == -1
    assert b"pi_rope_apply" in lib.pi_last_error()


@needs_lib
def test_mask_build_rejects_bad_arguments_before_launch():
    lib = Bd.lib()
    out = Bd.PiMask()
    need = lib.pi_mask_workspace_bytes(2, 100)
    assert lib.pi_mask_build(FAKE, FAKE, None, 0, 2, 100, P(0x100000), need - 1, ctypes.byref(out), None) == -3
    assert lib.pi_mask_build(FAKE, FAKE, None, 0, 0, 100, P(0x100000), need, ctypes.byref(out), None) == -1
    assert lib.pi_mask_build(FAKE, FAKE, None, 1 << 16, 2, 100, P(0x100000), need, ctypes.byref(out), None) == -1
    assert lib.pi_mask_build(FAKE, FAKE, None, 0, 2, 100, P(0x100010), need, ctypes.byref(out), None) == -1


@needs_lib
def test_expert_sampler_rejects_bad_arguments_before_launch():
    lib = Bd.lib()
    cache = Bd.PiKvCache(FAKE, FAKE, FAKE, 18, 2, 816, 1, 256, 816)
    ada = Bd.PiLayerStream(1024, 4096, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE)
    plain = Bd.PiLayerStream(1024, 4096, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None)
    narrow = Bd.PiLayerStream(512, 2048, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE)

    def net(layers, width=1024, A=32, n=None):
        arr = (Bd.PiLayerStream * len(layers))(*layers)
        return Bd.PiExpertNet(width, A, len(layers) if n is None else n, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                              ctypes.cast(arr, ctypes.POINTER(Bd.PiLayerStream)), FAKE, FAKE, FAKE), arr

    good, keep = net([ada] * 18)
    need = lib.pi_expert_flow_workspace_bytes(ctypes.byref(good), 2, 50, 816, 10)
    need1 = lib.pi_expert_flow_workspace_bytes(ctypes.byref(good), 2, 50, 816, 1)
    assert need > need1 > 2 * 50 * 4096 * 2           # at least the FFN activations
    for bad in (net([plain] * 18), net([ada] * 17 + [narrow]), net([ada] * 18, width=1000), net([ada] * 18, A=0),
                net([ada] * 18, A=257)):
        assert lib.pi_expert_flow_workspace_bytes(ctypes.byref(bad[0]), 2, 50, 816, 10) == 0
    assert lib.pi_expert_flow_workspace_bytes(ctypes.byref(good), 2, 129, 816, 10) == 0     # H > 128
    assert lib.pi_expert_flow_workspace_bytes(ctypes.byref(good), 2, 50, 816, 1001) == 0    # too many steps
    samp = lambda n=good, **kw: lib.pi_expert_flow_sample(
        ctypes.byref(n), ctypes.byref(kw.get("cache", cache)), FAKE, FAKE, kw.get("B", 2), 50, kw.get("A", 32),
        kw.get("steps", 10), kw.get("ws", P(0x100000)), kw.get("ws_bytes", need), None)
    assert samp(B=3) == -1                              # cache built for another batch
    assert samp(A=16) == -1                             # action dim differs from the net's
    assert samp(steps=0) == -1
    assert samp(ws=None) == -3 and samp(ws_bytes=need - 1) == -3
    assert samp(ws=P(0x100010)) == -1                   # misaligned workspace
    deep, keep2 = net([ada] * 19)
    assert samp(n=deep, ws_bytes=1 << 40) == -1         # more layers than the cache
    assert b"pi_expert_flow_sample" in lib.pi_last_error()
    ev = lambda **kw: lib.pi_expert_velocity_eval(
        ctypes.byref(good), ctypes.byref(cache), FAKE, FAKE, kw.get("t", 0.5), kw.get("vel", FAKE), 2, 50, 32,
        P(0x100000), kw.get("ws_bytes", need1), None)
    assert ev(vel=None) == -1 and ev(t=float("nan")) == -1 and ev(ws_bytes=need1 - 1) == -3
    assert b"pi_expert_velocity_eval" in lib.pi_last_error()


@needs_lib
def test_prefix_layer_rejects_bad_arguments_before_launch():
    lib = Bd.lib()
    sp = Bd.PiLayerStream(2048, 8192, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None)
    m = Bd.PiMask(B=2, N=60, n_qt=4, n_kt=2, forbid_bits=0, bid=FAKE, pos=FAKE, tok=FAKE, tiles=FAKE)
    need = lib.pi_prefix_layer_workspace_bytes(ctypes.byref(sp), 2, 60)
    assert need == lib.pi_joint_layer_workspace_bytes(ctypes.byref(sp), ctypes.byref(sp), 2, 60, 0) > 0
    cache = Bd.PiKvCache(FAKE, FAKE, FAKE, 18, 2, 816, 1, 256, 60)
    call = lambda c=cache, **kw: lib.pi_prefix_layer_forward(
        ctypes.byref(sp), FAKE, None, 2, kw.get("Np", 60), 0.0625, ctypes.byref(m),
        ctypes.byref(c) if c is not None else None, kw.get("layer", 0), P(0x100000), kw.get("ws_bytes", need), None)
    assert call(c=None) == -1                                   # the prefix pass writes the cache
    assert call(c=Bd.PiKvCache(FAKE, FAKE, FAKE, 18, 2, 816, 1, 256, 59)) == -1   # cache length != Np
    assert call(layer=18) == -1                                 # past the cache's layers
    assert call(ws_bytes=need - 1) == -3
    assert b"pi_" in lib.pi_last_error()

"""The Python binding rejects a tensor whose shape or dtype does not match the
sizes it passes to the C ABI, before anything reaches the library (the ABI sees
only pointers and sizes, so such a tensor would otherwise be read or written
out of bounds on the device).  Runs on the CPU: the shape checks come before the
device checks, and a correctly shaped host tensor is then refused as not being
on the device."""
import types

import pytest
import torch

from prefix_lm_joint_amd import binding as Bd

bf, f32, u8 = torch.bfloat16, torch.float32, torch.uint8


def z(*shape, dtype=bf):
    return torch.zeros(shape, dtype=dtype)


def fake_mask(B, N):
    return Bd.Mask(Bd.PiMask(B=B, N=N), z(16, dtype=u8))


def fake_cache(B=2, cap=40, Hkv=1, d=256, layers=3, length=40):
    return types.SimpleNamespace(struct=Bd.PiKvCache(None, None, None, layers, B, cap, Hkv, d, length),
                                 k=z(1), v=z(1))


def raises_shape(fn, what):
    with pytest.raises(ValueError, match=what):
        fn()


def test_prefill_shapes():
    B, L = 2, 64
    q, k, v = z(B, L, 8, 256), z(B, L, 1, 256), z(B, L, 1, 256)
    m = fake_mask(B, L)
    raises_shape(lambda: Bd.pi_joint_attn_prefill(q, k, z(B, L - 1, 1, 256), m), "v has shape")
    raises_shape(lambda: Bd.pi_joint_attn_prefill(q, k, z(B, L, 1, 256, dtype=f32), m), "v must be")
    raises_shape(lambda: Bd.pi_joint_attn_prefill(q, k, v, m, o=z(B, L, 8, 128)), "o has shape")
    raises_shape(lambda: Bd.pi_joint_attn_prefill(q, k, v, m, lse=z(B, L, 4, dtype=f32)), "lse has shape")
    raises_shape(lambda: Bd.pi_joint_attn_prefill(q, k, v, fake_mask(B, L + 1)), "mask built")
    raises_shape(lambda: Bd.pi_joint_attn_prefill(q, k, v, m, cache=fake_cache(B=B + 1)), "cache")
    # correct shapes pass the checks and stop at the device check
    raises_shape(lambda: Bd.pi_joint_attn_prefill(q, k, v, m), "device tensor")


def test_backward_shapes():
    B, L = 1, 48
    q, k, v = z(B, L, 8, 256), z(B, L, 1, 256), z(B, L, 1, 256)
    lse, ws, m = z(B, L, 8, dtype=f32), z(64, dtype=u8), fake_mask(B, L)
    raises_shape(lambda: Bd.pi_joint_attn_backward(q, k, v, q, z(B, L, 8, 64), lse, m, ws), "dout has shape")
    raises_shape(lambda: Bd.pi_joint_attn_backward(q, k, v, q, q, lse, m, ws, dk=z(B, L, 2, 256)), "dk has shape")
    raises_shape(lambda: Bd.pi_joint_attn_backward(q, k, v, q, q, z(B, L, 8), m, ws), "lse must be")
    raises_shape(lambda: Bd.pi_joint_attn_backward(q, k, v, q, q, lse, m, ws), "device tensor")


def test_mask_build_shapes():
    raises_shape(lambda: Bd.pi_mask_build(z(2, 30, dtype=u8), z(29, dtype=u8)), "ar has shape")
    raises_shape(lambda: Bd.pi_mask_build(z(2, 30, dtype=u8), z(30, dtype=u8), seg=z(31, dtype=u8)), "seg has shape")
    raises_shape(lambda: Bd.pi_mask_build(z(2, 30, dtype=torch.bool), z(30, dtype=u8)), "input_mask must be")
    raises_shape(lambda: Bd.pi_mask_materialize(fake_mask(2, 30), dense=z(2, 30, 29, dtype=u8)), "dense has shape")


def test_decode_shapes():
    c = fake_cache(B=2)
    q, kv, ar = z(2, 51, 8, 256), z(2, 51, 1, 256), z(51, dtype=u8)
    raises_shape(lambda: Bd.pi_suffix_decode_step(c, 0, q, z(2, 51, 1, 128), kv, ar), "k_s has shape")
    raises_shape(lambda: Bd.pi_suffix_decode_step(c, 0, q, kv, z(2, 50, 1, 256), ar), "v_s has shape")
    raises_shape(lambda: Bd.pi_suffix_decode_step(c, 0, q, kv, kv, z(50, dtype=u8)), "suffix_ar has shape")
    raises_shape(lambda: Bd.pi_suffix_decode_step(c, 0, q, kv, kv, ar, o_s=z(2, 51, 8, 255)), "o_s has shape")
    raises_shape(lambda: Bd.pi_suffix_decode_step(fake_cache(B=3), 0, q, kv, kv, ar), "cache holds")
    raises_shape(lambda: Bd.pi_suffix_decode_step(c, 0, q, kv, kv, ar), "device tensor")


def test_cache_rope_append_euler_shapes():
    raises_shape(lambda: Bd.KVCache(z(2, 3, 40, 1, 256), z(2, 3, 41, 1, 256), z(3, 40, dtype=u8)), "cache.v has")
    raises_shape(lambda: Bd.KVCache(z(2, 3, 40, 1, 256), z(2, 3, 40, 1, 256), z(3, 41, dtype=u8)), "prefix_mask")
    raises_shape(lambda: Bd.pi_rope_apply(z(2, 10, 8, 64), z(2, 10, dtype=torch.int64)), "pos must be")
    raises_shape(lambda: Bd.pi_rope_apply(z(2, 10, 8, 64), z(2, 9, dtype=torch.int32)), "pos has shape")
    c = fake_cache(B=2, Hkv=1, d=256)
    raises_shape(lambda: Bd.pi_kv_cache_append(c, 0, z(2, 1, 1, 256), z(2, 2, 1, 256)), "v_new has shape")
    raises_shape(lambda: Bd.pi_kv_cache_append(c, 0, z(3, 1, 1, 256), z(3, 1, 1, 256)), "k_new has shape")
    raises_shape(lambda: Bd.pi_euler_update(z(2, 50, 32, dtype=f32), z(2, 32, 50, dtype=f32), -0.1), "v has shape")


def _net_tensors(W=64, A=4):
    return dict(w_state=z(W, A), b_state=z(W, dtype=f32), w_in=z(W, A), b_in=z(W, dtype=f32),
                w_time=z(W, dtype=f32), w_q=z(2048, W), w_k=z(256, W), w_v=z(256, W), w_o=z(W, 2048),
                w_out=z(A, W), b_out=z(A, dtype=f32))


def test_velocity_net_shapes():
    t = _net_tensors()
    raises_shape(lambda: Bd.VelocityNet(dict(t, w_o=z(64, 1024))), "w_o has shape")
    raises_shape(lambda: Bd.VelocityNet(dict(t, b_out=z(5, dtype=f32))), "b_out has shape")
    raises_shape(lambda: Bd.VelocityNet(t), "device tensor")
    net = types.SimpleNamespace(action_dim=4, struct=None)
    c = fake_cache(B=2)
    x, st, ar = z(2, 6, 4, dtype=f32), z(2, 4, dtype=f32), z(7, dtype=u8)
    raises_shape(lambda: Bd.pi_velocity_eval(net, c, ar, z(2, 5, dtype=f32), x, 0.5), "state has shape")
    raises_shape(lambda: Bd.pi_velocity_eval(net, c, z(6, dtype=u8), st, x, 0.5), "suffix_ar has shape")
    raises_shape(lambda: Bd.pi_velocity_eval(net, c, ar, st, z(2, 6, 3, dtype=f32), 0.5), "x has shape")
    raises_shape(lambda: Bd.pi_flow_sample(net, fake_cache(B=1), ar, st, None, x), "cache")
    raises_shape(lambda: Bd.pi_flow_sample(None, None, None, None, z(2, 6, 3, dtype=f32), x), "v_const has shape")


def test_layer_stream_shapes():
    W, F = 256, 1024
    ok = dict(w_qkv=z(2560, W), w_o=z(W, 2048), w_up=z(F, W), w_down=z(W, F))
    raises_shape(lambda: Bd.LayerStream(**dict(ok, w_down=z(W, F - 1))), "w_down has shape")
    raises_shape(lambda: Bd.LayerStream(**dict(ok, w_qkv=z(2304, W))), "w_qkv has")
    raises_shape(lambda: Bd.LayerStream(**ok, norm1=z(W + 1, dtype=f32), norm2=z(W, dtype=f32)), "norm1 has shape")
    raises_shape(lambda: Bd.LayerStream(**ok, mod1=z(W, W), mod2=z(2 * W, W)), "mod1 has shape")

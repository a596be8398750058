#!/usr/bin/env python3
"""Benchmark of the block prefix-LM joint-attention path on one MI355X.

One step = one π0 control step on synthetic inputs resident in HBM:
    mask build for the 816-token prefix
    18 x joint-attention prefill over the prefix (K/V read in place from the cache)
    10 x Euler flow step, each running the stand-in velocity net over 18 cached
         layers (QKV projection, cached suffix decode, output projection) with the
         output projection and the Euler update fused.
value = control steps per second (B = 1).

Besides the step, the two kernels the metric names are measured live with HIP
events on the stream they run on:
    prefill at the π0.5 training shape (B=32, L=962, three blocks) -> MFMA fraction
    cached decode at the serving shape (B=64, 816 slots)           -> HBM GB/s
plus the rotary embedding, single-token decode, attention backward, joint
layer and cached expert-layer legs,
and the fp64 oracle is timed on the host's cores over a bounded sample.
Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_FLOPS = 2.5e15   # MI355X dense bf16 matrix-core peak
PEAK_HBM_BYTES = 8.0e12    # MI355X HBM3E peak


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--kernel-iters", type=int, default=50)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-baseline-child", action="store_true", help=argparse.SUPPRESS)
    p.add_argument("--only", choices=["step", "prefill", "decode", "mmdit", "copy", "rope", "ar", "backward", "sampler", "pi05",
                                      "layer", "expert", "serving"],
                   default=None,
                   help="run just one leg (for profiling)")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Ctx:
    def __init__(self):
        import numpy as np
        import torch
        from prefix_lm_joint_amd import binding as Bd
        from prefix_lm_joint_amd import inputs as I
        self.np, self.torch, self.Bd, self.I = np, torch, Bd, I
        self.dev = torch.device("cuda:0")
        self.stream = torch.cuda.current_stream()

    def bf(self, bits):
        np, torch = self.np, self.torch
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(self.dev)

    def u8(self, a):
        return self.torch.from_numpy(self.np.ascontiguousarray(a, dtype=self.np.uint8)).to(self.dev)

    def f32(self, a):
        return self.torch.from_numpy(self.np.ascontiguousarray(a, dtype=self.np.float32)).to(self.dev)

    def time_ms(self, fn, iters, warmup=2, warm_s=0.1):
        """Average ms per call of fn over `iters` calls, HIP events on the launch stream,
        after at least `warmup` calls and `warm_s` seconds of back-to-back calls: the
        GPU's clocks ramp up under sustained load, and a leg that starts after its
        host-side setup would otherwise time its first milliseconds at idle clocks."""
        torch = self.torch
        t0, n = time.perf_counter(), 0
        while n < warmup or time.perf_counter() - t0 < warm_s:
            fn()
            n += 1
            if n % 4 == 0:
                torch.cuda.synchronize()      # the host stays within a few calls of the GPU
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(self.stream)
        for _ in range(iters):
            fn()
        b.record(self.stream)
        b.synchronize()
        return a.elapsed_time(b) / iters

    def time_dist_us(self, fn, iters):
        """p10 / p50 / p90 of the per-call time in µs: an event on the launch stream
        between consecutive calls (run right after time_ms, at the same clocks)."""
        torch = self.torch
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(iters + 1)]
        torch.cuda.synchronize()
        ev[0].record(self.stream)
        for i in range(iters):
            fn()
            ev[i + 1].record(self.stream)
        ev[-1].synchronize()
        d = sorted(ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(iters))
        pick = lambda q: d[min(iters - 1, int(q * iters))]
        return {"p10": pick(0.1), "p50": pick(0.5), "p90": pick(0.9)}


# ---------------------------------------------------------------------------
# π0 control step (B = 1)
# ---------------------------------------------------------------------------

def build_control_step(cx: Ctx):
    np, torch, Bd, I = cx.np, cx.torch, cx.Bd, cx.I
    w = I.pi0_step()
    s = w.structure
    P, H, A, L = s.n_prefix, w.horizon, w.action_dim, w.layers
    seed = w.seed_base
    q = torch.stack([cx.bf(I.bf16_normal(seed + 16 * l + 1, (1, P, 8, 256))) for l in range(L)])
    ck = cx.bf(I.bf16_normal(seed + 500, (L, 1, P, 1, 256)))
    cv = cx.bf(I.bf16_normal(seed + 501, (L, 1, P, 1, 256)))
    pmask = np.ones((1, P), np.uint8)
    cache = Bd.KVCache(ck, cv, cx.u8(pmask))
    ar_pre, seg_pre = cx.u8(s.ar[:P]), cx.u8(s.seg[:P])
    in_mask = cx.u8(pmask)
    mask_ws = torch.empty(Bd.pi_mask_workspace_bytes(1, P), dtype=torch.uint8, device=cx.dev)
    o = torch.empty((1, P, 8, 256), dtype=torch.bfloat16, device=cx.dev)
    pre_ws = Bd.prefill_workspace(1, P, 8, 1, 256, cx.dev)   # key split: one sample alone cannot fill the chip
    net = Bd.VelocityNet.from_numpy(I.net_weights(seed + 600, width=w.width, action_dim=A), cx.dev)
    flow_ws = Bd.flow_workspace(net, 1, H, cx.dev)
    sar = cx.u8(s.ar[P:])
    state = cx.f32(I.f32_normal(seed + 601, (1, A)))
    noise = cx.f32(I.f32_normal(seed + 602, (1, H, A)))
    x = torch.empty_like(noise)

    def step():
        m = Bd.pi_mask_build(in_mask, ar_pre, seg_pre, 0, workspace=mask_ws)
        for l in range(L):
            Bd.pi_joint_attn_prefill(q[l], ck[l], cv[l], m, o=o, workspace=pre_ws)
        x.copy_(noise)
        Bd.pi_flow_sample(net, cache, sar, state, None, x, num_steps=w.steps, workspace=flow_ws)

    parts = {
        "mask_build": lambda: Bd.pi_mask_build(in_mask, ar_pre, seg_pre, 0, workspace=mask_ws),
        "prefill_layer": None,
        "decode_layer": None,
    }
    m0 = Bd.pi_mask_build(in_mask, ar_pre, seg_pre, 0, workspace=mask_ws)
    parts["prefill_layer"] = lambda: Bd.pi_joint_attn_prefill(q[0], ck[0], cv[0], m0, o=o, workspace=pre_ws)
    qs = cx.bf(I.bf16_normal(seed + 700, (1, H + 1, 8, 256)))
    ks = cx.bf(I.bf16_normal(seed + 701, (1, H + 1, 1, 256)))
    vs = cx.bf(I.bf16_normal(seed + 702, (1, H + 1, 1, 256)))
    os_ = torch.empty_like(qs)
    dec_ws = Bd.decode_workspace(cache, H + 1)
    parts["decode_layer"] = lambda: Bd.pi_suffix_decode_step(cache, 0, qs, ks, vs, sar, o_s=os_, workspace=dec_ws)
    parts["flow_sample_10_steps"] = lambda: (x.copy_(noise), Bd.pi_flow_sample(
        net, cache, sar, state, None, x, num_steps=w.steps, workspace=flow_ws))
    pairs_prefill = P * P
    return w, step, parts, pairs_prefill


# ---------------------------------------------------------------------------
# prefill at the π0.5 training shape and decode at the serving shape
# ---------------------------------------------------------------------------

def prefill_kernel_leg(cx: Ctx, iters: int, workload: str):
    torch, Bd, I = cx.torch, cx.Bd, cx.I
    w = I.WORKLOADS[workload]()
    s = w.structure
    q, k, v = (cx.bf(t) for t in w.qkv())
    valid = cx.u8(w.input_mask())
    m = Bd.pi_mask_build(valid, cx.u8(s.ar), cx.u8(s.seg), I.forbid_bits(s.forbid))
    pairs = int(Bd.pi_mask_materialize(m).sum(dtype=torch.int64).item())
    o = torch.empty_like(q)
    ms = cx.time_ms(lambda: Bd.pi_joint_attn_prefill(q, k, v, m, o=o), iters)
    dist = cx.time_dist_us(lambda: Bd.pi_joint_attn_prefill(q, k, v, m, o=o), iters)
    flops = 4.0 * w.d * w.Hq * pairs   # QK^T and PV, 2 flops per multiply-add, per head
    byts = (q.numel() + k.numel() + v.numel() + o.numel()) * 2
    tflops = flops / (ms * 1e-3) / 1e12
    return {
        "workload": w.name, "B": w.B, "L": w.N, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d,
        "allowed_pairs": pairs, "gflop_per_launch": flops / 1e9, "us_per_launch": ms * 1e3, "us_per_call": dist,
        "achieved_tflops": tflops, "mfma_frac": tflops * 1e12 / PEAK_BF16_FLOPS,
        "algorithmic_bytes": byts, "kernel": "prefill_kernel",
    }


def backward_leg(cx: Ctx, iters: int):
    """Backward of the joint attention at the π0.5 training shape (B=32, L=962,
    three blocks): one pi_joint_attn_backward call (row statistics, dK/dV, dQ)
    for a unit-variance upstream gradient, after a forward that keeps the rows'
    log-sum-exp.  Algorithmic FLOPs: five products of 2 d flops per allowed
    (query, key) pair and query head (Q K^T, dO V^T, dV, dK, dQ)."""
    torch, Bd, I = cx.torch, cx.Bd, cx.I
    w = I.WORKLOADS["pi05_three_block_prefill"]()
    s = w.structure
    q, k, v = (cx.bf(t) for t in w.qkv())
    u = cx.bf(I.bf16_normal(w.seed_base + 21, (w.B, w.N, w.Hq, w.d)))
    valid = cx.u8(w.input_mask())
    m = Bd.pi_mask_build(valid, cx.u8(s.ar), cx.u8(s.seg), I.forbid_bits(s.forbid))
    pairs = int(Bd.pi_mask_materialize(m).sum(dtype=torch.int64).item())
    lse = torch.empty((w.B, w.N, w.Hq), dtype=torch.float32, device=cx.dev)
    o = Bd.pi_joint_attn_prefill(q, k, v, m, lse=lse)
    ws = Bd.backward_workspace(w.B, w.N, w.Hq, w.Hkv, w.d, cx.dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ms = cx.time_ms(lambda: Bd.pi_joint_attn_backward(q, k, v, o, u, lse, m, ws, dq=dq, dk=dk, dv=dv), iters)
    ms_fwd = cx.time_ms(lambda: Bd.pi_joint_attn_prefill(q, k, v, m, o=o, lse=lse), iters)
    flops = 10.0 * w.d * w.Hq * pairs
    tflops = flops / (ms * 1e-3) / 1e12
    return {
        "workload": w.name, "B": w.B, "L": w.N, "allowed_pairs": pairs, "gflop_per_launch": flops / 1e9,
        "us_per_launch": ms * 1e3, "achieved_tflops": tflops, "mfma_frac": tflops * 1e12 / PEAK_BF16_FLOPS,
        "forward_with_lse_us": ms_fwd * 1e3, "kernel": "bwd_prep_kernel + dkdv32_kernel + dq32_kernel",
    }


def layer_leg(cx: Ctx, iters: int):
    """One π0.5 joint layer (pi_joint_layer_forward) at the training shape: B=32,
    the prefix stream (848 prefix + 64 FAST tokens, width 2048, FFN 8192, plain
    RMS norm) and the expert stream (50 tokens, width 1024, FFN 4096, adaptive
    RMS norm) around the joint attention.  Algorithmic FLOPs: 2 per multiply-add
    of every projection and FFN product, plus 8192 per allowed attention pair."""
    torch, Bd, I = cx.torch, cx.Bd, cx.I
    np = cx.np
    w = I.WORKLOADS["pi05_three_block_prefill"]()
    s = w.structure
    B, N = w.B, w.N
    Np = int(s.n_prefix + (s.seg == I.SEG_FAST).sum())
    Ne = N - Np
    Wp, We = 2048, 1024

    def dev_stream(wt):
        t = {k: (cx.bf(v) if v.dtype == np.uint16 else cx.f32(v)) for k, v in wt.items()}
        return Bd.LayerStream(t["w_qkv"], t["w_o"], t["w_up"], t["w_down"], t.get("norm1"), t.get("norm2"),
                              t.get("mod1"), t.get("mod2"))

    sp = dev_stream(I.layer_weights(w.seed_base + 31, Wp, False))
    se = dev_stream(I.layer_weights(w.seed_base + 41, We, True))
    valid = cx.u8(w.input_mask())
    m = Bd.pi_mask_build(valid, cx.u8(s.ar), cx.u8(s.seg), I.forbid_bits(s.forbid))
    pairs = int(Bd.pi_mask_materialize(m).sum(dtype=torch.int64).item())
    ws = Bd.layer_workspace(sp, se, B, Np, Ne, cx.dev)
    h_p = cx.f32(I.f32_normal(w.seed_base + 51, (B, Np, Wp)))
    h_e = cx.f32(I.f32_normal(w.seed_base + 52, (B, Ne, We)))
    c = cx.f32(I.f32_normal(w.seed_base + 53, (B, We)))
    ms = cx.time_ms(lambda: Bd.pi_joint_layer_forward(sp, se, h_p, h_e, c, m, ws), iters)
    gemm = 2.0 * B * (Np * Wp * (2560 + 2048 + 2 * 4 * Wp) + Ne * We * (2560 + 1024 + 2 * 4 * We)) \
        + 2.0 * B * We * 4 * We
    attn = 8192.0 * pairs
    tflops = (gemm + attn) / (ms * 1e-3) / 1e12
    return {"workload": "pi05_joint_layer", "B": B, "prefix_stream_tokens": Np, "expert_stream_tokens": Ne,
            "widths": [Wp, We], "ffn": [4 * Wp, 4 * We], "us_per_layer": ms * 1e3,
            "gemm_gflop": gemm / 1e9, "attention_gflop": attn / 1e9, "achieved_tflops": tflops,
            "mfma_frac": tflops * 1e12 / PEAK_BF16_FLOPS,
            "kernel": "norm_kernel + gemm_nt_kernel (QKV, out, FFN up/down) + prefill_kernel"}


def expert_decode_leg(cx: Ctx, iters: int):
    """The expert stream's π0.5 layer in the cached form (pi_expert_layer_decode)
    at the serving shape: B=64 robots, 50 action tokens of width 1024 (FFN 4096,
    adaptive norm) against one cache layer of 816 slots (valid U[600, 816])."""
    torch, Bd, I, np = cx.torch, cx.Bd, cx.I, cx.np
    w = I.serving_decode()
    B, P, S, W = w.B, w.structure.n_prefix, 50, 1024
    pm = w.input_mask()[:, :P]
    gen = torch.Generator(device=cx.dev)
    gen.manual_seed(w.seed_base + 61)
    ck = torch.randn((1, B, P, 1, 256), generator=gen, device=cx.dev, dtype=torch.float32).to(torch.bfloat16)
    cv = torch.randn((1, B, P, 1, 256), generator=gen, device=cx.dev, dtype=torch.float32).to(torch.bfloat16)
    cache = Bd.KVCache(ck, cv, cx.u8(pm), P)
    wt = I.layer_weights(w.seed_base + 62, W, True)
    t = {k: (cx.bf(v) if v.dtype == np.uint16 else cx.f32(v)) for k, v in wt.items()}
    se = Bd.LayerStream(t["w_qkv"], t["w_o"], t["w_up"], t["w_down"], None, None, t["mod1"], t["mod2"])
    h = cx.f32(I.f32_normal(w.seed_base + 63, (B, S, W)))
    c = cx.f32(I.f32_normal(w.seed_base + 64, (B, W)))
    sar = np.zeros(S, np.uint8)
    sar[0] = 1
    sar = cx.u8(sar)
    ws = Bd.expert_decode_workspace(se, cache, S)
    ms = cx.time_ms(lambda: Bd.pi_expert_layer_decode(se, cache, 0, h, c, sar, ws), iters)
    lens = pm.sum(axis=1)
    pairs = int(S * 8 * lens.sum() + B * 8 * S * S)      # every action token sees the valid slots and the chunk
    gemm = 2.0 * B * S * W * (2560 + 2048 + 2 * 4 * W) + 2.0 * 2 * B * W * 2 * W
    flops = gemm + 4.0 * 256 * pairs
    weights = 2 * (2560 * W + W * 2048 + 2 * 4 * W * W + 2 * 2 * W * W)
    byts = weights + int(lens.sum()) * 256 * 2 * 2 + B * S * W * 4 * 2
    return {"workload": "pi05_expert_layer_decode", "B": B, "slots": P, "tokens": S, "width": W,
            "us_per_layer": ms * 1e3, "gflop_per_layer": flops / 1e9,
            "achieved_tflops": flops / (ms * 1e-3) / 1e12, "mfma_frac": flops / (ms * 1e-3) / PEAK_BF16_FLOPS,
            "algorithmic_bytes": byts, "achieved_gbs": byts / (ms * 1e-3) / 1e9,
            "kernel": "norm_kernel + gemm_nt_kernel + decode_kernel (+ combine)"}


def expert_sampler_leg(cx: Ctx, iters: int, B: int):
    """π0.5's control step after the prefix: the Euler sampler with the action expert at
    its true shape (pi_expert_flow_sample: 18 expert layers of width 1024, FFN 4096,
    adaptive norms from the time MLP, 10 steps) for B robots over an 816-slot cache
    (valid U[600, 816] for B > 1, all valid for B = 1), 50 action tokens of dim 32.
    Weights and cache are drawn on the device from a seeded generator (bench-only
    inputs; parity is covered by the tests)."""
    torch, Bd, I, np = cx.torch, cx.Bd, cx.I, cx.np
    w = I.serving_decode()
    P, H, A, W, F, L, N = w.structure.n_prefix, 50, 32, 1024, 4096, w.layers, w.steps
    pm = w.input_mask()[:B, :P] if B > 1 else np.ones((1, P), np.uint8)
    gen = torch.Generator(device=cx.dev)
    gen.manual_seed(w.seed_base + 71 + B)

    def bf(shape, std):
        return (torch.randn(shape, generator=gen, device=cx.dev, dtype=torch.float32) * std).to(torch.bfloat16)

    def f32(shape, std):
        return torch.randn(shape, generator=gen, device=cx.dev, dtype=torch.float32) * std

    ck = bf((L, B, P, 1, 256), 1.0)
    cv = bf((L, B, P, 1, 256), 1.0)
    cache = Bd.KVCache(ck, cv, cx.u8(pm), P)
    layers = [Bd.LayerStream(bf((2560, W), W ** -0.5), bf((W, 2048), 2048 ** -0.5), bf((F, W), W ** -0.5),
                             bf((W, F), F ** -0.5), None, None, bf((2 * W, W), 0.5 * W ** -0.5),
                             bf((2 * W, W), 0.5 * W ** -0.5)) for _ in range(L)]
    t = {"w_in": bf((W, A), A ** -0.5), "b_in": f32((W,), 0.1), "w_t1": bf((W, W), W ** -0.5),
         "b_t1": f32((W,), 0.1), "w_t2": bf((W, W), W ** -0.5), "b_t2": f32((W,), 0.1),
         "mod_f": bf((2 * W, W), 0.5 * W ** -0.5), "w_out": bf((A, W), W ** -0.5), "b_out": f32((A,), 0.1)}
    net = Bd.ExpertNet(t, layers)
    sar = np.zeros(H, np.uint8)
    sar[0] = 1
    sar = cx.u8(sar)
    noise = f32((B, H, A), 1.0)
    x = torch.empty_like(noise)
    ws = Bd.expert_flow_workspace(net, cache, H, N)
    ms = cx.time_ms(lambda: (x.copy_(noise), Bd.pi_expert_flow_sample(net, cache, sar, x, N, ws)), iters)
    lens = pm.sum(axis=1)
    M = B * H
    pairs = int(H * 8 * lens.sum() + B * 8 * H * H)
    per_layer = 2.0 * M * W * (2560 + 2048 + 2 * F) + 2.0 * 2 * B * W * 2 * W + 4.0 * 256 * pairs
    per_step = L * per_layer + 2.0 * M * A * W * 2 + 2.0 * B * W * 2 * W
    flops = N * per_step + 2.0 * 2 * N * W * W
    return {"workload": "pi05_expert_sampler", "B": B, "slots": P, "actions": H, "action_dim": A, "width": W,
            "ffn": F, "layers": L, "euler_steps": N, "ms_per_control_step": ms,
            "control_steps_per_s": 1e3 / ms, "robot_steps_per_s": B * 1e3 / ms,
            "tflop_per_control_step": flops / 1e12, "achieved_tflops": flops / (ms * 1e-3) / 1e12,
            "mfma_frac": flops / (ms * 1e-3) / PEAK_BF16_FLOPS}


def pi05_control_step_leg(cx: Ctx, iters: int):
    """π0.5's whole control step at the true layer shapes, B = 1: the prefix (3 x 256
    image + 48 text + 32 discrete-state tokens = 848, bidirectional) through 18
    prefix-stream layers (width 2048, FFN 8192, plain RMS norm; pi_prefix_layer_forward
    writing each layer's K/V into the cache), then the expert sampler
    (pi_expert_flow_sample, 18 expert layers, 10 Euler steps, 50 actions of dim 32).
    Weights and inputs are drawn on the device from a seeded generator."""
    torch, Bd, I, np = cx.torch, cx.Bd, cx.I, cx.np
    P, H, A, Wp, We, L, N = 848, 50, 32, 2048, 1024, 18, 10
    gen = torch.Generator(device=cx.dev)
    gen.manual_seed(9001)

    def bf(shape, std):
        return (torch.randn(shape, generator=gen, device=cx.dev, dtype=torch.float32) * std).to(torch.bfloat16)

    def f32(shape, std):
        return torch.randn(shape, generator=gen, device=cx.dev, dtype=torch.float32) * std

    def stream(W, adaptive):
        F = 4 * W
        norms = (None, None, bf((2 * W, W), 0.5 * W ** -0.5), bf((2 * W, W), 0.5 * W ** -0.5)) if adaptive else \
            (1.0 + f32((W,), 0.1), 1.0 + f32((W,), 0.1), None, None)
        return Bd.LayerStream(bf((2560, W), W ** -0.5), bf((W, 2048), 2048 ** -0.5), bf((F, W), W ** -0.5),
                              bf((W, F), F ** -0.5), *norms)

    prefix = [stream(Wp, False) for _ in range(L)]
    t = {"w_in": bf((We, A), A ** -0.5), "b_in": f32((We,), 0.1), "w_t1": bf((We, We), We ** -0.5),
         "b_t1": f32((We,), 0.1), "w_t2": bf((We, We), We ** -0.5), "b_t2": f32((We,), 0.1),
         "mod_f": bf((2 * We, We), 0.5 * We ** -0.5), "w_out": bf((A, We), We ** -0.5), "b_out": f32((A,), 0.1)}
    net = Bd.ExpertNet(t, [stream(We, True) for _ in range(L)])
    ck = torch.zeros((L, 1, P, 1, 256), dtype=torch.bfloat16, device=cx.dev)
    cv = torch.zeros_like(ck)
    valid = cx.u8(np.ones((1, P), np.uint8))
    cache = Bd.KVCache(ck, cv, valid, P)
    mask_ws = torch.empty(Bd.pi_mask_workspace_bytes(1, P), dtype=torch.uint8, device=cx.dev)
    zeros = cx.u8(np.zeros(P, np.uint8))
    emb = f32((1, P, Wp), 1.0)
    h = torch.empty_like(emb)
    pws = Bd.prefix_layer_workspace(prefix[0], 1, P, cx.dev)
    sar = np.zeros(H, np.uint8)
    sar[0] = 1
    sar = cx.u8(sar)
    noise = f32((1, H, A), 1.0)
    x = torch.empty_like(noise)
    fws = Bd.expert_flow_workspace(net, cache, H, N)

    def prefix_pass():
        m = Bd.pi_mask_build(valid, zeros, zeros, 0, workspace=mask_ws)
        h.copy_(emb)
        for l in range(L):
            Bd.pi_prefix_layer_forward(prefix[l], h, m, cache, l, pws)

    def step():
        prefix_pass()
        x.copy_(noise)
        Bd.pi_expert_flow_sample(net, cache, sar, x, N, fws)

    ms = cx.time_ms(step, iters)
    ms_prefix = cx.time_ms(prefix_pass, iters)
    return {"workload": "pi05_control_step_true_shape", "B": 1, "prefix_tokens": P, "actions": H, "layers": L,
            "euler_steps": N, "prefix_width": Wp, "expert_width": We, "ms_per_control_step": ms,
            "control_steps_per_s": 1e3 / ms, "ms_prefix_pass": ms_prefix}


def decode_kernel_leg(cx: Ctx, iters: int):
    np, torch, Bd, I = cx.np, cx.torch, cx.Bd, cx.I
    w = I.serving_decode()
    s = w.structure
    P, S, B = s.n_prefix, s.n - s.n_prefix, w.B
    pm = w.input_mask()[:, :P]
    lens = pm.sum(axis=1)
    # all 18 layers (963 MB, larger than the 256 MB Infinity Cache), rotated so every
    # launch streams its layer's K/V from HBM; drawn on the device from a seeded
    # generator (bench-only inputs; parity is covered by the tests)
    layers = w.layers
    gen = torch.Generator(device=cx.dev)
    gen.manual_seed(w.seed_base + 1)
    ck = torch.randn((layers, B, P, 1, 256), generator=gen, device=cx.dev, dtype=torch.float32).to(torch.bfloat16)
    cv = torch.randn((layers, B, P, 1, 256), generator=gen, device=cx.dev, dtype=torch.float32).to(torch.bfloat16)
    cache = Bd.KVCache(ck, cv, cx.u8(pm))
    qs = cx.bf(I.bf16_normal(w.seed_base + 3, (B, S, 8, 256)))
    ks = cx.bf(I.bf16_normal(w.seed_base + 4, (B, S, 1, 256)))
    vs = cx.bf(I.bf16_normal(w.seed_base + 5, (B, S, 1, 256)))
    sar = cx.u8(s.ar[P:])
    o = torch.empty_like(qs)
    state = {"l": 0}

    def call():
        Bd.pi_suffix_decode_step(cache, state["l"] % layers, qs, ks, vs, sar, o_s=o)
        state["l"] += 1

    ms = cx.time_ms(call, iters)
    dist = cx.time_dist_us(call, iters)
    kv_bytes = int(lens.sum()) * 256 * 2 * 2
    qo_bytes = B * S * 8 * 256 * 2 * 2
    skv_bytes = B * S * 256 * 2 * 2
    byts = kv_bytes + qo_bytes + skv_bytes
    # suffix self pairs: state token sees itself, actions see state + all actions
    pairs = int(lens.sum()) * S + B * (1 + (S - 1) * S)
    flops = 4.0 * 256 * 8 * pairs
    gbs = byts / (ms * 1e-3) / 1e9
    return {
        "workload": w.name, "B": B, "slots": P, "valid_len_mean": float(lens.mean()), "S": S,
        "algorithmic_bytes_per_launch": byts, "us_per_launch": ms * 1e3, "us_per_call": dist, "achieved_gbs": gbs,
        "hbm_frac": gbs * 1e9 / PEAK_HBM_BYTES, "gflop_per_launch": flops / 1e9,
        "achieved_tflops": flops / (ms * 1e-3) / 1e12, "kernel": "decode_kernel",
    }


def rope_leg(cx: Ctx, iters: int):
    """Rotary embedding at the π0.5 training shape (B=32, L=962): the standalone
    rotation of Q and of K (HBM-bound: every element read and written once), and
    the prefill with and without the rotary embedding (its cost on the hot path)."""
    torch, Bd, I = cx.torch, cx.Bd, cx.I
    w = I.WORKLOADS["pi05_three_block_prefill"]()
    s = w.structure
    q, k, v = (cx.bf(t) for t in w.qkv())
    valid = cx.u8(w.input_mask())
    m = Bd.pi_mask_build(valid, cx.u8(s.ar), cx.u8(s.seg), I.forbid_bits(s.forbid))
    pos = m.pos()
    ws = Bd.prefill_workspace(w.B, w.N, w.Hq, w.Hkv, w.d, cx.dev)
    o = torch.empty_like(q)
    yq, yk = torch.empty_like(q), torch.empty_like(k)
    ms_q = cx.time_ms(lambda: Bd.pi_rope_apply(q, pos, 10000.0, y=yq), iters)
    ms_k = cx.time_ms(lambda: Bd.pi_rope_apply(k, pos, 10000.0, y=yk), iters)
    ms_plain = cx.time_ms(lambda: Bd.pi_joint_attn_prefill(q, k, v, m, o=o, workspace=ws), iters)
    ms_rope = cx.time_ms(lambda: Bd.pi_joint_attn_prefill(q, k, v, m, o=o, workspace=ws, rope_base=10000.0), iters)
    q_bytes, k_bytes = 2 * q.numel() * 2, 2 * k.numel() * 2
    return {
        "workload": w.name, "B": w.B, "L": w.N, "base": 10000.0,
        "rope_q": {"kernel": "rope_kernel (Q, 8 heads)", "algorithmic_bytes_per_launch": q_bytes,
                   "us_per_launch": ms_q * 1e3, "achieved_gbs": q_bytes / (ms_q * 1e-3) / 1e9,
                   "hbm_frac": q_bytes / (ms_q * 1e-3) / PEAK_HBM_BYTES},
        "rope_k": {"kernel": "rope_kernel (K, 1 head)", "algorithmic_bytes_per_launch": k_bytes,
                   "us_per_launch": ms_k * 1e3, "achieved_gbs": k_bytes / (ms_k * 1e-3) / 1e9,
                   "hbm_frac": k_bytes / (ms_k * 1e-3) / PEAK_HBM_BYTES},
        "prefill_us": ms_plain * 1e3, "prefill_rope_us": ms_rope * 1e3,
        "rope_overhead_us": (ms_rope - ms_plain) * 1e3,
    }


def ar_decode_leg(cx: Ctx, iters: int):
    """Single-token autoregressive decode at the serving shape (B=64, 816 slots, valid
    length U[600,816]): one new token per sample against one cache layer (the 18
    layers rotated as in the decode leg), then its K/V appended.  HBM-bound: each
    valid slot's K and V are read once."""
    torch, Bd, I = cx.torch, cx.Bd, cx.I
    w = I.serving_decode()
    s = w.structure
    P, B = s.n_prefix, w.B
    pm = w.input_mask()[:, :P]
    lens = pm.sum(axis=1)
    layers = w.layers
    gen = torch.Generator(device=cx.dev)
    gen.manual_seed(w.seed_base + 11)
    cap = P + 16
    ck = torch.randn((layers, B, cap, 1, 256), generator=gen, device=cx.dev, dtype=torch.float32).to(torch.bfloat16)
    cv = torch.randn((layers, B, cap, 1, 256), generator=gen, device=cx.dev, dtype=torch.float32).to(torch.bfloat16)
    pmask = torch.zeros((B, cap), dtype=torch.uint8, device=cx.dev)
    pmask[:, :P] = cx.u8(pm)
    cache = Bd.KVCache(ck, cv, pmask, P)
    qs = cx.bf(I.bf16_normal(w.seed_base + 13, (B, 1, 8, 256)))
    ks = cx.bf(I.bf16_normal(w.seed_base + 14, (B, 1, 1, 256)))
    vs = cx.bf(I.bf16_normal(w.seed_base + 15, (B, 1, 1, 256)))
    sar = cx.u8(cx.np.array([1], cx.np.uint8))
    o = torch.empty_like(qs)
    ws = Bd.decode_workspace(cache, 1)
    state = {"l": 0}

    def step():
        Bd.pi_suffix_decode_step(cache, state["l"] % layers, qs, ks, vs, sar, o_s=o, workspace=ws)
        state["l"] += 1

    def step_append():
        # the new token goes to slot P of this layer each time (len stays P)
        layer = state["l"] % layers
        Bd.pi_suffix_decode_step(cache, layer, qs, ks, vs, sar, o_s=o, workspace=ws)
        Bd.pi_kv_cache_append(cache, layer, ks, vs)
        state["l"] += 1

    ms = cx.time_ms(step, iters)
    ms_app = cx.time_ms(step_append, iters)
    byts = int(lens.sum()) * 256 * 2 * 2 + B * 8 * 256 * 2 * 2 + B * 256 * 2 * 2
    gbs = byts / (ms * 1e-3) / 1e9
    return {"workload": "ar_decode_serving", "B": B, "slots": P, "valid_len_mean": float(lens.mean()),
            "algorithmic_bytes_per_launch": byts, "us_per_step": ms * 1e3, "achieved_gbs": gbs,
            "hbm_frac": gbs * 1e9 / PEAK_HBM_BYTES, "us_per_step_with_append": ms_app * 1e3,
            "kernel": "decode_kernel (one wave, S=1) + decode_combine_kernel"}


def serving_control_step_leg(cx: Ctx, iters: int):
    """The batched serving control step on the stand-in path: B = 64 robots, each
    with its own 816-slot cache of 18 layers (valid lengths U[600, 816]), the whole
    10-step Euler loop of pi_flow_sample with the stand-in velocity net (width
    1024, 18 cache layers, 51 suffix tokens, 50 actions of dim 32) per control step.
    Cache and noise are drawn on the device from a seeded generator, the weights by
    the seeded host generator (bench-only inputs; parity is covered by the tests)."""
    torch, Bd, I = cx.torch, cx.Bd, cx.I
    w = I.serving_decode()
    s = w.structure
    P, S, B, L, N, A = s.n_prefix, s.n - s.n_prefix, w.B, w.layers, w.steps, w.action_dim
    H = S - 1
    pm = w.input_mask()[:, :P]
    lens = pm.sum(axis=1)
    gen = torch.Generator(device=cx.dev)
    gen.manual_seed(w.seed_base + 91)
    ck = torch.randn((L, B, P, 1, 256), generator=gen, device=cx.dev, dtype=torch.float32).to(torch.bfloat16)
    cv = torch.randn((L, B, P, 1, 256), generator=gen, device=cx.dev, dtype=torch.float32).to(torch.bfloat16)
    cache = Bd.KVCache(ck, cv, cx.u8(pm), P)
    net = Bd.VelocityNet.from_numpy(I.net_weights(w.seed_base + 92, width=1024, action_dim=A), cx.dev)
    ws = Bd.flow_workspace(net, B, H, cx.dev)
    sar = cx.u8(s.ar[P:])
    state = torch.randn((B, A), generator=gen, device=cx.dev, dtype=torch.float32)
    noise = torch.randn((B, H, A), generator=gen, device=cx.dev, dtype=torch.float32)
    x = torch.empty_like(noise)
    ms = cx.time_ms(lambda: (x.copy_(noise), Bd.pi_flow_sample(net, cache, sar, state, None, x, num_steps=N,
                                                                  workspace=ws)), iters)
    # attention bytes per Euler step (each layer's valid K/V, the queries, outputs and suffix K/V)
    att_bytes = L * (int(lens.sum()) * 256 * 2 * 2 + B * S * 8 * 256 * 2 * 2 + B * S * 256 * 2 * 2)
    W, M = 1024, B * S
    gemm_flops = L * 2.0 * M * W * (2048 + 512 + 2048) + 2.0 * M * W * A
    pairs = int(lens.sum()) * S + B * (1 + (S - 1) * S)
    att_flops = L * 4.0 * 256 * 8 * pairs
    return {"workload": "batched_serving_control_step", "B": B, "slots": P, "valid_len_mean": float(lens.mean()),
            "suffix_tokens": S, "layers": L, "euler_steps": N, "ms_per_control_step": ms,
            "control_steps_per_s": 1e3 / ms, "robot_steps_per_s": B * 1e3 / ms,
            "attention_bytes_per_control_step": N * att_bytes,
            "attention_gbs_over_the_step": N * att_bytes / (ms * 1e-3) / 1e9,
            "tflop_per_control_step": N * (gemm_flops + att_flops) / 1e12,
            "achieved_tflops": N * (gemm_flops + att_flops) / (ms * 1e-3) / 1e12}


def mmdit_leg(cx: Ctx, iters: int):
    """The MM-DiT contrast: B = 2, 4096 image + 154 text tokens, full bidirectional,
    24 heads of d = 64, the whole joint attention recomputed at each of 28 sampling
    steps (no cache): 28 prefill calls per sample."""
    w = cx.I.mmdit()
    one = prefill_kernel_leg(cx, iters, "mmdit_full_bidirectional")
    calls = w.steps
    return {**one, "calls_per_sample": calls, "ms_per_sample": calls * one["us_per_launch"] / 1e3,
            "gflop_per_sample": calls * one["gflop_per_launch"],
            "pairs_per_sample_per_head": calls * one["allowed_pairs"]}


def copy_kernel_leg(cx: Ctx, iters: int):
    """A plain device-to-device copy of known size.  Its HBM byte counters give
    the scale factor that turns the counters of the path's kernels into bytes."""
    torch = cx.torch
    n = 1 << 28                                  # 256 Mi fp32 = 1 GiB each way
    src = torch.ones(n, dtype=torch.float32, device=cx.dev)
    dst = torch.empty_like(src)
    ms = cx.time_ms(lambda: dst.copy_(src), iters)
    return {"bytes_read": 4 * n, "bytes_written": 4 * n, "us_per_launch": ms * 1e3,
            "achieved_gbs": 8 * n / (ms * 1e-3) / 1e9, "kernel": "torch copy (1 GiB)"}


# HBM bytes per launch from the committed counter summaries; a summary only counts
# while the kernel sources it was taken from are unchanged.
_ENGINE = ["prefix_lm_joint_amd/csrc/attention.hip", "prefix_lm_joint_amd/csrc/attention32.hip",
           "prefix_lm_joint_amd/csrc/common.h", "prefix_lm_joint_amd/csrc/engine.h"]
KERNEL_SOURCES = {"decode_kernel": _ENGINE, "prefill_kernel": _ENGINE}


def source_digest(kernel):
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counted_traffic(kernel, summary):
    import re
    path = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"kernel_source_digest:\s*([0-9a-f]+)", text)
    m_b = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m_src and m_b) or m_src.group(1) != source_digest(kernel):
        return None
    return float(m_b.group(1))


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on the host cores, bounded sample.  It runs in a
# child process of its own (`--cpu-baseline-child`) that never touches the GPU,
# so its process pool can fork freely.
# ---------------------------------------------------------------------------

_CPU = {}   # the sample's inputs, set before the pool forks (workers inherit them)


def _cpu_worker_init():
    from threadpoolctl import threadpool_limits
    _CPU["limit"] = threadpool_limits(1)      # one BLAS thread per worker process


def _cpu_prefill_rows(task):
    from oracle import attention as OA
    layer, rows = task
    q, k, v = _CPU["qkv"][layer]
    out = OA.joint_attention(q, k, v, _CPU["valid"], _CPU["ar"], rows=rows)
    return [out[b, i] for b, i in rows]


def cpu_baseline_child(sample_prefill_layers=3, sample_evals=2):
    """The oracle's π0 control step (prefill of the 816-token prefix x 18 layers,
    then 10 velocity evaluations through the 18 cache layers), timed on a bounded
    sample and scaled: once on one core (every BLAS pool limited to one thread),
    once on all usable cores (prefill rows over a process pool of one-thread
    workers; the velocity net, sequential over layers, with that many BLAS
    threads).  Prints one JSON object."""
    import multiprocessing as mp
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import attention as OA
    from oracle import flow as OF
    from prefix_lm_joint_amd import inputs as I
    host_cores = os.cpu_count() or 1
    usable = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else host_cores
    workers = max(1, min(usable, 16))
    w = I.pi0_step()
    s = w.structure
    P, H, A, L = s.n_prefix, w.horizon, w.action_dim, w.layers
    f64 = I.bf16_bits_to_f64
    valid = np.ones((1, P), np.uint8)
    _CPU.update(valid=valid, ar=s.ar[:P], qkv=[
        (f64(I.bf16_normal(9000 + l, (1, P, 8, 256))), f64(I.bf16_normal(9100 + l, (1, P, 1, 256))),
         f64(I.bf16_normal(9200 + l, (1, P, 1, 256)))) for l in range(sample_prefill_layers)])
    nw = I.net_weights(9300, width=w.width, action_dim=A)
    wf = {f: (f64(getattr(nw, f)) if getattr(nw, f).dtype == np.uint16 else getattr(nw, f).astype(np.float64))
          for f in nw.__dataclass_fields__}
    ck = f64(I.bf16_normal(9400, (L, 1, P, 1, 256)))
    cv = f64(I.bf16_normal(9401, (L, 1, P, 1, 256)))
    state = I.f32_normal(9402, (1, A)).astype(np.float64)
    x0 = I.f32_normal(9403, (1, H, A)).astype(np.float64)

    def evals():
        x = x0
        t0 = time.perf_counter()
        for k in range(sample_evals):
            x = OF.euler_update(x, OF.velocity_net(x, 1.0 - 0.1 * k, state, wf, ck, cv, valid, s.ar[P:], 8, 1, 256),
                                -0.1)
        return (time.perf_counter() - t0) / sample_evals

    with threadpool_limits(1):
        t0 = time.perf_counter()
        for l in range(sample_prefill_layers):
            q, k, v = _CPU["qkv"][l]
            OA.joint_attention(q, k, v, valid, s.ar[:P])
        pre_1 = (time.perf_counter() - t0) / sample_prefill_layers
        eval_1 = evals()
    rows = [(0, i) for i in range(P)]
    chunks = [rows[j::workers] for j in range(workers)]
    with mp.get_context("fork").Pool(workers, initializer=_cpu_worker_init) as pool:
        pool.map(_cpu_prefill_rows, [(0, c) for c in chunks])          # start the workers
        t0 = time.perf_counter()
        for l in range(sample_prefill_layers):
            pool.map(_cpu_prefill_rows, [(l, c) for c in chunks])
        pre_n = (time.perf_counter() - t0) / sample_prefill_layers
    with threadpool_limits(workers):
        eval_n = evals()
    step_1 = L * pre_1 + w.steps * eval_1
    step_n = L * pre_n + w.steps * eval_n
    print(json.dumps({
        "value": 1.0 / step_n, "unit": "control steps/s", "cores": workers, "kind": "oracle",
        "extrapolated": True, "host_cores": host_cores, "usable_cores": usable, "threads_used": workers,
        "single_core_s": step_1, "seconds_per_control_step": step_n,
        "sample": (f"pi0 control step (B=1, 816-token prefix x 18 layers, then 10 velocity evaluations x 18 layers), "
                   f"extrapolated from {sample_prefill_layers} timed prefill layers and {sample_evals} timed velocity "
                   f"evaluations; all cores: {pre_n:.3f} s/prefill layer over {workers} one-thread processes, "
                   f"{eval_n:.3f} s/evaluation with {workers} BLAS threads; one core: {pre_1:.3f} and {eval_1:.3f} s; "
                   f"fp64 numpy oracle"),
    }))


def cpu_baseline():
    """Run cpu_baseline_child in a child process (the oracle never shares a process with the GPU work)."""
    import subprocess
    r = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-baseline-child"], capture_output=True,
                       text=True, timeout=600)
    if r.returncode != 0:
        raise RuntimeError(f"cpu baseline failed ({r.returncode}): {r.stderr[-2000:]}")
    return json.loads(r.stdout.strip().splitlines()[-1])


def main():
    args = parse()
    if args.cpu_baseline_child:
        cpu_baseline_child()
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): this path is "
              f"built and measured for a single MI355X; see the sharding note in DESIGN.md.", file=sys.stderr)
        sys.exit(2)
    import torch
    cx = Ctx()
    result = {}
    if args.only in (None, "step"):
        log("building the pi0 control step")
        w, step, parts, _ = build_control_step(cx)
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        log(f"timing {args.steps} control steps")
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(cx.stream)
        for _ in range(args.steps):
            step()
        b.record(cx.stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / args.steps
        breakdown = {k: cx.time_ms(fn, 10) * 1e3 for k, fn in parts.items()}
        result.update(ms_per_step=ms, value=1000.0 / ms, breakdown_us=breakdown)
        log(f"control step {ms:.3f} ms ({1000 / ms:.1f}/s); parts {breakdown}")
    kernels = {}
    if args.only in (None, "prefill"):
        log("prefill kernel leg (pi05 B=32 L=962)")
        kernels["prefill"] = prefill_kernel_leg(cx, args.kernel_iters, "pi05_three_block_prefill")
        log(str(kernels["prefill"]))
    if args.only in (None, "decode"):
        log("decode kernel leg (B=64 816 slots)")
        kernels["decode"] = decode_kernel_leg(cx, args.kernel_iters)
        log(str(kernels["decode"]))
    if args.only == "copy":
        kernels["copy"] = copy_kernel_leg(cx, 5)
        log(str(kernels["copy"]))
    if args.only in (None, "mmdit"):
        log("MM-DiT contrast leg (B=2, 4250 tokens, 24 heads d=64, 28 calls)")
        kernels["mmdit"] = mmdit_leg(cx, max(5, args.kernel_iters // 5))
        log(str(kernels["mmdit"]))
    if args.only in (None, "serving"):
        log("batched serving control step (B=64, 18 layers x 10 Euler steps, stand-in net)")
        kernels["serving"] = serving_control_step_leg(cx, 3)
        log(str(kernels["serving"]))
    if args.only in (None, "ar"):
        log("autoregressive single-token decode leg (B=64 816 slots)")
        kernels["ar"] = ar_decode_leg(cx, args.kernel_iters)
        log(str(kernels["ar"]))
    if args.only in (None, "rope"):
        log("rotary embedding leg (pi05 B=32 L=962)")
        kernels["rope"] = rope_leg(cx, args.kernel_iters)
        log(str(kernels["rope"]))
    if args.only in (None, "layer"):
        log("joint layer leg (pi05 B=32, 912 + 50 tokens)")
        kernels["layer"] = layer_leg(cx, max(3, args.kernel_iters // 10))
        log(str(kernels["layer"]))
    if args.only in (None, "expert"):
        log("expert layer, cached form (B=64, 816 slots, 50 tokens)")
        kernels["expert"] = expert_decode_leg(cx, max(5, args.kernel_iters // 5))
        log(str(kernels["expert"]))
    if args.only in (None, "pi05"):
        log("pi05 control step at the true shapes (B=1: 18 prefix layers, then the expert sampler)")
        kernels["pi05"] = pi05_control_step_leg(cx, 3)
        log(str(kernels["pi05"]))
    if args.only in (None, "sampler"):
        for B in (1, 64):
            log(f"pi05 expert sampler leg (B={B}, 18 layers, 10 Euler steps)")
            kernels[f"sampler_b{B}"] = expert_sampler_leg(cx, 3, B)
            log(str(kernels[f"sampler_b{B}"]))
    if args.only in (None, "backward"):
        log("attention backward leg (pi05 B=32 L=962)")
        kernels["backward"] = backward_leg(cx, max(5, args.kernel_iters // 5))
        log(str(kernels["backward"]))
    if args.only is not None:
        print(json.dumps({"only": args.only, **result, "kernels": kernels}))
        return

    dec = kernels["decode"]
    pre = kernels["prefill"]
    roofline = {
        "kernel": "decode_kernel (cached suffix decode, B=64, 816 slots)",
        "bound": "hbm", "achieved": dec["achieved_gbs"], "peak": PEAK_HBM_BYTES / 1e9, "unit": "GB/s",
        "frac": dec["achieved_gbs"] * 1e9 / PEAK_HBM_BYTES,
        "traffic": counted_traffic("decode_kernel", "decode_kernel_serving_B64_816slots_traffic.md"),
        "algorithmic_bytes_per_launch": dec["algorithmic_bytes_per_launch"], "us_per_launch": dec["us_per_launch"],
        "us_per_call": dec["us_per_call"],
    }
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on the host")
        cpu = cpu_baseline()
        log(str(cpu))
    out = {
        "metric": "control steps/s (10-step Euler, cached prefix); MFMA% prefill, HBM GB/s decode",
        "value": result["value"], "unit": "control steps/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": result["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "pi0_control_step", "B": 1, "prefix_tokens": 816, "suffix_tokens": 51,
                   "layers": 18, "euler_steps": 10, "Hq": 8, "Hkv": 1, "head_dim": 256,
                   "velocity_net": "stand-in, width 1024, one weight set shared by the 18 cache layers"},
        "roofline": roofline,
        "prefill_mfma": {"kernel": "prefill_kernel (pi05 B=32 L=962)", "bound": "mfma",
                         "achieved": pre["achieved_tflops"], "peak": PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s",
                         "frac": pre["mfma_frac"], "us_per_launch": pre["us_per_launch"],
                         "us_per_call": pre["us_per_call"], "gflop_per_launch": pre["gflop_per_launch"],
                         "traffic": counted_traffic("prefill_kernel", "prefill_kernel_pi05_B32_L962_traffic.md"),
                         "algorithmic_bytes_per_launch": pre["algorithmic_bytes"]},
        "decode_hbm": {"kernel": "decode_kernel (B=64 816 slots)", "achieved_gbs": dec["achieved_gbs"],
                       "frac": dec["hbm_frac"], "us_per_launch": dec["us_per_launch"]},
        "ar_decode": {"kernel": kernels["ar"]["kernel"] + " (B=64, 816 slots)", "bound": "hbm",
                      "achieved": kernels["ar"]["achieved_gbs"], "peak": PEAK_HBM_BYTES / 1e9, "unit": "GB/s",
                      "frac": kernels["ar"]["hbm_frac"], "us_per_step": kernels["ar"]["us_per_step"],
                      "us_per_step_with_append": kernels["ar"]["us_per_step_with_append"]},
        "rope": {"kernel": "rope_kernel (pi05 B=32 L=962, Q)", "bound": "hbm",
                 "achieved": kernels["rope"]["rope_q"]["achieved_gbs"], "peak": PEAK_HBM_BYTES / 1e9, "unit": "GB/s",
                 "frac": kernels["rope"]["rope_q"]["hbm_frac"],
                 "us_per_launch": kernels["rope"]["rope_q"]["us_per_launch"],
                 "k_us_per_launch": kernels["rope"]["rope_k"]["us_per_launch"],
                 "prefill_us": kernels["rope"]["prefill_us"], "prefill_rope_us": kernels["rope"]["prefill_rope_us"]},
        "backward": {"kernel": kernels["backward"]["kernel"] + " (pi05 B=32 L=962)", "bound": "mfma",
                     "achieved": kernels["backward"]["achieved_tflops"], "peak": PEAK_BF16_FLOPS / 1e12,
                     "unit": "TFLOP/s", "frac": kernels["backward"]["mfma_frac"],
                     "us_per_launch": kernels["backward"]["us_per_launch"],
                     "gflop_per_launch": kernels["backward"]["gflop_per_launch"],
                     "forward_with_lse_us": kernels["backward"]["forward_with_lse_us"]},
        "joint_layer": {"kernel": kernels["layer"]["kernel"] + " (pi05 B=32, 912 + 50 tokens, widths 2048 / 1024)",
                        "bound": "mfma", "achieved": kernels["layer"]["achieved_tflops"],
                        "peak": PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s", "frac": kernels["layer"]["mfma_frac"],
                        "us_per_layer": kernels["layer"]["us_per_layer"],
                        "gflop_per_layer": kernels["layer"]["gemm_gflop"] + kernels["layer"]["attention_gflop"]},
        "expert_layer_decode": {"kernel": kernels["expert"]["kernel"] + " (B=64, 816 slots, 50 tokens, width 1024)",
                                "bound": "mfma", "achieved": kernels["expert"]["achieved_tflops"],
                                "peak": PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s",
                                "frac": kernels["expert"]["mfma_frac"], "us_per_layer": kernels["expert"]["us_per_layer"],
                                "achieved_gbs": kernels["expert"]["achieved_gbs"]},
        "serving_control_step": {
            "what": "B = 64 robots, 816-slot caches (valid U[600, 816]), pi_flow_sample with the stand-in net: "
                    "18 cache layers x 10 Euler steps, 51 suffix tokens, 50 actions of dim 32",
            **{k: kernels["serving"][k] for k in ("ms_per_control_step", "control_steps_per_s", "robot_steps_per_s",
                                                  "attention_gbs_over_the_step", "achieved_tflops")}},
        "mmdit": {"kernel": "prefill_kernel (MM-DiT: B=2, 4096 + 154 tokens, full bidirectional, Hq=Hkv=24, d=64)",
                  "bound": "mfma", "achieved": kernels["mmdit"]["achieved_tflops"], "peak": PEAK_BF16_FLOPS / 1e12,
                  "unit": "TFLOP/s", "frac": kernels["mmdit"]["mfma_frac"],
                  "us_per_launch": kernels["mmdit"]["us_per_launch"], "calls_per_sample": 28,
                  "ms_per_sample": kernels["mmdit"]["ms_per_sample"],
                  "gflop_per_launch": kernels["mmdit"]["gflop_per_launch"]},
        "pi05_expert_sampler": {
            "what": "control step after the cached prefix: 10 Euler steps of the true-shape action expert "
                    "(18 layers, width 1024, FFN 4096, adaptive norms), 50 actions of dim 32, 816-slot cache",
            **{f"B{b}": {k: kernels[f"sampler_b{b}"][k] for k in ("ms_per_control_step", "robot_steps_per_s",
                                                                 "achieved_tflops", "mfma_frac")}
               for b in (1, 64)}},
        "pi05_control_step": {
            "what": "B = 1: 848 prefix tokens through 18 prefix-stream layers (width 2048, FFN 8192) writing the "
                    "cache, then the expert sampler (18 layers, 10 Euler steps)",
            **{k: kernels["pi05"][k] for k in ("ms_per_control_step", "control_steps_per_s", "ms_prefix_pass")}},
        "breakdown_us": result["breakdown_us"],
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()

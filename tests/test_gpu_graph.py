"""The hot path under HIP graph capture: the π0 control step (mask build, 18 prefill
layers, the 10-step sampler, as the benchmark runs it) and the π0.5 expert sampler are
captured once and replayed; every replay, with eager work between replays, is
bit-identical to the eager run (the library records no memset or allocation)."""
import pytest
import torch

from prefix_lm_joint_amd import binding as Bd
from tests import gpu_util as G
from tests.test_oracle_expert_flow import real_case

pytestmark = pytest.mark.gpu


def _replays_match_eager(run, out):
    run()
    torch.cuda.synchronize()
    ref = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()                                   # warm the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        run()
    torch.cuda.synchronize()
    for i in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        G.note(f"replay {i}: max diff {(out - ref).abs().max().item():.3e}")
        assert torch.equal(out, ref), f"replay {i} differs from the eager run"
        run()                                   # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, ref)


def _control_step():
    """The π0 control step at B = 1: the prefix's mask, 18 prefix prefills reading the
    cache layers in place, then the 10-step sampler with the stand-in net over the
    cache.  Returns the step and its output x."""
    from prefix_lm_joint_amd import inputs as I
    w = I.pi0_step()
    s = w.structure
    P, H, A, L = s.n_prefix, w.horizon, w.action_dim, w.layers
    seed = w.seed_base
    dev = G.dev()
    q = torch.stack([G.bf16_dev(I.bf16_normal(seed + 16 * l + 1, (1, P, 8, 256))) for l in range(L)])
    ck = G.bf16_dev(I.bf16_normal(seed + 500, (L, 1, P, 1, 256)))
    cv = G.bf16_dev(I.bf16_normal(seed + 501, (L, 1, P, 1, 256)))
    in_mask = torch.ones((1, P), dtype=torch.uint8, device=dev)
    cache = Bd.KVCache(ck, cv, in_mask)
    ar_pre, seg_pre = G.u8_dev(s.ar[:P]), G.u8_dev(s.seg[:P])
    mask_ws = torch.empty(Bd.pi_mask_workspace_bytes(1, P), dtype=torch.uint8, device=dev)
    o = torch.empty((1, P, 8, 256), dtype=torch.bfloat16, device=dev)
    pre_ws = Bd.prefill_workspace(1, P, 8, 1, 256, dev)
    net = Bd.VelocityNet.from_numpy(I.net_weights(seed + 600, width=w.width, action_dim=A), dev)
    flow_ws = Bd.flow_workspace(net, 1, H, dev)
    sar = G.u8_dev(s.ar[P:])
    state = G.f32_dev(I.f32_normal(seed + 601, (1, A)))
    noise = G.f32_dev(I.f32_normal(seed + 602, (1, H, A)))
    x = torch.empty_like(noise)

    def step():
        m = Bd.pi_mask_build(in_mask, ar_pre, seg_pre, 0, workspace=mask_ws)
        for l in range(L):
            Bd.pi_joint_attn_prefill(q[l], ck[l], cv[l], m, o=o, workspace=pre_ws)
        x.copy_(noise)
        Bd.pi_flow_sample(net, cache, sar, state, None, x, num_steps=w.steps, workspace=flow_ws)

    return step, x


def test_control_step_replays_bit_identical():
    G.note("graph: pi0 control step (B=1, 816 + 51 tokens, 18 layers, 10 steps)")
    step, x = _control_step()
    _replays_match_eager(step, x)


def test_expert_sampler_replays_bit_identical():
    G.note("graph: pi05 expert sampler (B=2, 40 slots, 2 layers, 3 steps)")
    net, ck, cv, pm, ar, x = real_case(21, 2, 40, 50, 2)
    dnet = Bd.ExpertNet.from_numpy(net, G.dev())
    cache = Bd.KVCache(G.bf16_dev(ck), G.bf16_dev(cv), G.u8_dev(pm))
    sar = G.u8_dev(ar)
    ws = Bd.expert_flow_workspace(dnet, cache, 50, 3)
    noise = G.f32_dev(x)
    xd = torch.empty_like(noise)

    def run():
        xd.copy_(noise)
        Bd.pi_expert_flow_sample(dnet, cache, sar, xd, num_steps=3, workspace=ws)

    _replays_match_eager(run, xd)

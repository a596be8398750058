"""The hot path under HIP graph capture: the π0 control step the benchmark times
(mask build, 18 prefill layers, the 10-step sampler) and the π0.5 expert sampler are
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


def test_control_step_replays_bit_identical():
    G.note("graph: pi0 control step (B=1, 816 + 51 tokens, 18 layers, 10 steps)")
    import bench
    cx = bench.Ctx()
    _, step, _, _ = bench.build_control_step(cx)
    x = step.__closure__[step.__code__.co_freevars.index("x")].cell_contents
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

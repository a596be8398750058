"""The allocation-free cached decode (pi_suffix_decode_step_noalloc, the library's
own per-GPU scratch) against pi_suffix_decode_step with a caller workspace: two
calls in a row, the second smaller (the scratch keeps the first call's contents),
each bit-identical to the workspace call (same key split) and within the
parity bound (max-abs 1e-2, mean-abs 1e-3) of the fp64 oracle."""
import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import rope as R
from prefix_lm_joint_amd import inputs as I
from tests.gpu_util import assert_close, bf16_dev, f64, host64, note, u8_dev

pytestmark = pytest.mark.gpu


def _case(seed, B, P, S, lens):
    ck = I.bf16_normal(seed + 1, (2, B, P, 1, 256))
    cv = I.bf16_normal(seed + 2, (2, B, P, 1, 256))
    pm = I.tail_padding_mask(np.array(lens), P)
    sar = np.array([1, 1] + [0] * (S - 2), np.uint8)
    qs = I.bf16_normal(seed + 3, (B, S, 8, 256))
    ks = I.bf16_normal(seed + 4, (B, S, 1, 256))
    vs = I.bf16_normal(seed + 5, (B, S, 1, 256))
    return ck, cv, pm, sar, qs, ks, vs


@pytest.mark.parametrize("rope", [False, True])
def test_noalloc_decode_matches_workspace_decode(rope):
    from prefix_lm_joint_amd import binding as Bd
    base = 10000.0 if rope else 0.0
    layer = 1
    for seed, B, P, S, lens in ((7100, 2, 300, 51, [300, 233]), (7200, 1, 200, 20, [171])):
        note(f"noalloc decode B={B} P={P} S={S} rope={rope}")
        ck, cv, pm, sar, qs, ks, vs = _case(seed, B, P, S, lens)
        cache = Bd.KVCache(bf16_dev(ck), bf16_dev(cv), u8_dev(pm))
        q_d, k_d, v_d, ar_d = bf16_dev(qs), bf16_dev(ks), bf16_dev(vs), u8_dev(sar)
        ws = Bd.decode_workspace(cache, S)
        assert ws is not None and ws.numel() <= 16 << 20      # the shape splits its keys inside the scratch
        want_gpu = Bd.pi_suffix_decode_step(cache, layer, q_d, k_d, v_d, ar_d, workspace=ws, rope_base=base)
        got = torch.empty_like(q_d)
        Bd.pi_suffix_decode_step_noalloc(cache, layer, q_d, k_d, v_d, ar_d, got, rope_base=base)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want_gpu.view(torch.int16)), "differs from the workspace call"
        qf, kf = f64(qs), f64(ks)
        if rope:
            # cache keys are taken as already rotated; suffix token t sits at (valid slots) + t
            pos = pm.sum(1)[:, None] + np.arange(S)[None, :]
            qf, kf = R.rope(qf, pos, base), R.rope(kf, pos, base)
        want = A.cached_decode(qf, kf, f64(vs), f64(ck[layer]), f64(cv[layer]), pm, sar)
        assert_close(host64(got), want, f"noalloc decode B={B} S={S} rope={rope}")

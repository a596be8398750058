"""Pins of the oracle's Euler sampler (closed forms, the page's loop rule) and of
its bf16 rounding; structural checks of the stand-in velocity net."""
import numpy as np
import pytest
import torch

from oracle import flow as F
from oracle import attention as A
from oracle.bf16 import round_bf16
from prefix_lm_joint_amd import inputs as I


@pytest.mark.parametrize("N", [1, 3, 10, 28])
def test_constant_velocity_returns_noise_minus_v(N):
    r = np.random.default_rng(N)
    noise = r.standard_normal((2, 50, 32))
    v = r.standard_normal((2, 50, 32))
    x = F.euler_sample(noise, lambda x, t: v, N)
    np.testing.assert_allclose(x, noise - v, rtol=0, atol=1e-12)


def test_tiny_closed_form_recovers_action():
    """With the target velocity noise - action held fixed, 10 Euler steps land on the action."""
    r = np.random.default_rng(11)
    noise = r.standard_normal((1, 8, 4))
    action = r.standard_normal((1, 8, 4))
    x = F.euler_sample(noise, lambda x, t: noise - action, 10)
    np.testing.assert_allclose(x, action, rtol=0, atol=1e-12)


@pytest.mark.parametrize("lam", [-0.7, 0.3, 2.0])
def test_linear_velocity_closed_form(lam):
    N = 10
    noise = np.random.default_rng(3).standard_normal((4, 5))
    x = F.euler_sample(noise, lambda x, t: lam * x, N)
    np.testing.assert_allclose(x, (1 - lam / N) ** N * noise, rtol=1e-12)


def test_time_dependent_velocity_sees_the_time_grid():
    """v = c*t: x_N = noise + dt*c*sum_k t_k = noise - c*(N+1)/(2N)."""
    N = 10
    c = np.array([1.5, -2.0])
    x = F.euler_sample(np.zeros(2), lambda x, t: c * t, N)
    np.testing.assert_allclose(x, -c * (N + 1) / (2 * N), rtol=1e-13)


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_while_loop_rule_runs_exactly_n_steps(dtype):
    """The page's loop keeps stepping while t >= -dt/2, accumulating t += dt;
    that yields exactly N steps, which the oracle's fixed count reproduces."""
    for N in range(1, 60):
        dt = dtype(-1.0 / N)
        t, count = dtype(1.0), 0
        while t >= -dt / dtype(2):
            t = dtype(t + dt)
            count += 1
        assert count == N == len(F.time_grid(N))
    g = F.time_grid(10)
    assert g[0] == 1.0 and abs(g[-1] - 0.1) < 1e-15 and (np.diff(g) < 0).all()


def test_bf16_rounding_matches_torch():
    r = np.random.default_rng(9)
    x = np.concatenate([r.standard_normal(100000).astype(np.float32),
                        np.float32([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, 3.0e-30])])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(round_bf16(x.astype(np.float64)), want)


def _net_inputs(seed, B=2, P=12, layers=3):
    W, A_, Hq, Hkv, d, H = 64, 4, 8, 1, 16, 5
    w = I.net_weights(seed, width=W, action_dim=A_, Hq=Hq, Hkv=Hkv, d=d)
    wf = {f: (I.bf16_bits_to_f64(getattr(w, f)) if getattr(w, f).dtype == np.uint16
              else getattr(w, f).astype(np.float64)) for f in w.__dataclass_fields__}
    r = np.random.default_rng(seed)
    ck = r.standard_normal((layers, B, P, Hkv, d))
    cv = r.standard_normal((layers, B, P, Hkv, d))
    pre = np.ones((B, P), np.uint8)
    pre[0, P - 3:] = 0
    s = I.pi0_structure(P, H)
    x = r.standard_normal((B, H, A_))
    state = r.standard_normal((B, A_))
    return wf, ck, cv, pre, s.ar[P:], x, state, (Hq, Hkv, d)


def test_net_without_out_projection_ignores_the_cache():
    wf, ck, cv, pre, sar, x, st, (Hq, Hkv, d) = _net_inputs(1)
    wf["w_o"] = np.zeros_like(wf["w_o"])
    v1 = F.velocity_net(x, 0.4, st, wf, ck, cv, pre, sar, Hq, Hkv, d)
    v2 = F.velocity_net(x, 0.4, st, wf, ck * 3 + 1, cv[::-1], pre, sar, Hq, Hkv, d)
    assert np.array_equal(v1, v2)


def test_net_layers_use_the_pinned_decode():
    """Each layer's attention output is the cached decode of that layer's cache."""
    wf, ck, cv, pre, sar, x, st, (Hq, Hkv, d) = _net_inputs(2)
    _, trace = F.velocity_net(x, 0.7, st, wf, ck, cv, pre, sar, Hq, Hkv, d, return_trace=True)
    for layer, tr in enumerate(trace):
        o = A.cached_decode(tr["q"], tr["k"], tr["v"], ck[layer], cv[layer], pre, sar)
        np.testing.assert_array_equal(round_bf16(o), tr["o"])


def test_net_padded_cache_slots_do_not_matter():
    wf, ck, cv, pre, sar, x, st, (Hq, Hkv, d) = _net_inputs(3)
    v1 = F.velocity_net(x, 0.2, st, wf, ck, cv, pre, sar, Hq, Hkv, d)
    ck2, cv2 = ck.copy(), cv.copy()
    ck2[:, 0, -3:] = 1e3
    cv2[:, 0, -3:] = -1e3
    v2 = F.velocity_net(x, 0.2, st, wf, ck2, cv2, pre, sar, Hq, Hkv, d)
    assert np.array_equal(v1, v2)


def _net_fp32(x, t, state, w, ck, cv, pm, sar):
    """The stand-in net's definition evaluated in float32 with the same bf16
    rounding points (torch CPU): what any fp32-accumulating implementation gets."""
    def r(a):
        return a.to(torch.bfloat16).to(torch.float32)
    W = {k: torch.from_numpy(v.astype(np.float32)) for k, v in w.items()}
    x, state = torch.from_numpy(x.astype(np.float32)), torch.from_numpy(state.astype(np.float32))
    h = torch.cat([(r(state) @ W["w_state"].T + W["b_state"])[:, None],
                   r(x) @ W["w_in"].T + W["b_in"] + np.float32(t) * W["w_time"]], 1)
    B, S, _ = h.shape
    from oracle.mask import decode_mask
    vis = torch.from_numpy(decode_mask(pm, np.ones((B, S), np.uint8), sar))
    for layer in range(ck.shape[0]):
        a = r(h)
        rr = torch.sqrt((a * a).mean(-1, keepdim=True) + 1e-6)
        q = r(a @ W["w_q"].T / rr).view(B, S, 8, 256)
        k, v = r(a @ W["w_k"].T / rr), r(a @ W["w_v"].T / rr)
        kk = torch.cat([torch.from_numpy(ck[layer][:, :, 0].astype(np.float32)), k], 1)
        vv = torch.cat([torch.from_numpy(cv[layer][:, :, 0].astype(np.float32)), v], 1)
        s = torch.einsum("bshd,bkd->bshk", q, kk) / 16.0
        s = s.masked_fill(~vis[:, :, None, :], float("-inf"))
        o = r(torch.einsum("bshk,bkd->bshd", torch.softmax(s, -1), vv))
        h = h + o.reshape(B, S, 2048) @ W["w_o"].T
    aa = r(h[:, 1:])
    return (aa @ W["w_out"].T / torch.sqrt((aa * aa).mean(-1, keepdim=True) + 1e-6) + W["b_out"]).numpy()


def test_net_tolerance_is_twice_the_fp32_floor():
    """Derives the velocity-net bound used by the GPU tests: at the π0 control-step
    shape an fp32 evaluation of the same definition sits this far from the fp64
    oracle, only because bf16 rounding points turn accumulation-order differences
    into whole-ulp flips.  The GPU bound is about twice that floor."""
    from tests.gpu_util import NET_MAX_ABS, NET_MEAN_ABS
    B, P, H, A, W, L = 1, 816, 50, 32, 1024, 18
    nw = I.net_weights(2100, width=W, action_dim=A)
    wf = {f: (I.bf16_bits_to_f64(getattr(nw, f)) if getattr(nw, f).dtype == np.uint16
              else getattr(nw, f).astype(np.float64)) for f in nw.__dataclass_fields__}
    ck = I.bf16_bits_to_f64(I.bf16_normal(2120, (L, B, P, 1, 256)))
    cv = I.bf16_bits_to_f64(I.bf16_normal(2121, (L, B, P, 1, 256)))
    pm = np.ones((B, P), np.uint8)
    sar = I.pi0_structure(P, H).ar[P:]
    st, x = I.f32_normal(2123, (B, A)), I.f32_normal(2124, (B, H, A))
    ref = F.velocity_net(x.astype(np.float64), 0.7, st.astype(np.float64), wf, ck, cv, pm, sar, 8, 1, 256)
    err = np.abs(_net_fp32(x, 0.7, st, wf, ck, cv, pm, sar) - ref)
    floor_mean, floor_max = float(err.mean()), float(err.max())
    assert 5e-4 < floor_mean < 2e-3 and floor_max < 1e-2
    assert 1.5 * floor_mean <= NET_MEAN_ABS <= 3.0 * floor_mean
    assert 1.5 * floor_max <= NET_MAX_ABS


# ---------------------------------------------------------------------------
# Pins of the stand-in velocity net's definition ("VLA 代码精读" §1.4: a state
# token, the action in-projection, the expert's attention over the cached prefix
# and the suffix, the action out-projection of the last H tokens; "π0.5 vs
# MM-DiT joint attention", first section: an RMS norm ahead of each stream's
# projections).  Each check is written independently of oracle/flow.py.
# ---------------------------------------------------------------------------

def _nearest_bf16(x):
    """Brute-force nearest bf16 (ties to even) of float64 values: the two bf16
    neighbours bracket x, compare the exact float64 distances."""
    x = np.asarray(x, np.float64)
    f = x.astype(np.float32)
    bits = f.view(np.uint32) & np.uint32(0xFFFF0000)            # truncation toward zero
    lo = bits.view(np.float32).astype(np.float64)
    hi_bits = bits + np.uint32(0x10000)
    hi = hi_bits.view(np.float32).astype(np.float64)
    # truncation of the float32 image can overshoot x when float32 rounded away from zero
    over = np.abs(lo) > np.abs(x)
    lo_bits = np.where(over, bits - np.uint32(0x10000), bits)
    lo = np.where(over, lo_bits.view(np.float32).astype(np.float64), lo)
    hi = np.where(over, bits.view(np.float32).astype(np.float64), hi)
    hi_bits = np.where(over, bits, hi_bits)
    dlo, dhi = np.abs(x - lo), np.abs(hi - x)
    even_lo = ((lo_bits >> np.uint32(16)) & np.uint32(1)) == 0
    pick_lo = (dlo < dhi) | ((dlo == dhi) & even_lo)
    out = np.where(pick_lo, lo, hi)
    return np.where(x == 0, x, out)


def test_bf16_rounding_of_float64_is_single():
    """round_bf16 rounds the exact float64 value once: brute force over values
    that sit just beside bf16 midpoints (where rounding through float32 first
    would land on the midpoint and tie differently)."""
    r = np.random.default_rng(12)
    base = r.standard_normal(20000).astype(np.float32).astype(np.float64)
    mid = (I.bf16_bits_to_f64(I.f32_to_bf16_bits(base.astype(np.float32))) +
           np.float64(2.0) ** (np.floor(np.log2(np.abs(base))) - 8))           # a bf16 midpoint near each value
    x = np.concatenate([base, mid * (1 + 2.0 ** -40), mid * (1 - 2.0 ** -40), mid,
                        r.standard_normal(20000) * 10.0 ** r.integers(-6, 6, 20000)])
    assert np.array_equal(round_bf16(x), _nearest_bf16(x))


def _t64(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float64))


def _pi0_suffix_visibility(prefix_mask, S):
    """bool [B, S, P+S] written out from the π0 permission rule ("VLA 代码精读"
    §1.2): every suffix token reads the valid prefix slots; the state token
    (row 0) opens its own block and reads itself; the action tokens (rows 1..)
    form one block that reads the state token and every action token."""
    B, P = prefix_mask.shape
    vis = np.zeros((B, S, P + S), bool)
    vis[:, :, :P] = prefix_mask[:, None, :].astype(bool)
    vis[:, 0, P] = True
    vis[:, 1:, P:] = True
    return vis


def _net_torch_f64(x, t, state, w, ck, cv, pm, rounding):
    """The stand-in net as a float64 composition of library calls: F.linear for
    every projection, F.scaled_dot_product_attention with a boolean mask for the
    attention, the RMS from torch.linalg.vector_norm; with `rounding`, one
    round-to-nearest-even to bf16 at the definition's rounding points (torch's
    own float64 -> bf16 conversion rounds twice, through float32, so the
    separately pinned single rounding is used)."""
    import torch.nn.functional as TF

    def r(a):
        return torch.from_numpy(round_bf16(a.numpy())) if rounding else a

    def rms(a):
        n = torch.linalg.vector_norm(a, dim=-1, keepdim=True)
        return torch.sqrt(n * n / a.shape[-1] + 1e-6)

    W = {k: _t64(v) for k, v in w.items()}
    x, state = _t64(x), _t64(state)
    h = torch.cat([TF.linear(r(state), W["w_state"], W["b_state"])[:, None],
                   TF.linear(r(x), W["w_in"], W["b_in"]) + float(t) * W["w_time"]], 1)
    B, S, _ = h.shape
    P, d = ck.shape[2], ck.shape[-1]
    Hq = W["w_q"].shape[0] // d
    vis = torch.from_numpy(_pi0_suffix_visibility(pm, S))[:, None]          # [B, 1, S, P+S]
    for layer in range(ck.shape[0]):
        a = r(h)
        rr = rms(a)
        q = r(TF.linear(a, W["w_q"]) / rr).view(B, S, Hq, d).transpose(1, 2)
        k = r(TF.linear(a, W["w_k"]) / rr)
        v = r(TF.linear(a, W["w_v"]) / rr)
        kk = torch.cat([_t64(ck[layer][:, :, 0]), k], 1)[:, None].expand(B, Hq, P + S, d)
        vv = torch.cat([_t64(cv[layer][:, :, 0]), v], 1)[:, None].expand(B, Hq, P + S, d)
        o = r(TF.scaled_dot_product_attention(q, kk, vv, attn_mask=vis))
        h = h + TF.linear(o.transpose(1, 2).reshape(B, S, Hq * d), W["w_o"])
    aa = r(h[:, 1:])
    return (TF.linear(aa, W["w_out"]) / rms(aa) + W["b_out"]).numpy()


def _net_case(seed, B=2, P=20, H=6, A_=5, W=64, layers=3):
    """Stand-in net inputs at the true head geometry (8 heads, 1 KV head, d = 256),
    with padded prefix slots in one sample."""
    nw = I.net_weights(seed, width=W, action_dim=A_)
    wf = {f: (I.bf16_bits_to_f64(getattr(nw, f)) if getattr(nw, f).dtype == np.uint16
              else getattr(nw, f).astype(np.float64)) for f in nw.__dataclass_fields__}
    ck = I.bf16_bits_to_f64(I.bf16_normal(seed + 20, (layers, B, P, 1, 256)))
    cv = I.bf16_bits_to_f64(I.bf16_normal(seed + 21, (layers, B, P, 1, 256)))
    pm = np.ones((B, P), np.uint8)
    pm[1, P - 7:] = 0
    sar = I.pi0_structure(P, H).ar[P:]
    x = I.f32_normal(seed + 22, (B, H, A_)).astype(np.float64)
    st = I.f32_normal(seed + 23, (B, A_)).astype(np.float64)
    return wf, ck, cv, pm, sar, x, st


def test_net_equals_library_composition_with_rounding_off(monkeypatch):
    """With the bf16 rounding points switched off, the oracle net equals the
    float64 library composition to rounding error (a dropped term, a wrong
    sign, a transposed operand, a misplaced norm or token would not)."""
    wf, ck, cv, pm, sar, x, st = _net_case(31)
    ident = lambda a: np.asarray(a, np.float64)
    monkeypatch.setattr(F, "round_bf16", ident)
    got = F.velocity_net(x, 0.7, st, wf, ck, cv, pm, sar, 8, 1, 256)
    want = _net_torch_f64(x, 0.7, st, wf, ck, cv, pm, rounding=False)
    assert got.shape == want.shape == x.shape
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_net_equals_library_composition_with_rounding_on():
    """The same with the rounding points on (the single bf16 rounding, pinned by
    test_bf16_rounding_matches_torch and test_bf16_rounding_of_float64_is_single)."""
    wf, ck, cv, pm, sar, x, st = _net_case(32)
    got = F.velocity_net(x, 0.3, st, wf, ck, cv, pm, sar, 8, 1, 256)
    want = _net_torch_f64(x, 0.3, st, wf, ck, cv, pm, rounding=True)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_net_closed_form_without_attention_path():
    """W_q = W_k = W_v = W_o = 0: every layer adds nothing, so the velocity is the
    out-projection of the embedded action tokens, written out here by hand:
    h = r(x) W_in^T + b_in + t w_time;  v = r(h) W_out^T / rms(r(h)) + b_out."""
    wf, ck, cv, pm, sar, x, st = _net_case(33)
    for f in ("w_q", "w_k", "w_v", "w_o"):
        wf[f] = np.zeros_like(wf[f])
    t = 0.6
    xr = I.bf16_bits_to_f64(I.f32_to_bf16_bits(x.astype(np.float32)))   # x is float32-exact
    B, H, A_ = x.shape
    W = wf["w_in"].shape[0]
    h = np.zeros((B, H, W))
    for b in range(B):
        for i in range(H):
            h[b, i] = wf["w_in"] @ xr[b, i] + wf["b_in"] + t * wf["w_time"]
    hr = _nearest_bf16(h)
    want = np.zeros((B, H, A_))
    for b in range(B):
        for i in range(H):
            scale = np.sqrt(np.dot(hr[b, i], hr[b, i]) / W + 1e-6)
            want[b, i] = wf["w_out"] @ hr[b, i] / scale + wf["b_out"]
    got = F.velocity_net(x, t, st, wf, ck, cv, pm, sar, 8, 1, 256)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    # the time enters with a plus sign: a different t moves v
    assert not np.allclose(F.velocity_net(x, -t, st, wf, ck, cv, pm, sar, 8, 1, 256), got)


def test_net_state_token_is_row_zero():
    """The state token only reaches the actions through the attention: with W_o = 0
    a different state leaves v unchanged; with the attention path on it moves v,
    and the library composition (state token at row 0) agrees."""
    wf, ck, cv, pm, sar, x, st = _net_case(34)
    st2 = st + 1.5
    w0 = dict(wf, w_o=np.zeros_like(wf["w_o"]))
    assert np.array_equal(F.velocity_net(x, 0.4, st, w0, ck, cv, pm, sar, 8, 1, 256),
                          F.velocity_net(x, 0.4, st2, w0, ck, cv, pm, sar, 8, 1, 256))
    v1 = F.velocity_net(x, 0.4, st, wf, ck, cv, pm, sar, 8, 1, 256)
    v2 = F.velocity_net(x, 0.4, st2, wf, ck, cv, pm, sar, 8, 1, 256)
    assert np.abs(v1 - v2).max() > 1e-3
    np.testing.assert_allclose(v2, _net_torch_f64(x, 0.4, st2, wf, ck, cv, pm, rounding=True), rtol=0, atol=1e-12)


def test_oracle_rms_equals_vector_norm():
    a = np.random.default_rng(5).standard_normal((3, 7, 96))
    n = torch.linalg.vector_norm(_t64(a), dim=-1, keepdim=True).numpy()
    np.testing.assert_allclose(F.rms(a), np.sqrt(n * n / 96 + 1e-6), rtol=1e-14)


def test_embed_suffix_rows():
    """Row 0 is the state token's projection, rows 1.. the action tokens' (with the
    time term), each an F.linear of the bf16-rounded input."""
    import torch.nn.functional as TF
    wf, ck, cv, pm, sar, x, st = _net_case(35)
    h = F.embed_suffix(x, 0.25, st, wf)
    r = lambda a: _t64(_nearest_bf16(a))
    want0 = TF.linear(r(st), _t64(wf["w_state"]), _t64(wf["b_state"])).numpy()
    want1 = (TF.linear(r(x), _t64(wf["w_in"]), _t64(wf["b_in"])) + 0.25 * _t64(wf["w_time"])).numpy()
    np.testing.assert_allclose(h[:, 0], want0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(h[:, 1:], want1, rtol=0, atol=1e-12)

"""GPU parity of the software exp2 (the exponential moved off the transcendental unit
for part of the softmax, [HW] section 0x09) and of the forward that uses it."""
import numpy as np
import pytest
import torch

import attn_inputs
from oracle import dense, exp2soft
from gpu_common import (TOL_OUT, assert_close_lse, assert_close_out, need_gpu, say, to_dev)

pytestmark = pytest.mark.gpu

F32_MIN_NORMAL = np.float32(2.0 ** -126)


def _inputs():
    rng = np.random.default_rng(31)
    return np.concatenate([
        np.linspace(-160.0, 10.0, 400_001),
        rng.uniform(-30.0, 8.0, 200_000),
        np.arange(-155, 11),                      # integers: f = 0
        [-np.inf, -1e30, -150.0, -149.5, -126.0, -125.999, 0.0, -0.0, 1e-8, -1e-8, 7.999999],
    ]).astype(np.float32)


def test_exp2_soft_matches_oracle():
    need_gpu()
    import exact_tiled_attention_amd as eta
    x = _inputs()
    say(f"[exp2_soft] n={x.size}")
    y = eta.exp2_soft(torch.from_numpy(x).cuda()).cpu().numpy()
    ref = exp2soft.soft_exp2_f32(x)
    normal = ref >= F32_MIN_NORMAL
    # the oracle's fma rounds twice (float64 then float32): at most one ulp apart
    ulps = np.abs(y[normal].view(np.int32).astype(np.int64) - ref[normal].view(np.int32).astype(np.int64))
    assert ulps.max() <= 1, f"max ulp difference {ulps.max()}"
    # below the normal range a flush to zero is allowed
    assert np.all(np.abs(y[~normal] - ref[~normal]) <= F32_MIN_NORMAL)
    assert np.all(y >= 0.0) and np.all(np.isfinite(y))
    # at integers the result is the scaled constant term, exactly
    n = np.arange(-100, 9).astype(np.float32)
    yn = eta.exp2_soft(torch.from_numpy(n).cuda()).cpu().numpy()
    assert np.array_equal(yn, exp2soft.soft_exp2_f32(n))
    # against the exact exponential, over the range the softmax feeds it
    sel = (x >= -120.0) & (x <= 8.0)
    rel = np.abs(y[sel].astype(np.float64) / np.exp2(x[sel].astype(np.float64)) - 1.0)
    assert rel.max() <= 7.6e-5, rel.max()
    # -inf and deep underflow give 0
    assert np.all(y[np.isneginf(x) | (x <= -150.0)] == 0.0)


def test_exp2_soft_empty_and_ragged():
    need_gpu()
    import exact_tiled_attention_amd as eta
    e = torch.empty(0, dtype=torch.float32, device="cuda")
    assert eta.exp2_soft(e).numel() == 0
    x = np.linspace(-5, 5, 257 * 3 + 11).astype(np.float32).reshape(-1)
    y = eta.exp2_soft(torch.from_numpy(x).cuda()).cpu().numpy()
    ulps = np.abs(y.view(np.int32).astype(np.int64) - exp2soft.soft_exp2_f32(x).view(np.int32).astype(np.int64))
    assert ulps.max() <= 1


def _check(w, emu, rows=None):
    import exact_tiled_attention_amd as eta
    t, p = w.tensors, w.params
    q, k, v = (to_dev(t[n]) for n in ("q", "k", "v"))
    say(f"[fwd_exp_emulated] {w.name} causal={p['causal']} emulated_per_8={emu}")
    o, lse = eta.attn_fwd_exp_emulated(q, k, v, emu, scale=p["scale"], causal=p["causal"])
    torch.cuda.synchronize()
    O, L = dense.forward(t["q"], t["k"], t["v"], p["scale"], p["causal"], rows=rows)
    oo, ll = o.cpu(), lse.cpu()
    if rows is not None:
        oo, ll = oo[:, :, rows], ll[:, :, rows]
    e1 = assert_close_out(oo, O, TOL_OUT[t["q"].dtype], w.name)
    e2 = assert_close_lse(ll, L, w.name)
    say(f"    max|dO|={e1:.2e} max|dLSE|={e2:.2e}")


@pytest.mark.parametrize("emu", [2, 4])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk", [
    (2, 4, 1, 257, 193),      # query and key tails, MQA
    (1, 8, 2, 200, 333),      # S_q < S_k, GQA 4
    (1, 2, 2, 300, 100),      # S_q > S_k: causal rows with no visible key
])
def test_fwd_exp_emulated_small_elementwise(emu, dtype, d, causal, B, Hq, Hkv, Sq, Sk):
    need_gpu()
    w = attn_inputs.prefill(B, Hq, Hkv, Sq, Sk, d, dtype, seed=300 + Sq + Sk + d, causal=causal)
    _check(w, emu)


@pytest.mark.parametrize("emu", [2, 4])
def test_fwd_exp_emulated_full_size_sampled_rows(emu):
    need_gpu()
    w = attn_inputs.CONFIGS["fwd_f16_1x8x4096_d64"]()
    rows = np.unique(np.concatenate([np.arange(0, 4096, 131), [4095]]))
    _check(w, emu, rows=rows)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_exp_emulated_zero_is_attn_fwd(d, causal):
    need_gpu()
    import exact_tiled_attention_amd as eta
    w = attn_inputs.prefill(1, 4, 2, 333, 411, d, "bf16", seed=77 + d, causal=causal)
    q, k, v = (to_dev(w.tensors[n]) for n in ("q", "k", "v"))
    o0, l0 = eta.attn_fwd(q, k, v, causal=causal)
    o1, l1 = eta.attn_fwd_exp_emulated(q, k, v, 0, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)


def test_fwd_exp_emulated_rejects_other_fractions():
    need_gpu()
    import exact_tiled_attention_amd as eta
    q = torch.zeros((1, 1, 8, 64), dtype=torch.float16, device="cuda")
    with pytest.raises(eta.AttnError):
        eta.attn_fwd_exp_emulated(q, q, q, 3)

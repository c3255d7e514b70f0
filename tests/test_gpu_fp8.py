"""GPU parity of attn_fwd_fp8 against the oracle's step-by-step quantised forward."""
import numpy as np
import pytest
import torch

import attn_inputs
from oracle import dense, fp8
from gpu_common import TOL_FP8, assert_close_lse, assert_close_out, need_gpu, say, to_dev

pytestmark = pytest.mark.gpu

# Relative distance to an E4M3 midpoint below which a float32 probability's rounding is
# treated as undecided: the kernel's u carries a relative error of about
# ln2 * 2^-24 * (|score| + |max|) in base-2 units, below 2^-12 for |score| < 2^10.
AMBIGUITY_REL = 2.0 ** -12


def _gpu(w, o_dtype, causal=False, scale=None):
    import exact_tiled_attention_amd as eta
    t, p = w.tensors, w.params
    args = [to_dev(t[n]) for n in ("q8", "k8", "v8", "q_scale", "k_scale", "v_scale")]
    o, lse = eta.attn_fwd_fp8(*args, scale=p["scale"] if scale is None else scale, o_dtype=o_dtype, causal=causal)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def _check(w, rows=None, heads=None, causal=False, scale=None):
    import exact_tiled_attention_amd as eta
    t, p = w.tensors, w.params
    scale = p["scale"] if scale is None else scale
    tile = eta.fp8_kv_tile()
    say(f"[fp8] {w.name} tile={tile} causal={causal} scale={scale}")
    o32, l32 = _gpu(w, torch.float32, causal, scale)
    obf, lbf = _gpu(w, torch.bfloat16, causal, scale)
    # the bf16 output is the round-to-nearest-even of the float32 result
    assert torch.equal(obf, o32.to(torch.bfloat16)) and torch.equal(lbf, l32)
    O, L, E = fp8.forward(t["q8"], t["k8"], t["v8"], t["q_scale"], t["k_scale"], t["v_scale"], scale,
                          block_c=tile, rows=rows, heads=heads, envelope_rel=AMBIGUITY_REL, causal=causal)
    if rows is not None:
        o32, l32 = o32[:, :, rows], l32[:, :, rows]
    if heads is not None:
        sel = tuple(np.array(heads).T)
        o32, l32, O, L, E = o32[sel], l32[sel], O[sel], L[sel], E[sel]
    # 5e-2 plus, per element, what E4M3 roundings left undecided by float32 scores
    # could move the output (either neighbour is a correct rounding there)
    err = np.abs(o32.double().numpy() - O)
    bad = err > TOL_FP8 + E
    assert not bad.any(), f"{w.name}: max err {err.max():.3e} at {np.argwhere(bad)[:5].tolist()}"
    e1 = float(err.max())
    say(f"    elements whose bound was widened by ambiguous roundings: {(E > 0).mean():.2%}, max E {E.max():.3e}")
    e2 = assert_close_lse(l32, L, w.name)
    # informational: error of the quantised path against dense attention on the
    # dequantised inputs (the FA3 accuracy table reports RMSE against float64)
    Od, _ = dense.forward(fp8.dequantized(t["q8"], t["q_scale"]), fp8.dequantized(t["k8"], t["k_scale"]),
                          fp8.dequantized(t["v8"], t["v_scale"]), scale, causal, rows=rows, heads=heads)
    if heads is not None:
        Od = Od[sel]
    rmse = float(np.sqrt(np.mean((o32.double().numpy() - Od) ** 2)))
    say(f"    max|dO| vs oracle {e1:.2e}, max|dLSE| {e2:.2e}, RMSE vs unquantised P {rmse:.3e}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk", [(1, 2, 2, 128, 128), (2, 4, 2, 200, 333), (1, 2, 1, 64, 1),
                                            (1, 1, 1, 300, 64), (1, 2, 2, 300, 100),
                                            # three and four key tiles: every slot of the
                                            # three-stage K/V ring, and its first reuse
                                            (1, 2, 2, 150, 150), (1, 2, 1, 100, 250)])
def test_fp8_small_elementwise(d, causal, B, Hq, Hkv, Sq, Sk):
    need_gpu()
    _check(attn_inputs.fp8_prefill(B, Hq, Hkv, Sq, Sk, d, seed=500 + Sq + Sk + d), causal=causal)


@pytest.mark.parametrize("d", [64, 128])
def test_fp8_zero_descales_and_zero_scale(d):
    """An all-zero value block (descale 0), an all-zero key tail block (descale 0) and
    a zero score scale give the oracle's finite result, never NaN."""
    need_gpu()
    w = attn_inputs.fp8_prefill(1, 2, 2, 200, 300, d, seed=71)
    t = w.tensors
    t["v8"][:, :, 128:256] = 0
    t["v_scale"][:, :, 1] = 0.0
    t["k8"][:, :, 256:] = 0
    t["k_scale"][:, :, 2] = 0.0
    for causal in (False, True):
        _check(w, causal=causal)
        _check(w, causal=causal, scale=0.0)


def test_fp8_4x16x8192_full_size_sampled():
    need_gpu()
    w = attn_inputs.CONFIGS["fwd_fp8_4x16x8192_d128"]()
    rows = np.unique(np.concatenate([np.arange(0, 8192, 331), [0, 127, 128, 8191]]))
    _check(w, rows=rows, heads=[(0, 0), (1, 7), (3, 15)])


def test_fp8_eight_wave_tiles_with_tails():
    # a grid of at least one 256-row workgroup per compute unit takes the eight-wave
    # launch: here 4 x 32 heads x ceil(600 / 256) = 384 workgroups; query and key tails
    # (600 = 2 x 256 + 88, 777 keys) and GQA 4
    need_gpu()
    w = attn_inputs.fp8_prefill(4, 32, 8, 600, 777, 128, seed=61)
    rows = np.array([0, 1, 127, 128, 255, 256, 300, 511, 512, 513, 599])
    _check(w, rows=rows, heads=[(0, 0), (1, 13), (2, 22), (3, 31)])


def test_fp8_bitwise_repeatable():
    need_gpu()
    w = attn_inputs.fp8_prefill(1, 4, 4, 512, 512, 128, seed=9)
    a, b = _gpu(w, torch.bfloat16), _gpu(w, torch.bfloat16)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_fp8_causal_eight_waves_and_gqa_sampled():
    """The eight-wave launch (>= one 256-row workgroup per compute unit) under causal
    masking, with query and key tails (S_q < S_k) and GQA 4."""
    need_gpu()
    w = attn_inputs.fp8_prefill(4, 32, 8, 600, 777, 128, seed=62)
    rows = np.array([0, 1, 127, 128, 255, 256, 300, 511, 512, 513, 599])
    _check(w, rows=rows, heads=[(0, 0), (1, 13), (2, 22), (3, 31)], causal=True)

"""GPU parity of attn_fwd against the float64 oracle (elementwise on small shapes,
sampled rows at the full workload sizes)."""
import numpy as np
import pytest
import torch

import attn_inputs
from oracle import dense
from gpu_common import (TOL_OUT, assert_close_lse, assert_close_out, need_gpu, say, to_dev)

pytestmark = pytest.mark.gpu


def _run(w, rows=None, heads=None):
    import exact_tiled_attention_amd as eta
    t, p = w.tensors, w.params
    q, k, v = (to_dev(t[n]) for n in ("q", "k", "v"))
    say(f"[fwd] {w.name} causal={p['causal']}")
    o, lse = eta.attn_fwd(q, k, v, scale=p["scale"], causal=p["causal"])
    torch.cuda.synchronize()
    O, L = dense.forward(t["q"], t["k"], t["v"], p["scale"], p["causal"], rows=rows, heads=heads)
    return o, lse, O, L


def _check(w, rows=None, heads=None):
    o, lse, O, L = _run(w, rows, heads)
    dt = w.tensors["q"].dtype
    oo, ll = o.cpu(), lse.cpu()
    if rows is not None:
        oo, ll = oo[:, :, rows], ll[:, :, rows]
    if heads is not None:
        sel = tuple(np.array(heads).T)
        oo, ll, O, L = oo[sel], ll[sel], O[sel], L[sel]
    e1 = assert_close_out(oo, O, TOL_OUT[dt], w.name)
    e2 = assert_close_lse(ll, L, w.name)
    say(f"    max|dO|={e1:.2e} max|dLSE|={e2:.2e}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk", [
    (1, 4, 4, 128, 128),      # the small listing shape
    (2, 4, 1, 257, 193),      # query and key tails, MQA
    (1, 8, 2, 200, 333),      # S_q < S_k (bottom-right causal), GQA 4
    (1, 2, 2, 300, 100),      # S_q > S_k: causal rows with no visible key
    (1, 3, 3, 64, 1),         # a single key
])
def test_fwd_small_elementwise(dtype, d, causal, B, Hq, Hkv, Sq, Sk):
    need_gpu()
    w = attn_inputs.prefill(B, Hq, Hkv, Sq, Sk, d, dtype, seed=100 + Sq + Sk + d, causal=causal)
    _check(w)


def test_fwd_listing_shape_1x4x128():
    need_gpu()
    _check(attn_inputs.CONFIGS["fwd_f16_1x4x128_d64"]())


def test_fwd_empty_keys_and_zero_scale():
    need_gpu()
    import exact_tiled_attention_amd as eta
    w = attn_inputs.prefill(1, 2, 2, 70, 90, 64, "f16", seed=7, scale=0.0)
    _check(w)
    q = to_dev(w.tensors["q"])
    k = torch.empty((1, 2, 0, 64), dtype=torch.float16, device="cuda")
    o, lse = eta.attn_fwd(q, k, k, scale=0.125)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_fwd_1x8x4096_full_size_sampled_rows():
    need_gpu()
    w = attn_inputs.CONFIGS["fwd_f16_1x8x4096_d64"]()
    rows = np.unique(np.concatenate([np.arange(0, 4096, 97), [4095]]))
    _check(w, rows=rows)


def test_fwd_causal_gqa_full_size_sampled():
    need_gpu()
    w = attn_inputs.CONFIGS["causal_gqa_bf16_2x32x8192_kv8_d128"]()
    rows = np.unique(np.concatenate([np.arange(0, 8192, 211), [0, 1, 127, 128, 8191]]))
    heads = [(0, 0), (0, 5), (1, 31), (1, 12)]
    _check(w, rows=rows, heads=heads)


@pytest.mark.parametrize("d,dtype", [(64, "f16"), (64, "bf16"), (128, "bf16")])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_large_grid_sampled(d, dtype, causal):
    """Grids of at least one 256-row workgroup per compute unit (the single-key-range
    and two-key-range launch shapes), with query and key tails."""
    need_gpu()
    w = attn_inputs.prefill(2, 64, 16, 1100, 1070, d, dtype, seed=31 + d, causal=causal)
    rows = np.unique(np.concatenate([np.arange(0, 1100, 37), [0, 255, 256, 1023, 1024, 1099]]))
    heads = [(0, 0), (0, 63), (1, 17), (1, 40)]
    _check(w, rows=rows, heads=heads)


def test_fwd_bitwise_repeatable():
    need_gpu()
    import exact_tiled_attention_amd as eta
    w = attn_inputs.prefill(2, 8, 2, 1000, 1000, 128, "bf16", seed=9, causal=True)
    q, k, v = (to_dev(w.tensors[n]) for n in ("q", "k", "v"))
    o1, l1 = eta.attn_fwd(q, k, v, causal=True)
    o2, l2 = eta.attn_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)

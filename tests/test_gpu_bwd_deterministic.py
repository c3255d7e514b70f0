"""GPU parity of the deterministic backward (query-owner dQ over fixed key ranges, fixed
tree over their partials) against the float64 oracle, and bitwise repeatability."""
import numpy as np
import pytest
import torch

import attn_inputs
from oracle import dense
from gpu_common import TOL_GRAD, assert_close_out, need_gpu, say, to_dev

pytestmark = pytest.mark.gpu


def _grads(w, deterministic=True, dq_splits=1, grad_dtype=torch.float32):
    import exact_tiled_attention_amd as eta
    t, p = w.tensors, w.params
    q, k, v, do = (to_dev(t[n]) for n in ("q", "k", "v", "do"))
    o, lse = eta.attn_fwd(q, k, v, scale=p["scale"], causal=p["causal"])
    g = eta.attn_bwd(q, k, v, o, lse, do, scale=p["scale"], causal=p["causal"], grad_dtype=grad_dtype,
                     deterministic=deterministic, dq_splits=dq_splits)
    torch.cuda.synchronize()
    return tuple(x.cpu() for x in g)


def _check(w, dq_splits):
    t, p = w.tensors, w.params
    say(f"[bwd-det] {w.name} causal={p['causal']} splits={dq_splits}")
    got = _grads(w, dq_splits=dq_splits)
    ref = dense.backward(t["q"], t["k"], t["v"], t["do"], p["scale"], p["causal"], o_storage=t["q"].dtype)[:3]
    errs = [assert_close_out(g_, r_, TOL_GRAD, f"{w.name} {n}") for n, g_, r_ in zip(("dq", "dk", "dv"), got, ref)]
    say("    max err dq/dk/dv = " + " ".join(f"{e:.2e}" for e in errs))
    return got


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk", [
    (1, 2, 2, 128, 128),
    (2, 4, 1, 257, 193),      # query and key tails, MQA
    (1, 8, 2, 200, 333),      # S_q < S_k, GQA 4
    (1, 2, 2, 300, 100),      # S_q > S_k: causal rows with no visible key
    (1, 4, 2, 70, 1),         # one key
    (1, 2, 2, 32, 96),        # one query tile: the column owner's loop has one step
    (1, 2, 2, 64, 64),        # two steps
])
def test_deterministic_elementwise(dtype, d, causal, B, Hq, Hkv, Sq, Sk):
    need_gpu()
    w = attn_inputs.prefill(B, Hq, Hkv, Sq, Sk, d, dtype, seed=700 + Sq + Sk + d, causal=causal, with_grad=True)
    _check(w, 1)


@pytest.mark.parametrize("dq_splits", [2, 4, 16])
def test_deterministic_split_partials_tree(dq_splits):
    need_gpu()
    w = attn_inputs.prefill(1, 8, 2, 333, 1100, 128, "bf16", seed=71, causal=True, with_grad=True)
    _check(w, dq_splits)


@pytest.mark.parametrize("dq_splits", [1, 4])
def test_deterministic_is_bitwise_repeatable(dq_splits):
    need_gpu()
    w = attn_inputs.prefill(2, 8, 2, 700, 700, 128, "bf16", seed=72, causal=True, with_grad=True)
    a = _grads(w, dq_splits=dq_splits)
    b = _grads(w, dq_splits=dq_splits)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_deterministic_dk_dv_equal_atomic_path():
    """dK and dV come from the same column-owner arithmetic in both modes."""
    need_gpu()
    w = attn_inputs.prefill(1, 4, 2, 256, 384, 64, "f16", seed=73, causal=False, with_grad=True)
    a = _grads(w, deterministic=True)
    b = _grads(w, deterministic=False)
    assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])
    assert (a[0] - b[0]).abs().max().item() < 1e-3


def test_deterministic_16bit_gradients():
    need_gpu()
    w = attn_inputs.prefill(1, 8, 2, 384, 384, 128, "bf16", seed=74, causal=True, with_grad=True)
    got = _grads(w, grad_dtype=torch.bfloat16)
    f32 = _grads(w, grad_dtype=torch.float32)
    for x, y in zip(got, f32):
        assert torch.equal(x, y.to(torch.bfloat16))


@pytest.mark.parametrize("dq_splits", [1, 4])
def test_deterministic_bf16_power_of_two_inputs(dq_splits):
    """bf16 operands run on fp16 copies scaled by one power of two per tensor.  Inputs
    scaled as q 2^10, k 2^-10 (S unchanged), v 2^20 and dO 2^-30 give the same copies, so
    the gradients are the unscaled ones times 2^-20 (dQ), 1 (dK) and 2^-30 (dV), bit for
    bit: a wrong exponent, a factor applied twice or a lost one shows here."""
    need_gpu()
    import exact_tiled_attention_amd as eta
    w = attn_inputs.prefill(1, 8, 2, 333, 517, 128, "bf16", seed=75, causal=True, with_grad=True)
    t, p = w.tensors, w.params
    q, k, v, do = (to_dev(t[n]) for n in ("q", "k", "v", "do"))

    def grads(q, k, v, do):
        o, lse = eta.attn_fwd(q, k, v, scale=p["scale"], causal=True)
        g = eta.attn_bwd(q, k, v, o, lse, do, scale=p["scale"], causal=True, grad_dtype=torch.float32,
                         deterministic=True, dq_splits=dq_splits)
        torch.cuda.synchronize()
        return [x.cpu() for x in g]

    say(f"[bwd-det] power-of-two scaled bf16 inputs, splits={dq_splits}")
    base = grads(q, k, v, do)
    scaled = grads(q * 2.0 ** 10, k * 2.0 ** -10, v * 2.0 ** 20, do * 2.0 ** -30)
    assert torch.equal(scaled[0] * 2.0 ** 20, base[0])
    assert torch.equal(scaled[1], base[1])
    assert torch.equal(scaled[2] * 2.0 ** 30, base[2])
    ref = dense.backward(t["q"], t["k"], t["v"], t["do"], p["scale"], True, o_storage=t["q"].dtype)[:3]
    for n, g_, r_ in zip(("dq", "dk", "dv"), base, ref):
        assert_close_out(g_, r_, TOL_GRAD, f"power-of-two base {n}")


def test_deterministic_bf16_small_gradients():
    """dO of magnitude 2^-40 (a loss averaged over many tokens): the copies carry it at
    full fp16 precision, so the gradients keep their relative accuracy."""
    need_gpu()
    import exact_tiled_attention_amd as eta
    w = attn_inputs.prefill(1, 4, 2, 200, 300, 64, "bf16", seed=76, causal=False, with_grad=True)
    t, p = w.tensors, w.params
    q, k, v, do = (to_dev(t[n]) for n in ("q", "k", "v", "do"))
    o, lse = eta.attn_fwd(q, k, v, scale=p["scale"], causal=False)
    g = eta.attn_bwd(q, k, v, o, lse, do * 2.0 ** -40, scale=p["scale"], causal=False, grad_dtype=torch.float32,
                     deterministic=True)
    torch.cuda.synchronize()
    ref = dense.backward(t["q"], t["k"], t["v"], t["do"], p["scale"], False, o_storage=t["q"].dtype)[:3]
    for n, g_, r_ in zip(("dq", "dk", "dv"), g, ref):
        assert_close_out(g_.cpu() * 2.0 ** 40, r_, TOL_GRAD, f"dO 2^-40 {n}")

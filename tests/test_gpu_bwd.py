"""GPU parity of attn_bwd and attn_bwd_atomic (from the GPU forward's O and LSE) against
the float64 oracle."""
import numpy as np
import pytest
import torch

import attn_inputs
from oracle import dense
from gpu_common import TOL_GRAD, assert_close_out, need_gpu, say, to_dev

pytestmark = pytest.mark.gpu


def _gpu_grads(w, grad_dtype=torch.float32, atomic=False, deterministic=False):
    import exact_tiled_attention_amd as eta
    t, p = w.tensors, w.params
    q, k, v, do = (to_dev(t[n]) for n in ("q", "k", "v", "do"))
    o, lse = eta.attn_fwd(q, k, v, scale=p["scale"], causal=p["causal"])
    dq, dk, dv = eta.attn_bwd(q, k, v, o, lse, do, scale=p["scale"], causal=p["causal"], grad_dtype=grad_dtype,
                              atomic=atomic, deterministic=deterministic)
    torch.cuda.synchronize()
    return dq, dk, dv


def _check(w, grad_dtype=torch.float32, heads=None, atomic=False):
    t, p = w.tensors, w.params
    say(f"[bwd] {w.name} causal={p['causal']} grad={grad_dtype} atomic={atomic}")
    dq, dk, dv = _gpu_grads(w, grad_dtype, atomic=atomic)
    # D is formed from the forward output as stored in the element type
    dQ, dK, dV, _ = dense.backward(t["q"], t["k"], t["v"], t["do"], p["scale"], p["causal"], heads=heads,
                                   o_storage=t["q"].dtype)
    g = p["Hq"] // p["Hkv"]
    gq, gk, gv = dq.cpu(), dk.cpu(), dv.cpu()
    if heads is not None:
        qsel = [(b, h) for b, kv in heads for h in range(kv * g, (kv + 1) * g)]
        qi = tuple(np.array(qsel).T)
        ki = tuple(np.array(heads).T)
        gq, dQ = gq[qi], dQ[qi]
        gk, gv, dK, dV = gk[ki], gv[ki], dK[ki], dV[ki]
    errs = []
    for name, got, ref in (("dq", gq, dQ), ("dk", gk, dK), ("dv", gv, dV)):
        if grad_dtype == torch.float32:
            errs.append(assert_close_out(got, ref, TOL_GRAD, f"{w.name} {name}"))
        else:
            # a 16-bit gradient is the rounding of the float32 one: allow half an ulp of
            # the stored type on top of the float32 tolerance
            r = np.abs(ref)
            ulp = 2.0 ** (np.floor(np.log2(np.maximum(r, 1e-30))) - (7 if grad_dtype == torch.bfloat16 else 10))
            err = np.abs(got.float().double().numpy() - ref)
            assert np.all(err <= TOL_GRAD + 0.5 * ulp), f"{name} max err {err.max():.3e}"
            errs.append(float(err.max()))
    say("    max err dq/dk/dv = " + " ".join(f"{e:.2e}" for e in errs))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk", [
    (1, 2, 2, 128, 128),
    (2, 4, 1, 257, 193),      # query and key tails, MQA
    (1, 8, 2, 200, 333),      # S_q < S_k, GQA 4
    (1, 2, 2, 300, 100),      # S_q > S_k: causal rows with no visible key
    (1, 4, 2, 70, 1),         # one key
])
def test_bwd_small_elementwise(dtype, d, causal, B, Hq, Hkv, Sq, Sk):
    need_gpu()
    w = attn_inputs.prefill(B, Hq, Hkv, Sq, Sk, d, dtype, seed=300 + Sq + Sk + d, causal=causal, with_grad=True)
    _check(w)


@pytest.mark.parametrize("gd", [torch.bfloat16, torch.float16])
def test_bwd_16bit_gradient_outputs(gd):
    need_gpu()
    w = attn_inputs.prefill(1, 8, 2, 384, 384, 128, "bf16", seed=31, causal=True, with_grad=True)
    _check(w, grad_dtype=gd)


def test_bwd_atomic_dq_repeat_within_tolerance():
    need_gpu()
    w = attn_inputs.prefill(1, 8, 2, 640, 640, 128, "bf16", seed=41, causal=True, with_grad=True)
    a = _gpu_grads(w)
    b = _gpu_grads(w)
    assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])        # dK, dV: no atomics
    assert (a[0] - b[0]).abs().max().item() <= 1e-5                    # dQ: unordered float adds


@pytest.mark.parametrize("atomic", [False, True])
def test_bwd_causal_gqa_full_size_one_kv_head(atomic):
    need_gpu()
    w = attn_inputs.CONFIGS["causal_gqa_bf16_2x32x8192_kv8_d128"]()
    _check(w, heads=[(1, 5)], atomic=atomic)


@pytest.mark.parametrize("dtype,causal", [("bf16", True), ("f16", False)])
def test_bwd_atomic_form_long_keys(dtype, causal):
    """attn_bwd_atomic keeps the column owner's atomic dQ where attn_bwd switches form."""
    need_gpu()
    w = attn_inputs.prefill(1, 8, 2, 700, 1100, 128, dtype, seed=42, causal=causal, with_grad=True)
    _check(w, atomic=True)


def test_bwd_long_keys_take_the_query_row_owner():
    """From 1024 keys on, attn_bwd is the deterministic form with one key range."""
    need_gpu()
    w = attn_inputs.prefill(1, 8, 2, 700, 1100, 128, "bf16", seed=43, causal=True, with_grad=True)
    _check(w)
    a = _gpu_grads(w)
    b = _gpu_grads(w, deterministic=True)
    for x, y in zip(a, b):
        assert torch.equal(x, y)

"""GPU parity of attn_bwd_fp8 (gradients with respect to the dequantised E4M3 operands)
against the float64 oracle, fed the same O and LSE."""
import numpy as np
import pytest
import torch

import attn_inputs
from oracle import dense, fp8
from gpu_common import TOL_GRAD, assert_close_out, need_gpu, say, to_dev

pytestmark = pytest.mark.gpu


def _inputs(w, seed):
    t = w.tensors
    do = attn_inputs.normal(tuple(t["q8"].shape), seed, 3, "bf16")
    return do


def _gpu_bwd(w, o, lse, do, causal, grad_dtype=torch.float32):
    import exact_tiled_attention_amd as eta
    t, p = w.tensors, w.params
    args = [to_dev(t[n]) for n in ("q8", "k8", "v8", "q_scale", "k_scale", "v_scale")]
    g = eta.attn_bwd_fp8(*args, to_dev(o), to_dev(lse), to_dev(do), scale=p["scale"], causal=causal,
                         grad_dtype=grad_dtype)
    torch.cuda.synchronize()
    return tuple(x.cpu() for x in g)


def _compare(w, got, o, lse, do, causal, grad_dtype=torch.float32):
    t, p = w.tensors, w.params
    ref = fp8.backward(t["q8"], t["k8"], t["v8"], t["q_scale"], t["k_scale"], t["v_scale"], o.double(), lse.double(),
                       do.double(), p["scale"], causal)
    errs = []
    for name, g_, r_ in zip(("dq", "dk", "dv"), got, ref):
        if grad_dtype == torch.float32:
            errs.append(assert_close_out(g_, r_, TOL_GRAD, f"{w.name} {name}"))
        else:
            # a 16-bit gradient is the rounding of the float32 one: half an ulp on top
            ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(r_), 1e-30))) - (7 if grad_dtype == torch.bfloat16 else 10))
            err = np.abs(g_.float().double().numpy() - r_)
            assert np.all(err <= TOL_GRAD + 0.5 * ulp), f"{name} max err {err.max():.3e}"
            errs.append(float(err.max()))
    say("    max err dq/dk/dv = " + " ".join(f"{e:.2e}" for e in errs)
        + "; max |dq|,|dk|,|dv| = " + " ".join(f"{np.nanmax(np.abs(r)):.1f}" for r in ref))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk", [(1, 2, 2, 128, 128), (1, 4, 2, 200, 333), (1, 2, 1, 300, 100),
                                            (2, 4, 4, 64, 1)])
def test_fp8_bwd_exact_forward_state(d, causal, B, Hq, Hkv, Sq, Sk):
    """O and LSE of the exact forward on the dequantised operands (O stored in bf16):
    the gradients are then the exact ones of that forward."""
    need_gpu()
    w = attn_inputs.fp8_prefill(B, Hq, Hkv, Sq, Sk, d, seed=700 + Sq + Sk + d)
    t, p = w.tensors, w.params
    say(f"[fp8-bwd] {w.name} causal={causal}")
    O, L = dense.forward(fp8.dequantized(t["q8"], t["q_scale"]), fp8.dequantized(t["k8"], t["k_scale"]),
                         fp8.dequantized(t["v8"], t["v_scale"]), p["scale"], causal)
    o = torch.from_numpy(O).to(torch.bfloat16)
    lse = torch.from_numpy(L).float()
    do = _inputs(w, 700 + Sq)
    got = _gpu_bwd(w, o, lse, do, causal)
    _compare(w, got, o, lse, do, causal)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_training_chain_forward_then_backward(causal):
    """attn_fwd_fp8 (bf16 O, LSE) then attn_bwd_fp8 on them, against the oracle given
    the same O and LSE; GQA 4, query and key tails."""
    need_gpu()
    import exact_tiled_attention_amd as eta
    w = attn_inputs.fp8_prefill(2, 8, 2, 300, 450, 128, seed=741)
    t, p = w.tensors, w.params
    say(f"[fp8-chain] {w.name} causal={causal}")
    args = [to_dev(t[n]) for n in ("q8", "k8", "v8", "q_scale", "k_scale", "v_scale")]
    o, lse = eta.attn_fwd_fp8(*args, scale=p["scale"], causal=causal)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    do = _inputs(w, 741)
    got = _gpu_bwd(w, o, lse, do, causal)
    _compare(w, got, o, lse, do, causal)


@pytest.mark.parametrize("gd", [torch.bfloat16, torch.float16])
def test_fp8_bwd_16bit_gradients(gd):
    need_gpu()
    w = attn_inputs.fp8_prefill(1, 4, 2, 256, 256, 128, seed=751)
    t, p = w.tensors, w.params
    O, L = dense.forward(fp8.dequantized(t["q8"], t["q_scale"]), fp8.dequantized(t["k8"], t["k_scale"]),
                         fp8.dequantized(t["v8"], t["v_scale"]), p["scale"], True)
    o, lse = torch.from_numpy(O).to(torch.bfloat16), torch.from_numpy(L).float()
    do = _inputs(w, 751)
    say(f"[fp8-bwd16] {w.name} {gd}")
    got = _gpu_bwd(w, o, lse, do, True, grad_dtype=gd)
    _compare(w, got, o, lse, do, True, grad_dtype=gd)

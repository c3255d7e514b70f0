"""GPU parity of the dropout forward and backward against the float64 oracle, and the
exact keep decisions (integer Philox words) against the oracle's."""
import numpy as np
import pytest
import torch

import attn_inputs
from oracle import dense, dropout
from gpu_common import TOL_GRAD, TOL_OUT, assert_close_lse, assert_close_out, need_gpu, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_dropout_keep_decisions_exact(d, causal):
    """Q = K = 0 makes every visible probability 1 / (visible keys); with V = I the
    output element (i, j) is nonzero exactly when (i, j) was kept."""
    need_gpu()
    import exact_tiled_attention_amd as eta
    B, Hq, Hkv, Sq, Sk = 2, 4, 2, 200, d
    p, seed, offset = 0.37, 0x1234_5678_9ABC_DEF0, 11
    q = torch.zeros(B, Hq, Sq, d, dtype=torch.float16)
    k = torch.zeros(B, Hkv, Sk, d, dtype=torch.float16)
    v = torch.eye(Sk, d, dtype=torch.float16).expand(B, Hkv, Sk, d).contiguous()
    say(f"[dropout-mask] d={d} causal={causal}")
    o, _ = eta.attn_fwd_dropout(to_dev(q), to_dev(k), to_dev(v), p, seed, offset, scale=0.1, causal=causal)
    got = (o.cpu().float().numpy() != 0)
    vis = dense.visible(Sq, Sk, causal)
    for b in range(B):
        for h in range(Hq):
            keep = dropout.keep_mask(b, h, Hq, np.arange(Sq), Sk, p, seed, offset)
            assert np.array_equal(got[b, h], keep & vis), (b, h)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk,p", [
    (1, 4, 2, 257, 193, 0.1),
    (2, 2, 1, 130, 300, 0.5),
    (1, 2, 2, 300, 100, 0.25),     # causal rows with no visible key
])
def test_dropout_forward_elementwise(dtype, d, causal, B, Hq, Hkv, Sq, Sk, p):
    need_gpu()
    import exact_tiled_attention_amd as eta
    w = attn_inputs.prefill(B, Hq, Hkv, Sq, Sk, d, dtype, seed=800 + Sq + d, causal=causal)
    t, prm = w.tensors, w.params
    seed, offset = 1000 + Sq, 3
    say(f"[dropout-fwd] {w.name} causal={causal} p={p}")
    o, lse = eta.attn_fwd_dropout(to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"]), p, seed, offset,
                                  scale=prm["scale"], causal=causal)
    torch.cuda.synchronize()
    O, L = dropout.forward(t["q"], t["k"], t["v"], prm["scale"], causal, p, seed, offset)
    # 1 / (1 - p) scales kept values past 2, where half an ulp of the stored 16-bit
    # output alone can exceed the absolute tolerance: allow it on top (as for 16-bit
    # gradients)
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(O), 1e-30))) - (7 if dtype == "bf16" else 10))
    err = np.abs(o.cpu().double().numpy() - O)
    assert np.all(err <= TOL_OUT[t["q"].dtype] + 0.5 * ulp), f"{w.name}: max err {err.max():.3e}"
    e1 = float(err.max())
    e2 = assert_close_lse(lse.cpu(), L, w.name)
    say(f"    max|dO|={e1:.2e} max|dLSE|={e2:.2e}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_dropout_zero_rate_is_the_plain_forward_and_repeatable(dtype):
    """p = 0 keeps everything: fp16 gives the plain forward bit for bit; bf16 carries the
    probabilities into P V as hi + lo bf16 pairs in the dropout forward, so its O is the
    more accurate one (same LSE, O within the bf16 tolerance of the plain forward's)."""
    need_gpu()
    import exact_tiled_attention_amd as eta
    w = attn_inputs.prefill(1, 8, 2, 333, 333, 128, dtype, seed=81, causal=True)
    q, k, v = (to_dev(w.tensors[n]) for n in ("q", "k", "v"))
    o0, l0 = eta.attn_fwd(q, k, v, causal=True)
    o1, l1 = eta.attn_fwd_dropout(q, k, v, 0.0, 5, 0, causal=True)
    assert torch.equal(l0, l1)
    if dtype == "f16":
        assert torch.equal(o0, o1)
    else:
        O, _ = dense.forward(w.tensors["q"], w.tensors["k"], w.tensors["v"], w.params["scale"], True)
        e_plain = assert_close_out(o0.cpu(), O, TOL_OUT[torch.bfloat16], "plain")
        e_split = assert_close_out(o1.cpu(), O, TOL_OUT[torch.bfloat16], "dropout p=0")
        say(f"    bf16 max err: plain {e_plain:.2e}, dropout p=0 {e_split:.2e}")
    a, la = eta.attn_fwd_dropout(q, k, v, 0.2, 5, 7, causal=True)
    b, lb = eta.attn_fwd_dropout(q, k, v, 0.2, 5, 7, causal=True)
    c, _ = eta.attn_fwd_dropout(q, k, v, 0.2, 5, 8, causal=True)
    assert torch.equal(a, b) and torch.equal(la, l0) and not torch.equal(a, c)


def _dropout_grads(w, p, seed, offset, deterministic, dq_splits=1):
    """Backward from the oracle's dropout forward: O (rounded to the element type, as
    a forward stores it) and LSE (float32) come from oracle/dropout.py, so the test
    isolates the backward; both sides form D from the same stored O."""
    import exact_tiled_attention_amd as eta
    t, prm = w.tensors, w.params
    O, L = dropout.forward(t["q"], t["k"], t["v"], prm["scale"], prm["causal"], p, seed, offset)
    o = to_dev(torch.from_numpy(O).to(t["q"].dtype))
    lse = to_dev(torch.from_numpy(L).float())
    q, k, v, do = (to_dev(t[n]) for n in ("q", "k", "v", "do"))
    g = eta.attn_bwd(q, k, v, o, lse, do, scale=prm["scale"], causal=prm["causal"], dropout_p=p, seed=seed,
                     offset=offset, deterministic=deterministic, dq_splits=dq_splits)
    torch.cuda.synchronize()
    return tuple(x.cpu() for x in g)


@pytest.mark.parametrize("deterministic", [False, True])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk,p", [
    (1, 4, 2, 257, 193, 0.15),
    (1, 2, 2, 300, 100, 0.4),      # causal rows with no visible key
])
def test_dropout_backward_elementwise(deterministic, dtype, d, causal, B, Hq, Hkv, Sq, Sk, p):
    need_gpu()
    w = attn_inputs.prefill(B, Hq, Hkv, Sq, Sk, d, dtype, seed=900 + Sq + d, causal=causal, with_grad=True)
    t, prm = w.tensors, w.params
    seed, offset = 4242 + Sk, 1
    say(f"[dropout-bwd] {w.name} causal={causal} p={p} det={deterministic}")
    got = _dropout_grads(w, p, seed, offset, deterministic)
    ref = dropout.backward(t["q"], t["k"], t["v"], t["do"], prm["scale"], causal, p, seed, offset,
                           o_storage=t["q"].dtype)
    errs = [assert_close_out(g_, r_, TOL_GRAD, f"{w.name} {n}") for n, g_, r_ in zip(("dq", "dk", "dv"), got, ref)]
    say("    max err dq/dk/dv = " + " ".join(f"{e:.2e}" for e in errs))


def test_dropout_backward_deterministic_repeatable_and_split():
    need_gpu()
    w = attn_inputs.prefill(1, 8, 2, 500, 700, 128, "bf16", seed=91, causal=True, with_grad=True)
    a = _dropout_grads(w, 0.3, 77, 5, True, 4)
    b = _dropout_grads(w, 0.3, 77, 5, True, 4)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    t, prm = w.tensors, w.params
    ref = dropout.backward(t["q"], t["k"], t["v"], t["do"], prm["scale"], True, 0.3, 77, 5, o_storage=t["q"].dtype)
    for g_, r_ in zip(a, ref):
        assert_close_out(g_, r_, TOL_GRAD, w.name)


@pytest.mark.parametrize("deterministic", [False, True])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk,p", [
    (1, 4, 2, 257, 193, 0.15),     # query and key tails, GQA 2
    (1, 2, 2, 300, 100, 0.4),      # causal rows with few or no visible keys
    (2, 8, 2, 200, 333, 0.25),     # S_q < S_k, GQA 4
])
def test_dropout_training_chain_end_to_end(deterministic, dtype, d, causal, B, Hq, Hkv, Sq, Sk, p):
    """attn_fwd_dropout, then attn_bwd with the same dropout_p, seed and offset on the
    forward's own O and LSE, against the oracle's exact gradients (D from the oracle's
    O rounded to the element type, as a forward stores it)."""
    need_gpu()
    import exact_tiled_attention_amd as eta
    w = attn_inputs.prefill(B, Hq, Hkv, Sq, Sk, d, dtype, seed=950 + Sq + d, causal=causal, with_grad=True)
    t, prm = w.tensors, w.params
    seed, offset = 9090 + Sk, 4
    say(f"[dropout-chain] {w.name} causal={causal} p={p} det={deterministic}")
    q, k, v, do = (to_dev(t[n]) for n in ("q", "k", "v", "do"))
    o, lse = eta.attn_fwd_dropout(q, k, v, p, seed, offset, scale=prm["scale"], causal=causal)
    g = eta.attn_bwd(q, k, v, o, lse, do, scale=prm["scale"], causal=causal, dropout_p=p, seed=seed,
                     offset=offset, deterministic=deterministic)
    torch.cuda.synchronize()
    ref = dropout.backward(t["q"], t["k"], t["v"], t["do"], prm["scale"], causal, p, seed, offset,
                           o_storage=t["q"].dtype)
    errs = [assert_close_out(g_.cpu(), r_, TOL_GRAD, f"{w.name} {n}") for n, g_, r_ in zip(("dq", "dk", "dv"), g, ref)]
    say("    max err dq/dk/dv = " + " ".join(f"{e:.2e}" for e in errs))

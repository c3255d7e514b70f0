"""Pins of the oracle's backward: finite differences, identities, torch autograd in float64."""
import numpy as np
import pytest
import torch

from oracle import dense
from conftest import golden


def _rand(shape, seed):
    return np.random.default_rng(seed).normal(size=shape)


def _loss(q, k, v, do, scale, causal):
    O, _ = dense.forward(q, k, v, scale, causal)
    return float((O * do).sum())


@pytest.mark.parametrize("causal", [False, True])
def test_central_finite_differences(causal):
    B, Hq, Hkv, Sq, Sk, d = 1, 4, 2, 4, 5, 3
    q, k, v, do = _rand((B, Hq, Sq, d), 1), _rand((B, Hkv, Sk, d), 2), _rand((B, Hkv, Sk, d), 3), _rand((B, Hq, Sq, d), 4)
    scale = 0.6
    dq, dk, dv, _ = dense.backward(q, k, v, do, scale, causal)
    eps = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            fp = _loss(args["q"], args["k"], args["v"], do, scale, causal)
            args[name] = xm
            fm = _loss(args["q"], args["k"], args["v"], do, scale, causal)
            num[idx] = (fp - fm) / (2 * eps)
        assert np.abs(num - grad).max() < 1e-8, name


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_autograd_float64(causal):
    B, Hq, Hkv, S, d = 2, 6, 3, 17, 8
    q, k, v, do = _rand((B, Hq, S, d), 5), _rand((B, Hkv, S, d), 6), _rand((B, Hkv, S, d), 7), _rand((B, Hq, S, d), 8)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_() for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=0.3, enable_gqa=True)
    out.backward(torch.from_numpy(do))
    dq, dk, dv, _ = dense.backward(q, k, v, do, 0.3, causal)
    assert np.allclose(dq, tq.grad.numpy(), atol=1e-12)
    assert np.allclose(dk, tk.grad.numpy(), atol=1e-12)
    assert np.allclose(dv, tv.grad.numpy(), atol=1e-12)


def test_D_identity_masked_dS_and_unused_keys():
    B, H, Sq, Sk, d = 1, 2, 6, 9, 4
    q, k, v, do = _rand((B, H, Sq, d), 9), _rand((B, H, Sk, d), 10), _rand((B, H, Sk, d), 11), _rand((B, H, Sq, d), 12)
    scale = 0.5
    O, _ = dense.forward(q, k, v, scale, True)
    _, dk, dv, D = dense.backward(q, k, v, do, scale, True)
    assert np.allclose(D, (do * O).sum(-1), atol=1e-13)            # D_i = dO_i . O_i
    P = dense.probabilities(q, k, scale, True)
    dP = do @ np.swapaxes(v, -1, -2)
    dS = P * (dP - D[..., None])
    vis = dense.visible(Sq, Sk, True)
    assert np.all(dS[..., ~vis] == 0.0)
    # Under causal masking key S-1 is seen only by the last query row; with that row's
    # dO set to zero the key receives no gradient at all (dP = 0 and D = 0 there).
    q3, k3, v3, do3 = _rand((1, 2, 7, 4), 17), _rand((1, 2, 7, 4), 18), _rand((1, 2, 7, 4), 19), _rand((1, 2, 7, 4), 20)
    do3[:, :, -1] = 0.0
    _, dk3, dv3, _ = dense.backward(q3, k3, v3, do3, scale, True)
    assert np.all(dk3[:, :, -1] == 0.0) and np.all(dv3[:, :, -1] == 0.0)
    assert np.all(np.abs(dv3[:, :, :-1]).sum(-1) > 0)


def test_group_sum_example():
    g = golden("gqa_group_sum.json")["group_sum"]
    expanded = np.array(g["expanded"], float)
    grp = g["Hq"] // g["Hkv"]
    reduced = expanded.reshape(g["Hkv"], grp, -1).sum(1)
    assert reduced.tolist() == g["reduced"]
    # and the oracle's grouped dK equals the sum of per-query-head dK computed with
    # explicitly repeated K/V heads
    q, k, v, do = _rand((1, 6, 5, 3), 13), _rand((1, 2, 5, 3), 14), _rand((1, 2, 5, 3), 15), _rand((1, 6, 5, 3), 16)
    _, dk, dv, _ = dense.backward(q, k, v, do, 0.7, True)
    _, dke, dve, _ = dense.backward(q, np.repeat(k, 3, 1), np.repeat(v, 3, 1), do, 0.7, True)
    assert np.allclose(dk, dke.reshape(1, 2, 3, 5, 3).sum(2), atol=1e-14)
    assert np.allclose(dv, dve.reshape(1, 2, 3, 5, 3).sum(2), atol=1e-14)


def test_stored_output_D_reading():
    """D from the output as stored in a 16-bit type: equal to the exact gradient when
    the stored O is exact, and different by exactly the rounding term otherwise."""
    q, k, do = _rand((1, 2, 6, 4), 21), _rand((1, 2, 6, 4), 22), _rand((1, 2, 6, 4), 23)
    v = np.full((1, 2, 6, 4), 0.75)               # every O row is exactly 0.75
    for dt in (torch.float16, torch.bfloat16):
        exact = dense.backward(q, k, v, do, 0.5, True)
        stored = dense.backward(q, k, v, do, 0.5, True, o_storage=dt)
        for a, b in zip(exact, stored):
            assert np.allclose(a, b, atol=1e-13)
    v = _rand((1, 2, 6, 4), 24)
    O, _ = dense.forward(q, k, v, 0.5, True)
    _, _, _, D_exact = dense.backward(q, k, v, do, 0.5, True)
    _, _, _, D_st = dense.backward(q, k, v, do, 0.5, True, o_storage=torch.bfloat16)
    O_bf = torch.from_numpy(O).to(torch.bfloat16).double().numpy()
    assert np.allclose(D_st - D_exact, (do * (O_bf - O)).sum(-1), atol=1e-13)
    assert np.abs(D_st - D_exact).max() > 0

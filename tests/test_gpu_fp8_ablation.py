"""Scale granularity x incoherent processing on the fp8 forward (GPU quantiser and
forward, float64 oracle reference): "M4.6 - FlashAttention-3/4 Hardware Pipelines ...",
section 0x06 and its ablation table.  The output RMSE of each variant is printed; the
checks are the ones the pages support: every variant stays close to the reference,
and on the controlled outlier-channel geometry the transform lowers the error."""
import math

import numpy as np
import pytest
import torch

from oracle import dense
from gpu_common import need_gpu, say, to_dev

pytestmark = pytest.mark.gpu


def _variants(q, k, v, scale, seed):
    import exact_tiled_attention_amd as eta
    d = q.shape[-1]
    signs = to_dev(torch.from_numpy(np.random.default_rng(seed).choice([-1.0, 1.0], size=d).astype(np.float32)))
    ref, _ = dense.forward(q, k, v, scale, False)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    out = {}
    for per_tensor in (True, False):
        for had in (False, True):
            s = signs if had else None
            cq, dq = eta.fp8_quantize(qd, s, per_tensor=per_tensor)
            ck, dk = eta.fp8_quantize(kd, s, per_tensor=per_tensor)
            cv, dv = eta.fp8_quantize(vd, None, per_tensor=per_tensor)
            o, _ = eta.attn_fwd_fp8(cq, ck, cv, dq, dk, dv, scale=scale, o_dtype=torch.float32)
            torch.cuda.synchronize()
            name = ("tensor" if per_tensor else "block") + ("+hadamard" if had else "")
            out[name] = math.sqrt(np.mean((o.cpu().double().numpy() - ref) ** 2))
    o16, _ = eta.attn_fwd(qd, kd, vd, scale=scale)
    torch.cuda.synchronize()
    out["bf16"] = math.sqrt(np.mean((o16.cpu().double().numpy() - ref) ** 2))
    return out


def test_ablation_on_the_pages_distribution():
    """N(0,1) + N(0,100) Bernoulli(0.001) for Q, K, V (the distribution of the pages'
    ablation table)."""
    need_gpu()
    B, H, S, d = 1, 4, 1024, 128
    rng = np.random.default_rng(2024)
    def draw():
        x = rng.standard_normal((B, H, S, d)) + rng.normal(0, 10, (B, H, S, d)) * (rng.random((B, H, S, d)) < 1e-3)
        return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)
    q, k, v = draw(), draw(), draw()
    r = _variants(q, k, v, 1 / math.sqrt(d), 7)
    say("[fp8-ablation] pages' distribution RMSE: " + ", ".join(f"{k_} {v_:.3e}" for k_, v_ in r.items()))
    assert all(x < 5e-2 for x in r.values()), r


def test_ablation_on_the_outlier_channel_geometry():
    """Persistent +-10 excursions in channel 0 of Q and K (the pages' controlled
    fixture): the signed Hadamard spreads them and lowers the block-scale error."""
    need_gpu()
    B, H, S, d = 1, 4, 512, 128
    rng = np.random.default_rng(2025)
    q = rng.standard_normal((B, H, S, d))
    k = rng.standard_normal((B, H, S, d))
    v = rng.standard_normal((B, H, S, d))
    q[..., 0] += 10 * rng.choice([-1, 1], size=(B, H, S))
    k[..., 0] += 10 * rng.choice([-1, 1], size=(B, H, S))
    q, k, v = (torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16) for x in (q, k, v))
    r = _variants(q, k, v, 1 / math.sqrt(d), 8)
    say("[fp8-ablation] outlier-channel RMSE: " + ", ".join(f"{k_} {v_:.3e}" for k_, v_ in r.items()))
    assert r["block+hadamard"] < 0.7 * r["block"], r

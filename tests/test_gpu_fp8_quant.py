"""GPU parity of attn_fp8_quantize (E4M3 codes and descales, block or tensor scales,
optional incoherent transform) against the float64 oracle."""
import numpy as np
import pytest
import torch

import attn_inputs
from oracle import fp8
from gpu_common import need_gpu, say, to_dev

pytestmark = pytest.mark.gpu


def _signs(d, seed):
    return torch.from_numpy(np.random.default_rng(seed).choice([-1.0, 1.0], size=d).astype(np.float32))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("hadamard", [False, True])
@pytest.mark.parametrize("per_tensor", [False, True])
def test_quantize_matches_oracle(dtype, d, hadamard, per_tensor):
    need_gpu()
    import exact_tiled_attention_amd as eta
    B, H, S = 2, 3, 300
    x32 = attn_inputs.outlier_normal((B, H, S, d), 61 + d, 0)
    x = x32.to(torch.float16 if dtype == "f16" else torch.bfloat16)
    s = _signs(d, 62) if hadamard else None
    say(f"[fp8-quant] {dtype} d={d} hadamard={hadamard} per_tensor={per_tensor}")
    codes, desc = eta.fp8_quantize(to_dev(x), None if s is None else to_dev(s), per_tensor=per_tensor)
    torch.cuda.synchronize()
    xr = fp8.incoherent(x, s.numpy()) if hadamard else x.double().numpy()
    oc, od = fp8.quantize(xr, per_tensor=per_tensor)
    gd = desc.cpu().numpy()
    assert np.allclose(gd, od, rtol=2e-6, atol=0), np.abs(gd / od - 1).max()
    gc = codes.cpu().numpy()
    drow = gd[:, :, np.arange(S) // 128][..., None].astype(np.float64)
    back = fp8.decode(gc) * drow
    allowed = np.maximum(2 ** -4 * np.abs(xr), 2 ** -10 * drow) + 1e-5 * np.abs(xr).max()
    assert np.all(np.abs(back - xr) <= allowed)
    # The oracle rounds the exact quotient x / descale once; the kernel rounds its
    # float32 quotient (correctly rounded, so within 2^-24 relative of the exact one).
    # The two roundings can differ only where the exact quotient lies that close to an
    # E4M3 midpoint; the transform adds its own float32 error (the butterflies: 1e-5).
    # There either neighbour is accepted, with the sign of x.
    rel = 2.0 ** -23 if not hadamard else 1e-5
    u = xr / drow
    alt_code = fp8.encode_rne_sat(np.copysign(fp8.rounding_alternative(np.abs(u), rel), u))
    assert np.all((gc == oc) | (gc == alt_code))
    # (ambiguous quotients are not rare here: with 8- or 11-bit inputs, 448 x / amax is
    # often exactly an E4M3 midpoint, and the rounded descale then decides the side;
    # the bound below only guards against a systematic error)
    same = float((gc == oc).mean())
    say(f"    identical codes: {same:.5f}")
    assert same >= 0.99


def test_incoherent_quantized_scores_stay_close():
    """Q R and K R quantised with the same signs give scores close to Q K^T (the
    identity holds before quantisation; after it, within the E4M3 error)."""
    need_gpu()
    import exact_tiled_attention_amd as eta
    d = 128
    q = attn_inputs.normal((1, 1, 256, d), 63, 0, "bf16")
    k = attn_inputs.normal((1, 1, 256, d), 63, 1, "bf16")
    s = to_dev(_signs(d, 64))
    cq, dq = eta.fp8_quantize(to_dev(q), s)
    ck, dk = eta.fp8_quantize(to_dev(k), s)
    torch.cuda.synchronize()
    qd = fp8.dequantized(cq.cpu(), dq.cpu())
    kd = fp8.dequantized(ck.cpu(), dk.cpu())
    ref = q.double().numpy() @ np.swapaxes(k.double().numpy(), -1, -2)
    got = qd @ np.swapaxes(kd, -1, -2)
    rel = np.sqrt(np.mean((got - ref) ** 2) / np.mean(ref ** 2))
    assert rel < 0.08, rel

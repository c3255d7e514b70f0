"""Pins of the E4M3FN codebook and the quantised forward's step order."""
import math

import numpy as np
import pytest
import torch

import attn_inputs
from oracle import dense, fp8
from conftest import golden


def test_codebook_matches_torch_float8_for_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = fp8.decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours)) and nan.sum() == 2      # 0x7F and 0xFF
    assert np.array_equal(ref[~nan], ours[~nan])
    g = golden("fp8_e4m3.json")
    assert np.nanmax(ours) == g["max_finite"]
    assert ours[ours > 0].min() == g["min_positive_subnormal"] == 2.0 ** -9


def test_encoder_matches_torch_rne_cast():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.normal(size=20000) * 30, rng.uniform(-448, 448, 20000),
                        rng.uniform(-0.02, 0.02, 20000)])
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = fp8.encode_rne_sat(x.astype(np.float32).astype(np.float64))
    assert np.array_equal(ref, ours)
    # exact midpoints between neighbouring codes round to the even code
    vals = fp8._POS_VALUES
    mids = (vals[:-1] + vals[1:]) / 2
    got = fp8.encode_rne_sat(mids)
    assert np.all(got % 2 == 0)
    # saturation instead of NaN beyond the largest finite value
    assert fp8.decode(fp8.encode_rne_sat(np.array([1e6, -500.0]))).tolist() == [448.0, -448.0]


def _small_inputs(seed=7, B=1, H=2, S=200, d=32):
    w = attn_inputs.fp8_prefill(B, H, H, S, S, d, seed=seed)
    return w


@pytest.mark.parametrize("block_c", [32, 64, 128])
def test_without_probability_rounding_steps_reduce_to_dense(block_c):
    """Removing the P rounding, the 2^8 offset, the scale placement and the LSE shift
    must reproduce the dense definition on the dequantised inputs exactly (fp64)."""
    w = _small_inputs()
    t, p = w.tensors, w.params
    O, L = fp8.forward(t["q8"], t["k8"], t["v8"], t["q_scale"], t["k_scale"], t["v_scale"], p["scale"],
                       block_c=block_c, prob_round=lambda u: u)
    Qd = fp8.dequantized(t["q8"], t["q_scale"])
    Kd = fp8.dequantized(t["k8"], t["k_scale"])
    Vd = fp8.dequantized(t["v8"], t["v_scale"])
    Od, Ld = dense.forward(Qd, Kd, Vd, p["scale"], False)
    assert np.allclose(O, Od, atol=1e-11, rtol=1e-11)
    assert np.allclose(L, Ld, atol=1e-11)


def test_two_to_the_eight_cancels_exactly():
    rng = np.random.default_rng(3)
    s = rng.normal(size=50) * 4
    v = rng.normal(size=(50, 3))
    m = s.max()
    u = 2.0 ** 8 * np.exp(s - m)
    plain = np.exp(s - m)
    assert np.allclose((u @ v) / u.sum(), (plain @ v) / plain.sum(), atol=1e-15)
    assert abs((m + math.log(u.sum()) - 8 * math.log(2)) - (m + math.log(plain.sum()))) < 1e-14


def test_quantised_output_is_close_to_dense_and_frames_differ_little():
    w = _small_inputs(seed=11, S=256, d=64)
    t, p = w.tensors, w.params
    args = (t["q8"], t["k8"], t["v8"], t["q_scale"], t["k_scale"], t["v_scale"], p["scale"])
    O, L = fp8.forward(*args, block_c=64)
    Of, _ = fp8.forward(*args, block_c=64, frame="final")
    Ou, Lu = fp8.forward(*args, block_c=64, prob_round=lambda u: u)
    rmse = np.sqrt(np.mean((O - Ou) ** 2))
    assert 0 < rmse < 5e-2
    assert np.sqrt(np.mean((Of - Ou) ** 2)) < 5e-2
    assert np.allclose(L, Lu, atol=1e-12)          # the denominator uses unrounded u


def test_descales_enter_before_the_row_max():
    """Planting the mistake of applying the Q/K descales after the softmax changes O."""
    w = _small_inputs(seed=13, S=128, d=32)
    t, p = w.tensors, w.params
    ones = lambda x: torch.ones_like(x)
    O_right, _ = fp8.forward(t["q8"], t["k8"], t["v8"], t["q_scale"], t["k_scale"], t["v_scale"], p["scale"],
                             prob_round=lambda u: u)
    O_wrong, _ = fp8.forward(t["q8"], t["k8"], t["v8"], ones(t["q_scale"]), ones(t["k_scale"]), t["v_scale"],
                             p["scale"], prob_round=lambda u: u)
    assert np.abs(O_right - O_wrong).max() > 1e-2


def test_rounding_alternative_band():
    vals = fp8._POS_VALUES
    mids = 0.5 * (vals[1:-1] + vals[2:])
    alt = fp8.rounding_alternative(mids, 1e-6)
    rn = fp8.round_e4m3(mids)
    assert np.all(alt != rn)                                    # exact midpoints: both neighbours
    far = 0.5 * (vals[1:-1] + mids)                             # a quarter-step from a value
    assert np.array_equal(fp8.rounding_alternative(far, 1e-6), fp8.round_e4m3(far))


def test_envelope_is_zero_without_ambiguity_and_bounds_a_flip():
    w = _small_inputs(seed=17, S=128, d=32)
    t, p = w.tensors, w.params
    args = (t["q8"], t["k8"], t["v8"], t["q_scale"], t["k_scale"], t["v_scale"], p["scale"])
    O, L = fp8.forward(*args, block_c=64)
    O0, L0, E0 = fp8.forward(*args, block_c=64, envelope_rel=0.0)
    assert np.array_equal(O, O0) and np.all(E0 == 0)
    O1, _, E1 = fp8.forward(*args, block_c=64, envelope_rel=0.05)
    # rounding every ambiguous probability the other way stays inside the envelope
    Of, _ = fp8.forward(*args, block_c=64, prob_round=lambda u: fp8.rounding_alternative(u, 0.05))
    assert np.all(np.abs(Of - O1) <= E1 + 1e-12)
    assert E1.max() > 0

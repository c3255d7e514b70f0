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
@pytest.mark.parametrize("causal,Sq,Sk", [(False, 200, 200), (True, 200, 200), (True, 150, 260), (True, 260, 150)])
def test_without_probability_rounding_steps_reduce_to_dense(block_c, causal, Sq, Sk):
    """Removing the P rounding, the 2^8 offset, the scale placement and the LSE shift
    must reproduce the dense definition on the dequantised inputs exactly (fp64),
    causal masks included (S_q > S_k: rows that see no key get O = 0, LSE = -inf)."""
    w = attn_inputs.fp8_prefill(1, 2, 2, Sq, Sk, 32, seed=7)
    t, p = w.tensors, w.params
    O, L = fp8.forward(t["q8"], t["k8"], t["v8"], t["q_scale"], t["k_scale"], t["v_scale"], p["scale"],
                       block_c=block_c, prob_round=lambda u: u, causal=causal)
    Qd = fp8.dequantized(t["q8"], t["q_scale"])
    Kd = fp8.dequantized(t["k8"], t["k_scale"])
    Vd = fp8.dequantized(t["v8"], t["v_scale"])
    Od, Ld = dense.forward(Qd, Kd, Vd, p["scale"], causal)
    assert np.allclose(O, Od, atol=1e-11, rtol=1e-11)
    assert np.array_equal(np.isneginf(L), np.isneginf(Ld))
    fin = np.isfinite(Ld)
    assert np.allclose(L[fin], Ld[fin], atol=1e-11)
    if causal and Sq > Sk:
        assert np.isneginf(L).any() and np.all(O[np.isneginf(L)] == 0)


# ---------------------------------------------------------------------------------
# Hand-derived pins of the probability rounding ([HW] section 0x06, "Why The Source
# Raises Softmax Probabilities By 2^8" and "Derive Where Every Scale Must Enter").
# Each case uses head dimension 1 and hand-picked E4M3 codes, so every score is known
# exactly; the expected O and LSE are written out below from the stated step order:
# u = 2^8 e^(S - m) in the running-max frame, p8 = E4M3(u) (values typed in by hand
# from the codebook: sign, 4 exponent bits with bias 7, 3 fraction bits), l from the
# unrounded u, o += dV_j (p8 . V_j), O = o / l, LSE = m + ln l - 8 ln 2.

C_ZERO, C_ONE, C_TWO, C_FOUR = 0x00, 0x38, 0x40, 0x48     # +0, 1.0, 2.0, 4.0
C_MINUS_ONE, C_MINUS_EIGHT = 0xB8, 0xD0                     # -1.0, -8.0


def _codes(vals):
    return np.asarray(vals, dtype=np.uint8).reshape(1, 1, -1, 1)


def _descales(vals):
    return np.asarray(vals, dtype=np.float32).reshape(1, 1, -1)


def _run(k_codes, v_codes, v_scale, block_c, scale_rows=128, frame="running", prob_round=fp8.round_e4m3):
    nk = len(k_codes)
    nblk = -(-nk // scale_rows)
    O, L = fp8.forward(_codes([C_ONE]), _codes(k_codes), _codes(v_codes), _descales([1.0]),
                       _descales([1.0] * nblk), _descales(v_scale), 1.0, block_c=block_c,
                       scale_rows=scale_rows, frame=frame, prob_round=prob_round)
    return float(O[0, 0, 0, 0]), float(L[0, 0, 0])


def test_pin_offset_keeps_a_small_probability():
    """Scores (0, -8) in one tile.  u = (256, 256 e^-8 = 0.08588); the E4M3 value next
    to 0.08588 is 1.375 * 2^-4 = 0.0859375, so the second key survives.  Without the
    offset, e^-8 = 3.4e-4 is below half the smallest subnormal (2^-10) and rounds to 0."""
    O, L = _run([C_ZERO, C_MINUS_EIGHT], [C_ONE, C_TWO], [1.0], block_c=2)
    e8 = math.exp(-8.0)
    l = 256.0 * (1.0 + e8)
    want_O = (256.0 * 1.0 + 0.0859375 * 2.0) / l
    want_L = math.log(l) - 8 * math.log(2.0)          # m = 0
    assert abs(O - want_O) < 1e-13 and abs(L - want_L) < 1e-13
    # the planted mistake -- rounding e^(S - m) first, then applying 2^8 -- loses key 1
    wrong, _ = _run([C_ZERO, C_MINUS_EIGHT], [C_ONE, C_TWO], [1.0], block_c=2,
                    prob_round=lambda u: 256.0 * fp8.round_e4m3(u / 256.0))
    assert abs(wrong - 256.0 / l) < 1e-13 and abs(wrong - want_O) > 5e-4
    # the denominator sums the unrounded u: summing p8 instead moves O and LSE
    assert abs(want_O - (256.0 + 0.171875) / (256.0 + 0.0859375)) > 1e-7


def test_pin_running_frame_when_the_max_moves():
    """Scores (0, -2 | 2, 1) in two tiles of two keys, V = (1, 2, 4, -1).
    Tile 1 (m = 0): u = (256, 256 e^-2 = 34.646) -> p8 = (256, 36)   (step 4 in [32, 64)).
    Tile 2 (m = 2): alpha = e^-2; u = (256, 256 e^-1 = 94.176) -> p8 = (256, 96)
    (step 8 in [64, 128)).  Rounding in the final frame (m = 2) instead rounds tile 1's
    (256 e^-2, 256 e^-4) = (34.646, 4.689) to (36, 4.5) (step 0.5 in [4, 8))."""
    k = [C_ZERO, 0xC0, C_TWO, C_ONE]                        # q = 1: S = (0, -2, 2, 1)
    v = [C_ONE, C_TWO, C_FOUR, C_MINUS_ONE]
    O, L = _run(k, v, [1.0], block_c=2)
    a = math.exp(-2.0)
    l = a * (256.0 + 256.0 * math.exp(-2.0)) + (256.0 + 256.0 * math.exp(-1.0))
    o = a * (256.0 * 1.0 + 36.0 * 2.0) + (256.0 * 4.0 + 96.0 * -1.0)
    assert abs(O - o / l) < 1e-13
    assert abs(L - (2.0 + math.log(l) - 8 * math.log(2.0))) < 1e-13
    # the final-frame variant: tile 1 contributes 36 * 1 + 4.5 * 2 in the final scale
    Of, Lf = _run(k, v, [1.0], block_c=2, frame="final")
    o_final = (36.0 * 1.0 + 4.5 * 2.0) + (256.0 * 4.0 + 96.0 * -1.0)
    assert abs(Of - o_final / l) < 1e-13 and abs(Lf - L) < 1e-13
    assert abs(Of - O) > 1e-3
    # one tile of four keys (m = 2 from the start) is the final frame as well
    O4, _ = _run(k, v, [1.0], block_c=4)
    assert abs(O4 - Of) < 1e-13


def test_pin_per_tile_value_descale():
    """Scores (0, -1), one key per tile and per scale block, V codes (1, 1) with value
    descales (0.5, 3.0).  Tile 1: u = 256 -> p8 = 256, o = 0.5 * 256 = 128.  Tile 2
    (m stays 0): u = 256 e^-1 = 94.176 -> p8 = 96, o = 128 + 3.0 * 96 = 416."""
    O, L = _run([C_ZERO, C_MINUS_ONE], [C_ONE, C_ONE], [0.5, 3.0], block_c=1, scale_rows=1)
    l = 256.0 * (1.0 + math.exp(-1.0))
    assert abs(O - 416.0 / l) < 1e-13
    assert abs(L - (math.log(l) - 8 * math.log(2.0))) < 1e-13
    # one descale for both tiles (either one) gives a different O
    for dv in (0.5, 3.0):
        Ow, _ = _run([C_ZERO, C_MINUS_ONE], [C_ONE, C_ONE], [dv, dv], block_c=1, scale_rows=1)
        assert abs(Ow - 416.0 / l) > 0.1


def test_pin_key_descales_enter_before_the_max():
    """K codes (1, 2) with key descales (1.0, 0.25): the scores are (1, 0.5), so key 0
    holds the maximum although its code is the smaller one.  u = (256, 256 e^-0.5 =
    155.27) -> p8 = (256, 160) (step 16 in [128, 256)), V = (1, -1)."""
    O, L = fp8.forward(_codes([C_ONE]), _codes([C_ONE, C_TWO]), _codes([C_ONE, C_MINUS_ONE]), _descales([1.0]),
                       _descales([1.0, 0.25]), _descales([1.0, 1.0]), 1.0, block_c=1, scale_rows=1)
    l = 256.0 * (1.0 + math.exp(-0.5))
    assert abs(float(O[0, 0, 0, 0]) - (256.0 - 160.0) / l) < 1e-13
    assert abs(float(L[0, 0, 0]) - (1.0 + math.log(l) - 8 * math.log(2.0))) < 1e-13


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


def test_pin_causal_row_sees_only_its_keys():
    """Causal, S_q = S_k = 2 (one tile): row 0 sees key 0 only, so its O is V_0 (the
    value 1.0 exactly: u = 256, p8 = 256) and LSE = S_00 = 0; row 1 sees both keys,
    scores (0, -1): u = (256, 94.18) -> p8 = (256, 96)."""
    q = _codes([C_ONE, C_ONE])
    O, L = fp8.forward(q, _codes([C_ZERO, C_MINUS_ONE]), _codes([C_ONE, C_TWO]), _descales([1.0]),
                       _descales([1.0]), _descales([1.0]), 1.0, block_c=2, causal=True)
    assert O[0, 0, 0, 0] == 1.0 and L[0, 0, 0] == 0.0
    l = 256.0 * (1.0 + math.exp(-1.0))
    assert abs(O[0, 0, 1, 0] - (256.0 * 1.0 + 96.0 * 2.0) / l) < 1e-13


@pytest.mark.parametrize("causal,Sq,Sk", [(False, 96, 80), (True, 96, 96), (True, 120, 70)])
def test_backward_with_exact_o_and_lse_is_the_dense_gradient(causal, Sq, Sk):
    """Given the exact forward's O and LSE on the dequantised operands, the fp8 backward
    is the (pinned) exact gradient of the dense definition on those operands."""
    w = attn_inputs.fp8_prefill(1, 4, 2, Sq, Sk, 16, seed=21)
    t, p = w.tensors, w.params
    Qd = fp8.dequantized(t["q8"], t["q_scale"])
    Kd = fp8.dequantized(t["k8"], t["k_scale"])
    Vd = fp8.dequantized(t["v8"], t["v_scale"])
    dO = np.random.default_rng(3).standard_normal(Qd.shape)
    O, L = dense.forward(Qd, Kd, Vd, p["scale"], causal)
    got = fp8.backward(t["q8"], t["k8"], t["v8"], t["q_scale"], t["k_scale"], t["v_scale"], O, L, dO,
                       p["scale"], causal)
    want = dense.backward(Qd, Kd, Vd, dO, p["scale"], causal)[:3]
    for g_, w_ in zip(got, want):
        assert np.allclose(g_, w_, atol=1e-9, rtol=1e-9)


def test_backward_descales_matter():
    """Planted mistakes: ignoring the key descale in S, or the value descale in dP,
    changes the gradients."""
    w = attn_inputs.fp8_prefill(1, 2, 2, 64, 200, 16, seed=22)
    t, p = w.tensors, w.params
    Qd = fp8.dequantized(t["q8"], t["q_scale"])
    Kd = fp8.dequantized(t["k8"], t["k_scale"])
    Vd = fp8.dequantized(t["v8"], t["v_scale"])
    dO = np.random.default_rng(4).standard_normal(Qd.shape)
    O, L = dense.forward(Qd, Kd, Vd, p["scale"], False)
    args = (t["q8"], t["k8"], t["v8"], t["q_scale"])
    right = fp8.backward(*args, t["k_scale"], t["v_scale"], O, L, dO, p["scale"])
    for ks, vs in ((torch.ones_like(t["k_scale"]), t["v_scale"]), (t["k_scale"], torch.ones_like(t["v_scale"]))):
        with np.errstate(all="ignore"):
            wrong = fp8.backward(*args, ks, vs, O, L, dO, p["scale"])
        assert any(not np.allclose(a, b, atol=1e-2) for a, b in zip(right, wrong))

"""Pins of the oracle's software exp2 ([HW] section 0x09: range reduction plus a
degree-3 polynomial for 2^f), fitted here as the relative-error minimax."""
import numpy as np

from oracle import exp2soft

# The page's float32 maximum relative error for its own degree-3 coefficients: a
# minimax fit of the same degree cannot do worse.
PAGE_DEG3_F32_MAX_REL = 8.77e-5


def _rel_err(coef, f):
    return (np.polyval(np.asarray(coef)[::-1], f) - np.exp2(f)) / np.exp2(f)


def test_float32_error_against_exact_exp2():
    x = np.linspace(-30.0, 8.0, 2_000_001).astype(np.float32)
    y = exp2soft.soft_exp2_f32(x).astype(np.float64)
    rel = np.abs(y / np.exp2(x.astype(np.float64)) - 1.0)
    assert rel.max() <= 7.6e-5
    assert rel.max() < PAGE_DEG3_F32_MAX_REL


def test_fit_equioscillates():
    # the minimax error alternates in sign with equal magnitude at deg + 2 points,
    # among them both ends of [0, 1]
    coef, emax = exp2soft.fit_coefficients()
    f = np.linspace(0.0, 1.0, 200_001)
    err = _rel_err(coef, f)
    assert abs(abs(err[0]) - emax) < 1e-3 * emax and abs(abs(err[-1]) - emax) < 1e-3 * emax
    d = np.diff(err)
    ext = np.concatenate([[0], np.nonzero(d[:-1] * d[1:] < 0)[0] + 1, [len(f) - 1]])
    assert len(ext) == exp2soft.DEGREE + 2
    vals = err[ext]
    assert np.all(np.sign(vals[1:]) == -np.sign(vals[:-1]))
    assert np.all(np.abs(np.abs(vals) - emax) < 1e-3 * emax)


def test_fit_is_locally_optimal():
    # no small change of the coefficients lowers the maximum relative error (a fit of
    # the absolute error, a least-squares fit or a sign slip in the exchange would)
    coef, emax = exp2soft.fit_coefficients()
    f = np.linspace(0.0, 1.0, 20_001)
    base = np.abs(_rel_err(coef, f)).max()
    rng = np.random.default_rng(7)
    for _ in range(200):
        step = rng.standard_normal(len(coef)) * rng.choice([1e-7, 1e-6, 1e-5])
        assert np.abs(_rel_err(coef + step, f)).max() >= base * (1 - 1e-9)


def test_special_values_and_exact_scaling():
    y = exp2soft.soft_exp2_f32(np.array([-np.inf, -1e30, -150.0, -151.5], dtype=np.float32))
    assert np.all(y == 0.0)
    c0 = exp2soft.coefficients_f32()[0]
    n = np.arange(-100, 9, dtype=np.float32)
    # at integers f = 0: the polynomial gives c0 and the exponent scaling is exact
    assert np.array_equal(exp2soft.soft_exp2_f32(n), np.ldexp(np.float32(c0), n.astype(np.int32)))
    # beats the degree-3 Taylor polynomial of 2^f at 0 by more than an order of magnitude
    f = np.linspace(0.0, 1.0, 10_001)
    ln2 = np.log(2.0)
    taylor = 1 + ln2 * f + (ln2 * f) ** 2 / 2 + (ln2 * f) ** 3 / 6
    assert np.abs(taylor / np.exp2(f) - 1).max() > 10 * exp2soft.fit_coefficients()[1]

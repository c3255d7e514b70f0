"""Pins of the dropout oracle (oracle/dropout.py): the generator against its published
known-answer vectors, the dropout forward and backward against the dense definition,
statistics of the decisions and central finite differences."""
import numpy as np
import pytest

from oracle import dense, dropout


# Known-answer vectors of Philox4x32-10 published with the generator's reference
# implementation (Random123, "kat_vectors"): counter words, key words, output words.
KAT = [
    ((0x00000000, 0x00000000, 0x00000000, 0x00000000), (0x00000000, 0x00000000),
     (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
    ((0xffffffff, 0xffffffff, 0xffffffff, 0xffffffff), (0xffffffff, 0xffffffff),
     (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
    ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
     (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1)),
]


@pytest.mark.parametrize("ctr,key,out", KAT)
def test_philox_known_answers(ctr, key, out):
    got = dropout.philox4x32_10(np.array(ctr, dtype=np.uint32), np.array(key, dtype=np.uint32))
    assert [int(x) for x in got] == list(out)


def test_philox_vectorised_equals_scalar():
    rng = np.random.default_rng(5)
    ctr = rng.integers(0, 2 ** 32, size=(7, 4), dtype=np.uint64).astype(np.uint32)
    key = np.array([0x1234567, 0x89abcdef], dtype=np.uint32)
    batch = dropout.philox4x32_10(ctr, key)
    for i in range(7):
        assert np.array_equal(batch[i], dropout.philox4x32_10(ctr[i], key))


def _inputs(B, Hq, Hkv, Sq, Sk, d, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, Sq, d))
    k = rng.standard_normal((B, Hkv, Sk, d))
    v = rng.standard_normal((B, Hkv, Sk, d))
    do = rng.standard_normal((B, Hq, Sq, d))
    return q, k, v, do


@pytest.mark.parametrize("causal", [False, True])
def test_zero_rate_is_the_dense_definition(causal):
    q, k, v, do = _inputs(1, 4, 2, 9, 13, 8, 1)
    O, L = dropout.forward(q, k, v, 0.3, causal, 0.0, seed=7)
    O2, L2 = dense.forward(q, k, v, 0.3, causal)
    assert np.allclose(O, O2, atol=1e-13) and np.array_equal(np.isneginf(L), np.isneginf(L2))
    g = dropout.backward(q, k, v, do, 0.3, causal, 0.0, seed=7)
    g2 = dense.backward(q, k, v, do, 0.3, causal)[:3]
    for a, b in zip(g, g2):
        assert np.allclose(a, b, atol=1e-12)


def test_lse_is_undropped_and_output_changes():
    q, k, v, _ = _inputs(1, 2, 2, 16, 40, 8, 2)
    O, L = dropout.forward(q, k, v, 0.35, False, 0.25, seed=11)
    O2, L2 = dense.forward(q, k, v, 0.35, False)
    assert np.allclose(L, L2, atol=1e-13)
    assert np.abs(O - O2).max() > 1e-3


def test_keep_rate_and_scale():
    p = 0.3
    keep = dropout.keep_mask(0, 1, 4, np.arange(256), 512, p, seed=123, offset=9)
    n = keep.size
    frac = keep.mean()
    sigma = np.sqrt(p * (1 - p) / n)
    assert abs(frac - (1 - p)) < 5 * sigma
    assert dropout.threshold(0.0) == 0 and dropout.threshold(0.5) == 2 ** 31
    # with V = 1 every row of O is sum_k P_k Z_k, whose mean over rows is close to 1
    q, k, _, _ = _inputs(1, 1, 1, 400, 300, 4, 3)
    v = np.ones((1, 1, 300, 2))
    O, _ = dropout.forward(q, k, v, 0.1, False, p, seed=5)
    assert abs(O[..., 0].mean() - 1.0) < 0.02


def test_decisions_are_coordinate_stable():
    full = dropout.keep_mask(1, 3, 4, np.arange(50), 37, 0.4, seed=2 ** 40 + 17, offset=3)
    rows = np.array([49, 0, 17, 18])
    part = dropout.keep_mask(1, 3, 4, rows, 37, 0.4, seed=2 ** 40 + 17, offset=3)
    assert np.array_equal(part, full[rows])
    # the decision of key j only depends on the Philox word j % 4 of counter j // 4
    longer = dropout.keep_mask(1, 3, 4, np.arange(50), 64, 0.4, seed=2 ** 40 + 17, offset=3)
    assert np.array_equal(longer[:, :37], full)
    other = dropout.keep_mask(1, 3, 4, np.arange(50), 37, 0.4, seed=2 ** 40 + 17, offset=4)
    assert not np.array_equal(other, full)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_finite_differences(causal):
    q, k, v, do = _inputs(1, 2, 1, 5, 7, 4, 4)
    scale, p, seed = 0.7, 0.4, 99
    g = dropout.backward(q, k, v, do, scale, causal, p, seed)

    def f(q_, k_, v_):
        return (dropout.forward(q_, k_, v_, scale, causal, p, seed)[0] * do).sum()

    eps = 1e-6
    for which, grad in ((0, g[0]), (1, g[1]), (2, g[2])):
        base = [q, k, v]
        num = np.zeros_like(base[which])
        it = np.nditer(base[which], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            plus = [x.copy() for x in base]
            minus = [x.copy() for x in base]
            plus[which][idx] += eps
            minus[which][idx] -= eps
            num[idx] = (f(*plus) - f(*minus)) / (2 * eps)
        assert np.allclose(grad, num, atol=1e-6), (which, np.abs(grad - num).max())

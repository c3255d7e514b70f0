"""Pins of the online state algebra against the pages' printed traces and laws."""
import itertools
import math

import numpy as np
import pytest

from oracle import state as st
from conftest import golden


def _close(a, b, digits):
    return np.allclose(np.asarray(a, float), np.asarray(b, float), atol=0.6 * 10.0 ** (-digits), rtol=0)


def test_three_block_trace_printed_values():
    g = golden("three_block_trace.json")
    x = np.array(g["scores"], float)
    V = np.array(g["values"], float)
    parts = [st.of_set(x[b], V[b]) for b in g["blocks"]]
    first = st.merge(parts[0], parts[1])
    a = g["after_first_merge"]
    assert first.m == a["m"]
    assert _close(first.l, a["l"], 6) and _close(first.u, a["u"], 6)
    fin = st.fold_sequential(parts)
    f = g["final"]
    assert fin.m == f["m"]
    assert abs(fin.l - f["l"]) < 1e-14
    assert np.allclose(fin.u, f["u"], atol=1e-14, rtol=0)
    O, lse = st.finalize(fin)
    assert np.allclose(O, f["O"], atol=1e-14, rtol=0)
    assert abs(lse - f["LSE"]) < 1e-13
    assert fin.n == len(x)


def test_two_block_trace_printed_values():
    g = golden("two_block_trace.json")
    A = st.of_set(g["block_a"]["scores"], g["block_a"]["values"])
    B = st.of_set(g["block_b"]["scores"], g["block_b"]["values"])
    for s, ref in ((A, g["block_a"]), (B, g["block_b"]), (st.merge(A, B), g["union"])):
        assert s.m == ref["m"]
        assert _close(s.l, ref["l"], 6)
        assert _close(s.u, ref["u"], 6)
        assert _close(st.finalize(s)[0], ref["O"], 6)
        # u = l * O (the two coordinates describe one row)
        assert np.allclose(s.u, s.l * st.finalize(s)[0], atol=1e-14)


def test_naive_block_softmax_is_wrong_and_merge_is_right():
    g = golden("naive_block_trap.json")
    naive = st.naive_block_softmax(g["scores"], g["values"], g["blocks"])
    assert naive[0] == pytest.approx(g["naive"], abs=1e-12)
    parts = [st.of_set(np.array(g["scores"], float)[b], np.array(g["values"], float)[b]) for b in g["blocks"]]
    O, _ = st.finalize(st.fold_sequential(parts))
    assert O[0] == pytest.approx(g["correct"], abs=1e-9)


def test_row_trace_with_masked_tail():
    g = golden("row_trace_masked_tail.json")
    x = np.array(g["scores"], float)
    x[g["allowed_keys"]:] = -np.inf
    V = np.zeros((len(x), 1))
    tiles = st.chunked(x, V, g["tile"])
    assert not tiles[2].valid                   # fully masked tile is the identity
    s0 = tiles[0]
    assert s0.m == g["after_tile_0"]["m"] and _close(s0.l, g["after_tile_0"]["l"], 12)
    assert _close(math.exp(s0.m - max(s0.m, tiles[1].m)), g["alpha_old"], 12)
    s1 = st.merge(s0, tiles[1])
    assert s1.m == g["after_tile_1"]["m"] and _close(s1.l, g["after_tile_1"]["l"], 12)
    s2 = st.merge(s1, tiles[2])
    assert (s2.m, s2.l, s2.n) == (s1.m, s1.l, s1.n)


def _rand_row(seed, n, dv):
    r = np.random.default_rng(seed)
    return r.normal(size=n) * 3, r.normal(size=(n, dv))


@pytest.mark.parametrize("n,chunk", [(1, 1), (7, 3), (64, 16), (257, 32)])
def test_identity_commutativity_associativity_partition(n, chunk):
    x, V = _rand_row(n, n, 3)
    dense = st.of_set(x, V)
    parts = st.chunked(x, V, chunk)
    e = st.empty(3)
    for p in parts:
        for a, b in ((st.merge(e, p), p), (st.merge(p, e), p)):
            assert (a.valid, a.m, a.l, a.n) == (b.valid, b.m, b.l, b.n) and np.array_equal(a.u, b.u)
    trees = [st.fold_sequential(parts), st.fold_balanced(parts),
             st.fold_sequential(parts[::-1]),
             st.fold_balanced([parts[i] for i in np.random.default_rng(1).permutation(len(parts))])]
    O_dense, L_dense = st.finalize(dense)
    for t in trees:
        O, L = st.finalize(t)
        assert t.n == n
        assert np.allclose(O, O_dense, atol=1e-12, rtol=0) and abs(L - L_dense) < 1e-12
    if len(parts) >= 2:
        ab = st.merge(parts[0], parts[1])
        ba = st.merge(parts[1], parts[0])
        assert ab.m == ba.m and abs(ab.l - ba.l) < 1e-13 and np.allclose(ab.u, ba.u, atol=1e-13)


def test_three_coordinate_forms_agree():
    x, V = _rand_row(5, 40, 4)
    parts = st.chunked(x, V, 7)
    O_ref, L_ref = st.finalize(st.fold_sequential(parts))
    norm = [(p.valid, p.m, p.l, st.finalize(p)[0]) for p in parts]
    acc = (False, -math.inf, 0.0, np.zeros(4))
    for p in norm:
        acc = st.merge_normalized(acc, p)
    assert np.allclose(acc[3], O_ref, atol=1e-12)
    lse_acc = (-math.inf, np.zeros(4))
    for p in parts:
        O, L = st.finalize(p)
        lse_acc = st.merge_lse(lse_acc, (L, O))
    assert abs(lse_acc[0] - L_ref) < 1e-12 and np.allclose(lse_acc[1], O_ref, atol=1e-12)


def test_online_normalizer_and_bounds():
    x = [-np.inf, 0.5, -2.0, -np.inf, 4.0, 3.0]
    m, d = st.online_normalizer(x)
    finite = np.array([v for v in x if v != -np.inf])
    assert m == finite.max() and abs(d - np.exp(finite - m).sum()) < 1e-14
    assert 1.0 <= d <= len(finite)
    assert st.online_normalizer([-np.inf, -np.inf]) is None


def test_all_masked_row_policy():
    s = st.of_set([-np.inf] * 4, np.ones((4, 2)))
    assert not s.valid
    O, L = st.finalize(s)
    assert np.array_equal(O, np.zeros(2)) and L == -math.inf


def test_finite_precision_witnesses():
    g = golden("finite_precision.json")
    f32 = np.float32
    a, b, c = (f32(v) for v in g["float32_order"]["a"])
    assert float((a + b) + c) == g["float32_order"]["left_first"]
    a, b, c = (f32(v) for v in g["float32_order"]["b"])
    assert float((a + b) + c) == g["float32_order"]["left_first_b"]
    w = g["binary16_row"]
    h = [np.float16(v) for v in w["payloads"]]
    seq = np.float16(0)
    for v in h:
        seq = np.float16(seq + v)
    assert float(seq) / len(h) == w["sequential"]
    lvl = h
    while len(lvl) > 1:
        lvl = [np.float16(lvl[i] + lvl[i + 1]) for i in range(0, len(lvl), 2)]
    assert float(lvl[0]) / len(h) == w["balanced"]
    assert sum(float(v) for v in h) / len(h) == w["exact"]

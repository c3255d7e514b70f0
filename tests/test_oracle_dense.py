"""Pins of the dense float64 oracle: brute force, closed forms, invariants, library cross-checks."""
import math

import numpy as np
import pytest
import torch

from oracle import dense, state as st, tiles
from conftest import golden


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).normal(size=shape) * scale


def _brute_force(Q, K, V, scale, causal):
    """Pure-Python loops over one (b, h) pair; bottom-right causal alignment."""
    Sq, d = len(Q), len(Q[0])
    Sk, dv = len(K), len(V[0])
    delta = Sk - Sq
    O, L = [], []
    for i in range(Sq):
        s = []
        for k in range(Sk):
            if causal and k > i + delta:
                continue
            s.append((k, scale * sum(Q[i][t] * K[k][t] for t in range(d))))
        if not s:
            O.append([0.0] * dv)
            L.append(-math.inf)
            continue
        m = max(v for _, v in s)
        z = sum(math.exp(v - m) for _, v in s)
        O.append([sum(math.exp(v - m) / z * V[k][c] for k, v in s) for c in range(dv)])
        L.append(m + math.log(z))
    return np.array(O), np.array(L)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Sq,Sk,Hq,Hkv", [(5, 7, 2, 1), (7, 5, 2, 2), (6, 6, 4, 2), (1, 9, 3, 3)])
def test_brute_force(causal, Sq, Sk, Hq, Hkv):
    d, B = 3, 2
    q, k, v = _rand((B, Hq, Sq, d), 1), _rand((B, Hkv, Sk, d), 2), _rand((B, Hkv, Sk, d), 3)
    scale = 0.7
    O, L = dense.forward(q, k, v, scale, causal)
    g = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            Ob, Lb = _brute_force(q[b, h].tolist(), k[b, h // g].tolist(), v[b, h // g].tolist(), scale, causal)
            assert np.allclose(O[b, h], Ob, atol=1e-13)
            assert np.array_equal(np.isinf(L[b, h]), np.isinf(Lb))
            fin = np.isfinite(Lb)
            assert np.allclose(L[b, h][fin], Lb[fin], atol=1e-13)


def test_rectangular_causal_masks_are_bottom_right():
    for c in golden("rect_causal_masks.json")["cases"]:
        m = dense.visible(c["Sq"], c["Sk"], True).astype(int)
        assert m.tolist() == c["bottom_right"]
        assert m.tolist() != c["top_left"]


def test_rows_sum_to_one_and_uniform_v():
    q, k = _rand((1, 2, 9, 4), 4), _rand((1, 2, 11, 4), 5)
    for causal in (False, True):
        P = dense.probabilities(q, k, 0.5, causal)
        assert np.allclose(P.sum(-1), 1.0, atol=1e-14)
        v = np.full((1, 2, 11, 3), 2.5)
        O, _ = dense.forward(q, k, v, 0.5, causal)
        assert np.allclose(O, 2.5, atol=1e-14)


def test_scale_zero_gives_mean_and_log_count():
    q, k, v = _rand((1, 1, 6, 4), 6), _rand((1, 1, 8, 4), 7), _rand((1, 1, 8, 2), 8)
    O, L = dense.forward(q, k, v, 0.0, True)
    delta = 8 - 6
    for i in range(6):
        n = i + delta + 1
        assert np.allclose(O[0, 0, i], v[0, 0, :n].mean(0), atol=1e-14)
        assert abs(L[0, 0, i] - math.log(n)) < 1e-14


def test_single_key_and_first_causal_row():
    q, k, v = _rand((1, 1, 4, 3), 9), _rand((1, 1, 1, 3), 10), _rand((1, 1, 1, 3), 11)
    O, L = dense.forward(q, k, v, 0.3, False)
    assert np.allclose(O[0, 0], v[0, 0, 0], atol=1e-15)
    assert np.allclose(L[0, 0], 0.3 * q[0, 0] @ k[0, 0, 0], atol=1e-14)
    q, k, v = _rand((1, 1, 5, 3), 12), _rand((1, 1, 5, 3), 13), _rand((1, 1, 5, 3), 14)
    O, L = dense.forward(q, k, v, 0.3, True)
    assert np.allclose(O[0, 0, 0], v[0, 0, 0], atol=1e-15)
    assert abs(L[0, 0, 0] - 0.3 * q[0, 0, 0] @ k[0, 0, 0]) < 1e-14


def test_key_permutation_invariance():
    q, k, v = _rand((1, 2, 5, 4), 15), _rand((1, 2, 9, 4), 16), _rand((1, 2, 9, 3), 17)
    perm = np.random.default_rng(0).permutation(9)
    O1, L1 = dense.forward(q, k, v, 0.5, False)
    O2, L2 = dense.forward(q, k[:, :, perm], v[:, :, perm], 0.5, False)
    assert np.allclose(O1, O2, atol=1e-13) and np.allclose(L1, L2, atol=1e-13)


def test_gqa_direct_map_equals_repetition_and_wrong_map_differs():
    g = golden("gqa_group_sum.json")["head_map"]
    assert [h // (g["Hq"] // g["Hkv"]) for h in range(g["Hq"])] == g["kv_of_q"]
    q, k, v = _rand((2, 6, 7, 5), 18), _rand((2, 2, 7, 5), 19), _rand((2, 2, 7, 5), 20)
    O, L = dense.forward(q, k, v, 0.4, True)
    rep_k, rep_v = np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1)
    Or, Lr = dense.forward(q, rep_k, rep_v, 0.4, True)
    assert np.array_equal(O, Or) and np.array_equal(L, Lr)
    wrong = [h % 2 for h in range(6)]
    Ow, _ = dense.forward(q, k[:, wrong], v[:, wrong], 0.4, True)
    assert np.abs(Ow - O).max() > 1e-2


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_sdpa_float64(causal):
    q, k, v = _rand((2, 8, 33, 16), 21), _rand((2, 2, 33, 16), 22), _rand((2, 2, 33, 16), 23)
    O, L = dense.forward(q, k, v, 0.25, causal)
    t = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        is_causal=causal, scale=0.25, enable_gqa=True)
    assert np.allclose(O, t.numpy(), atol=1e-12)
    S = 0.25 * torch.from_numpy(q) @ torch.from_numpy(np.repeat(k, 4, axis=1)).transpose(-1, -2)
    if causal:
        S = S.masked_fill(torch.ones(33, 33, dtype=torch.bool).triu(1), -math.inf)
    assert np.allclose(L, torch.logsumexp(S, -1).numpy(), atol=1e-12)


def test_all_masked_rows_policy():
    q, k, v = _rand((1, 1, 5, 3), 24), _rand((1, 1, 2, 3), 25), _rand((1, 1, 2, 3), 26)
    O, L = dense.forward(q, k, v, 1.0, True)    # S_q > S_k: rows 0..2 see nothing
    assert np.array_equal(O[0, 0, :3], np.zeros((3, 3))) and np.all(L[0, 0, :3] == -np.inf)
    assert np.all(np.isfinite(L[0, 0, 3:]))


def test_split_kv_fold_equals_dense_decode():
    """An associative merge of per-chunk (m, l, u) states equals the full softmax."""
    q, kc, vc = _rand((3, 4, 1, 8), 27), _rand((3, 2, 40, 8), 28), _rand((3, 2, 40, 8), 29)
    lens = np.array([40, 17, 1])
    O, L = dense.decode(q, kc, vc, lens, 0.35)
    for b in range(3):
        for h in range(4):
            x = 0.35 * kc[b, h // 2, :lens[b]] @ q[b, h, 0]
            for chunk in (1, 4, 16):
                parts = st.chunked(x, vc[b, h // 2, :lens[b]], chunk)
                for tree in (st.fold_sequential(parts), st.fold_balanced(parts)):
                    Ot, Lt = st.finalize(tree)
                    assert np.allclose(Ot, O[b, h, 0], atol=1e-12) and abs(Lt - L[b, h, 0]) < 1e-12


def test_causal_tile_census_matches_printed_counts():
    for c in golden("causal_tiles.json")["cases"]:
        got = tiles.census(c["Sq"], c["Sk"], c["Br"], c["Bc"], c["delta"])
        for key in ("full", "partial", "skipped", "visited", "visited_cells", "allowed_cells"):
            if key in c:
                assert got[key] == c[key], key
        if "visits_per_query_tile_first" in c:
            per = tiles.visited_per_query_tile(c["Sq"], c["Sk"], c["Br"], c["Bc"], c["delta"])
            assert per[0] == c["visits_per_query_tile_first"] and per[-1] == c["visits_per_query_tile_last"]
            assert sum(per) == c["visited"]

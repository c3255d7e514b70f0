"""Pins of the oracle's packed variable-length forward, paged-cache decode and packed
launch census (CPU)."""
import numpy as np

import attn_inputs
from conftest import golden
from oracle import dense, tiles


def _rng(seed):
    return np.random.default_rng(seed)


def test_census_matches_printed_packed_fixture():
    c = golden("varlen_census.json")["case"]
    got = tiles.varlen_census(c["seqlens_q"], c["seqlens_k"], c["Br"], c["max_seqlen_q"], c["Hq"])
    for key in ("launched", "active", "full", "tail", "row_slots", "valid_rows"):
        assert got[key] == c[key], key
    assert got["launched"] - got["active"] == c["early_return"]


def _pack(x):
    """[B, H, S, d] -> token-major [B*S, H, d] (all sequences of length S)."""
    B, H, S, d = x.shape
    return x.transpose(0, 2, 1, 3).reshape(B * S, H, d)


def test_equal_lengths_reduce_to_the_padded_forward():
    r = _rng(1)
    B, Hq, Hkv, S, d = 3, 4, 2, 37, 16
    q, k, v = (r.standard_normal((B, h, S, d)) for h in (Hq, Hkv, Hkv))
    cu = np.arange(B + 1) * S
    for causal in (False, True):
        O, L = dense.forward(q, k, v, 0.3, causal)
        Ov, Lv = dense.forward_varlen(_pack(q), _pack(k), _pack(v), cu, cu, 0.3, causal)
        assert np.allclose(Ov, _pack(O), rtol=0, atol=1e-13)
        assert np.allclose(Lv, L.transpose(1, 0, 2).reshape(Hq, B * S), rtol=0, atol=1e-13)


def test_sequences_are_independent_and_use_their_own_causal_alignment():
    r = _rng(2)
    Hq, Hkv, d = 4, 1, 8
    sq, sk = [5, 0, 9, 3], [7, 4, 2, 0]
    cq, ck = np.concatenate([[0], np.cumsum(sq)]), np.concatenate([[0], np.cumsum(sk)])
    q = r.standard_normal((cq[-1], Hq, d))
    k = r.standard_normal((ck[-1], Hkv, d))
    v = r.standard_normal((ck[-1], Hkv, d))
    O, L = dense.forward_varlen(q, k, v, cq, ck, 0.5, True)
    for b in range(4):
        if sq[b] == 0:
            continue
        qb = q[cq[b]:cq[b + 1]].transpose(1, 0, 2)[None]
        kb = k[ck[b]:ck[b + 1]].transpose(1, 0, 2)[None]
        vb = v[ck[b]:ck[b + 1]].transpose(1, 0, 2)[None]
        Ob, Lb = dense.forward(qb, kb, vb, 0.5, True)
        assert np.allclose(O[cq[b]:cq[b + 1]], Ob[0].transpose(1, 0, 2), atol=1e-13, equal_nan=True)
        assert np.array_equal(np.isneginf(L[:, cq[b]:cq[b + 1]]), np.isneginf(Lb[0]))
    # a sequence with no keys: every row takes the empty-row policy
    assert np.all(O[cq[3]:cq[4]] == 0) and np.all(np.isneginf(L[:, cq[3]:cq[4]]))
    # sequence 2 (S_q = 9 > S_k = 2): rows 0..6 see nothing under bottom-right alignment
    assert np.all(np.isneginf(L[:, cq[2]:cq[2] + 7])) and np.all(np.isfinite(L[:, cq[2] + 7:cq[3]]))
    # perturbing sequence 2 leaves sequence 0 unchanged
    k2 = k.copy()
    k2[ck[2]:ck[3]] += 5.0
    O2, _ = dense.forward_varlen(q, k2, v, cq, ck, 0.5, True)
    assert np.array_equal(O2[cq[0]:cq[1]], O[cq[0]:cq[1]])


def test_paged_gather_inverts_a_random_page_scatter():
    r = _rng(3)
    B, H, P, d = 3, 2, 16, 8
    lens = np.array([33, 16, 1])
    maxp = 3
    contiguous = r.standard_normal((B, H, maxp * P, d))
    npages = B * maxp + 2
    perm = r.permutation(npages)
    pages = r.standard_normal((npages, H, P, d))          # unused pages hold noise
    bt = np.zeros((B, maxp), dtype=np.int64)
    for b in range(B):
        for i in range(maxp):
            bt[b, i] = perm[b * maxp + i]
            pages[bt[b, i]] = contiguous[b, :, i * P:(i + 1) * P]
    got = dense.gather_pages(pages, bt, lens)
    for b in range(B):
        assert np.array_equal(got[b], contiguous[b, :, :lens[b]])


def test_paged_decode_equals_contiguous_decode():
    r = _rng(4)
    B, Hq, Hkv, P, d = 2, 4, 2, 8, 16
    lens = np.array([19, 8])
    maxp = 3
    q = r.standard_normal((B, Hq, 1, d))
    kc = r.standard_normal((B, Hkv, maxp * P, d))
    vc = r.standard_normal((B, Hkv, maxp * P, d))
    npages = B * maxp
    perm = r.permutation(npages)
    kp = np.zeros((npages, Hkv, P, d)); vp = np.zeros((npages, Hkv, P, d))
    bt = perm.reshape(B, maxp)
    for b in range(B):
        for i in range(maxp):
            kp[bt[b, i]] = kc[b, :, i * P:(i + 1) * P]
            vp[bt[b, i]] = vc[b, :, i * P:(i + 1) * P]
    O, L = dense.decode_paged(q, kp, vp, bt, lens, 0.25)
    O2, L2 = dense.decode(q, kc, vc, lens, 0.25)
    assert np.array_equal(O, O2) and np.array_equal(L, L2)

"""Attention dropout with coordinate-stable counter-based replay (float64 oracle).

Test infrastructure only (see the package docstring).

The contract ([FA2] section 0x03I; [IO] section 0x0DF):
  1. m, l and the shifted numerators are those of the undropped softmax, so the LSE
     is unchanged by dropout;
  2. a keep decision is drawn for every probability element;
  3. the decision is applied before P V,
  4. with the reciprocal keep probability as the scale of what is kept;
  5. the backward regenerates the same decisions, so the draw must be a function of
     the element's coordinates (batch, head, query row, key), not of the order in
     which a kernel visits tiles.

The pages leave the generator and the coordinate map open.  This library's reading:
Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2,
3", SC 2011), a counter-based generator whose output is a pure function of (counter,
key).  Element (b, h, i, j) of a call with seed s and offset f uses

    counter = (j // 4, i, b * H_q + h, f),   key = (s mod 2^32, s div 2^32)

and word j % 4 of the output; it is kept iff that word is >= floor(p 2^32), so the
keep probability is 1 - floor(p 2^32) / 2^32, and kept values are scaled by 1 / (1 - p).
With dropout, for Z = keep / (1 - p) (element-wise):

    O = (P * Z) V                       (P the undropped, normalised probabilities)
    dV = (P * Z)^T dO,   dP = Z * (dO V^T),   D_i = sum_k P_ik dP_ik = dO_i . O_i,
    dS = P * (dP - D),   dQ = scale dS K,   dK = scale dS^T Q.
"""
from __future__ import annotations

import numpy as np

from .dense import _f64, _round_to, visible

_M0 = np.uint64(0xD2511F53)
_M1 = np.uint64(0xCD9E8D57)
_W0 = np.uint32(0x9E3779B9)
_W1 = np.uint32(0xBB67AE85)
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(ctr, key):
    """Philox4x32 with 10 rounds.  ctr uint32 [..., 4], key uint32 [..., 2] (broadcast).

    Each round multiplies words 0 and 2 by the two round constants (full 64-bit
    products), and the new state is (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1,
    lo(M0 c0)); the key is bumped by the two Weyl constants between rounds.
    """
    c = np.array(ctr, dtype=np.uint32)
    k = np.array(key, dtype=np.uint32)
    c0, c1, c2, c3 = (c[..., i].astype(np.uint64) for i in range(4))
    k0 = np.broadcast_to(k[..., 0], c0.shape).astype(np.uint32)
    k1 = np.broadcast_to(k[..., 1], c0.shape).astype(np.uint32)
    for r in range(10):
        if r:   # the key bump wraps modulo 2^32
            k0 = ((k0.astype(np.uint64) + np.uint64(_W0)) & _MASK32).astype(np.uint32)
            k1 = ((k1.astype(np.uint64) + np.uint64(_W1)) & _MASK32).astype(np.uint32)
        p0 = _M0 * c0
        p1 = _M1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c0 = hi1 ^ c1 ^ k0.astype(np.uint64)
        c1 = lo1
        c2 = hi0 ^ c3 ^ k1.astype(np.uint64)
        c3 = lo0
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def threshold(p_drop: float) -> int:
    """Words below this value are dropped: floor(p 2^32), capped to 2^32 - 1."""
    return min(int(np.floor(float(p_drop) * 2.0 ** 32)), 2 ** 32 - 1)


def keep_mask(b: int, h: int, Hq: int, rows, Sk: int, p_drop: float, seed: int, offset: int) -> np.ndarray:
    """Boolean [len(rows), Sk] keep decisions of (batch b, query head h) for the given
    query rows, from the coordinate map in the module docstring."""
    rows = np.asarray(rows, dtype=np.int64)
    ngrp = (Sk + 3) // 4
    jj, ii = np.meshgrid(np.arange(ngrp, dtype=np.uint64), rows.astype(np.uint64))
    ctr = np.stack([jj, ii, np.full_like(jj, b * Hq + h), np.full_like(jj, offset)], axis=-1)
    ctr = (ctr & np.uint64(0xFFFFFFFF)).astype(np.uint32)
    s = int(seed) & (2 ** 64 - 1)
    key = np.array([s & 0xFFFFFFFF, s >> 32], dtype=np.uint32)
    words = philox4x32_10(ctr, key).reshape(len(rows), ngrp * 4)[:, :Sk]
    return words >= np.uint32(threshold(p_drop))


def _head(Qh, Kh, Vh, scale, vis, keep, rp):
    S = scale * (Qh @ Kh.T)
    S = np.where(vis, S, -np.inf)
    m = S.max(axis=1, initial=-np.inf)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    E = np.exp(S - m_safe[:, None])
    l = E.sum(axis=1)
    P = np.divide(E, l[:, None], out=np.zeros_like(E), where=~empty[:, None])
    Z = keep * rp
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, l)))
    return P, Z, (P * Z) @ Vh, lse


def forward(q, k, v, scale: float, causal: bool, p_drop: float, seed: int, offset: int = 0):
    """Dropout forward: (O [B,Hq,Sq,dv], LSE [B,Hq,Sq]) float64; LSE is undropped."""
    Q, K, V = _f64(q), _f64(k), _f64(v)
    B, Hq, Sq, _ = Q.shape
    Hkv, Sk = K.shape[1], K.shape[2]
    g = Hq // Hkv
    vis = visible(Sq, Sk, causal)
    rp = 1.0 / (1.0 - float(p_drop))
    O = np.empty((B, Hq, Sq, V.shape[3]))
    LSE = np.empty((B, Hq, Sq))
    for b in range(B):
        for h in range(Hq):
            keep = keep_mask(b, h, Hq, np.arange(Sq), Sk, p_drop, seed, offset)
            _, _, O[b, h], LSE[b, h] = _head(Q[b, h], K[b, h // g], V[b, h // g], float(scale), vis, keep, rp)
    return O, LSE


def backward(q, k, v, do, scale: float, causal: bool, p_drop: float, seed: int, offset: int = 0,
             o_storage=None):
    """Gradients of the dropout forward with the same decisions: (dQ, dK, dV) float64.
    ``o_storage`` as in dense.backward (D from the stored, rounded O)."""
    Q, K, V, dO = _f64(q), _f64(k), _f64(v), _f64(do)
    B, Hq, Sq, _ = Q.shape
    Hkv, Sk = K.shape[1], K.shape[2]
    g = Hq // Hkv
    vis = visible(Sq, Sk, causal)
    rp = 1.0 / (1.0 - float(p_drop))
    s = float(scale)
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    for b in range(B):
        for h in range(Hq):
            kv = h // g
            keep = keep_mask(b, h, Hq, np.arange(Sq), Sk, p_drop, seed, offset)
            P, Z, Oh, _ = _head(Q[b, h], K[b, kv], V[b, kv], s, vis, keep, rp)
            dV[b, kv] += (P * Z).T @ dO[b, h]
            dP = Z * (dO[b, h] @ V[b, kv].T)
            if o_storage is None:
                D = (P * dP).sum(axis=1)
            else:
                D = (dO[b, h] * _round_to(Oh, o_storage)).sum(axis=1)
            dS = P * (dP - D[:, None])
            dQ[b, h] = s * (dS @ K[b, kv])
            dK[b, kv] += s * (dS.T @ Q[b, h])
    return dQ, dK, dV

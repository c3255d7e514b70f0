"""Dense float64 attention: the plain definition the tiled kernels must reach.

Test infrastructure only (see the package docstring).

Forward, per batch item b and query head h, with kv(h) = h // (H_q / H_kv)
([FA2] section 0x06A, the direct head map):

    S      = scale * Q_h K_kv(h)^T                    (float64)
    S[i,k] = -inf where the cell is not visible       ([IO] 0x02A: mask before softmax)
    m_i    = max_k S[i,k]
    P      = exp(S - m) / sum_k exp(S - m)            ([IO] 0x06B-C safe softmax)
    O      = P V_kv(h)
    LSE_i  = m_i + ln sum_k exp(S[i,k] - m_i)         ([IO] 0x09E; [FA2] 0x02D)

Causal visibility is k <= i + delta with delta = S_k - S_q, the bottom-right
alignment ([FA2] 0x05.1F).  A row with no visible key (possible only when
S_q > S_k under causal masking) takes the declared empty-row policy: O = 0,
LSE = -inf, and it contributes nothing to any gradient ([FA2] 0x02F).

Backward ([FA2] 0x06.1A; [IO] 0x0DB, no dropout):

    dV = P^T dO,   dP = dO V^T,   D_i = sum_k P_ik dP_ik,
    dS = P * (dP - D),   dQ = scale dS K,   dK = scale dS^T Q,

and for grouped heads dK, dV of a K/V head are the sums over its query heads
([FA2] 0x06E).
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    """Widen a torch tensor or array to a float64 numpy array (no other change)."""
    if hasattr(x, "detach"):
        x = x.detach().cpu()
        if x.dtype.is_floating_point:
            x = x.double()
        x = x.numpy()
    return np.asarray(x, dtype=np.float64)


def _round_to(x, dtype):
    """Round float64 values to a 16-bit storage type (torch's round-to-nearest-even)."""
    import torch
    return torch.from_numpy(np.asarray(x, dtype=np.float64)).to(dtype).double().numpy()


def visible(sq: int, sk: int, causal: bool, rows=None) -> np.ndarray:
    """Boolean [len(rows), sk]: True where query row i may see key k."""
    rows = np.arange(sq) if rows is None else np.asarray(rows)
    keys = np.arange(sk)
    if not causal:
        return np.ones((len(rows), sk), dtype=bool)
    delta = sk - sq
    return keys[None, :] <= rows[:, None] + delta


def _head_forward(Qh, Kh, Vh, scale, mask):
    S = scale * (Qh @ Kh.T)
    S = np.where(mask, S, -np.inf)
    m = S.max(axis=1, initial=-np.inf)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    E = np.exp(S - m_safe[:, None])          # masked cells give exp(-inf) = 0
    l = E.sum(axis=1)
    P = np.divide(E, l[:, None], out=np.zeros_like(E), where=~empty[:, None])
    O = P @ Vh
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, l)))
    return O, lse, P


def forward(q, k, v, scale: float, causal: bool = False, rows=None, heads=None):
    """Dense attention.

    q [B,Hq,Sq,d], k/v [B,Hkv,Sk,d] (torch or numpy, any float dtype).
    ``rows``: optional query-row subset (indices into Sq); ``heads``: optional list of
    (b, h) pairs to evaluate (others are left as NaN).
    Returns (O [B,Hq,R,dv] float64, LSE [B,Hq,R] float64).
    """
    Q, K, V = _f64(q), _f64(k), _f64(v)
    B, Hq, Sq, _ = Q.shape
    Hkv, Sk = K.shape[1], K.shape[2]
    assert Hq % Hkv == 0, "H_q must be a multiple of H_kv"
    g = Hq // Hkv
    rows = np.arange(Sq) if rows is None else np.asarray(rows)
    mask = visible(Sq, Sk, causal, rows)
    O = np.full((B, Hq, len(rows), V.shape[3]), np.nan)
    LSE = np.full((B, Hq, len(rows)), np.nan)
    pairs = [(b, h) for b in range(B) for h in range(Hq)] if heads is None else heads
    s = float(scale)
    for b, h in pairs:
        kv = h // g
        O[b, h], LSE[b, h], _ = _head_forward(Q[b, h][rows], K[b, kv], V[b, kv], s, mask)
    return O, LSE


def probabilities(q, k, scale: float, causal: bool = False):
    """The full probability tensor P [B,Hq,Sq,Sk] (small shapes only)."""
    Q, K = _f64(q), _f64(k)
    B, Hq, Sq, _ = Q.shape
    Hkv, Sk = K.shape[1], K.shape[2]
    g = Hq // Hkv
    mask = visible(Sq, Sk, causal)
    P = np.zeros((B, Hq, Sq, Sk))
    for b in range(B):
        for h in range(Hq):
            _, _, P[b, h] = _head_forward(Q[b, h], K[b, h // g], np.zeros((Sk, 1)), float(scale), mask)
    return P


def backward(q, k, v, do, scale: float, causal: bool = False, heads=None, o_storage=None):
    """Gradients of ``forward`` contracted with dO.

    Returns (dQ [B,Hq,Sq,d], dK [B,Hkv,Sk,d], dV [B,Hkv,Sk,dv], D [B,Hq,Sq]) in float64.
    ``heads``: optional list of (b, h_kv) pairs; only their query groups are evaluated
    (the rest of dQ/dK/dV is NaN).

    ``o_storage``: None gives the exact gradient (D = rowsum(P * dP)).  A torch dtype
    (float16 / bfloat16) forms D = rowsum(dO * O_stored) from the forward output
    rounded (to nearest even) to that storage type: the backward reads the O that the
    forward wrote in the element type ([FA2] 0x03H: O is written in the input dtype;
    0x06.1D: the preprocessing pass reads O and dO to form D).
    """
    Q, K, V, dO = _f64(q), _f64(k), _f64(v), _f64(do)
    B, Hq, Sq, _ = Q.shape
    Hkv, Sk = K.shape[1], K.shape[2]
    g = Hq // Hkv
    mask = visible(Sq, Sk, causal)
    s = float(scale)
    dQ = np.full_like(Q, np.nan)
    dK = np.full_like(K, np.nan)
    dV = np.full_like(V, np.nan)
    Dout = np.full((B, Hq, Sq), np.nan)
    pairs = [(b, kv) for b in range(B) for kv in range(Hkv)] if heads is None else heads
    for b, kv in pairs:
        dK[b, kv] = 0.0
        dV[b, kv] = 0.0
        for h in range(kv * g, (kv + 1) * g):
            _, _, P = _head_forward(Q[b, h], K[b, kv], V[b, kv], s, mask)
            dV[b, kv] += P.T @ dO[b, h]
            dP = dO[b, h] @ V[b, kv].T
            if o_storage is None:
                D = (P * dP).sum(axis=1)
            else:
                O_st = _round_to(P @ V[b, kv], o_storage)
                D = (dO[b, h] * O_st).sum(axis=1)
            dS = P * (dP - D[:, None])
            dQ[b, h] = s * (dS @ K[b, kv])
            dK[b, kv] += s * (dS.T @ Q[b, h])
            Dout[b, h] = D
    return dQ, dK, dV, Dout


def decode(q, k_cache, v_cache, seqlens, scale: float, batches=None):
    """One-query decode over per-sequence prefixes of a padded cache.

    q [B,Hq,1,d]; k_cache/v_cache [B,Hkv,Smax,d]; seqlens int [B].  Sequence b attends
    to keys 0..seqlens[b]-1 with no other mask (for S_q = 1 the bottom-right causal
    rule sees every cached key).  Returns (O [B,Hq,1,dv], LSE [B,Hq,1]) float64.
    """
    Q, K, V = _f64(q), _f64(k_cache), _f64(v_cache)
    lens = np.asarray(seqlens.cpu() if hasattr(seqlens, "cpu") else seqlens).astype(np.int64)
    B, Hq = Q.shape[:2]
    O = np.full((B, Hq, 1, V.shape[3]), np.nan)
    LSE = np.full((B, Hq, 1), np.nan)
    for b in (range(B) if batches is None else batches):
        n = int(lens[b])
        O[b:b + 1], LSE[b:b + 1] = forward(Q[b:b + 1], K[b:b + 1, :, :n], V[b:b + 1, :, :n], scale, False)
    return O, LSE


def _seq_lengths(cu):
    cu = np.asarray(cu.cpu() if hasattr(cu, "cpu") else cu).astype(np.int64)
    return cu, cu[1:] - cu[:-1]


def forward_varlen(q, k, v, cu_q, cu_k, scale: float, causal: bool = False, seqs=None):
    """Packed variable-length forward ([FA2] section 0x06F: each packed sequence has
    its own query and key extents, causal alignment and tile classes).

    q [total_q, Hq, d], k/v [total_k, Hkv, d] token-major; cu_q, cu_k int [B+1]
    cumulative offsets.  Sequence b is the dense definition above on its own rows
    cu_q[b] .. cu_q[b+1]-1 and keys cu_k[b] .. cu_k[b+1]-1.
    Returns (O [total_q, Hq, dv], LSE [Hq, total_q]) float64.
    """
    Q, K, V = _f64(q), _f64(k), _f64(v)
    cq, nq = _seq_lengths(cu_q)
    ck, nk = _seq_lengths(cu_k)
    O = np.full((Q.shape[0], Q.shape[1], V.shape[2]), np.nan)
    LSE = np.full((Q.shape[1], Q.shape[0]), np.nan)
    for b in (range(len(nq)) if seqs is None else seqs):
        qb = Q[cq[b]:cq[b + 1]].transpose(1, 0, 2)[None]        # [1, Hq, Sq_b, d]
        kb = K[ck[b]:ck[b + 1]].transpose(1, 0, 2)[None]
        vb = V[ck[b]:ck[b + 1]].transpose(1, 0, 2)[None]
        ob, lb = forward(qb, kb, vb, scale, causal)
        O[cq[b]:cq[b + 1]] = ob[0].transpose(1, 0, 2)
        LSE[:, cq[b]:cq[b + 1]] = lb[0]
    return O, LSE


def gather_pages(pages, block_table, seqlens):
    """Logical K (or V) rows of each sequence from a paged pool.

    pages [num_pages, H, P, d]; block_table int [B, max_pages]: logical page i of
    sequence b is physical page block_table[b, i]; key j of sequence b is row j % P of
    page block_table[b, j // P].  Returns a list of [H, seqlens[b], d] arrays.
    """
    X = _f64(pages)
    bt = np.asarray(block_table.cpu() if hasattr(block_table, "cpu") else block_table).astype(np.int64)
    lens = np.asarray(seqlens.cpu() if hasattr(seqlens, "cpu") else seqlens).astype(np.int64)
    P = X.shape[2]
    out = []
    for b in range(len(lens)):
        n = int(lens[b])
        npg = -(-n // P)
        rows = [X[bt[b, i]] for i in range(npg)]                 # each [H, P, d]
        full = np.concatenate(rows, axis=1) if rows else np.zeros((X.shape[1], 0, X.shape[3]))
        out.append(full[:, :n])
    return out


def decode_paged(q, k_pages, v_pages, block_table, seqlens, scale: float):
    """One-query decode over a paged K/V pool: the contiguous decode above applied to
    the gathered logical rows of each sequence.  Returns (O [B,Hq,1,dv], LSE [B,Hq,1])."""
    Q = _f64(q)
    Ks = gather_pages(k_pages, block_table, seqlens)
    Vs = gather_pages(v_pages, block_table, seqlens)
    B, Hq = Q.shape[:2]
    O = np.full((B, Hq, 1, Vs[0].shape[2] if Vs else Q.shape[3]), np.nan)
    LSE = np.full((B, Hq, 1), np.nan)
    for b in range(B):
        O[b:b + 1], LSE[b:b + 1] = forward(Q[b:b + 1], Ks[b][None], Vs[b][None], scale, False)
    return O, LSE


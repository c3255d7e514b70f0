"""E4M3FN arithmetic and the quantised attention forward.  Test infrastructure only.

Codebook ([HW] section 0x06, "E4M3 Names The Operand"): one sign bit, four exponent
bits (bias 7), three fraction bits; finite-only, largest magnitude 448, smallest
positive subnormal 2^-9; the all-ones exponent with all-ones fraction is NaN.

Quantised forward ([HW] 0x06, "Derive Where Every Scale Must Enter" and "Why The
Source Raises Softmax Probabilities By 2^8"), per batch item, query head and K/V
tile j taken in ascending key order:

    S     = scale * dQ_i * dK_j * (Q8 K8_j^T)          (descales before the row max)
    m_new = max(m, rowmax S),  alpha = exp(m - m_new)
    u     = 2^8 exp(S - m_new)                         (float, unrounded)
    p8    = E4M3(u)                                    (round to nearest even, saturating)
    l     = alpha l + rowsum(u)                        (denominator from unrounded u)
    o     = alpha o + dV_j * (p8 V8_j)                 (per-tile V descale)
    O     = o / l,   LSE = m + ln l - 8 ln 2.

Parity of this quantised output is unpinned by printed values: the pages print no
result for this input distribution.  What is pinned: the codebook against an
independent float8 implementation, the exact 2^8 cancellation, and that with the
probability rounding removed the steps reproduce the dense definition.
"""
from __future__ import annotations

import math

import numpy as np

from . import dense

E4M3_MAX = 448.0
PROB_OFFSET_LOG2 = 8


def decode_code(c: int) -> float:
    """Value of one E4M3FN byte from its bit fields."""
    c = int(c) & 0xFF
    sign = -1.0 if c & 0x80 else 1.0
    e = (c >> 3) & 0xF
    f = c & 0x7
    if e == 0xF and f == 0x7:
        return math.nan
    if e == 0:
        return sign * (f / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + f / 8.0) * 2.0 ** (e - 7)


_TABLE = np.array([decode_code(c) for c in range(256)], dtype=np.float64)
# non-negative finite codes 0x00..0x7E are increasing in value
_POS_VALUES = _TABLE[:0x7F]


def decode(codes) -> np.ndarray:
    """Array of E4M3FN bytes (uint8, any shape) -> float64 values."""
    c = np.asarray(codes.cpu().numpy() if hasattr(codes, "cpu") else codes).astype(np.uint8)
    return _TABLE[c]


def encode_rne_sat(x) -> np.ndarray:
    """float64 -> E4M3FN codes: round to nearest, ties to even code, saturate at 448."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_POS_VALUES, a, side="left")          # first value >= a
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _POS_VALUES[lo]
    dhi = _POS_VALUES[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(a == _POS_VALUES[hi], hi, code).astype(np.uint8)
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)


def round_e4m3(x) -> np.ndarray:
    return _TABLE[encode_rne_sat(x)]


def rounding_alternative(u, rel: float):
    """For each u >= 0: the other E4M3 neighbour when u lies within ``rel * u`` of the
    midpoint between its two neighbours (the rounding is then not decided by float32
    arithmetic of that accuracy), else the rounded value itself."""
    u = np.minimum(np.asarray(u, dtype=np.float64), E4M3_MAX)
    hi = np.minimum(np.searchsorted(_POS_VALUES, u, side="left"), len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    vlo, vhi = _POS_VALUES[lo], _POS_VALUES[hi]
    mid = 0.5 * (vlo + vhi)
    near = (vhi > vlo) & (np.abs(u - mid) <= rel * u)
    r = _TABLE[encode_rne_sat(u)]
    return np.where(near, np.where(r == vlo, vhi, vlo), r)


def forward(q8, k8, v8, q_scale, k_scale, v_scale, scale: float, block_c: int = 64,
            scale_rows: int = 128, rows=None, heads=None, prob_round=round_e4m3, frame="running",
            envelope_rel=None, causal: bool = False):
    """The quantised forward, step by step.

    ``causal``: the bottom-right causal mask (key k visible to row i iff
    k <= i + S_k - S_q), applied to S before the row max; masked cells give u = 0, a
    tile with no visible key leaves a row's state unchanged, and a row that sees no key
    at all gets O = 0 and LSE = -inf (as in the dense definition).

    q8/k8/v8: E4M3FN codes [B,H,S,d] (uint8); *_scale: float32 [B,H,ceil(S/128)].
    ``block_c``: K/V tile width; each tile must lie inside one 128-row scale block.
    ``prob_round``: the probability rounding (identity removes it).
    ``frame``: "running" rounds u in the running-max frame (the kernel's order);
    "final" rounds it in the final row-max frame (an informational variant).
    ``envelope_rel``: when set, also return E [B,Hq,R,d], the largest change of O that
    flipping every probability whose rounding lies within ``envelope_rel`` (relative)
    of an E4M3 midpoint could cause: u is specified in float32, so such a rounding is
    not determined by the method's own arithmetic and either neighbour is correct.
    Returns (O [B,Hq,R,d], LSE [B,Hq,R]) in float64 (and E).
    """
    assert scale_rows % block_c == 0, "a K/V tile must lie inside one scale block"
    Q, K, V = decode(q8), decode(k8), decode(v8)
    qs, ks, vs = (np.asarray(t.cpu().numpy() if hasattr(t, "cpu") else t, dtype=np.float64)
                  for t in (q_scale, k_scale, v_scale))
    B, Hq, Sq, _ = Q.shape
    Hkv, Sk = K.shape[1], K.shape[2]
    g = Hq // Hkv
    rows = np.arange(Sq) if rows is None else np.asarray(rows)
    O = np.full((B, Hq, len(rows), V.shape[3]), np.nan)
    LSE = np.full((B, Hq, len(rows)), np.nan)
    pairs = [(b, h) for b in range(B) for h in range(Hq)] if heads is None else heads
    off = float(2 ** PROB_OFFSET_LOG2)
    E = np.full_like(O, np.nan) if envelope_rel is not None else None
    for b, h in pairs:
        kv = h // g
        Qi = Q[b, h][rows]
        dq = qs[b, h][rows // scale_rows]
        vis_all = dense.visible(Sq, Sk, causal, rows=rows)
        if frame == "final":
            S_all = float(scale) * dq[:, None] * (Qi @ K[b, kv].T) * ks[b, kv][np.arange(Sk) // scale_rows][None, :]
            m_final = np.where(vis_all, S_all, -np.inf).max(axis=1)
        m = np.full(len(rows), -np.inf)
        l = np.zeros(len(rows))
        o = np.zeros((len(rows), V.shape[3]))
        e = np.zeros((len(rows), V.shape[3]))
        for k0 in range(0, Sk, block_c):
            k1 = min(Sk, k0 + block_c)
            dk = ks[b, kv][k0 // scale_rows]
            dv = vs[b, kv][k0 // scale_rows]
            vis = vis_all[:, k0:k1]
            S = float(scale) * dq[:, None] * dk * (Qi @ K[b, kv][k0:k1].T)
            S = np.where(vis, S, -np.inf)
            m_new = np.maximum(m, S.max(axis=1))
            with np.errstate(invalid="ignore"):
                # a row that has seen no visible key yet keeps m = -inf and alpha = 1
                alpha = np.where(m_new == -np.inf, 1.0, np.exp(m - m_new))
                u = np.where(vis, off * np.exp(S - m_new[:, None]), 0.0)
            if frame == "final":
                # the same u expressed in the final frame, rounded there, brought back
                with np.errstate(invalid="ignore", over="ignore"):
                    shift = np.where(m_new == -np.inf, 1.0, np.exp(m_new - m_final))[:, None]
                p8 = np.where(u > 0, prob_round(u * shift) / shift, 0.0)
            else:
                p8 = prob_round(u)
            l = alpha * l + u.sum(axis=1)
            o = alpha[:, None] * o + dv * (p8 @ V[b, kv][k0:k1])
            if envelope_rel is not None:
                flip = np.abs(rounding_alternative(u, envelope_rel) - p8)
                e = alpha[:, None] * e + dv * (flip @ np.abs(V[b, kv][k0:k1]))
            m = m_new
        empty = ~(l > 0)
        with np.errstate(invalid="ignore", divide="ignore"):
            O[b, h] = np.where(empty[:, None], 0.0, o / l[:, None])
            LSE[b, h] = np.where(empty, -np.inf, m + np.log(l) - PROB_OFFSET_LOG2 * math.log(2.0))
            if E is not None:
                E[b, h] = np.where(empty[:, None], 0.0, e / l[:, None])
    if E is not None:
        return O, LSE, E
    return O, LSE


def dequantized(codes, scales, scale_rows: int = 128) -> np.ndarray:
    """float64 values decode(code) * descale of each row's block: [B,H,S,d]."""
    X = decode(codes)
    s = np.asarray(scales.cpu().numpy() if hasattr(scales, "cpu") else scales, dtype=np.float64)
    S = X.shape[2]
    return X * s[:, :, np.arange(S) // scale_rows][..., None]


# ---------------------------------------------------------------------------------
# Incoherent processing and scale granularity ([HW] section 0x06, "Incoherent
# Processing Is Exact Before Quantization Only" and the block-vs-tensor ablation that
# follows it).  With R = diag(s) H / sqrt(d) (random signs s, Sylvester Hadamard H) R
# is orthogonal, so (Q R)(K R)^T = Q K^T in exact arithmetic; V is not transformed.
# After E4M3 rounding the identity no longer holds and whether the error shrinks
# depends on the data's geometry.

def hadamard_matrix(d: int) -> np.ndarray:
    """Normalised Sylvester Hadamard matrix of order d (a power of two): H_1 = [1],
    H_2n = [[H_n, H_n], [H_n, -H_n]] / sqrt(2) at every doubling."""
    assert d >= 1 and d & (d - 1) == 0, "order must be a power of two"
    H = np.ones((1, 1))
    while H.shape[0] < d:
        H = np.block([[H, H], [H, -H]]) / math.sqrt(2.0)
    return H


def incoherent(x, signs) -> np.ndarray:
    """x R along the last axis, R = diag(signs) H / sqrt(d) (orthogonal for +-1 signs)."""
    X = np.asarray(x.detach().cpu().double().numpy() if hasattr(x, "detach") else x, dtype=np.float64)
    s = np.asarray(signs, dtype=np.float64)
    return (X * s) @ hadamard_matrix(X.shape[-1])


def quantize(x, block_rows: int = 128, per_tensor: bool = False):
    """E4M3 codes and float32 descales [B,H,ceil(S/block_rows)] of float64 x [B,H,S,d].

    Block mode: descale = amax(block) / 448 per (b, h, 128-row block) (1 for an all-zero
    block).  Tensor mode: one descale from the amax of the whole tensor, repeated in
    every entry.  Codes = E4M3(x / descale) with the descale as stored (float32): one
    rounding to nearest even of the quotient (the plain definition; formed in float64,
    i.e. exact to 2^-53 relative, far finer than the 2^-4 spacing of E4M3 values).
    """
    X = np.asarray(x, dtype=np.float64)
    B, H, S, d = X.shape
    nb = (S + block_rows - 1) // block_rows
    pad = np.zeros((B, H, nb * block_rows - S, d))
    Xb = np.concatenate([X, pad], axis=2).reshape(B, H, nb, block_rows, d)
    if per_tensor:
        amax = np.full((B, H, nb), np.abs(X).max() if X.size else 0.0)
    else:
        amax = np.abs(Xb).max(axis=(3, 4))
    desc = np.where(amax > 0, amax / E4M3_MAX, 1.0).astype(np.float32)
    u = Xb / desc.astype(np.float64)[..., None, None]
    codes = encode_rne_sat(u).reshape(B, H, nb * block_rows, d)[:, :, :S]
    return codes, desc


# ---------------------------------------------------------------------------------
# Backward on E4M3 operands.  The pages define no FP8 backward ([HW] section 0x06 leaves
# FP8 training to future work), so this follows the plainest reading: the gradients of
# attention on the dequantised operands, by the FA2 backward formulas ([FA2] section
# 0x06.1): P recomputed from the given LSE, D = rowsum(dO * O) from the given O.

def backward(q8, k8, v8, q_scale, k_scale, v_scale, o, lse, do, scale: float, causal: bool = False,
             heads=None, scale_rows: int = 128):
    """dQ [B,Hq,Sq,d], dK, dV [B,Hkv,Sk,d] (float64; dK/dV summed over each K/V head's
    query group) with respect to Q_d = decode(q8) dQ, K_d, V_d:

        S  = scale Q_d K_d^T (masked cells excluded),  P = exp(S - LSE)
        dV = P^T dO,  dP = dO V_d^T,  D = rowsum(dO * O),  dS = P * (dP - D)
        dQ = scale dS K_d,  dK = scale dS^T Q_d.

    ``o``, ``lse``: the forward's output and log-sum-exp as the backward receives them.
    ``heads``: optional (b, h_kv) pairs to evaluate (the rest is NaN)."""
    Qd = dequantized(q8, q_scale, scale_rows)
    Kd = dequantized(k8, k_scale, scale_rows)
    Vd = dequantized(v8, v_scale, scale_rows)
    O = np.asarray(o.detach().cpu().double().numpy() if hasattr(o, "detach") else o, dtype=np.float64)
    dO = np.asarray(do.detach().cpu().double().numpy() if hasattr(do, "detach") else do, dtype=np.float64)
    L = np.asarray(lse.detach().cpu().double().numpy() if hasattr(lse, "detach") else lse, dtype=np.float64)
    B, Hq, Sq, _ = Qd.shape
    Hkv, Sk = Kd.shape[1], Kd.shape[2]
    g = Hq // Hkv
    vis = dense.visible(Sq, Sk, causal)
    s = float(scale)
    dQ = np.full_like(Qd, np.nan)
    dK = np.full_like(Kd, np.nan)
    dV = np.full_like(Vd, np.nan)
    pairs = [(b, kv) for b in range(B) for kv in range(Hkv)] if heads is None else heads
    for b, kv in pairs:
        dK[b, kv] = 0.0
        dV[b, kv] = 0.0
        for h in range(kv * g, (kv + 1) * g):
            S = s * (Qd[b, h] @ Kd[b, kv].T)
            with np.errstate(invalid="ignore", over="ignore"):
                P = np.where(vis, np.exp(S - L[b, h][:, None]), 0.0)
            P = np.where(np.isneginf(L[b, h])[:, None], 0.0, P)     # rows with no visible key
            dV[b, kv] += P.T @ dO[b, h]
            dP = dO[b, h] @ Vd[b, kv].T
            D = (dO[b, h] * O[b, h]).sum(axis=1)
            dS = P * (dP - D[:, None])
            dQ[b, h] = s * (dS @ Kd[b, kv])
            dK[b, kv] += s * (dS.T @ Qd[b, h])
    return dQ, dK, dV

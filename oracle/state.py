"""The online softmax state algebra, in float64.  Test infrastructure only.

[IO] section 0x08A: a non-empty set A of allowed, finite scores x_j with payload
rows v_j is summarised by

    m_A = max x_j,   l_A = sum exp(x_j - m_A),   u_A = sum exp(x_j - m_A) v_j,
    n_A = |A|.

[IO] 0x08B-C: two disjoint summaries merge in one common maximum frame,

    m = max(m_A, m_B),  alpha = exp(m_A - m),  beta = exp(m_B - m),
    l = alpha l_A + beta l_B,  u = alpha u_A + beta u_B,  n = n_A + n_B,

and the empty set (valid = False, m = -inf, l = 0, u = 0, n = 0) is the identity,
taken by an explicit branch so exp(-inf - -inf) is never evaluated.

[IO] 0x09C-E / [FA2] 0x02A-D: the finished row is O = u / l and LSE = m + ln l;
the same row can be carried as (m, l, O) (normalised merge) or (LSE, O)
(log-domain merge).  [IO] 0x07B-D: the scalar online normaliser starts from the
first unmasked element with d = 1.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


@dataclass
class State:
    valid: bool
    m: float
    l: float
    u: np.ndarray
    n: int = 0


def empty(dv: int) -> State:
    """The identity element ([IO] 0x08C)."""
    return State(False, -math.inf, 0.0, np.zeros(dv), 0)


def of_set(scores, values) -> State:
    """Canonical summary of one index set; -inf scores are masked (absent)."""
    x = np.asarray(scores, dtype=np.float64).reshape(-1)
    V = np.asarray(values, dtype=np.float64).reshape(len(x), -1)
    keep = x != -np.inf
    if not keep.any():
        return empty(V.shape[1])
    x, V = x[keep], V[keep]
    m = float(x.max())
    w = np.exp(x - m)
    return State(True, m, float(w.sum()), w @ V, int(len(x)))


def merge(a: State, b: State) -> State:
    """The binary merge with its identity branch ([IO] 0x08B-C)."""
    if not a.valid:
        return b
    if not b.valid:
        return a
    m = max(a.m, b.m)
    alpha = math.exp(a.m - m)
    beta = math.exp(b.m - m)
    return State(True, m, alpha * a.l + beta * b.l, alpha * a.u + beta * b.u, a.n + b.n)


def fold_sequential(states):
    acc = empty(len(states[0].u))
    for s in states:
        acc = merge(acc, s)
    return acc


def fold_balanced(states):
    level = list(states)
    while len(level) > 1:
        nxt = [merge(level[i], level[i + 1]) for i in range(0, len(level) - 1, 2)]
        if len(level) % 2:
            nxt.append(level[-1])
        level = nxt
    return level[0]


def finalize(s: State):
    """(O, LSE) of a finished row; an invalid row gives (0, -inf) (declared policy)."""
    if not s.valid:
        return np.zeros_like(s.u), -math.inf
    return s.u / s.l, s.m + math.log(s.l)


def chunked(scores, values, chunk: int, order=None):
    """Per-chunk states of one row, in key order (or a permuted ``order`` of chunks)."""
    x = np.asarray(scores, dtype=np.float64).reshape(-1)
    V = np.asarray(values, dtype=np.float64).reshape(len(x), -1)
    parts = [of_set(x[i:i + chunk], V[i:i + chunk]) for i in range(0, len(x), chunk)]
    if order is not None:
        parts = [parts[i] for i in order]
    return parts


# ---- alternative coordinates ([IO] 0x09D-E) -------------------------------------------

def merge_normalized(a, b):
    """(valid, m, l, O) merge in normalised coordinates."""
    va, ma, la, Oa = a
    vb, mb, lb, Ob = b
    if not va:
        return b
    if not vb:
        return a
    m = max(ma, mb)
    left = math.exp(ma - m) * la
    right = math.exp(mb - m) * lb
    l = left + right
    return (True, m, l, (left * Oa + right * Ob) / l)


def merge_lse(a, b):
    """(LSE, O) merge in log-partition coordinates; LSE = -inf is the empty part."""
    La, Oa = a
    Lb, Ob = b
    if La == -math.inf:
        return b
    if Lb == -math.inf:
        return a
    L = float(np.logaddexp(La, Lb))
    return (L, math.exp(La - L) * Oa + math.exp(Lb - L) * Ob)


def online_normalizer(x):
    """Scalar streaming (m, d) from the first unmasked element ([IO] 0x07B-D)."""
    x = [float(v) for v in x]
    first = next((i for i, v in enumerate(x) if v != -math.inf), None)
    if first is None:
        return None                      # all-masked row: policy decided by the caller
    m, d = x[first], 1.0
    for xj in x[first + 1:]:
        if xj == -math.inf:
            continue
        m_new = max(m, xj)
        d = d * math.exp(m - m_new) + math.exp(xj - m_new)
        m = m_new
    return m, d


def naive_block_softmax(scores, values, blocks):
    """The wrong local-normalisation answer ([IO] 0x09H): sum of per-block outputs."""
    x = np.asarray(scores, dtype=np.float64)
    V = np.asarray(values, dtype=np.float64).reshape(len(x), -1)
    out = np.zeros(V.shape[1])
    for blk in blocks:
        e = np.exp(x[blk] - x[blk].max())
        out += (e / e.sum()) @ V[blk]
    return out

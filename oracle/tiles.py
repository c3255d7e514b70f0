"""Causal tile geometry from integer coordinates.  Test infrastructure only.

[FA2] section 0x05.1A-B: query tile i covers [q0, q1) = [i B_r, min(S_q,(i+1)B_r)),
key tile j covers [k0, k1) = [j B_c, min(S_k,(j+1)B_c)); a cell is visible iff
k <= q + delta.  A tile is skipped (fully future) iff k0 > (q1 - 1) + delta, fully
visible iff (k1 - 1) <= q0 + delta, and partial otherwise.
"""
from __future__ import annotations


def tile_class(q0, q1, k0, k1, delta):
    if k0 > (q1 - 1) + delta:
        return "skipped"
    if (k1 - 1) <= q0 + delta:
        return "full"
    return "partial"


def ranges(n, block):
    return [(s, min(n, s + block)) for s in range(0, n, block)]


def census(sq, sk, br, bc, delta):
    """Counts of tile classes and cells over the whole [S_q, S_k] grid."""
    out = {"full": 0, "partial": 0, "skipped": 0, "visited_cells": 0, "allowed_cells": 0}
    for q0, q1 in ranges(sq, br):
        for k0, k1 in ranges(sk, bc):
            c = tile_class(q0, q1, k0, k1, delta)
            out[c] += 1
            if c != "skipped":
                out["visited_cells"] += (q1 - q0) * (k1 - k0)
                for q in range(q0, q1):
                    hi = min(k1, q + delta + 1)
                    out["allowed_cells"] += max(0, hi - k0)
    out["visited"] = out["full"] + out["partial"]
    return out


def visited_per_query_tile(sq, sk, br, bc, delta):
    """Number of non-skipped key tiles for each query tile."""
    return [sum(1 for k0, k1 in ranges(sk, bc) if tile_class(q0, q1, k0, k1, delta) != "skipped")
            for q0, q1 in ranges(sq, br)]


def varlen_census(seqlens_q, seqlens_k, br, max_seqlen_q, n_heads):
    """Workgroup populations of a packed launch ([FA2] section 0x04B): the grid is
    ceil(max_seqlen_q / br) query tiles x sequences x heads; a workgroup is active when
    its first row exists (i br < S_q) and the sequence has keys (S_k > 0), full when it
    owns br valid rows, tail otherwise.  Row slots are br per active workgroup."""
    ntiles = -(-max_seqlen_q // br)
    out = {"launched": ntiles * len(seqlens_q) * n_heads, "active": 0, "full": 0, "tail": 0,
           "row_slots": 0, "valid_rows": 0}
    for sq, sk in zip(seqlens_q, seqlens_k):
        for i in range(ntiles):
            if i * br >= sq or sk == 0:
                continue
            rows = min(br, sq - i * br)
            out["active"] += n_heads
            out["full" if rows == br else "tail"] += n_heads
            out["row_slots"] += br * n_heads
            out["valid_rows"] += rows * n_heads
    return out


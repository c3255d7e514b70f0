// tile_plan.h -- causal / tail tile geometry shared by the kernels and the host API.
//
// Query tile [q0, q1), key tile [k0, k1); a cell is visible iff k <= q + delta with
// delta = S_k - S_q under causal masking ("M4.4 - FlashAttention-2 Work Partitioning
// and the Decode Boundary", sections 0x05.1A-0x05.1B and 0x05.1F).  A key tile is
// skipped when k0 > (q1 - 1) + delta and fully visible when k1 - 1 <= q0 + delta.
// Every visited tile that is not fully visible for the rows in question, or that
// runs past S_k, needs an element mask before the row maximum (section 0x05.1D).
#pragma once

#if defined(__HIPCC__)
#define ATTN_HD __host__ __device__ inline
#else
#define ATTN_HD inline
#endif

struct TilePlan {
  int n_visit;       // key tiles 0 .. n_visit-1 are visited, in ascending order
  int first_masked;  // tiles first_masked .. n_visit-1 need an element mask
};

ATTN_HD int ceil_div_i(int a, int b) { return (a + b - 1) / b; }

// Plan for the query rows [q0, q1) (q1 > q0) against S_k keys in tiles of bk.
ATTN_HD TilePlan plan_rows(int q0, int q1, int Sq, int Sk, int bk, int causal) {
  TilePlan p;
  int kend = Sk;                       // exclusive bound of keys any row may see
  int kfull = Sk;                      // keys [0, kfull) are visible to every row
  if (causal) {
    const int delta = Sk - Sq;
    const int last_visible = (q1 - 1) + delta;   // largest key the last row sees
    kend = last_visible + 1 < Sk ? last_visible + 1 : Sk;
    if (kend < 0) kend = 0;
    const int first_row_sees = q0 + delta + 1;    // keys [0, q0+delta] for the first row
    kfull = first_row_sees < Sk ? first_row_sees : Sk;
    if (kfull < 0) kfull = 0;
  }
  p.n_visit = ceil_div_i(kend, bk);
  int full_tiles = kfull / bk;         // tiles entirely inside [0, kfull)
  p.first_masked = full_tiles < p.n_visit ? full_tiles : p.n_visit;
  return p;
}

// Column view used by the backward's K/V-column owner: for the key tile [k0, k1)
// (k1 <= S_k), the query tiles of height bq that see at least one of its keys are
// first_qtile .. n_qtiles-1, and the ones before nomask_qtile intersect the causal
// band (need an element mask).  A query row q sees key k iff k <= q + delta, so the
// first row seeing key k0 is k0 - delta and the first row seeing every key of the
// tile is (k1 - 1) - delta ("M4.4 - FlashAttention-2 ...", section 0x06.1G: causality
// makes the producer set of each column triangular).
struct ColPlan {
  int first_qtile;
  int nomask_qtile;
  int n_qtiles;
};

ATTN_HD ColPlan plan_cols(int k0, int k1, int Sq, int Sk, int bq, int causal) {
  ColPlan p;
  p.n_qtiles = ceil_div_i(Sq, bq);
  if (!causal) {
    p.first_qtile = 0;
    p.nomask_qtile = 0;
    return p;
  }
  const int delta = Sk - Sq;
  int first_row = k0 - delta;
  if (first_row < 0) first_row = 0;
  if (first_row >= Sq) {
    p.first_qtile = p.n_qtiles;
    p.nomask_qtile = p.n_qtiles;
    return p;
  }
  p.first_qtile = first_row / bq;
  int full_row = (k1 - 1) - delta;
  if (full_row < 0) full_row = 0;
  int nm = ceil_div_i(full_row, bq);
  if (nm < p.first_qtile) nm = p.first_qtile;
  if (nm > p.n_qtiles) nm = p.n_qtiles;
  p.nomask_qtile = nm;
  return p;
}

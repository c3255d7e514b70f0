// attn_fwd.hip -- tiled attention forward for gfx950 (fp16 / bf16, d = 64 / 128).
//
// Schedule ("M4.4 - FlashAttention-2 Work Partitioning and the Decode Boundary",
// section 0x03, Algorithm 1, and section 0x05C, split-Q): one workgroup owns one
// query tile of one (batch, query head); each wave owns 32 disjoint query rows, so no
// output is merged across waves that share a key range.  The workgroup streams K/V
// tiles of BC keys through an LDS ring and every wave carries the online state
// (m, l, u) of its rows in registers ("M4.3 - IO-Aware Attention ...", section 0x09C;
// FA2 section 0x02C: u <- alpha u + P~ V, normalised once at the end).
//
// Orientation.  The kernel computes the transposed score tile S^T = K Q^T on the
// 32x32x16 matrix core: in the accumulator layout each lane then holds ONE query
// column and 16 keys of it, so the running max, the rescale factor alpha and l are
// per-lane scalars (one cross-lane exchange, lane l <-> l^32, for the max).  The
// probabilities stay in registers and feed O^T += V^T P^T directly as the B operand:
// slot j of lane group g in key chunk c is key 16c + 8(j/4) + 4g + j%4, the same
// keys the S^T accumulator put in registers 8(c%2) .. 8(c%2)+7.
//
// Staging.  K and V tiles are staged row-major in LDS through registers, K and V in
// rings of two slots each.  The V^T operand of the P V product comes from
// ds_read_b64_tr_b16, which hands each lane of a 16-lane group one column of a 4-row
// x 16-column block (4 consecutive keys of one d), so V needs no transpose on the way
// in.  Rows are not padded; each row's 16-byte chunks are XOR-swizzled instead (LDS
// chunk p of row r holds global chunk p ^ swz(r)), with swizzles chosen so that the
// K reads, the V transpose reads and the 16-byte tile writes all hit distinct banks.
//
// Software pipeline.  Step t of a wave runs, chunk by chunk over the 16-key chunks
// of the tile, the score product of tile t+1, the probabilities of tile t and the
// P V product of tile t, so that each chunk's exponentials sit between matrix-core
// instructions that do not depend on them; the row maximum of tile t+1 (and the
// rescale decision) ends the step, under the tail of the P V product.  The rescale of
// the output accumulator, when one is needed, follows the P V product of tile t,
// whose terms still belong to the old maximum.  Staging runs one tile ahead: step t
// writes K(t+2) and V(t+1) into LDS from registers, then loads K(t+3) and V(t+2) into
// those registers; one workgroup barrier per step publishes the writes of the step
// before and frees the slots read in it.
//
// Exponentials run in base 2: p = exp2(s * c - m) with c = scale * log2(e) in one FMA.
// Masking (key tail and causal band) sets the invisible scores to -inf before the row
// max, and only on the tiles the tile plan marks (tile_plan.h); a zero scale uses the
// smallest c that keeps c * (-inf) = -inf while c * s rounds to 0 for finite s.  Loads
// past the tensor return zeros (the buffer range check), so tails need no branches.
//
// Conditional rescale ("M4.6 - FlashAttention-3/4 Hardware Pipelines", section 0x09:
// the reference maximum may stay stale while the new maximum exceeds it by at most a
// threshold; numerator and denominator share that reference, so the result is exact):
// the running max m moves only when some row of the wave sees a score more than
// TAU = 8 (base 2) above it.  Otherwise alpha = 1 and the O / l rescale is skipped;
// probabilities then stay below 2^8, well inside fp16 / bf16 range.  The denominator
// sums the fp32 probabilities (before their rounding to the element type), which
// keeps the log-sum-exp at fp32 accuracy.
#include "attn_device.h"
#include "attn_launch.h"
#include "tile_plan.h"

namespace {

constexpr int kWave = 64;
constexpr float kTau = 8.f;   // conditional-rescale threshold, base-2 units
constexpr int BC = 64;        // keys per K/V tile

typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Tile geometry for head dimension D: rows of D*2 bytes, CPR 16-byte chunks per row.
template <int D>
struct Tile {
  static constexpr int ROWB = D * 2;
  static constexpr int CPR = D / 8;
  static constexpr int BYTES = BC * ROWB;          // one K or V tile
  static constexpr int CHUNKS = BYTES / 16;        // 16-byte chunks per tile
  // K: 16 consecutive rows must use 16 distinct bank groups for the b128 reads.
  static __device__ inline int swz_k(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
  // V: the 4 rows x 4 chunks read by one 32-lane pass of the transpose read must be
  // 16 distinct bank groups.
  static __device__ inline int swz_v(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
};

// Maximum for scores: no NaN can occur, and the NaN-propagating form maps to
// v_maximum3_f32 without operand canonicalisation.
__device__ inline float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// max over the two lanes l and l ^ 32 (one VALU lane swap).
__device__ inline float max_pair32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <typename T, int D, int NW, int KS, bool CAUSAL>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(2)))
void fwd_kernel(FwdArgs a) {
  typedef Elem<T> E;
  typedef typename E::v8 V8;
  typedef Tile<D> TL;
  constexpr int RB = NW / KS;                 // 32-row query blocks per workgroup
  constexpr int BQ = RB * 32;
  constexpr int KC = D / 16;                  // contraction chunks for S^T
  constexpr int KB = BC / 32;                 // key blocks of 32 per tile
  constexpr int DB = D / 32;                  // output d blocks of 32
  constexpr int PC = BC / 16;                 // key chunks of 16 for P V
  constexpr int RING = 4 * TL::BYTES;         // K slots 0, 1 then V slots 0, 1
  constexpr int NTK = RB * kWave;             // threads staging one key range
  constexpr int LOADS = TL::CHUNKS / NTK;     // 16-byte K (and V) chunks per thread
  static_assert(TL::CHUNKS % NTK == 0, "chunks must split evenly over the threads");

  __shared__ __attribute__((aligned(1024))) uint8_t lds_all[KS * RING];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int kh = wave / RB;                   // key range of this wave
  const int w = wave % RB;                    // query block of this wave
  const int n = lane & 31;
  const int grp = lane >> 5;
  const int tid = threadIdx.x % NTK;          // index among the threads of this key range
  uint8_t* kring = lds_all + kh * RING;
  uint8_t* vring = kring + 2 * TL::BYTES;

  const int BH = a.B * a.Hq;
  const int wg = blockIdx.x;
  const int bh = wg % BH;
  const int qt = CAUSAL ? (a.nqt - 1 - wg / BH) : (wg / BH);   // heavy causal tiles first
  const int b = bh / a.Hq;
  const int h = bh - b * a.Hq;
  const int kvh = h / a.group;

  const T* qb = reinterpret_cast<const T*>(a.q) + ((int64_t)(b * a.Hq + h) * a.Sq) * D;
  const T* kb = reinterpret_cast<const T*>(a.k) + ((int64_t)(b * a.Hkv + kvh) * a.Sk) * D;
  const T* vb = reinterpret_cast<const T*>(a.v) + ((int64_t)(b * a.Hkv + kvh) * a.Sk) * D;
  const __amdgpu_buffer_rsrc_t qr = make_rsrc(qb, (uint32_t)a.Sq * D * 2);
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(kb, (uint32_t)a.Sk * D * 2);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(vb, (uint32_t)a.Sk * D * 2);

  const int q0 = qt * BQ;
  const int q1 = min(q0 + BQ, a.Sq);
  const int qrow = q0 + w * 32 + n;
  const TilePlan plan = plan_rows(q0, q1, a.Sq, a.Sk, BC, CAUSAL);
  const int w0 = q0 + w * 32;
  const int w1 = max(min(w0 + 32, a.Sq), w0 + 1);
  const TilePlan wplan = plan_rows(w0, w1, a.Sq, a.Sk, BC, CAUSAL);
  // keys at or past klim are invisible to this lane's query row
  const int klim = CAUSAL ? min(a.Sk, qrow + (a.Sk - a.Sq) + 1) : a.Sk;

  // Q^T fragments (B operand): lane column = its query row, slots = d 16kc+8g .. +8.
  // A negative score scale is moved into Q (sign flip) so that c > 0 below and the
  // row max can be taken on the raw accumulator values.
  const uint32_t qsign = a.scale_log2 < 0.f ? 0x80008000u : 0u;
  const float c = fmaxf(fabsf(a.scale_log2), 1e-30f);
  V8 qf[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    u32x4 raw = buf_load_16(qr, (uint32_t)(qrow * D + 16 * kc + 8 * grp) * 2);
    raw.x ^= qsign;
    raw.y ^= qsign;
    raw.z ^= qsign;
    raw.w ^= qsign;
    qf[kc] = as_v8<V8>(raw);
  }

  f32x16 o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) o[i] = f32x16{};
  float m_i = -INFINITY;   // running max (base-2 units)
  float l_i = 0.f;         // this lane's share of the running denominator

  // Staging: chunk idx = r * NTK + tid of a tile is LDS (row, pos) = (idx / CPR,
  // idx % CPR) and holds global chunk pos ^ swz(row) of that row.
  u32x4 kreg[LOADS], vreg[LOADS];
  auto load_k = [&](int t) {
#pragma unroll
    for (int r = 0; r < LOADS; ++r) {
      const int idx = r * NTK + tid;
      const int row = idx / TL::CPR;
      const int pos = idx % TL::CPR;
      kreg[r] = buf_load_16(kr, (uint32_t)((t * BC + row) * D) * 2 + (uint32_t)((pos ^ TL::swz_k(row)) * 16));
    }
  };
  auto load_v = [&](int t) {
#pragma unroll
    for (int r = 0; r < LOADS; ++r) {
      const int idx = r * NTK + tid;
      const int row = idx / TL::CPR;
      const int pos = idx % TL::CPR;
      vreg[r] = buf_load_16(vr, (uint32_t)((t * BC + row) * D) * 2 + (uint32_t)((pos ^ TL::swz_v(row)) * 16));
    }
  };
  auto store_k = [&](int slot) {
#pragma unroll
    for (int r = 0; r < LOADS; ++r) st_lds_16(kring + slot * TL::BYTES + (r * NTK + tid) * 16, kreg[r]);
  };
  auto store_v = [&](int slot) {
#pragma unroll
    for (int r = 0; r < LOADS; ++r) st_lds_16(vring + slot * TL::BYTES + (r * NTK + tid) * 16, vreg[r]);
  };

  // S^T MFMAs for contraction chunks [kc0, kc1) of one tile from K slot `slot`; the
  // chunk kc = 0 starts from a zero accumulator.
  auto score_part = [&](f32x16 (&sc)[KB], int slot, int kc0, int kc1) {
    const uint8_t* ks = kring + slot * TL::BYTES;
#pragma unroll
    for (int kc = kc0; kc < kc1; ++kc) {
#pragma unroll
      for (int kbk = 0; kbk < KB; ++kbk) {
        const int row = kbk * 32 + n;
        const int chunk = (2 * kc + grp) ^ TL::swz_k(row);
        const V8 av = as_v8<V8>(ld_lds_16(ks + row * TL::ROWB + chunk * 16));
        sc[kbk] = E::mfma(av, qf[kc], kc == 0 ? f32x16{} : sc[kbk]);
      }
    }
  };

  // O^T += V^T P^T for key chunk cc from V slot `slot`.  The 16-lane group G =
  // lane/16 reads the 4 keys x 16 d block at keys 16cc + 4g (+8 for slots 4..7),
  // d = 32db + 16(G%2); lane s of the group addresses key row s/4, d columns
  // 4(s%4) .. +3.
  const int s16 = lane & 15;
  const int dsub = 16 * ((lane >> 4) & 1) + 4 * (s16 & 3);
  auto pv_chunk = [&](const u32x4& p, int slot, int cc) {
    const uint8_t* vs = vring + slot * TL::BYTES;
    const int r0 = 16 * cc + 4 * grp + (s16 >> 2);
    const int r1 = r0 + 8;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int col = 32 * db + dsub;                 // multiple of 4: 8 bytes in one chunk
      const int ch = col >> 3;
      const int hf = (col & 7) * 2;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4*)(vs + r0 * TL::ROWB + ((ch ^ TL::swz_v(r0)) * 16) + hf));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4*)(vs + r1 * TL::ROWB + ((ch ^ TL::swz_v(r1)) * 16) + hf));
      const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
      const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
      const u32x4 av4 = {l2.x, l2.y, h2.x, h2.y};
      o[db] = E::mfma(as_v8<V8>(av4), as_v8<V8>(p), o[db]);
    }
  };

  // Probabilities of key chunk cc of a scored tile, packed to the element type
  // (slot j of lane group g = key 16cc + 8(j/4) + 4g + j%4, accumulator registers
  // 8(cc%2) .. +7 of key block cc/2); their fp32 sum goes to l.
  auto probs_chunk = [&](const f32x16 (&sc)[KB], int cc, float m_use, float& l0, float& l1) -> u32x4 {
    const int kbk = cc >> 1;
    const int hb = (cc & 1) * 8;
    uint32_t pk[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float e0 = fast_exp2(fmaf(sc[kbk][hb + 2 * j], c, -m_use));
      const float e1 = fast_exp2(fmaf(sc[kbk][hb + 2 * j + 1], c, -m_use));
      l0 += e0;
      l1 += e1;
      pk[j] = E::pack2(e0, e1);
    }
    return u32x4{pk[0], pk[1], pk[2], pk[3]};
  };

  // Row max of tile t and the rescale decision; l is rescaled here, O by the caller
  // (after the pending P V product).
  auto row_max = [&](f32x16 (&sc)[KB], int t, bool& moved) -> float {
    if (t >= wplan.first_masked) {
#pragma unroll
      for (int kbk = 0; kbk < KB; ++kbk)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = t * BC + kbk * 32 + 8 * (i >> 2) + 4 * grp + (i & 3);
          sc[kbk][i] = key < klim ? sc[kbk][i] : -INFINITY;
        }
    }
    float r0 = vmax(sc[0][0], sc[0][1]), r1 = vmax(sc[0][2], sc[0][3]);
#pragma unroll
    for (int kbk = 0; kbk < KB; ++kbk)
#pragma unroll
      for (int i = (kbk == 0 ? 4 : 0); i < 16; i += 4) {
        r0 = vmax(r0, vmax(sc[kbk][i], sc[kbk][i + 1]));
        r1 = vmax(r1, vmax(sc[kbk][i + 2], sc[kbk][i + 3]));
      }
    const float mx = max_pair32(vmax(r0, r1) * c);
    moved = wave_any(mx > m_i + kTau);
    float alpha = 1.f;
    if (moved) {
      const float m_new = fmaxf(m_i, mx);
      // the decision is per wave: a row with nothing visible yet keeps m = -inf, alpha 1
      alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_i - m_new);
      m_i = m_new;
      l_i *= alpha;
    }
    return alpha;
  };
  auto rescale_o = [&](float alpha) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
  };

  // The visited tiles are split into KS contiguous ranges, one per group of RB waves;
  // this wave's rows need the tiles of its range below we.  Every wave runs the same
  // number of steps so the workgroup barriers line up.
  const int nt = plan.n_visit;
  const int per = (nt + KS - 1) / KS;
  const int tb = min(nt, kh * per);
  const int te = min(nt, tb + per);
  const int we = max(tb, min(te, wplan.n_visit));
  const int nr = te - tb;

  if (nr > 0) {
    load_k(tb);
    store_k(0);
    load_v(tb);
    store_v(0);
  }
  if (nr > 1) {
    load_k(tb + 1);
    store_k(1);
    load_v(tb + 1);
  }
  if (nr > 2) load_k(tb + 2);
  __syncthreads();
  f32x16 sa[KB], sb[KB];
  if (tb < we) {
    score_part(sa, 0, 0, KC);
    bool moved;
    row_max(sa, tb, moved);   // O is still zero: no rescale needed
  }

  // One step: tile t = tb + i is in `cur` (scored, its max taken); tile t+1 is scored
  // into `nxt`.
  auto step = [&](int i, f32x16 (&cur)[KB], f32x16 (&nxt)[KB]) {
    const int t = tb + i;
    __syncthreads();   // writes of the step before are visible; the slots written below are free
    if (t + 2 < te) store_k(i & 1);
    if (t + 1 < te) store_v((i + 1) & 1);
    if (t + 3 < te) load_k(t + 3);
    if (t + 2 < te) load_v(t + 2);

    const bool has_cur = t < we;
    const bool has_nxt = t + 1 < we;
    const float m_use = (m_i == -INFINITY) ? 0.f : m_i;
    float l0 = 0.f, l1 = 0.f;
    if (has_cur && has_nxt) {
      // steady state: one basic block, chunk by chunk
#pragma unroll
      for (int cc = 0; cc < PC; ++cc) {
        score_part(nxt, (i + 1) & 1, cc * KC / PC, (cc + 1) * KC / PC);
        const u32x4 p = probs_chunk(cur, cc, m_use, l0, l1);
        pv_chunk(p, i & 1, cc);
      }
    } else if (has_cur) {
#pragma unroll
      for (int cc = 0; cc < PC; ++cc) pv_chunk(probs_chunk(cur, cc, m_use, l0, l1), i & 1, cc);
    } else if (has_nxt) {
      score_part(nxt, (i + 1) & 1, 0, KC);
    }
    l_i += l0 + l1;
    if (has_nxt) {
      bool moved;
      const float alpha = row_max(nxt, t + 1, moved);
      if (moved) rescale_o(alpha);
    }
  };
  for (int i = 0; i < per; i += 2) {
    step(i, sa, sb);
    if (i + 1 < per) step(i + 1, sb, sa);
  }

  if constexpr (KS == 2) {
    // Merge the two key ranges' states of each row in one max frame ("M4.3 -
    // IO-Aware Attention ...", section 0x08B); the second range hands its (m, l, u)
    // to the first through LDS.  Layout [block][value][lane] keeps lanes on banks.
    constexpr int NV = 2 + 16 * DB;
    static_assert(RB * NV * kWave * 4 <= KS * RING, "merge buffer fits in the ring");
    __syncthreads();                                   // every wave is done with the ring
    float* xf = reinterpret_cast<float*>(lds_all);
    float* mine = xf + (w * NV) * kWave + lane;
    if (kh == 1) {
      mine[0] = m_i;
      mine[kWave] = l_i;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) mine[(2 + 16 * db + i) * kWave] = o[db][i];
    }
    __syncthreads();
    if (kh == 0) {
      const float m1 = mine[0];
      const float l1 = mine[kWave];
      const float m = fmaxf(m_i, m1);
      const float a0 = (m == -INFINITY) ? 0.f : fast_exp2(m_i - m);
      const float a1 = (m == -INFINITY) ? 0.f : fast_exp2(m1 - m);
      l_i = a0 * l_i + a1 * l1;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] = a0 * o[db][i] + a1 * mine[(2 + 16 * db + i) * kWave];
      m_i = m;
    }
  }

  // Epilogue: O = u / l once per row; LSE = (m + log2 l) ln 2 (FA2 section 0x02D).
  const float l_tot = l_i + __shfl_xor(l_i, 32);
  const bool empty = (m_i == -INFINITY) || !(l_tot > 0.f);
  const float inv = empty ? 0.f : 1.f / l_tot;
  if (kh == 0 && qrow < a.Sq) {
    T* ob = reinterpret_cast<T*>(a.o) + ((int64_t)(b * a.Hq + h) * a.Sq + qrow) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        u32x2 pk;
        pk.x = E::pack2(o[db][4 * r4 + 0] * inv, o[db][4 * r4 + 1] * inv);
        pk.y = E::pack2(o[db][4 * r4 + 2] * inv, o[db][4 * r4 + 3] * inv);
        *reinterpret_cast<u32x2*>(ob + db * 32 + 8 * r4 + 4 * grp) = pk;
      }
    }
    if (a.lse != nullptr && grp == 0) {
      a.lse[(int64_t)(b * a.Hq + h) * a.Sq + qrow] = empty ? -INFINITY : (m_i + __log2f(l_tot)) * ATTN_LN2;
    }
  }
}

template <typename T, int D, int NW, int KS>
hipError_t launch_fwd_t(const FwdArgs& a0, hipStream_t stream) {
  FwdArgs a = a0;
  constexpr int BQ = (NW / KS) * 32;
  a.nqt = (a.Sq + BQ - 1) / BQ;
  const dim3 grid((unsigned)(a.nqt * a.B * a.Hq));
  const dim3 block(NW * kWave);
  if (a.causal)
    hipLaunchKernelGGL((fwd_kernel<T, D, NW, KS, true>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((fwd_kernel<T, D, NW, KS, false>), grid, block, 0, stream, a);
  return hipGetLastError();
}

// Eight waves per workgroup.  When 256-row query tiles would leave fewer than two
// workgroups per compute unit, the waves split into two groups that stream the two
// halves of the K/V range for 128-row tiles instead (merged at the end).
constexpr int kCUs = 256;

template <typename T, int D>
hipError_t launch_fwd_d(const FwdArgs& a, hipStream_t stream) {
  const int64_t wgs_full = (int64_t)((a.Sq + 255) / 256) * a.B * a.Hq;
  if (wgs_full >= 2 * kCUs) return launch_fwd_t<T, D, 8, 1>(a, stream);
  return launch_fwd_t<T, D, 8, 2>(a, stream);
}

template <typename T>
hipError_t launch_fwd_dtype(const FwdArgs& a, hipStream_t stream) {
  if (a.d == 64) return launch_fwd_d<T, 64>(a, stream);
  return launch_fwd_d<T, 128>(a, stream);
}

}  // namespace

hipError_t attn_launch_fwd(const FwdArgs& a, hipStream_t stream) {
  if (a.dtype_bf16) return launch_fwd_dtype<bf16>(a, stream);
  return launch_fwd_dtype<f16>(a, stream);
}

// attn_fwd.hip -- tiled attention forward for gfx950 (fp16 / bf16, d = 64 / 128).
//
// Schedule ("M4.4 - FlashAttention-2 Work Partitioning and the Decode Boundary",
// section 0x03, Algorithm 1, and section 0x05C, split-Q): one workgroup owns one
// query tile of one (batch, query head); each wave owns QB blocks of 32 disjoint query
// rows, so no output is merged across waves that share a key range.  The workgroup
// streams K/V tiles through an LDS ring and every wave carries the online state
// (m, l, u) of its rows in registers ("M4.3 - IO-Aware Attention ...", section 0x09C;
// FA2 section 0x02C: u <- alpha u + P~ V, normalised once at the end).  With two
// query blocks per wave (head dimension 64) every K and V fragment read from LDS feeds
// two matrix-core products, halving the LDS traffic per product; the tiles are then
// 32 keys long to bound the registers.  Small grids split the key range over KS
// groups of waves, merged at the end.
//
// Orientation.  The kernel computes the transposed score tile S^T = K Q^T on the
// 32x32x16 matrix core: in the accumulator layout each lane then holds ONE query
// column and 16 keys of it, so the running max, the rescale factor alpha and l are
// per-lane scalars (one cross-lane exchange, lane l <-> l^32, for the max).  The
// probabilities stay in registers and feed O^T += V^T P^T directly as the B operand:
// slot j of lane group g in key chunk c is key 16c + 8(j/4) + 4g + j%4, the same
// keys the S^T accumulator put in registers 8(c%2) .. 8(c%2)+7.
//
// Staging.  K and V tiles are loaded row-major from HBM straight into LDS (buffer loads
// with the LDS destination, no staging registers), K and V in rings of two slots
// each.  The V^T operand of the P V product comes from
// ds_read_b64_tr_b16, which hands each lane of a 16-lane group one column of a 4-row
// x 16-column block (4 consecutive keys of one d), so V needs no transpose on the way
// in.  Rows are not padded; each row's 16-byte chunks are XOR-swizzled instead (LDS
// chunk p of row r holds global chunk p ^ swz(r)), with swizzles chosen so that the
// K fragment reads and the V transpose reads hit distinct banks.
//
// Software pipeline.  Step t of a wave runs, chunk by chunk over the 16-key chunks
// of the tile, the score product of tile t+1, the probabilities of tile t and the
// P V product of tile t, so that each chunk's exponentials sit between matrix-core
// instructions that do not depend on them; the row maximum of tile t+1 (and the
// rescale decision) ends the step, under the tail of the P V product.  The rescale of
// the output accumulator, when one is needed, follows the P V product of tile t,
// whose terms still belong to the old maximum.  Staging runs one tile ahead: step t
// waits for its own loads of K(t+1) and V(t) (issued a step earlier), passes one
// workgroup barrier, which publishes every thread's part and frees the slots read in
// step t-1, then issues the loads of K(t+2) and V(t+1) into those slots.
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
// TAU = 8 (base 2) above it (tested per lane on its raw scores against (m + TAU) / c,
// the cross-lane maximum is taken only when m moves).  Otherwise alpha = 1 and the O / l rescale is skipped;
// probabilities then stay below 2^8, well inside fp16 / bf16 range.  The denominator
// sums the fp32 probabilities (before their rounding to the element type), which
// keeps the log-sum-exp at fp32 accuracy.
#include "attn_device.h"
#include "attn_launch.h"
#include "tile_plan.h"

#include <type_traits>

namespace {

constexpr int kWave = 64;
constexpr float kTau = 8.f;   // conditional-rescale threshold, base-2 units

typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Tile geometry for head dimension D and BC keys: rows of D*2 bytes, CPR 16-byte
// chunks per row.
template <int D, int BC>
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

// VL: packed variable-length layout.  DROP: dropout on the probabilities entering P V
// (padded layout only).  EMU: 0, 2 or 4 of every 8 exponentials of a key chunk by the
// software exp2 on the FMA pipe (padded layout without dropout only).
template <typename T, int D, int QB, int RW, int KS, bool VL, bool CAUSAL, bool DROP, int EMU = 0>
__global__ __launch_bounds__(RW * KS * kWave) __attribute__((amdgpu_waves_per_eu(RW * KS / 4)))
void fwd_kernel(FwdArgs a) {
  typedef Elem<T> E;
  typedef typename E::v8 V8;
  // bf16 dropout (training): the probabilities enter P V as a two-term bf16 sum hi + lo
  // (~16 significant bits), so the stored O is the rounding of an O accurate to fp32
  // level and the backward's D = rowsum(dO o O) sees only that storage rounding
  constexpr bool SPLIT = DROP && std::is_same<T, bf16>::value;
  constexpr int BC = QB == 2 ? 32 : 64;       // keys per K/V tile
  typedef Tile<D, BC> TL;
  constexpr int BQ = RW * QB * 32;            // query rows per workgroup
  constexpr int KC = D / 16;                  // contraction chunks for S^T
  constexpr int KB = BC / 32;                 // key blocks of 32 per tile
  constexpr int DB = D / 32;                  // output d blocks of 32
  constexpr int PC = BC / 16;                 // key chunks of 16 for P V
  constexpr int KPC = KC / PC;                // score contraction chunks per key chunk
  // K/V ring depth: three slots each where the key ranges' rings fit the LDS, else two.
  // K/V ring depth (slots per ring).  Two: with the loop unrolled by two steps the
  // slots are compile-time constants, so every LDS read address is a fixed register
  // plus an immediate; three slots (loads two tiles ahead) measured slower.
  constexpr int DEPTH = 2;
  constexpr int RING = 2 * DEPTH * TL::BYTES; // K slots then V slots
  constexpr int NTK = RW * kWave;             // threads staging one key range
  constexpr int LOADS = TL::CHUNKS / NTK;     // 16-byte K (and V) chunks per thread
  static_assert(TL::CHUNKS % NTK == 0 && LOADS >= 1, "chunks must split evenly over the threads");
  static_assert(KC % PC == 0, "score product must split evenly over the key chunks");
  constexpr int NV = 2 + 16 * DB;             // merged values per lane and query block
  constexpr int MERGE = (D == 64 ? KS : KS - 1) * RW * QB * NV * kWave * 4;   // the key ranges' states
  constexpr int LDS = (KS > 1 && MERGE > KS * RING) ? MERGE : KS * RING;

  __shared__ __attribute__((aligned(1024))) uint8_t lds_all[LDS];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int kh = wave / RW;                   // key range of this wave
  const int w = wave % RW;                    // query rows of this wave
  const int n = lane & 31;
  const int grp = lane >> 5;
  const int tid = threadIdx.x % NTK;          // index among the threads of this key range
  uint8_t* kring = lds_all + kh * RING;
  uint8_t* vring = kring + DEPTH * TL::BYTES;

  const int BH = a.B * a.Hq;
  const int wg = blockIdx.x;
  // Workgroups go round-robin to the 8 XCDs (each with its own L2).  Padded layout:
  // the K/V head index (b, kvh) varies fastest, so the g query heads sharing a K/V head
  // land on the same XCD whenever B Hkv is a multiple of 8.  Packed layout: the heads of
  // one sequence stay adjacent (sequences differ in length) and, among them, the K/V
  // head varies fastest, so the g query heads of a K/V head are Hkv workgroups apart
  // (one XCD when Hkv is a multiple of 8).
  const int bh = wg % BH;
  const int qt = CAUSAL ? (a.nqt - 1 - wg / BH) : (wg / BH);   // heavy causal tiles first
  int b, h, kvh;
  if constexpr (VL) {
    b = bh / a.Hq;
    const int hh = bh - b * a.Hq;
    const int nkvh = a.Hq / a.group;
    kvh = hh % nkvh;
    h = kvh * a.group + hh / nkvh;
  } else {
    const int nkv = a.B * a.Hkv;
    const int bkv = bh % nkv;
    b = bkv / a.Hkv;
    kvh = bkv - b * a.Hkv;
    h = kvh * a.group + bh / nkv;
  }

  // Geometry of this (sequence, head): lengths, first-row element offsets, row strides
  // (d for the padded layout, H d for the packed token-major layout), LSE row base.
  // VL: the packed layout; otherwise the strides are the compile-time d.
  int Sq, Sk;
  int q_rs = D, kv_rs = D;
  int64_t q_off, kv_off, lse_off;
  if constexpr (VL) {
    // extents clamped to the declared maxima and totals: inconsistent offsets can
    // give wrong rows but never an access outside the tensors
    const int tq = min(max(a.cu_q[b], 0), a.total_q);
    const int tk = min(max(a.cu_k[b], 0), a.total_k);
    Sq = min(min(max(a.cu_q[b + 1] - tq, 0), a.Sq), a.total_q - tq);
    Sk = min(min(max(a.cu_k[b + 1] - tk, 0), a.Sk), a.total_k - tk);
    q_rs = a.Hq * D;
    kv_rs = a.Hkv * D;
    q_off = ((int64_t)tq * a.Hq + h) * D;
    kv_off = ((int64_t)tk * a.Hkv + kvh) * D;
    lse_off = (int64_t)h * a.total_q + tq;
  } else {
    Sq = a.Sq;
    Sk = a.Sk;
    q_off = (int64_t)(b * a.Hq + h) * a.Sq * D;
    kv_off = (int64_t)(b * a.Hkv + kvh) * a.Sk * D;
    lse_off = (int64_t)(b * a.Hq + h) * a.Sq;
  }
  if (VL && qt * BQ >= Sq) return;   // whole workgroup, before any barrier
  const T* qb = reinterpret_cast<const T*>(a.q) + q_off;
  const T* kb = reinterpret_cast<const T*>(a.k) + kv_off;
  const T* vb = reinterpret_cast<const T*>(a.v) + kv_off;
  // range-checked spans: rows at or past the sequence end read as zero
  const __amdgpu_buffer_rsrc_t qr = make_rsrc(qb, Sq > 0 ? (uint32_t)((Sq - 1) * q_rs + D) * 2 : 0u);
  const int64_t kv_bytes = Sk > 0 ? ((int64_t)(Sk - 1) * kv_rs + D) * 2 : 0;

  const int q0 = qt * BQ;
  const int q1 = min(q0 + BQ, Sq);
  const TilePlan plan = plan_rows(q0, q1, Sq, Sk, BC, CAUSAL);
  const int w0 = q0 + w * QB * 32;
  const int w1 = max(min(w0 + QB * 32, Sq), w0 + 1);
  const TilePlan wplan = plan_rows(w0, w1, Sq, Sk, BC, CAUSAL);
  int qrow[QB], klim[QB];   // this lane's query row per block; keys at or past klim are invisible
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    qrow[j] = w0 + 32 * j + n;
    klim[j] = CAUSAL ? min(Sk, qrow[j] + (Sk - Sq) + 1) : Sk;
  }

  // Q^T fragments (B operand): lane column = its query row, slots = d 16kc+8g .. +8.
  // A negative score scale is moved into Q (sign flip) so that c > 0 below and the
  // row max can be taken on the raw accumulator values.
  const uint32_t qsign = a.scale_log2 < 0.f ? 0x80008000u : 0u;
  const float c = fmaxf(fabsf(a.scale_log2), 1e-30f);
  const float inv_c = 1.f / c;
  V8 qf[QB][KC];
#pragma unroll
  for (int j = 0; j < QB; ++j)
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      u32x4 raw = buf_load_16(qr, (uint32_t)(qrow[j] * q_rs + 16 * kc + 8 * grp) * 2);
      raw.x ^= qsign;
      raw.y ^= qsign;
      raw.z ^= qsign;
      raw.w ^= qsign;
      qf[j][kc] = as_v8<V8>(raw);
    }

  f32x16 o[QB][DB];
  // running max (base-2 units); this lane's share of l; the rescale threshold
  // (m + TAU) / c in raw score units
  float m_i[QB], l_i[QB], thr[QB];
#pragma unroll
  for (int j = 0; j < QB; ++j) {
#pragma unroll
    for (int i = 0; i < DB; ++i) o[j][i] = f32x16{};
    m_i[j] = -INFINITY;
    l_i[j] = 0.f;
    thr[j] = -INFINITY;
  }

  // Staging: chunk idx = r * NTK + tid of a tile is LDS (row, pos) = (idx / CPR,
  // idx % CPR) and holds global chunk pos ^ swz(row) of that row.  The loads go
  // straight from HBM/L2 to LDS (a wave's 64 lanes fill 1 KiB at consecutive 16-byte
  // positions), so staging takes no registers and no LDS writes; each thread waits for
  // its own loads (vmcnt) and the step's barrier publishes them.  Load round r covers
  // rows r*RS .. r*RS+RS-1 and the swizzles repeat every 16 rows, so a thread's column
  // offset is the same in every round.  Padded layout: one resource over the head's
  // rows, the tile's first row in the scalar offset.  Packed layout (runtime row stride): a per-round
  // resource (uniform base and remaining range) with one shared vector offset.
  constexpr int RS = NTK / TL::CPR;
  static_assert(RS % 16 == 0 && NTK % TL::CPR == 0, "load rounds must cover whole swizzle periods");
  const int trow = tid / TL::CPR, tpos = tid % TL::CPR;
  const uint32_t co_k = (uint32_t)((tpos ^ TL::swz_k(trow)) * 16);
  const uint32_t co_v = (uint32_t)((tpos ^ TL::swz_v(trow)) * 16);
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(kb, (uint32_t)kv_bytes);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(vb, (uint32_t)kv_bytes);
  const int wsub = tid / kWave;               // wave within this key range's group
  // LDS byte address of this wave's first 16-byte position in each ring (uniform; set
  // once, so a load's destination is scalar arithmetic on constants)
  const uint32_t kdst = __builtin_amdgcn_readfirstlane(lds_offset(kring + wsub * kWave * 16));
  const uint32_t vdst = __builtin_amdgcn_readfirstlane(lds_offset(vring + wsub * kWave * 16));
  auto load_tile = [&](int slot, const T* src, int t, bool is_v) {
    const uint32_t co = is_v ? co_v : co_k;
#pragma unroll
    for (int r = 0; r < LOADS; ++r) {
      const uint32_t dst = (is_v ? vdst : kdst) + slot * TL::BYTES + r * NTK * 16;
      if constexpr (VL) {
        // the resource must be uniform (SGPRs): t is, but not provably so
        const int64_t off = (int64_t)(__builtin_amdgcn_readfirstlane(t) * BC + r * RS) * kv_rs * 2;
        const uint32_t left = kv_bytes > off ? (uint32_t)(kv_bytes - off) : 0u;
        lds_load_16(make_rsrc(reinterpret_cast<const uint8_t*>(src) + off, left),
                    (uint32_t)(trow * kv_rs * 2) + co, 0u, dst);
      } else {
        // the tile's row offset goes in the scalar offset, the rest is loop-invariant
        lds_load_16(is_v ? vr : kr, (uint32_t)((r * RS + trow) * D * 2) + co,
                    (uint32_t)(__builtin_amdgcn_readfirstlane(t) * BC * D * 2), dst);
      }
    }
  };
  // S^T MFMAs for contraction chunks [kc0, kc1) of one tile from K slot `slot`, each K
  // fragment shared by the QB query blocks; chunk kc = 0 starts from zero.
  auto score_part = [&](f32x16 (&sc)[QB][KB], int slot, int kc0, int kc1) {
    const uint8_t* ks = kring + slot * TL::BYTES;
#pragma unroll
    for (int kc = kc0; kc < kc1; ++kc) {
#pragma unroll
      for (int kbk = 0; kbk < KB; ++kbk) {
        const int row = kbk * 32 + n;
        const int chunk = (2 * kc + grp) ^ TL::swz_k(row);
        const V8 av = as_v8<V8>(ld_lds_16(ks + row * TL::ROWB + chunk * 16));
#pragma unroll
        for (int j = 0; j < QB; ++j) sc[j][kbk] = E::mfma(av, qf[j][kc], kc == 0 ? f32x16{} : sc[j][kbk]);
      }
    }
  };

  // O^T += V^T P^T for key chunk cc from V slot `slot`, each V^T fragment shared by
  // the QB query blocks.  The 16-lane group G = lane/16 reads the 4 keys x 16 d block
  // at keys 16cc + 4g (+8 for slots 4..7), d = 32db + 16(G%2); lane s of the group
  // addresses key row s/4, d columns 4(s%4) .. +3.
  const int s16 = lane & 15;
  const int dsub = 16 * ((lane >> 4) & 1) + 4 * (s16 & 3);
  auto pv_chunk = [&](const u32x4 (&p)[QB], const u32x4 (&plo)[QB], int slot, int cc) {
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
#pragma unroll
      for (int j = 0; j < QB; ++j) {
        o[j][db] = E::mfma(as_v8<V8>(av4), as_v8<V8>(p[j]), o[j][db]);
        if constexpr (SPLIT) o[j][db] = E::mfma(as_v8<V8>(av4), as_v8<V8>(plo[j]), o[j][db]);
      }
    }
  };

  // Probabilities of key chunk cc of a scored tile for query block j, packed to the
  // element type (slot s of lane group g = key 16cc + 8(s/4) + 4g + s%4, accumulator
  // registers 8(cc%2) .. +7 of key block cc/2); their fp32 sum goes to l.
  //
  // Dropout ("M4.4 - FlashAttention-2 ...", section 0x03I): l sums the undropped
  // values; the operand of P V carries only the kept ones, and the epilogue scales by
  // 1 / (1 - p).  Registers 4q .. 4q+3 of a key block are 4 consecutive keys, so one
  // Philox call (counter (key / 4, query row, b H_q + h, offset)) decides all four.
  auto probs_chunk = [&](const f32x16 (&sc)[KB], int cc, float m_use, float& l0, float& l1, int t,
                         int j, u32x4& lo) -> u32x4 {
    const int kbk = cc >> 1;
    const int hb = (cc & 1) * 8;
    u32x4 w0 = {}, w1 = {};
    if constexpr (DROP) {
      const uint32_t grp4 = (uint32_t)(t * (BC / 4) + kbk * 8 + (hb >> 1) + grp);   // (key of register hb) / 4
      const uint32_t bhq = (uint32_t)(b * a.Hq + h);
      w0 = philox4x32_10(grp4, (uint32_t)qrow[j], bhq, a.drop.offset, a.drop.seed_lo, a.drop.seed_hi);
      w1 = philox4x32_10(grp4 + 2, (uint32_t)qrow[j], bhq, a.drop.offset, a.drop.seed_lo, a.drop.seed_hi);
    }
    uint32_t pk[4], pl[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const float e0 = fast_exp2(fmaf(sc[kbk][hb + 2 * jj], c, -m_use));
      const float x1 = fmaf(sc[kbk][hb + 2 * jj + 1], c, -m_use);
      const float e1 = (EMU == 4 || (EMU == 2 && (jj & 1))) ? soft_exp2(x1) : fast_exp2(x1);
      if (!DROP && EMU == 0 && cc == 0 && jj == 0) {
        // the step's first terms start the partial sums (0 + e is not folded by the
        // compiler, as it would be wrong for e = -0; e >= +0 here).  Not in the dropout
        // and emulated-exponential forms, where the changed schedule spills registers.
        l0 = e0;
        l1 = e1;
      } else {
        l0 += e0;
        l1 += e1;
      }
      if constexpr (DROP) {
        const u32x4& wv = jj < 2 ? w0 : w1;
        const float k0 = wv[2 * (jj & 1)] >= a.drop.thresh ? e0 : 0.f;
        const float k1 = wv[2 * (jj & 1) + 1] >= a.drop.thresh ? e1 : 0.f;
        pk[jj] = E::pack2(k0, k1);
        if constexpr (SPLIT) {
          // remainders after the bf16 rounding (bf16 -> f32 is a 16-bit shift)
          pl[jj] = E::pack2(k0 - __uint_as_float(pk[jj] << 16), k1 - __uint_as_float(pk[jj] & 0xFFFF0000u));
        }
      } else {
        pk[jj] = E::pack2(e0, e1);
      }
    }
    lo = u32x4{pl[0], pl[1], pl[2], pl[3]};
    return u32x4{pk[0], pk[1], pk[2], pk[3]};
  };

  // Row max of tile t and the rescale decision (one per wave, over its QB blocks); l
  // is rescaled here, O by the caller (after the pending P V product).
  // MASK (a compile-time tag): the tile may hold invisible keys; the unmasked form
  // carries no mask code at all.
  auto row_max = [&](auto mask_tag, f32x16 (&sc)[QB][KB], int t, float (&alpha)[QB]) -> bool {
    constexpr bool MASK = decltype(mask_tag)::value;
    float mx[QB];
    bool up = false;
#pragma unroll
    for (int j = 0; j < QB; ++j) {
      if (MASK && t >= wplan.first_masked) {
        // key offset within the tile against this lane's limit: the per-register
        // offsets are constants, so the test is one compare per register
        const int lim = klim[j] - t * BC - 4 * grp;
#pragma unroll
        for (int kbk = 0; kbk < KB; ++kbk)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            sc[j][kbk][i] = (kbk * 32 + 8 * (i >> 2) + (i & 3)) < lim ? sc[j][kbk][i] : -INFINITY;
      }
      // two chains of three-input maxima: 8 instructions per 16 values
      const f32x16& v = sc[j][0];
      float r0 = vmax(vmax(v[0], v[1]), v[2]), r1 = vmax(vmax(v[8], v[9]), v[10]);
      r0 = vmax(vmax(r0, v[3]), v[4]);
      r1 = vmax(vmax(r1, v[11]), v[12]);
      r0 = vmax(vmax(r0, v[5]), v[6]);
      r1 = vmax(vmax(r1, v[13]), v[14]);
#pragma unroll
      for (int kbk = 1; kbk < KB; ++kbk) {
        const f32x16& u = sc[j][kbk];
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          r0 = vmax(vmax(r0, u[i]), u[i + 1]);
          r1 = vmax(vmax(r1, u[8 + i]), u[8 + i + 1]);
        }
      }
      // this lane's maximum (raw units) against the row's threshold: some row of the
      // wave passes it exactly when some lane's maximum does
      mx[j] = vmax(vmax(r0, r1), vmax(v[7], v[15]));
      up = up || (mx[j] > thr[j]);
    }
    const bool moved = wave_any(up);
    if (moved) {
#pragma unroll
      for (int j = 0; j < QB; ++j) {
        const float m_new = fmaxf(m_i[j], max_pair32(mx[j]) * c);
        // the decision is per wave: a row with nothing visible yet keeps m = -inf, alpha 1
        alpha[j] = (m_new == -INFINITY) ? 1.f : fast_exp2(m_i[j] - m_new);
        m_i[j] = m_new;
        thr[j] = (m_new + kTau) * inv_c;
        l_i[j] *= alpha[j];
      }
    }
    return moved;
  };
  auto rescale_o = [&](const float (&alpha)[QB]) {
#pragma unroll
    for (int j = 0; j < QB; ++j)
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[j][db][r] *= alpha[j];
  };

  // The visited tiles are split into KS contiguous ranges, one per group of RW waves;
  // this wave's rows need the tiles of its range below we.  Every wave runs the same
  // number of steps so the workgroup barriers line up.
  const int nt = plan.n_visit;
  const int per = (nt + KS - 1) / KS;
  const int tb = min(nt, kh * per);
  const int te = min(nt, tb + per);
  const int we = max(tb, min(te, wplan.n_visit));
  const int nr = te - tb;

  // Relative tile i (absolute tb + i) lives in slot i % 2 of its ring.  Step i reads
  // K(i+1) and V(i) and loads K(i+2) and V(i+1), into the slots that K(i) and V(i-1)
  // held until step i-1.
  static_assert(DEPTH == 2, "the step schedule below is written for two slots");
  auto load_k = [&](int i) { load_tile(i % DEPTH, kb, tb + i, false); };
  auto load_v = [&](int i) { load_tile(i % DEPTH, vb, tb + i, true); };
  // Prologue: K0 V0 K1; K0 is needed first, V0 and K1 may stay in flight.
  if (nr > 0) {
    load_k(0);
    load_v(0);
  }
  if (nr > 1) {
    load_k(1);
    wait_vmcnt<2 * LOADS>();
  } else {
    wait_vmcnt<0>();
  }
  __syncthreads();
  f32x16 sa[QB][KB], sb[QB][KB];
  if (tb < we) {
    score_part(sa, 0, 0, KC);
    float alpha[QB];
    row_max(std::true_type{}, sa, tb, alpha);   // O is still zero: no rescale needed
  }

  // One step: tile t = tb + i is in `cur` (scored, its max taken); tile t+1 is scored
  // into `nxt`.
  auto step = [&](auto mask_tag, int i, f32x16 (&cur)[QB][KB], f32x16 (&nxt)[QB][KB]) {
    const int t = tb + i;
    // K(i+1) and V(i), the previous step's loads, must have landed; the barrier then
    // publishes every thread's part and frees the slots loaded below.
    wait_vmcnt<0>();
    __syncthreads();
    if (t + 2 < te) load_k(i + 2);
    if (t + 1 < te) load_v(i + 1);

    const bool has_cur = t < we;
    const bool has_nxt = t + 1 < we;
    float m_use[QB], l0[QB], l1[QB];
#pragma unroll
    for (int j = 0; j < QB; ++j) {
      m_use[j] = (m_i[j] == -INFINITY) ? 0.f : m_i[j];
      l0[j] = 0.f;
      l1[j] = 0.f;
    }
    auto probs = [&](int cc, u32x4 (&p)[QB], u32x4 (&plo)[QB]) {
#pragma unroll
      for (int j = 0; j < QB; ++j) p[j] = probs_chunk(cur[j], cc, m_use[j], l0[j], l1[j], t, j, plo[j]);
    };
    if (has_cur && has_nxt) {
      // steady state: one basic block, chunk by chunk.  The wave issues the next
      // tile's score MFMAs at raised priority, so that with several waves per SIMD the
      // matrix core gets its work ahead of the other waves' vector work.
#pragma unroll
      for (int cc = 0; cc < PC; ++cc) {
        __builtin_amdgcn_s_setprio(1);
        score_part(nxt, (i + 1) % DEPTH, cc * KPC, (cc + 1) * KPC);
        __builtin_amdgcn_s_setprio(0);
        u32x4 p[QB], plo[QB];
        probs(cc, p, plo);
        pv_chunk(p, plo, i % DEPTH, cc);
      }
    } else if (has_cur) {
#pragma unroll
      for (int cc = 0; cc < PC; ++cc) {
        u32x4 p[QB], plo[QB];
        probs(cc, p, plo);
        pv_chunk(p, plo, i % DEPTH, cc);
      }
    } else if (has_nxt) {
      score_part(nxt, (i + 1) % DEPTH, 0, KC);
    }
#pragma unroll
    for (int j = 0; j < QB; ++j) l_i[j] += l0[j] + l1[j];
    if (has_nxt) {
      float alpha[QB];
      if (row_max(mask_tag, nxt, t + 1, alpha)) rescale_o(alpha);
    }
  };
  // Step i takes the row max of tile tb + i + 1: the masked form from the first
  // masked tile of this wave's rows on.
  for (int i = 0; i < per; i += 2) {
    if (tb + i + 1 < wplan.first_masked)
      step(std::false_type{}, i, sa, sb);
    else
      step(std::true_type{}, i, sa, sb);
    if (i + 1 < per) {
      if (tb + i + 2 < wplan.first_masked)
        step(std::false_type{}, i + 1, sb, sa);
      else
        step(std::true_type{}, i + 1, sb, sa);
    }
  }

  wait_vmcnt<0>();   // no ring load may still be in flight when the LDS is reused
  if constexpr (KS > 1 && D == 64) {
    // Merge the key ranges' states of each row in one max frame ("M4.3 - IO-Aware
    // Attention ...", section 0x08B), then O = u / l and LSE = (m + log2 l) ln 2 (FA2
    // section 0x02D).  Every range hands its (m, l, u) over through LDS, and every range
    // then finishes its share of the output: units of four columns (one 8-byte store per
    // lane), unit u = 4 db + r4 going to range u % KS, so no range waits for another to
    // finish all the columns.  Layout [range][wave][block][value][lane] keeps lanes on
    // banks.
    float* xf = reinterpret_cast<float*>(lds_all);
    __syncthreads();                                   // the rings are free
#pragma unroll
    for (int j = 0; j < QB; ++j) {
      float* slot = xf + ((kh * RW + w) * QB + j) * NV * kWave + lane;
      slot[0] = m_i[j];
      slot[kWave] = l_i[j];
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int q = 0; q < 16; ++q) slot[(2 + 16 * db + q) * kWave] = o[j][db][q];
    }
    __syncthreads();
    constexpr int RSTR = RW * QB * NV * kWave;        // floats between two ranges' states
#pragma unroll
    for (int j = 0; j < QB; ++j) {
      const float* st = xf + (w * QB + j) * NV * kWave + lane;   // range r at st + r RSTR
      float mr[KS], sc[KS];
      float m = -INFINITY;
#pragma unroll
      for (int r = 0; r < KS; ++r) {
        mr[r] = st[r * RSTR];
        m = fmaxf(m, mr[r]);
      }
      float l = 0.f;
#pragma unroll
      for (int r = 0; r < KS; ++r) {
        sc[r] = (m == -INFINITY) ? 0.f : fast_exp2(mr[r] - m);
        l = fmaf(sc[r], st[r * RSTR + kWave], l);
      }
      const float l_tot = l + __shfl_xor(l, 32);
      const bool empty = (m == -INFINITY) || !(l_tot > 0.f);
      const float inv = empty ? 0.f : (DROP ? a.drop.rp : 1.f) / l_tot;
      if (qrow[j] < Sq) {
        T* ob = reinterpret_cast<T*>(a.o) + q_off + (int64_t)qrow[j] * q_rs;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            if ((4 * db + r4) % KS != kh) continue;
            float v[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              float acc = 0.f;
#pragma unroll
              for (int r = 0; r < KS; ++r) acc = fmaf(sc[r], st[r * RSTR + (2 + 16 * db + 4 * r4 + k) * kWave], acc);
              v[k] = acc * inv;
            }
            u32x2 pk;
            pk.x = E::pack2(v[0], v[1]);
            pk.y = E::pack2(v[2], v[3]);
            *reinterpret_cast<u32x2*>(ob + db * 32 + 8 * r4 + 4 * grp) = pk;
          }
        }
        if (kh == 0 && a.lse != nullptr && grp == 0) {
          a.lse[lse_off + qrow[j]] = empty ? -INFINITY : (m + __log2f(l_tot)) * ATTN_LN2;
        }
      }
    }
    return;
  }

  if constexpr (KS > 1 && D != 64) {
    // Merge the key ranges' states of each row in one max frame ("M4.3 - IO-Aware
    // Attention ...", section 0x08B): ranges 1 .. KS-1 hand their (m, l, u) to range 0
    // through LDS, all at once, and range 0 combines them (at d = 128 the shared
    // epilogue above costs the dropout form a spilled register).  Layout
    // [range][wave][block][value][lane] keeps lanes on banks.
    float* xf = reinterpret_cast<float*>(lds_all);
    __syncthreads();                                   // the rings are free
    if (kh > 0) {
#pragma unroll
      for (int j = 0; j < QB; ++j) {
        float* slot = xf + (((kh - 1) * RW + w) * QB + j) * NV * kWave + lane;
        slot[0] = m_i[j];
        slot[kWave] = l_i[j];
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int q = 0; q < 16; ++q) slot[(2 + 16 * db + q) * kWave] = o[j][db][q];
      }
    }
    __syncthreads();
    if (kh == 0) {
#pragma unroll
      for (int j = 0; j < QB; ++j) {
        float mr[KS], sc[KS];
        mr[0] = m_i[j];
        float m = m_i[j];
#pragma unroll
        for (int r = 1; r < KS; ++r) {
          mr[r] = xf[(((r - 1) * RW + w) * QB + j) * NV * kWave + lane];
          m = fmaxf(m, mr[r]);
        }
#pragma unroll
        for (int r = 0; r < KS; ++r) sc[r] = (m == -INFINITY) ? 0.f : fast_exp2(mr[r] - m);
        l_i[j] *= sc[0];
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int q = 0; q < 16; ++q) o[j][db][q] *= sc[0];
#pragma unroll
        for (int r = 1; r < KS; ++r) {
          const float* slot = xf + (((r - 1) * RW + w) * QB + j) * NV * kWave + lane;
          l_i[j] = fmaf(sc[r], slot[kWave], l_i[j]);
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int q = 0; q < 16; ++q) o[j][db][q] = fmaf(sc[r], slot[(2 + 16 * db + q) * kWave], o[j][db][q]);
        }
        m_i[j] = m;
      }
    }
  }

  // Epilogue: O = u / l once per row; LSE = (m + log2 l) ln 2 (FA2 section 0x02D).
  if (kh == 0) {
#pragma unroll
    for (int j = 0; j < QB; ++j) {
      const float l_tot = l_i[j] + __shfl_xor(l_i[j], 32);
      const bool empty = (m_i[j] == -INFINITY) || !(l_tot > 0.f);
      const float inv = empty ? 0.f : (DROP ? a.drop.rp : 1.f) / l_tot;
      if (qrow[j] < Sq) {
        T* ob = reinterpret_cast<T*>(a.o) + q_off + (int64_t)qrow[j] * q_rs;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            u32x2 pk;
            pk.x = E::pack2(o[j][db][4 * r4 + 0] * inv, o[j][db][4 * r4 + 1] * inv);
            pk.y = E::pack2(o[j][db][4 * r4 + 2] * inv, o[j][db][4 * r4 + 3] * inv);
            *reinterpret_cast<u32x2*>(ob + db * 32 + 8 * r4 + 4 * grp) = pk;
          }
        }
        if (a.lse != nullptr && grp == 0) {
          a.lse[lse_off + qrow[j]] = empty ? -INFINITY : (m_i[j] + __log2f(l_tot)) * ATTN_LN2;
        }
      }
    }
  }
}

template <typename T, int D, int QB, int RW, int KS>
hipError_t launch_fwd_t(const FwdArgs& a0, hipStream_t stream) {
  FwdArgs a = a0;
  constexpr int BQ = RW * QB * 32;
  a.nqt = (a.Sq + BQ - 1) / BQ;
  const dim3 grid((unsigned)(a.nqt * a.B * a.Hq));
  const dim3 block(RW * KS * kWave);
  const bool vl = a.cu_q != nullptr;
  if constexpr (D == 64 && QB == 1) {
    // the twelve-wave form is built for the plain forward only (the dropout and emulated
    // forms need more than its 168 registers): those take the eight-wave 2 x 4 form
    if (a.dropout || a.exp_emulated) return launch_fwd_t<T, 64, 2, 2, 4>(a0, stream);
    if (a.causal) {
      if (vl)
        hipLaunchKernelGGL((fwd_kernel<T, D, QB, RW, KS, true, true, false>), grid, block, 0, stream, a);
      else
        hipLaunchKernelGGL((fwd_kernel<T, D, QB, RW, KS, false, true, false>), grid, block, 0, stream, a);
    } else {
      if (vl)
        hipLaunchKernelGGL((fwd_kernel<T, D, QB, RW, KS, true, false, false>), grid, block, 0, stream, a);
      else
        hipLaunchKernelGGL((fwd_kernel<T, D, QB, RW, KS, false, false, false>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
  } else {
    if (a.causal) {
      if (vl)
        hipLaunchKernelGGL((fwd_kernel<T, D, QB, RW, KS, true, true, false>), grid, block, 0, stream, a);
      else if (a.dropout)
        hipLaunchKernelGGL((fwd_kernel<T, D, QB, RW, KS, false, true, true>), grid, block, 0, stream, a);
      else if (a.exp_emulated == 2)
        hipLaunchKernelGGL((fwd_kernel<T, D, QB, RW, KS, false, true, false, 2>), grid, block, 0, stream, a);
      else if (a.exp_emulated == 4)
        hipLaunchKernelGGL((fwd_kernel<T, D, QB, RW, KS, false, true, false, 4>), grid, block, 0, stream, a);
      else
        hipLaunchKernelGGL((fwd_kernel<T, D, QB, RW, KS, false, true, false>), grid, block, 0, stream, a);
    } else {
      if (vl)
        hipLaunchKernelGGL((fwd_kernel<T, D, QB, RW, KS, true, false, false>), grid, block, 0, stream, a);
      else if (a.dropout)
        hipLaunchKernelGGL((fwd_kernel<T, D, QB, RW, KS, false, false, true>), grid, block, 0, stream, a);
      else if (a.exp_emulated == 2)
        hipLaunchKernelGGL((fwd_kernel<T, D, QB, RW, KS, false, false, false, 2>), grid, block, 0, stream, a);
      else if (a.exp_emulated == 4)
        hipLaunchKernelGGL((fwd_kernel<T, D, QB, RW, KS, false, false, false, 4>), grid, block, 0, stream, a);
      else
        hipLaunchKernelGGL((fwd_kernel<T, D, QB, RW, KS, false, false, false>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
  }
}

// Head dimension 64: two query blocks per wave, 4 row waves x 2 key ranges (256 rows,
// eight waves, two per SIMD) when that gives every compute unit a workgroup; else one
// query block per wave (167 registers) in twelve-wave workgroups of 4 row waves x 3 key
// ranges (128 rows, three waves per SIMD: more waves to cover each other's stalls).
// Head dimension 128 (register bound): one query block per wave, 8 row waves (256
// rows), or 4 x 2 key ranges (128 rows) for grids under two workgroups per compute unit.
// The waves per SIMD of a launch are its waves / 4 (amdgpu_waves_per_eu above).
constexpr int kCUs = 256;

template <typename T>
hipError_t launch_fwd_dtype(const FwdArgs& a, hipStream_t stream) {
  const int64_t wgs256 = (int64_t)((a.Sq + 255) / 256) * a.B * a.Hq;
  if (a.d == 64) {
    if (wgs256 >= kCUs) return launch_fwd_t<T, 64, 2, 4, 2>(a, stream);
    return launch_fwd_t<T, 64, 1, 4, 3>(a, stream);
  }
  if (wgs256 >= 2 * kCUs) return launch_fwd_t<T, 128, 1, 8, 1>(a, stream);
  return launch_fwd_t<T, 128, 1, 4, 2>(a, stream);
}

// soft_exp2 element by element (the forward's software exponential, callable on its own)
__global__ __launch_bounds__(256) void exp2_soft_kernel(const float* x, float* y, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) y[i] = soft_exp2(x[i]);
}

}  // namespace

hipError_t attn_launch_exp2_soft(const float* x, float* y, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(exp2_soft_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, x, y, n);
  return hipGetLastError();
}

hipError_t attn_launch_fwd(const FwdArgs& a, hipStream_t stream) {
  if (a.dtype_bf16) return launch_fwd_dtype<bf16>(a, stream);
  return launch_fwd_dtype<f16>(a, stream);
}

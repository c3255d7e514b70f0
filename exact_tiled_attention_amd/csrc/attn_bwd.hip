// attn_bwd.hip -- backward of the tiled attention for gfx950 (fp16 / bf16, d = 64 / 128).
//
// "M4.4 - FlashAttention-2 Work Partitioning and the Decode Boundary", section 0x06.1:
//   1. preprocess: D_i = dO_i . O_i (section 0x06.1A) and a zeroed float32 dQ
//      accumulator;
//   2. main: one workgroup owns one K/V column tile of one (batch, K/V head) and keeps
//      its dK_j, dV_j in registers while it streams every visible query tile of every
//      query head of the group (sections 0x06.1B-0x06.1E; the group sum of section
//      0x06E happens in the owner, so no expanded dK/dV is ever written).  Per query
//      tile it recomputes S = Q K^T, P = exp(S - LSE) (masked before use), dP = dO V^T,
//      dS = P (dP - D), accumulates dV += P^T dO and dK += dS^T Q, and adds dS K into
//      the dQ accumulator with float32 atomics (section 0x06.1F: no lost update, no
//      fixed order);
//   3. convert: dQ = scale * accumulator in the requested gradient type.
//
// Wave layout of the column owner (bwd_kv_kernel, section 2 below): each 32-key group
// of the 128-key tile is served by a P wave and a dS wave on the 32x32x16 matrix core.
// S and dP are computed with the step's queries as M and the group's keys as N, so
// each lane holds ONE key: the A-operand shape of dV += P^T dO and dK += dS^T Q.  Their
// B operands (dO and Q with the query index as the contraction) come from the row-major
// staged tiles through ds_read_b64_tr_b16 (one column of 4 consecutive rows per lane).
// dQ needs dS with queries as rows: dS goes to LDS key-major and comes back through the
// same transpose read, against K (row-major in LDS).  Staged rows are unpadded, their
// 16-byte chunks XOR-swizzled so that the fragment reads and the transpose reads of a
// tile both hit distinct banks.
#include <type_traits>

#include "../../include/attn.h"
#include "attn_device.h"
#include "attn_launch.h"
#include "attn_philox.h"
#include "tile_plan.h"

namespace {

constexpr int kWave = 64;
constexpr int kNT = 256;      // preprocess / convert kernels

// ---------------------------------------------------------------------------------
// 1. D = rowsum(dO * O) and dQ accumulator clear.  One row per LPR lanes.
template <typename T, int D>
__global__ __launch_bounds__(kNT) void bwd_pre_kernel(BwdArgs a) {
  constexpr int LPR = D / 8;
  constexpr int RPB = kNT / LPR;       // rows per block
  const int64_t rows = (int64_t)a.B * a.Hq * a.Sq;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const int c8 = threadIdx.x % LPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 ov = ld_global_16(reinterpret_cast<const T*>(a.o) + row * D + 8 * c8);
    const u32x4 dv = ld_global_16(reinterpret_cast<const T*>(a.dO) + row * D + 8 * c8);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t x = ov[w], y = dv[w];
      acc += Elem<T>::to_f(__builtin_bit_cast(T, (uint16_t)(x & 0xFFFF))) *
             Elem<T>::to_f(__builtin_bit_cast(T, (uint16_t)(y & 0xFFFF)));
      acc += Elem<T>::to_f(__builtin_bit_cast(T, (uint16_t)(x >> 16))) *
             Elem<T>::to_f(__builtin_bit_cast(T, (uint16_t)(y >> 16)));
    }
    if (a.dq_acc != nullptr) {          // the atomic dQ accumulator (not in deterministic mode)
      float* dq = a.dq_acc + row * D + 8 * c8;
      const u32x4 z = {0u, 0u, 0u, 0u};
      st_global_16(dq, z);
      st_global_16(dq + 4, z);
    }
  }
  // sum over the LPR lanes of the row (LPR = 8 or 16 consecutive lanes)
#pragma unroll
  for (int s = 1; s < LPR; s <<= 1) acc += __shfl_xor(acc, s);
  // owners on fp16 copies of bf16 operands take D in the scale of dP (section 5)
  if (row < rows && c8 == 0) a.delta[row] = a.f16_fac != nullptr ? acc * a.f16_fac[1] : acc;
}

// ---------------------------------------------------------------------------------
// 3. dQ = scale * accumulator.
template <typename G>
__global__ __launch_bounds__(kNT) void bwd_convert_kernel(BwdArgs a, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * kNT + threadIdx.x;
  if (i >= n4) return;
  const f32x4 x = reinterpret_cast<const f32x4*>(a.dq_acc)[i];
  G* out = reinterpret_cast<G*>(a.dq) + 4 * i;
#pragma unroll
  for (int j = 0; j < 4; ++j) out[j] = (G)(x[j] * a.scale);
}

template <typename G> __device__ inline void store_grad(G* p, float x) { *p = (G)x; }

// bf16 keeps 8 significant bits; P and dS feed the dV / dK sums as hi + lo pairs.
template <typename T> constexpr bool kSplit = false;
template <> constexpr bool kSplit<bf16> = true;

typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ inline u32x2 tr_read(const uint8_t* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p));
}

template <typename T> struct M16;
template <> struct M16<f16> {
  static __device__ inline f32x4 run(const u32x4& a, const u32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};
template <> struct M16<bf16> {
  static __device__ inline f32x4 run(const u32x4& a, const u32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

// Pack 8 floats (two groups of 4) into element values (hi) and, for bf16, the
// residuals x - hi (lo).
template <typename T>
__device__ inline void split_pack4x2(const f32x4& x0, const f32x4& x1, u32x4& hi, u32x4& lo) {
  const float r[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
  hi.x = Elem<T>::pack2(r[0], r[1]);
  hi.y = Elem<T>::pack2(r[2], r[3]);
  hi.z = Elem<T>::pack2(r[4], r[5]);
  hi.w = Elem<T>::pack2(r[6], r[7]);
  if (kSplit<T>) {
    float e[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t hw = hi[j];
      e[2 * j] = r[2 * j] - __builtin_bit_cast(float, hw << 16);
      e[2 * j + 1] = r[2 * j + 1] - __builtin_bit_cast(float, hw & 0xFFFF0000u);
    }
    lo.x = Elem<T>::pack2(e[0], e[1]);
    lo.y = Elem<T>::pack2(e[2], e[3]);
    lo.z = Elem<T>::pack2(e[4], e[5]);
    lo.w = Elem<T>::pack2(e[6], e[7]);
  } else {
    lo = u32x4{0u, 0u, 0u, 0u};
  }
}

// 8 E4M3 codes -> 8 bf16 values, one instruction per pair (exact: every E4M3 value is
// a bf16 value, and the conversion's scale is 1).
__device__ inline u32x4 e4m3x8_bf16(const u32x2& w) {
  return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w.x, 1.f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w.x, 1.f, true)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w.y, 1.f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w.y, 1.f, true))};
}

// ---------------------------------------------------------------------------------
// 2. Column owner with split roles (every backward: 16-bit or fp8 operands, dropout).
// One workgroup owns a 128-key tile; four key groups of 32 keys, each served by two
// waves on one SIMD: wave w (role P) keeps the group's K rows in registers, computes
// S = Q K^T and P = exp(S - LSE) and accumulates dV += P^T dO; wave w + 4 (role dS)
// keeps the V rows, computes dP = dO V^T, takes P from its partner through LDS, forms
// dS = P (dP - D) and accumulates dK += dS^T Q.  Both products of a role use 32x32x16
// matrix-core tiles with the step's 32 queries and the group's 32 keys, whose
// accumulator layout (lane = key, registers = queries) is already the A-operand layout
// of the dV / dK products, and one wave holds one accumulator set (64 registers at
// d = 128), so two waves share each SIMD and cover each other's waits.  Per step the
// waves read only the staged Q and dO tiles (fragment and transpose reads).  With DQ,
// dS goes to LDS key-major and the eight waves compute dQ = dS K in 16x16 tiles over
// the tile's 128 keys (transpose reads of dS and of the K tile kept in LDS), added
// with float32 atomics ([FA2] section 0x06.1F).  Q and dO tiles go straight from
// HBM/L2 into LDS (one step ahead).  dS has two slots, so the dQ tiles of step t run at
// the start of step t + 1, after its first barrier: two barriers per step (staged tiles
// and the previous dS visible; P visible), and the atomics are issued a whole step
// before the wait that precedes the next barrier.  Without dQ (and with 16-bit operands
// and no dropout) the dS waves lag one query tile behind the P waves instead: step k
// runs S, P and dV of tile k and dP, dS and dK of tile k - 1, one barrier per step.
constexpr int kKW = 32;               // keys per group
constexpr int kKG = 4;                // key groups per workgroup
constexpr int kKVT = kKW * kKG;       // keys per workgroup
constexpr int kKVW = 2 * kKG;         // waves per workgroup
constexpr int kKVQ = 32;              // queries per step

// QS staged Q / dO slots and PSL P-handoff slots (4 and 2 in the lagged schedule); the
// K tile and the dS slots exist only with dQ.
template <int D, int QS, int PSL, bool DQ>
struct KvLds {
  static constexpr int ROWB = D * 2;
  static constexpr int QT = kKVQ * ROWB;            // one staged Q or dO tile
  static constexpr int Q0 = 0;                      // Q slots
  static constexpr int DO0 = QS * QT;               // dO slots
  static constexpr int K = 2 * QS * QT;             // K tile [128 keys][D]
  static constexpr int DS = K + (DQ ? kKVT * ROWB : 0);   // dS slots 0, 1: [128 keys][32 queries], 64-byte rows
  static constexpr int DSS = 2 * kKVT * kKVQ * 2;   // one slot: the values, then their bf16 residuals
  static constexpr int P = DS + (DQ ? 2 * DSS : 0); // P handoff [slot][group][16 registers][64 lanes] float32
  static constexpr int PS = kKG * 16 * kWave * 4;   // one P slot
  static constexpr int Z = P + PSL * PS;            // dropout keep bits [role][group][64 lanes] uint32 ([slot][half][group][lanes] when lagged)
  static constexpr int BYTES = Z + 4 * kKG * kWave * 4;
};

// Chunk swizzle of staged rows (Q, dO, K): chunk p of row r at position p ^ kv_swz(r).
// The fragment reads take one chunk of 16 consecutive rows (bank groups = low three
// bits of the position: 2(r&3) + bit 2 of r runs through all eight over 8 rows); the
// transpose reads take two adjacent chunks of 4 consecutive rows (XOR with 2j + const
// for j = 0..3 keeps the 8 positions distinct).
template <int D> __device__ inline int kv_swz(int r) {
  const int s = 2 * (r & 3) + ((r >> 2) & 1) + 8 * ((r >> 3) & 1);
  return D == 128 ? s : (s & 7);
}
// dS rows: 16-byte unit u of key row r at u ^ 2((r >> 1) & 1) (a transpose read's 4 rows
// x 2 units then cover the eight bank groups); the residuals follow the values.
__device__ inline int kv_ds_off(int key, int q) {
  const int u = q >> 3;
  return key * (kKVQ * 2) + ((u ^ (2 * ((key >> 1) & 1))) * 16) + (q & 7) * 2;
}

// F8 (T = bf16, with DQ): Q, K, V are E4M3 codes with per-128-row float32 descales,
// widened exactly to bf16; a 128-key tile is one descale block and a 32-query step lies
// in one, so S = (scale dQ dK) Q8 K8^T, dP = dV (dO V8^T), dK_d = scale sum (dQ dS)^T Q8,
// dQ_d = scale dK sum dS K8 and dV_d = P^T dO.  The Q tile is loaded into registers at
// the start of a step and widened into its LDS slot at the end (dO still goes straight
// to LDS).
// DROP: regenerate the forward's dropout decisions Z (keep / (1 - p)) and use
// dV += (P Z)^T dO, dS = P (Z dP - D).  The roles split the Philox work: in the lagged
// schedule the P wave draws query groups 2, 3 of its tile k and the dS wave groups 0, 1
// of tile k + 1 a step ahead, each handing its half to the other through LDS.
template <typename T, typename G, int D, bool CAUSAL, bool DQ, bool F8 = false, bool DROP = false>
__global__ __launch_bounds__(kKVW * kWave) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_kv_kernel(BwdArgs a) {
  typedef Elem<T> E;
  typedef typename E::v8 V8;
  typedef M16<T> MF;
  // Lagged schedule (no dQ, 16-bit operands): in step k the P waves take
  // query tile k (S, P, dV) while the dS waves take tile k - 1 (dP, dS) with the P their
  // partners handed over a step earlier, and the dK product of tile k - 2 (its dS kept
  // in registers): the roles never wait for each other within a step (one barrier per
  // step, four Q / dO slots, two P slots), and while the P wave of a SIMD issues its S
  // products, its exponentials and its dV products, its dS partner issues dK products,
  // dP products and the vector work of dS, so that the matrix core and the vector ALU
  // get work from the two waves in turn.
  constexpr bool LAG = !DQ && !F8;
  typedef KvLds<D, LAG ? 4 : 2, LAG ? 2 : 1, DQ> L;
  constexpr int KC = D / 16;                 // contraction chunks of S and dP
  constexpr int DB = D / 32;                 // 32-wide d blocks of dK, dV
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int WL = kKVQ * CPR / kWave;     // wave loads (1 KiB each) per staged tile
  constexpr int DQB = 2 * (D / 16);          // dQ tiles (16 queries x 16 d) per step
  static_assert(WL * kWave == kKVQ * CPR && kWave % CPR == 0, "staging splits evenly");

  __shared__ __attribute__((aligned(1024))) uint8_t lds[L::BYTES];
  __shared__ __attribute__((aligned(16))) float s_lse[LAG ? 4 : 2][kKVQ];
  __shared__ __attribute__((aligned(16))) float s_del[LAG ? 4 : 2][kKVQ];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int grp = w % kKG;                   // key group
  const bool role_p = w < kKG;               // P / dV wave, else dP / dS / dK wave
  const int n = lane & 31;
  const int g = lane >> 5;
  const int s16 = lane & 15;
  const int gh = (lane >> 4) & 1;            // which 16-column half a transpose read takes

  // key tiles slowest in the linear order: under causal masking the tiles with the most
  // visible query tiles start first
  const int nbkv = a.B * a.Hkv;
  const int lin = blockIdx.x + gridDim.x * blockIdx.y;
  const int jt = lin / nbkv;
  const int bkv = lin - jt * nbkv;
  const int b = bkv / a.Hkv;
  const int kvh = bkv - b * a.Hkv;
  const int k0 = jt * kKVT;
  const int k1 = min(k0 + kKVT, a.Sk);
  const bool key_tail = (k0 + kKVT) > a.Sk;
  const int delta = a.Sk - a.Sq;
  const int kr_own = kKW * grp + n;          // this lane's key row within the tile
  const int mykey = k0 + kr_own;             // this lane's key (column of S / dP)

  // The group's K rows (role P) or V rows (role dS) as B fragments (slots d 16kc + 8g
  // .. +7); role P also stores its K rows into the LDS tile for the dQ product.  Keys
  // past S_k read as zero.
  constexpr int EB = F8 ? 1 : 2;             // bytes per stored Q / K / V element
  const uint8_t* kvbase = reinterpret_cast<const uint8_t*>(role_p ? a.k : a.v) + ((int64_t)(b * a.Hkv + kvh) * a.Sk) * D * EB;
  const __amdgpu_buffer_rsrc_t kvrs = make_rsrc(kvbase, (uint32_t)a.Sk * D * EB);
  // fp8: this workgroup's key and value descales (its 128 keys are one scale block)
  float dk_s = 1.f, dv_s = 1.f;
  if constexpr (F8) {
    const int nkb = (a.Sk + kKVT - 1) / kKVT;
    dk_s = a.k_scale[(int64_t)(b * a.Hkv + kvh) * nkb + jt];
    dv_s = a.v_scale[(int64_t)(b * a.Hkv + kvh) * nkb + jt];
  }
  // fp16 copies of bf16 operands: the score factor (section 5; D arrives in the scale of
  // dP from the preprocess, the dK and dV factors are read at the end)
  const float sl2b = a.f16_fac != nullptr ? a.f16_fac[0] : a.scale_log2;
  V8 bf[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    u32x4 x;
    if constexpr (F8)
      x = e4m3x8_bf16(buf_load_8(kvrs, (uint32_t)(mykey * D + 16 * kc + 8 * g)));
    else
      x = buf_load_16(kvrs, (uint32_t)(mykey * D + 16 * kc + 8 * g) * 2);
    bf[kc] = as_v8<V8>(x);
    if (DQ && role_p) st_lds_16(lds + L::K + kr_own * L::ROWB + (((2 * kc + g) ^ kv_swz<D>(kr_own)) * 16), x);
  }

  f32x16 acc[DB];                            // dV (role P) or dK (role dS) of the group
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = f32x16{};

  const ColPlan cp = plan_cols(k0, k1, a.Sq, a.Sk, kKVQ, CAUSAL);
  const int nq = cp.n_qtiles - cp.first_qtile;
  const int nsteps = nq * a.group;
  auto step_coords = [&](int step, int& h, int& qt) {
    h = kvh * a.group + step / nq;
    qt = cp.first_qtile + step % nq;
  };

  // Direct HBM -> LDS staging of one step's Q and dO tiles into slot sb: wave load j
  // fills LDS bytes [1024 j, 1024 j + 1024) of the tile, i.e. row j 64 / CPR + lane / CPR
  // at position lane % CPR, which holds global chunk position ^ kv_swz(row).
  const int lrow = lane / CPR, lpos = lane % CPR;
  // fp8: the step's Q codes, 8 per thread (chunk tid of the 32 x D tile), loaded by
  // stage() and widened into the LDS slot by store_q()
  constexpr int Q8C = kKVQ * D / 8;          // 8-byte chunks of a Q8 tile
  u32x2 q8 = {0u, 0u};
  auto stage_at = [&](int h, int qt, int sb) {
    const int64_t base = ((int64_t)(b * a.Hq + h) * a.Sq) * D;
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(reinterpret_cast<const uint8_t*>(a.q) + base * EB, (uint32_t)a.Sq * D * EB);
    const __amdgpu_buffer_rsrc_t dr = make_rsrc(reinterpret_cast<const T*>(a.dO) + base, (uint32_t)a.Sq * D * 2);
#pragma unroll
    for (int j = w; j < WL; j += kKVW) {
      const int row = j * kWave / CPR + lrow;
      const uint32_t voff = (uint32_t)((row * D) + 8 * (lpos ^ kv_swz<D>(row))) * 2;
      const uint32_t soff = (uint32_t)(qt * kKVQ * D * 2);
      const uint32_t dq = __builtin_amdgcn_readfirstlane(lds_offset(lds + L::Q0 + sb * L::QT + j * kWave * 16));
      const uint32_t dd = __builtin_amdgcn_readfirstlane(lds_offset(lds + L::DO0 + sb * L::QT + j * kWave * 16));
      if constexpr (!F8) lds_load_16(qr, voff, soff, dq);
      lds_load_16(dr, voff, soff, dd);
    }
    if constexpr (F8) {
      if (tid < Q8C) q8 = buf_load_8(qr, (uint32_t)((qt * kKVQ + tid / (D / 8)) * D + 8 * (tid % (D / 8))));
    }
  };
  auto stage = [&](int step, int sb) {
    int h, qt;
    step_coords(step, h, qt);
    stage_at(h, qt, sb);
  };
  auto store_q = [&](int sb) {
    if constexpr (F8) {
      if (tid < Q8C) {
        const int row = tid / (D / 8), c = tid % (D / 8);
        st_lds_16(lds + L::Q0 + sb * L::QT + row * L::ROWB + ((c ^ kv_swz<D>(row)) * 16), e4m3x8_bf16(q8));
      }
    }
  };
  // fp8: the query descale of a step (its 32 rows lie in one 128-row block)
  const int nqb = (a.Sq + kKVT - 1) / kKVT;
  auto q_descale = [&](int h, int qt) {
    return F8 ? a.q_scale[(int64_t)(b * a.Hq + h) * nqb + (qt * kKVQ) / kKVT] : 1.f;
  };
  // LSE (base 2) and D of the step's rows, through registers
  float pre = 0.f;
  auto fetch_rows_at = [&](int h, int qt) {
    if (tid < 2 * kKVQ) {
      const int qr = qt * kKVQ + (tid & (kKVQ - 1));
      const int64_t ri = (int64_t)(b * a.Hq + h) * a.Sq + qr;
      pre = qr < a.Sq ? (tid < kKVQ ? a.lse[ri] * ATTN_LOG2E : a.delta[ri]) : (tid < kKVQ ? INFINITY : 0.f);
    }
  };
  auto fetch_rows = [&](int step) {
    int h, qt;
    step_coords(step, h, qt);
    fetch_rows_at(h, qt);
  };
  auto store_rows = [&](int sb) {
    if (tid < kKVQ) s_lse[sb][tid] = pre;
    else if (tid < 2 * kKVQ) s_del[sb][tid - kKVQ] = pre;
  };

  // Transpose read of a row-major staged tile: the 16-lane group reads rows r0 .. r0+3
  // at columns c0 .. c0+15 (lane s addresses row r0 + s/4, columns c0 + 4(s%4) .. +3);
  // lane i receives column c0 + i of the 4 rows.
  auto tr_rows = [&](const uint8_t* tile, int r0, int c0) -> u32x2 {
    const int r = r0 + (s16 >> 2);
    const int col = c0 + 4 * (s16 & 3);
    return tr_read(tile + r * L::ROWB + (((col >> 3) ^ kv_swz<D>(r)) * 16) + (col & 7) * 2);
  };
  float* const phand0 = reinterpret_cast<float*>(lds + L::P) + grp * 16 * kWave + lane;   // [reg][lane]
  uint32_t* zhand = reinterpret_cast<uint32_t*>(lds + L::Z) + grp * kWave + lane;  // [role][group][lane]
  uint32_t keep = 0;                         // dropout: this step's decisions (bit i = register i)
  int h_cur = 0;                             // this step's query head (the dropout counter)

  // Dropout decisions of a step (query head h, query tile qt) for this lane's key, as bit
  // i for query 8(i/4) + 4g + i%4; draw_at(h, qt, j0) makes query groups j0 and j0 + 1.
  // The four lanes of a key quad (n = 4c .. 4c+3) share the Philox counter word key / 4:
  // lane e = n % 4 makes the call of query 8j + 4g + e, and in round r it sends word
  // (e + r) % 4 and receives, from quad lane (e - r) % 4, word e (its own key) of that
  // lane's query.
  auto draw_at = [&](int h, int qt, int j0) -> uint32_t {
    const int e = n & 3;
    uint32_t kb = 0;
#pragma unroll
    for (int j = j0; j < j0 + 2; ++j) {
      const u32x4 wv = philox4x32_10((uint32_t)mykey >> 2, (uint32_t)(qt * kKVQ + 8 * j + 4 * g + e),
                                     (uint32_t)(b * a.Hq + h), a.drop.offset, a.drop.seed_lo, a.drop.seed_hi);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int wi = (e + r) & 3;
        const uint32_t send = wi == 0 ? wv[0] : wi == 1 ? wv[1] : wi == 2 ? wv[2] : wv[3];
        const uint32_t got = (uint32_t)__shfl((int)send, (lane & ~3) | ((e - r) & 3));
        kb |= (got >= a.drop.thresh ? 1u : 0u) << (4 * j + ((e - r) & 3));
      }
    }
    return kb;
  };

  // Phase 1: S (role P) or dP (role dS) for the group's 32 keys: A = Q / dO rows (row n,
  // chunk 2kc + g) of the staged tile, B = the group's K / V fragments.  Role P turns S
  // into P (masked) and hands it to its partner.
  auto phase1 = [&](auto masked_tag, int qt, int sb, float sl2, f32x16& x, int ps) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    float* const phand = phand0 + ps * (L::PS / 4);
    const uint8_t* src = lds + (role_p ? L::Q0 : L::DO0) + sb * L::QT;
    x = f32x16{};
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const V8 af = as_v8<V8>(ld_lds_16(src + n * L::ROWB + (((2 * kc + g) ^ kv_swz<D>(n)) * 16)));
      x = E::mfma(af, bf[kc], x);
    }
    // Two-barrier schedule: the roles split the step's dropout draws, the dS wave making
    // query groups 0, 1 after its dP product, the P wave groups 2, 3 after its
    // probabilities; each hands its half to the partner through LDS.
    auto draw = [&](int j0) -> uint32_t { return draw_at(h_cur, qt, j0); };
    if (DROP && !LAG && !role_p) {
      keep = draw(0);
      zhand[0] = keep;
    }
    if (role_p) {
      // register i holds query 8(i/4) + 4g + i%4 of the step
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 lv = *reinterpret_cast<const f32x4*>(&s_lse[sb][8 * j + 4 * g]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * j + e;
          float pv = fast_exp2(fmaf(x[i], sl2, -lv[e]));
          if constexpr (MASKED) {
            const int qr = qt * kKVQ + 8 * j + 4 * g + e;
            const bool vis = qr < a.Sq && mykey < a.Sk && (!CAUSAL || mykey <= qr + delta);
            pv = vis ? pv : 0.f;
          }
          x[i] = pv;
          phand[i * kWave] = pv;
        }
      }
      if constexpr (DROP && !LAG) {
        keep = draw(2);
        zhand[kKG * kWave] = keep;
      }
    }
  };

  // Phase 2: role P: dV += P^T dO; role dS: dS = P (dP - D), dK += dS^T Q, dS to LDS.
  // Chunk c: A = registers 8c .. 8c+7 (queries 16c + 4g + s%4 and 16c + 8 + 4g + s%4),
  // B = dO / Q columns by transpose reads of those rows; bf16 carries P and dS as
  // hi + lo pairs.
  auto phase2 = [&](int sb, float dq_s, f32x16& x, int ps) {
    const float* const phand = phand0 + ps * (L::PS / 4);
    uint8_t* dsv = lds + L::DS + sb * L::DSS;
    uint8_t* dsr = dsv + L::DSS / 2;
    const uint8_t* src = lds + (role_p ? L::DO0 : L::Q0) + sb * L::QT;
    if constexpr (DROP && !LAG) {
      keep |= role_p ? zhand[0] : zhand[kKG * kWave];
    }
    if (!role_p) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 dl = *reinterpret_cast<const f32x4*>(&s_del[sb][8 * j + 4 * g]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * j + e;
          const float z = DROP ? (((keep >> i) & 1u) ? a.drop.rp : 0.f) : 1.f;
          x[i] = phand[i * kWave] * (z * (F8 ? dv_s * x[i] : x[i]) - dl[e]);
        }
      }
    } else if constexpr (DROP) {
      // dV takes the kept probabilities, scaled by 1 / (1 - p)
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] *= ((keep >> i) & 1u) ? a.drop.rp : 0.f;
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int r0 = 16 * c + 4 * g;
      u32x4 hi, lo;
      split_pack4x2<T>(f32x4{x[8 * c + 0], x[8 * c + 1], x[8 * c + 2], x[8 * c + 3]},
                       f32x4{x[8 * c + 4], x[8 * c + 5], x[8 * c + 6], x[8 * c + 7]}, hi, lo);
      if (DQ && !role_p) {
        // dS key-major: this lane's key row, queries r0 .. r0+3 and r0+8 .. r0+11
        st_lds_8(dsv + kv_ds_off(kr_own, r0), u32x2{hi.x, hi.y});
        st_lds_8(dsv + kv_ds_off(kr_own, r0 + 8), u32x2{hi.z, hi.w});
        if constexpr (kSplit<T>) {
          st_lds_8(dsr + kv_ds_off(kr_own, r0), u32x2{lo.x, lo.y});
          st_lds_8(dsr + kv_ds_off(kr_own, r0 + 8), u32x2{lo.z, lo.w});
        }
      }
      if constexpr (F8) {
        // the dK product takes dS dQ (the stored dS stays unscaled for dQ)
        if (!role_p)
          split_pack4x2<T>(f32x4{x[8 * c + 0], x[8 * c + 1], x[8 * c + 2], x[8 * c + 3]} * dq_s,
                           f32x4{x[8 * c + 4], x[8 * c + 5], x[8 * c + 6], x[8 * c + 7]} * dq_s, hi, lo);
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int c0 = 32 * db + 16 * gh;
        const u32x2 t0 = tr_rows(src, r0, c0), t1 = tr_rows(src, r0 + 8, c0);
        const V8 bt = as_v8<V8>(u32x4{t0.x, t0.y, t1.x, t1.y});
        acc[db] = E::mfma(as_v8<V8>(hi), bt, acc[db]);
        if constexpr (kSplit<T>) acc[db] = E::mfma(as_v8<V8>(lo), bt, acc[db]);
      }
    }
  };

  // Lagged dS role: dS = P (dP - D) of the step in slot sb, packed (chunk c: queries 16c +
  // 4g + s%4 and + 8), and, a step later, its dK product against that step's Q tile.
  auto ds_make = [&](int sb, f32x16& x, int ps, u32x4 (&hi)[2], u32x4 (&lo)[2]) {
    const float* const phand = phand0 + ps * (L::PS / 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 dl = *reinterpret_cast<const f32x4*>(&s_del[sb][8 * j + 4 * g]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * j + e;
        const float z = DROP ? (((keep >> i) & 1u) ? a.drop.rp : 0.f) : 1.f;
        x[i] = phand[i * kWave] * (z * x[i] - dl[e]);
      }
    }
#pragma unroll
    for (int c = 0; c < 2; ++c)
      split_pack4x2<T>(f32x4{x[8 * c + 0], x[8 * c + 1], x[8 * c + 2], x[8 * c + 3]},
                       f32x4{x[8 * c + 4], x[8 * c + 5], x[8 * c + 6], x[8 * c + 7]}, hi[c], lo[c]);
  };
  auto dk_apply = [&](const u32x4 (&hi)[2], const u32x4 (&lo)[2], int sb) {
    const uint8_t* src = lds + L::Q0 + sb * L::QT;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int r0 = 16 * c + 4 * g;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int c0 = 32 * db + 16 * gh;
        const u32x2 t0 = tr_rows(src, r0, c0), t1 = tr_rows(src, r0 + 8, c0);
        const V8 bt = as_v8<V8>(u32x4{t0.x, t0.y, t1.x, t1.y});
        acc[db] = E::mfma(as_v8<V8>(hi[c]), bt, acc[db]);
        if constexpr (kSplit<T>) acc[db] = E::mfma(as_v8<V8>(lo[c]), bt, acc[db]);
      }
    }
  };

  // Phase 3: dQ = dS K over the tile's 128 keys in 16x16 tiles (16 queries x 16 d): wave w
  // takes query block w / 4 and TPW adjacent d blocks, so its dS reads serve all of them.
  // A = dS (lane = query column, slots = keys 32kc + 8G + s%4 and + 4, by transpose reads
  // of the key-major dS), B = K (lane = d column, same keys, transpose reads of the K
  // tile).  Result lane = d column, registers = queries 4G + i.
  constexpr int TPW = DQB / kKVW;            // dQ tiles per wave
  const int G4 = lane >> 4;
  auto phase3 = [&](int h, int qt, int sb) {
    const uint8_t* dsv = lds + L::DS + sb * L::DSS;
    const uint8_t* dsr = dsv + L::DSS / 2;
    float* dqb = a.dq_acc + ((int64_t)(b * a.Hq + h) * a.Sq) * D;
    const int tq = w / (kKVW / 2);
    const int db0 = (w % (kKVW / 2)) * TPW;
    f32x4 dq[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) dq[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < kKVT / 32; ++kc) {
      const int r0 = 32 * kc + 8 * G4;
      const int qc = 16 * tq + 4 * (s16 & 3);
      const int kr = r0 + (s16 >> 2);
      const u32x2 a0 = tr_read(dsv + kv_ds_off(kr, qc)), a1 = tr_read(dsv + kv_ds_off(kr + 4, qc));
      u32x2 e0 = {0u, 0u}, e1 = {0u, 0u};
      if constexpr (kSplit<T>) {
        e0 = tr_read(dsr + kv_ds_off(kr, qc));
        e1 = tr_read(dsr + kv_ds_off(kr + 4, qc));
      }
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const u32x2 b0 = tr_rows(lds + L::K, r0, 16 * (db0 + t)), b1 = tr_rows(lds + L::K, r0 + 4, 16 * (db0 + t));
        const u32x4 kb4 = {b0.x, b0.y, b1.x, b1.y};
        dq[t] = MF::run(u32x4{a0.x, a0.y, a1.x, a1.y}, kb4, dq[t]);
        if constexpr (kSplit<T>) dq[t] = MF::run(u32x4{e0.x, e0.y, e1.x, e1.y}, kb4, dq[t]);
      }
    }
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int dcol = 16 * (db0 + t) + s16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int qr = qt * kKVQ + 16 * tq + 4 * G4 + i;
        if (qr < a.Sq) unsafeAtomicAdd(dqb + (int64_t)qr * D + dcol, F8 ? dq[t][i] * dk_s : dq[t][i]);
      }
    }
  };

  if (nsteps > 0) {
    stage(0, 0);
    store_q(0);
    fetch_rows(0);
  }
  if constexpr (LAG) {
    // Step k: the rows of tile k are stored and tile k has landed; after the barrier
    // every wave has finished step k - 1 (P(k - 1) is visible, and the Q / dO slot of
    // tile k - 3 is free for tile k + 1).  One step more than tiles: the last dK.
    // coordinates of steps k - 1, k and k + 1, advanced without divisions
    int qt_prev = 0, h_k = 0, qt_k = 0, h_next = 0, qt_next = 0;
    if (nsteps > 0) step_coords(0, h_k, qt_k);
    auto advance = [&](int& h, int& qt) {
      if (++qt == cp.n_qtiles) {
        qt = cp.first_qtile;
        ++h;
      }
    };
    h_next = h_k;
    qt_next = qt_k;
    advance(h_next, qt_next);
    u32x4 dsh[2] = {}, dsl[2] = {};          // dS waves: the packed dS of the previous step
    // dropout halves [slot][half][group][lane]: half 0 (groups 2, 3) from the P wave of the
    // tile, half 1 (groups 0, 1) from the dS wave a step ahead; slot = tile & 1
    uint32_t* const zs = reinterpret_cast<uint32_t*>(lds + L::Z) + grp * kWave + lane;
    auto zslot = [&](int slot, int half) { return zs + (2 * slot + half) * (kKG * kWave); };
    if constexpr (DROP) {
      if (!role_p && nsteps > 0) *zslot(0, 1) = draw_at(h_k, qt_k, 0);
    }
    for (int k = 0; k <= nsteps + 1; ++k) {
      if (k < nsteps) store_rows(k % 4);
      wait_vmcnt<0>();
      __syncthreads();
      if (k + 1 < nsteps) {
        stage_at(h_next, qt_next, (k + 1) % 4);
        fetch_rows_at(h_next, qt_next);
      }
      if (role_p) {
        if (k < nsteps) {
          const int h = h_k, qt = qt_k;
          const bool masked = key_tail || qt < cp.nomask_qtile || (qt + 1) * kKVQ > a.Sq;
          f32x16 x;
          if (masked)
            phase1(std::true_type{}, qt, k % 4, sl2b, x, k & 1);
          else
            phase1(std::false_type{}, qt, k % 4, sl2b, x, k & 1);
          if constexpr (DROP) {
            const uint32_t half0 = draw_at(h, qt, 2);
            *zslot(k & 1, 0) = half0;
            keep = half0 | *zslot(k & 1, 1);
          }
          phase2(k % 4, 1.f, x, k & 1);
        }
      } else {
        if (k >= 2) dk_apply(dsh, dsl, (k - 2) % 4);
        uint32_t half1 = 0;
        if (DROP && k + 1 < nsteps) half1 = draw_at(h_next, qt_next, 0);
        if (k >= 1 && k <= nsteps) {
          f32x16 x;
          phase1(std::false_type{}, qt_prev, (k - 1) % 4, sl2b, x, (k - 1) & 1);   // dP (P carries the mask)
          if constexpr (DROP) keep = *zslot((k - 1) & 1, 0) | *zslot((k - 1) & 1, 1);
          ds_make((k - 1) % 4, x, (k - 1) & 1, dsh, dsl);
        }
        // tile k + 1's half goes where tile k - 1's was, after that was read above
        if (DROP && k + 1 < nsteps) *zslot((k + 1) & 1, 1) = half1;
      }
      qt_prev = qt_k;
      h_k = h_next;
      qt_k = qt_next;
      advance(h_next, qt_next);
    }
    wait_vmcnt<0>();
  } else {
    // With DQ one more pass runs the last step's dQ tiles.
    const int npass = (DQ && nsteps > 0) ? nsteps + 1 : nsteps;
    int ph = 0, pqt = 0;                       // the previous step's head and query tile
    for (int step = 0; step < npass; ++step) {
      const bool work = step < nsteps;
      int h = 0, qt = 0;
      if (work) step_coords(step, h, qt);
      h_cur = h;
      const int sb = step & 1;
      if (work) store_rows(sb);
      // this step's tiles have landed (own loads) and, after the barrier, everyone's;
      // every wave has finished step - 1 (its P handoff, its dS writes, and the staged
      // slot the loads below overwrite)
      wait_vmcnt<0>();
      __syncthreads();
      if (step + 1 < nsteps) {
        stage(step + 1, sb ^ 1);
        fetch_rows(step + 1);
      }
      if constexpr (DQ) {
        if (step > 0) phase3(ph, pqt, sb ^ 1);
      }
      if (work) {
        const bool masked = key_tail || qt < cp.nomask_qtile || (qt + 1) * kKVQ > a.Sq;
        const float dq_s = q_descale(h, qt);
        const float sl2 = F8 ? a.scale_log2 * dq_s * dk_s : sl2b;
        f32x16 x;
        if (masked)
          phase1(std::true_type{}, qt, sb, sl2, x, 0);
        else
          phase1(std::false_type{}, qt, sb, sl2, x, 0);
        __syncthreads();                       // P of every group visible
        phase2(sb, dq_s, x, 0);
      }
      if (step + 1 < nsteps) store_q(sb ^ 1);  // fp8: the next step's Q, widened
      ph = h;
      pqt = qt;
    }
    wait_vmcnt<0>();
  }

  // dV = sum P^T dO (role P), dK = scale sum dS^T Q (role dS); lane = d column 32db + n,
  // register i = key 8(i/4) + 4g + i%4 of the group's 32
  G* out = reinterpret_cast<G*>(role_p ? a.dv : a.dk) + ((int64_t)(b * a.Hkv + kvh) * a.Sk) * D;
  float f = role_p ? 1.f : a.scale, f2 = 1.f;
  if (a.f16_fac != nullptr) {
    f = role_p ? a.f16_fac[2] : a.f16_fac[3];
    f2 = role_p ? 1.f : a.f16_fac[4];
  }
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = k0 + kKW * grp + 8 * (i >> 2) + 4 * g + (i & 3);
      if (key < a.Sk) store_grad<G>(out + (int64_t)key * D + 32 * db + n, acc[db][i] * f * f2);
    }
  }
}

// ---------------------------------------------------------------------------------
// 4. Deterministic dQ: the query-row owner ("M4.4 - FlashAttention-2 ...", section
// 0x06.1G and its ownership table: with queries as the owner, dQ_i is a direct output).
// One workgroup owns a 128-row query tile of one (b, h_q) and one of dq_splits
// contiguous ranges of key tiles; it walks its key tiles in ascending order and keeps
// dQ in registers, so the summation order is fixed by the grid, not by arrival.  With
// dq_splits > 1 each range writes a float32 partial and bwd_tree_kernel sums them in
// a fixed binary tree (the materialised-partials alternative of section 0x06.1F).
//
// Layout as in the forward (32x32x16 matrix core, transposed products): a wave owns 32
// query rows as the N dimension.  Per 64-key tile:
//   S^T  = K Q^T     (A = K row fragments from LDS, B = Q^T fragments in registers)
//   dP^T = V dO^T    (A = V row fragments, B = dO^T fragments in registers)
//   P = exp2(S scale log2e - LSE log2e), dS = P (dP - D)   (per lane: one query)
//   dQ^T += K^T dS^T (A = K^T by transpose reads of the K tile, B = dS^T in registers:
//                     the accumulator layout of S^T is already the operand layout).
// K and V tiles go straight to LDS (two-slot rings, loaded one tile ahead).  fp16
// operands only: bf16 operands arrive as the exact fp16 copies of section 5.
constexpr int kDqRW = 4;                   // waves (32 query rows each) per workgroup
constexpr int kDqBQ = 32 * kDqRW;
constexpr int kDqBC = 64;                  // keys per tile

template <typename G, int D, bool CAUSAL, bool DROP>
__global__ __launch_bounds__(kDqRW * kWave) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_dq_kernel(BwdArgs a) {
  typedef f16 T;
  typedef Elem<T> E;
  typedef typename E::v8 V8;
  constexpr int BC = kDqBC;
  constexpr int KC = D / 16;               // contraction chunks of S^T / dP^T
  constexpr int KB = BC / 32;              // key blocks of 32
  constexpr int DB = D / 32;               // d blocks of dQ^T
  constexpr int CPR = D / 8;               // 16-byte chunks per row
  constexpr int ROWB = D * 2;
  constexpr int TB = BC * ROWB;            // one tile
  constexpr int NT = kDqRW * kWave;
  constexpr int LOADS = BC * CPR / NT;     // 16-byte chunks per thread per tile
  constexpr int RS = NT / CPR;             // rows per load round
  static_assert(RS % 16 == 0 && LOADS * NT == BC * CPR, "load rounds cover whole swizzle periods");

  __shared__ __attribute__((aligned(1024))) uint8_t lds[4 * TB];   // K slots 0, 1; V slots 0, 1

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int n = lane & 31;
  const int grp = lane >> 5;

  const int BH = a.B * a.Hq;
  const int nqt = (a.Sq + kDqBQ - 1) / kDqBQ;
  const int wg = blockIdx.x;
  const int bh = wg % BH;
  const int qt = CAUSAL ? (nqt - 1 - wg / BH) : (wg / BH);
  const int split = blockIdx.y;
  const int b = bh / a.Hq;
  const int h = bh - b * a.Hq;
  const int kvh = h / a.group;

  const int q0 = qt * kDqBQ;
  const int q1 = min(q0 + kDqBQ, a.Sq);
  const TilePlan plan = plan_rows(q0, q1, a.Sq, a.Sk, BC, CAUSAL);
  const int ntk = (a.Sk + BC - 1) / BC;
  const int per = (ntk + a.dq_splits - 1) / a.dq_splits;
  const int tb = min(plan.n_visit, split * per);
  const int te = min(plan.n_visit, tb + per);

  // swizzle of the 16-byte chunks of a staged row: 16 consecutive rows on distinct
  // bank groups for the fragment reads and, at d = 128, the transpose reads of the dQ
  // product (4 rows x 2 chunks) on 8 distinct positions too, as in the column owner
  auto swz = [](int r) { return D == 128 ? kv_swz<128>(r) : ((r >> 1) & 7); };

  const int64_t rowq0 = (int64_t)(b * a.Hq + h) * a.Sq;
  const T* qb = reinterpret_cast<const T*>(a.q) + rowq0 * D;
  const T* dob = reinterpret_cast<const T*>(a.dO) + rowq0 * D;
  const T* kb = reinterpret_cast<const T*>(a.k) + (int64_t)(b * a.Hkv + kvh) * a.Sk * D;
  const T* vb = reinterpret_cast<const T*>(a.v) + (int64_t)(b * a.Hkv + kvh) * a.Sk * D;
  const __amdgpu_buffer_rsrc_t qr = make_rsrc(qb, (uint32_t)a.Sq * D * 2);
  const __amdgpu_buffer_rsrc_t dr = make_rsrc(dob, (uint32_t)a.Sq * D * 2);

  // this lane's query row; Q^T and dO^T fragments (column = query, slots d 16kc + 8g)
  const int qrow = q0 + 32 * w + n;
  V8 qf[KC], df[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    const uint32_t off = (uint32_t)(qrow * D + 16 * kc + 8 * grp) * 2;
    qf[kc] = as_v8<V8>(buf_load_16(qr, off));
    df[kc] = as_v8<V8>(buf_load_16(dr, off));
  }
  // rows past S_q: P = exp2(-inf) = 0, so they contribute nothing
  const float lse2 = qrow < a.Sq ? a.lse[rowq0 + qrow] * ATTN_LOG2E : INFINITY;
  // fp16 copies of bf16 operands: the score factor (section 5; D arrives in the scale of
  // dP from the preprocess, the dQ factors are read at the end)
  const float sl2b = a.f16_fac != nullptr ? a.f16_fac[0] : a.scale_log2;
  const float dl = qrow < a.Sq ? a.delta[rowq0 + qrow] : 0.f;
  const int klim = CAUSAL ? min(a.Sk, qrow + (a.Sk - a.Sq) + 1) : a.Sk;

  f32x16 dq[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) dq[i] = f32x16{};

  // K / V tile t into slot s: chunk idx = r NT + tid is LDS (row, pos) = (idx / CPR,
  // idx % CPR) holding global chunk pos ^ swz(row)
  const int trow = tid / CPR, tpos = tid % CPR;
  const uint32_t co = (uint32_t)((tpos ^ swz(trow)) * 16);
  // The tile's and the round's row offsets go into a per-round resource (uniform base,
  // remaining range), so each thread keeps one vector offset.
  const int64_t kv_bytes = (int64_t)a.Sk * D * 2;
  const uint32_t vo = (uint32_t)(trow * ROWB) + co;
  auto load_tile = [&](int t, int slot) {
    const int tu = __builtin_amdgcn_readfirstlane(t);
#pragma unroll
    for (int r = 0; r < LOADS; ++r) {
      const int64_t off = (int64_t)(tu * BC + r * RS) * ROWB;
      const uint32_t left = kv_bytes > off ? (uint32_t)(kv_bytes - off) : 0u;
      const uint32_t kd = __builtin_amdgcn_readfirstlane(lds_offset(lds + slot * TB + (r * NT + w * kWave) * 16));
      const uint32_t vd = __builtin_amdgcn_readfirstlane(lds_offset(lds + (2 + slot) * TB + (r * NT + w * kWave) * 16));
      lds_load_16(make_rsrc(reinterpret_cast<const uint8_t*>(kb) + off, left), vo, 0u, kd);
      lds_load_16(make_rsrc(reinterpret_cast<const uint8_t*>(vb) + off, left), vo, 0u, vd);
    }
  };

  const int s16 = lane & 15;
  const int dsub = 16 * ((lane >> 4) & 1) + 4 * (s16 & 3);
  // One key tile, one 32-key block at a time (keeps two score accumulators live).
  auto step = [&](auto mask_tag, int t, int slot) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const uint8_t* ks = lds + slot * TB;
    const uint8_t* vs = lds + (2 + slot) * TB;
#pragma unroll 1
    for (int kbk = 0; kbk < KB; ++kbk) {
      // dropout decisions of this key block, first: bit i for register i (registers
      // 4q .. 4q+3 are four consecutive keys, one Philox call each q)
      uint32_t keepbits = 0;
      if constexpr (DROP) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const u32x4 wv = philox4x32_10((uint32_t)(t * (BC / 4) + 8 * kbk + 2 * q4 + grp), (uint32_t)qrow,
                                         (uint32_t)(b * a.Hq + h), a.drop.offset, a.drop.seed_lo, a.drop.seed_hi);
#pragma unroll
          for (int e = 0; e < 4; ++e) keepbits |= (wv[e] >= a.drop.thresh ? 1u : 0u) << (4 * q4 + e);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      f32x16 sc, dp;
      const int row = kbk * 32 + n;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const int off = row * ROWB + (((2 * kc + grp) ^ swz(row)) * 16);
        const V8 ak = as_v8<V8>(ld_lds_16(ks + off));
        const V8 av = as_v8<V8>(ld_lds_16(vs + off));
        sc = E::mfma(ak, qf[kc], kc == 0 ? f32x16{} : sc);
        dp = E::mfma(av, df[kc], kc == 0 ? f32x16{} : dp);
        if ((kc & 1) == 1) __builtin_amdgcn_sched_barrier(0);   // bound the reads in flight
      }
      // P and dS; register i is key t BC + 32 kbk + 8(i/4) + 4 grp + i%4
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float pv = fast_exp2(fmaf(sc[i], sl2b, -lse2));
        if constexpr (MASK) {
          const int key = t * BC + 32 * kbk + 8 * (i >> 2) + 4 * grp + (i & 3);
          pv = key < klim ? pv : 0.f;
        }
        const float z = DROP ? (((keepbits >> i) & 1u) ? a.drop.rp : 0.f) : 1.f;
        dp[i] = pv * (z * dp[i] - dl);
      }
      // dQ^T += K^T dS^T, key chunk cc: slots of lane group g = keys 16cc + 8(s/4) + 4g + s%4
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int cc = 2 * kbk + half;
        const int hb = half * 8;
        // dS^T operand
        const u32x4 dsp = {E::pack2(dp[hb + 0], dp[hb + 1]), E::pack2(dp[hb + 2], dp[hb + 3]),
                           E::pack2(dp[hb + 4], dp[hb + 5]), E::pack2(dp[hb + 6], dp[hb + 7])};
        const int r0 = 16 * cc + 4 * grp + (s16 >> 2);
        const int r1 = r0 + 8;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int col = 32 * db + dsub;
          const int ch = col >> 3;
          const int hf = (col & 7) * 2;
          const u32x2 lo = tr_read(ks + r0 * ROWB + ((ch ^ swz(r0)) * 16) + hf);
          const u32x2 hi = tr_read(ks + r1 * ROWB + ((ch ^ swz(r1)) * 16) + hf);
          const V8 kt8 = as_v8<V8>(u32x4{lo.x, lo.y, hi.x, hi.y});
          dq[db] = E::mfma(kt8, as_v8<V8>(dsp), dq[db]);
        }
        __builtin_amdgcn_sched_barrier(0);   // bound the transpose reads in flight
      }
    }
  };

  if (tb < te) load_tile(tb, 0);
  for (int t = tb; t < te; ++t) {
    const int slot = (t - tb) & 1;
    wait_vmcnt<0>();              // this thread's loads of tile t have landed
    __syncthreads();              // everyone's have; tile t-1's slot is free
    if (t + 1 < te) load_tile(t + 1, slot ^ 1);
    if (t >= plan.first_masked)
      step(std::true_type{}, t, slot);
    else
      step(std::false_type{}, t, slot);
  }

  // dQ^T registers: lane column = query row, register i = d 32db + 8(i/4) + 4grp + i%4.
  // fdq: the factor of a partial (the tree applies the scale) or of dQ itself
  float fds = 1.f, fdq = a.dq_splits > 1 ? 1.f : a.scale;
  if (a.f16_fac != nullptr) {
    fds = a.f16_fac[3];
    fdq = a.dq_splits > 1 ? a.f16_fac[6] : a.f16_fac[5];
  }
  if (qrow < a.Sq) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int dcol = 32 * db + 8 * r4 + 4 * grp;
        if (a.dq_splits > 1) {
          float* out = a.dq_part + ((int64_t)split * a.B * a.Hq * a.Sq + rowq0 + qrow) * D + dcol;
          st_global_16(out, __builtin_bit_cast(u32x4, f32x4{dq[db][4 * r4] * fds * fdq, dq[db][4 * r4 + 1] * fds * fdq,
                                                            dq[db][4 * r4 + 2] * fds * fdq, dq[db][4 * r4 + 3] * fds * fdq}));
        } else {
          G* out = reinterpret_cast<G*>(a.dq) + (rowq0 + qrow) * D + dcol;
#pragma unroll
          for (int e = 0; e < 4; ++e) store_grad<G>(out + e, dq[db][4 * r4 + e] * fds * fdq);
        }
      }
  }
}

// dQ = scale * (fixed binary tree over the dq_splits partials): level by level, the
// partial 2^l (2m + 1) is added into 2^l (2m).
template <typename G>
__global__ __launch_bounds__(kNT) void bwd_tree_kernel(BwdArgs a, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * kNT + threadIdx.x;
  if (i >= n4) return;
  const f32x4* part = reinterpret_cast<const f32x4*>(a.dq_part);
  f32x4 v[16];
  const int np = a.dq_splits;
#pragma unroll
  for (int p = 0; p < 16; ++p)
    if (p < np) v[p] = part[(int64_t)p * n4 + i];
#pragma unroll
  for (int st = 1; st < 16; st <<= 1)
#pragma unroll
    for (int p = 0; p + st < 16; p += 2 * st)
      if (p + st < np) v[p] = v[p] + v[p + st];
  G* out = reinterpret_cast<G*>(a.dq) + 4 * i;
#pragma unroll
  for (int j = 0; j < 4; ++j) out[j] = (G)(v[0][j] * a.scale);
}

// ---------------------------------------------------------------------------------
// 5. Deterministic mode with bf16 operands: exact fp16 copies.  A bf16 value has 8
// significant bits, an fp16 value 11, so 2^k x of a bf16 x is an fp16 value whenever it
// lies in fp16's normal range.  k is chosen per tensor so that its largest magnitude
// lands in [4, 8) (for v, the larger of v's and o's, which bounds D).  Then |dP| and |D|
// stay below d * 64 and |dS| = P |dP - D| below 2 d * 64 <= 16384, inside fp16's range,
// and P and dS enter the dV, dK and dQ products as single fp16 operands (relative
// rounding 2^-12) instead of bf16 hi + lo pairs.  Scaled values below 2^-14 become fp16
// subnormals (absolute error at most 2^-25 in the scaled units).  The exponents are
// clamped to [-60, 60] (largest magnitudes from 2^-58 to 2^63 are fully normalised), so
// that every factor below is a float32: S carries 2^(eq+ek), dP and dS 2^(ed+ev) (D is
// scaled to match), dV 2^ed, dK 2^(ed+ev+eq) and dQ 2^(ed+ev+ek); the owners multiply by
//   [0] scale log2(e) 2^-(eq+ek)   [1] 2^(ed+ev) (D, in the preprocess)   [2] 2^-ed (dV)
//   [3] 2^-(ed+ev), then [4] scale 2^-eq (dK) or [5] scale 2^-ek (dQ) or [6] 2^-ek (dQ
//   partials; the tree applies the scale).  The powers of two are exact, so each result
//   is rounded once.
constexpr int kAmaxBlocks = kBwdAmaxBlocks;
constexpr int kNumF16 = 4;                 // copies: q, k, v, dO

// Largest magnitude of q, k, v, dO, o (blockIdx.y) over a grid-strided range of 16-byte
// chunks, as bf16 bits without the sign (for values that are not NaN their order is the
// order of the magnitudes; NaN sorts above infinity).
__global__ __launch_bounds__(kNT) void bwd_amax_kernel(const void* q, const void* k, const void* v, const void* dO,
                                                       const void* o, int64_t nq16, int64_t nk16, uint32_t* amax) {
  const int t = blockIdx.y;
  const u32x4* src = reinterpret_cast<const u32x4*>(t == 0 ? q : t == 1 ? k : t == 2 ? v : t == 3 ? dO : o);
  const int64_t n16 = (t == 1 || t == 2) ? nk16 : nq16;
  uint32_t m = 0;
  for (int64_t i = (int64_t)blockIdx.x * kNT + threadIdx.x; i < n16; i += (int64_t)kAmaxBlocks * kNT) {
    const u32x4 x = ld_global_16(src + i);
#pragma unroll
    for (int j = 0; j < 4; ++j) m = max(m, max(x[j] & 0x7FFFu, (x[j] >> 16) & 0x7FFFu));
  }
#pragma unroll
  for (int st = 1; st < kWave; st <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, st));
  __shared__ uint32_t wm[kNT / kWave];
  if ((threadIdx.x & (kWave - 1)) == 0) wm[threadIdx.x / kWave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int i = 1; i < kNT / kWave; ++i) m = max(m, wm[i]);
    amax[t * kAmaxBlocks + blockIdx.x] = m;
  }
}

// k with 2^k |x|max in [4, 8) from the bf16 bits of |x|max; 0 for zero, infinity, NaN
__device__ inline int f16_exponent(uint32_t m) {
  if (m == 0u || m >= 0x7F80u) return 0;
  const int e = max((int)(m >> 7), 1);       // biased exponent (subnormals as 1)
  return min(60, max(-60, 129 - e));
}

// One workgroup: reduce the per-block maxima, store the four exponents and the factors.
__global__ __launch_bounds__(kNT) void bwd_f16_exp_kernel(uint32_t* amax, float scale, float scale_log2) {
  const uint32_t* part = amax;
  __shared__ uint32_t wm[5][kNT / kWave];
#pragma unroll
  for (int t = 0; t < 5; ++t) {
    uint32_t m = 0;
    for (int i = threadIdx.x; i < kAmaxBlocks; i += kNT) m = max(m, part[t * kAmaxBlocks + i]);
#pragma unroll
    for (int st = 1; st < kWave; st <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, st));
    if ((threadIdx.x & (kWave - 1)) == 0) wm[t][threadIdx.x / kWave] = m;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int ex[kNumF16];
#pragma unroll
    for (int t = 0; t < kNumF16; ++t) {
      uint32_t m = 0;
#pragma unroll
      for (int i = 0; i < kNT / kWave; ++i) {
        m = max(m, wm[t][i]);
        if (t == 2) m = max(m, wm[4][i]);    // v's exponent also covers o
      }
      ex[t] = f16_exponent(m);
    }
    int* eo = reinterpret_cast<int*>(amax + 5 * kAmaxBlocks);
    float* fo = reinterpret_cast<float*>(eo + kNumF16);
#pragma unroll
    for (int t = 0; t < kNumF16; ++t) eo[t] = ex[t];
    const int eq = ex[0], ek = ex[1], ev = ex[2], ed = ex[3];
    fo[0] = ldexpf(scale_log2, -(eq + ek));
    fo[1] = ldexpf(1.f, ed + ev);
    fo[2] = ldexpf(1.f, -ed);
    fo[3] = ldexpf(1.f, -(ed + ev));
    fo[4] = ldexpf(scale, -eq);
    fo[5] = ldexpf(scale, -ek);
    fo[6] = ldexpf(1.f, -ek);
  }
}

// fp16 copy 2^k x of q, k, v, dO (blockIdx.y), 8 values per thread and iteration.
__global__ __launch_bounds__(kNT) void bwd_to_f16_kernel(const void* q, const void* k, const void* v, const void* dO,
                                                         BwdF16Ws ws, int64_t nq16, int64_t nk16) {
  const int t = blockIdx.y;
  const int e = reinterpret_cast<const int*>(ws.amax + 5 * kAmaxBlocks)[t];
  const u32x4* src = reinterpret_cast<const u32x4*>(t == 0 ? q : t == 1 ? k : t == 2 ? v : dO);
  u32x4* dst = reinterpret_cast<u32x4*>(ws.copy[t]);
  const int64_t n16 = (t == 1 || t == 2) ? nk16 : nq16;
  for (int64_t i = (int64_t)blockIdx.x * kNT + threadIdx.x; i < n16; i += (int64_t)gridDim.x * kNT) {
    const u32x4 x = ld_global_16(src + i);
    u32x4 y;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      y[j] = Elem<f16>::pack2(ldexpf(__uint_as_float(x[j] << 16), e), ldexpf(__uint_as_float(x[j] & 0xFFFF0000u), e));
    st_global_16(dst + i, y);
  }
}

// column-owner launch (16-bit operands) for one DQ form
template <typename T, typename G, int D, bool DQ>
void kv_k(const BwdArgs& a, dim3 gkv, hipStream_t stream) {
  const dim3 blk(kKVW * kWave);
  if (a.dropout) {
    if (a.causal)
      hipLaunchKernelGGL((bwd_kv_kernel<T, G, D, true, DQ, false, true>), gkv, blk, 0, stream, a);
    else
      hipLaunchKernelGGL((bwd_kv_kernel<T, G, D, false, DQ, false, true>), gkv, blk, 0, stream, a);
  } else {
    if (a.causal)
      hipLaunchKernelGGL((bwd_kv_kernel<T, G, D, true, DQ>), gkv, blk, 0, stream, a);
    else
      hipLaunchKernelGGL((bwd_kv_kernel<T, G, D, false, DQ>), gkv, blk, 0, stream, a);
  }
}

// deterministic mode after the preprocess, on fp16 operands: column owner without dQ,
// query-row owner, and the partials' tree when dq_splits > 1
template <typename G, int D>
hipError_t launch_det(const BwdArgs& a, dim3 gkv, int64_t n4, hipStream_t stream) {
  kv_k<f16, G, D, false>(a, gkv, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nqt = (a.Sq + kDqBQ - 1) / kDqBQ;
  const dim3 gq((unsigned)(nqt * a.B * a.Hq), (unsigned)a.dq_splits);
  if (a.dropout) {
    if (a.causal)
      hipLaunchKernelGGL((bwd_dq_kernel<G, D, true, true>), gq, dim3(kDqRW * kWave), 0, stream, a);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<G, D, false, true>), gq, dim3(kDqRW * kWave), 0, stream, a);
  } else {
    if (a.causal)
      hipLaunchKernelGGL((bwd_dq_kernel<G, D, true, false>), gq, dim3(kDqRW * kWave), 0, stream, a);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<G, D, false, false>), gq, dim3(kDqRW * kWave), 0, stream, a);
  }
  e = hipGetLastError();
  if (e != hipSuccess || a.dq_splits == 1) return e;
  hipLaunchKernelGGL((bwd_tree_kernel<G>), dim3((unsigned)((n4 + kNT - 1) / kNT)), dim3(kNT), 0, stream, a, n4);
  return hipGetLastError();
}

template <typename T, typename G, int D>
hipError_t launch_bwd_tg(const BwdArgs& a, const BwdF16Ws* cw, hipStream_t stream) {
  const int64_t rows = (int64_t)a.B * a.Hq * a.Sq;
  constexpr int RPB = kNT / (D / 8);
  auto pre = [&](const BwdArgs& x) {
    hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(kNT), 0, stream, x);
    return hipGetLastError();
  };
  hipError_t e = hipSuccess;
  const bool copies = std::is_same<T, bf16>::value && a.deterministic;
  if (!copies) {
    e = pre(a);
    if (e != hipSuccess) return e;
  }
  const int64_t n4 = rows * D / 4;
  const dim3 gkv((unsigned)((a.Sk + kKVT - 1) / kKVT), (unsigned)(a.B * a.Hkv));
  if constexpr (std::is_same<T, bf16>::value) {
    if (a.fp8) {
      // E4M3 operands: the split-role column owner with atomic dQ
      if (a.causal)
        hipLaunchKernelGGL((bwd_kv_kernel<T, G, D, true, true, true>), gkv, dim3(kKVW * kWave), 0, stream, a);
      else
        hipLaunchKernelGGL((bwd_kv_kernel<T, G, D, false, true, true>), gkv, dim3(kKVW * kWave), 0, stream, a);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((bwd_convert_kernel<G>), dim3((unsigned)((n4 + kNT - 1) / kNT)), dim3(kNT), 0, stream, a, n4);
      return hipGetLastError();
    }
  }
  if (a.deterministic) {
    if constexpr (std::is_same<T, bf16>::value) {
      // exact fp16 copies of q, k, v, dO, then the fp16 owners on them
      if (cw == nullptr || cw->amax == nullptr) return hipErrorInvalidValue;
      const int64_t nq16 = rows * D / 8, nk16 = (int64_t)a.B * a.Hkv * a.Sk * D / 8;
      hipLaunchKernelGGL(bwd_amax_kernel, dim3(kAmaxBlocks, 5), dim3(kNT), 0, stream, a.q, a.k, a.v, a.dO, a.o,
                         nq16, nk16, cw->amax);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(bwd_f16_exp_kernel, dim3(1), dim3(kNT), 0, stream, cw->amax, a.scale, a.scale_log2);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(bwd_to_f16_kernel, dim3(1024, kNumF16), dim3(kNT), 0, stream, a.q, a.k, a.v, a.dO, *cw,
                         nq16, nk16);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      BwdArgs c = a;
      c.f16_fac = reinterpret_cast<const float*>(cw->amax + 5 * kAmaxBlocks + kNumF16);
      e = pre(c);                        // D from the bf16 o and dO, in the scale of dP
      if (e != hipSuccess) return e;
      c.q = cw->copy[0]; c.k = cw->copy[1]; c.v = cw->copy[2]; c.dO = cw->copy[3];
      c.dtype_bf16 = 0;
      return launch_det<G, D>(c, gkv, n4, stream);
    } else {
      return launch_det<G, D>(a, gkv, n4, stream);
    }
  }
  kv_k<T, G, D, true>(a, gkv, stream);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_convert_kernel<G>), dim3((unsigned)((n4 + kNT - 1) / kNT)), dim3(kNT), 0, stream, a, n4);
  return hipGetLastError();
}

template <typename T, typename G>
hipError_t launch_bwd_d(const BwdArgs& a, const BwdF16Ws* cw, hipStream_t stream) {
  if (a.d == 64) return launch_bwd_tg<T, G, 64>(a, cw, stream);
  return launch_bwd_tg<T, G, 128>(a, cw, stream);
}

template <typename T>
hipError_t launch_bwd_t(const BwdArgs& a, const BwdF16Ws* cw, hipStream_t stream) {
  if (a.grad_type == ATTN_F32) return launch_bwd_d<T, float>(a, cw, stream);
  if (a.grad_type == ATTN_BF16) return launch_bwd_d<T, bf16>(a, cw, stream);
  return launch_bwd_d<T, f16>(a, cw, stream);
}

}  // namespace

hipError_t attn_launch_bwd(const BwdArgs& a, const BwdF16Ws* cw, hipStream_t stream) {
  if (a.dtype_bf16) return launch_bwd_t<bf16>(a, cw, stream);
  return launch_bwd_t<f16>(a, cw, stream);
}

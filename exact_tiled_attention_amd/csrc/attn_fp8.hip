// attn_fp8.hip -- forward on E4M3FN operands with 128-row block descales (gfx950).
//
// "M4.6 - FlashAttention-3/4 Hardware Pipelines: Hopper, Blackwell, and the Moving
// Bottleneck", section 0x06:
//   * Q/K descales enter the scores before the row maximum ("Derive Where Every Scale
//     Must Enter"): S = scale * dQ_i * dK_j * (Q8 K8_j^T);
//   * probabilities are raised by 2^8 before they are rounded to E4M3 for the P V
//     product, the denominator sums the unrounded values, and LSE removes the 2^8
//     ("Why The Source Raises Softmax Probabilities By 2^8");
//   * the V descale varies per K/V block, so each tile's P V contribution enters the
//     accumulator in its own scale frame (the block-varying V scale case).
//
// Same schedule and orientation as the 16-bit forward (S^T = K Q^T on the matrix
// core, one query column per lane, P kept in registers as the B operand of
// O^T += V^T P^T).  The score product runs on the bf16 matrix core: every E4M3 value
// is exact in bf16 and the products are exact in the float32 accumulator, so S is the
// float32 accumulation the method specifies ("QK WGMMA accumulator S: FP32"); the
// K=64 fp8 instruction accumulates internally with ~2^-14 relative precision, which
// at the score magnitudes of outlier-heavy inputs moves the E4M3 rounding of P.
// The P V product, whose error stays continuous, runs on the 32x32x64 fp8
// instruction.  The V scale is
// folded into the rescale that the online softmax does anyway: the accumulator is
// kept in units of the current tile's V descale s_v, and moving to a tile with
// descale dV_j multiplies it by alpha * s_v / dV_j.
//
// V goes from HBM straight into LDS (buffer loads with the LDS destination), row-major
// with its rows permuted and its 16-byte chunks swizzled; the V^T operand of the P V
// product comes from ds_read_b64_tr_b8, which hands each lane of a 16-lane group one
// byte column (one d) of 8 rows.  Slot j of lane group g of a 64-key contraction is key
// 8 (j / 4) + 4 g + j % 4 (the keys the S^T accumulator put in that lane's registers), so
// LDS row r holds key r with bits 2 and 3 exchanged: the 8 slots 8m .. 8m+7 of group g
// are then the 8 consecutive rows 16m + 8g .. +7.
#include <type_traits>

#include "attn_device.h"
#include "attn_launch.h"
#include "tile_plan.h"

namespace {

constexpr int kWave = 64;
constexpr int BC = 64;
constexpr int SCALE_ROWS = 128;
constexpr int kStages = 3;      // LDS stages of the K/V tile ring

typedef __attribute__((ext_vector_type(8))) int i32x8;

template <int D>
struct Fp8Lds {
  static constexpr int KSTR = D + 8;      // bf16 elements per K row (widened from E4M3)
  static constexpr int K_BYTES = BC * KSTR * 2;
  static constexpr int V_BYTES = BC * D;  // E4M3 rows, permuted and swizzled
  static constexpr int STAGE = K_BYTES + V_BYTES;
};

// LDS row r of a V tile holds key r with bits 2 and 3 exchanged.
__device__ inline int v_row_key(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }
// Chunk p of LDS V row r holds the row's 16-byte chunk p ^ v_swz(r): the 8 rows a
// transpose read takes then fall on distinct banks.
template <int D> __device__ inline int v_swz(int r) { return D == 128 ? (r & 7) : ((r >> 2) & 1); }

typedef __attribute__((ext_vector_type(2))) int i32x2;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
// ds_read_b64_tr_b8: in each 16-lane group, lanes 2k and 2k+1 address the two 8-byte
// halves of row k of an 8 x 16-byte block; lane i receives byte i of rows 0 .. 7.
__device__ inline u32x2 tr8_read(const uint8_t* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)p));
}

__device__ inline f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  // format 0 (E4M3) for both operands, block scales fixed at 2^0 (E8M0 code 127)
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// 8 E4M3 bytes (two dwords) -> 8 bf16 values, one instruction per pair (exact: every
// E4M3 value is a bf16 value, and the conversion's scale is 1).
__device__ inline u32x4 e4m3x8_to_bf16(uint32_t w0, uint32_t w1) {
  u32x4 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, 1.f, false));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, 1.f, true));
  r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, 1.f, false));
  r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, 1.f, true));
  return r;
}

__device__ inline float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// max over the two lanes l and l ^ 32 (one VALU lane swap).
__device__ inline float max_pair32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <int D, int NW, bool OF32>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(2))) void fp8_fwd_kernel(Fp8Args a) {
  // causal masking is a runtime flag: the plans and the per-lane key limit below carry it
  const bool CAUSAL = a.causal != 0;
  typedef Fp8Lds<D> L;
  constexpr int NT = NW * kWave;
  constexpr int BQ = NW * 32;
  constexpr int K_LOADS = (BC * D / 16 + NT - 1) / NT;     // 16-byte K chunks per thread
  constexpr int CPR = D / 16;                              // 16-byte chunks per V row
  constexpr int V_LOADS = (BC * CPR + NT - 1) / NT;        // direct V loads per thread

  __shared__ __attribute__((aligned(16))) uint8_t lds[kStages * L::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int n = lane & 31;
  const int grp = lane >> 5;

  const int BH = a.B * a.Hq;
  const int wg = blockIdx.x;
  const int bh = wg % BH;
  const int qt = CAUSAL ? (a.nqt - 1 - wg / BH) : (wg / BH);   // heavy causal tiles first
  const int b = bh / a.Hq;
  const int h = bh - b * a.Hq;
  const int kvh = h / a.group;

  const uint8_t* qb = a.q + ((int64_t)(b * a.Hq + h) * a.Sq) * D;
  const uint8_t* kb = a.k + ((int64_t)(b * a.Hkv + kvh) * a.Sk) * D;
  const uint8_t* vb = a.v + ((int64_t)(b * a.Hkv + kvh) * a.Sk) * D;
  const int nqb = (a.Sq + SCALE_ROWS - 1) / SCALE_ROWS;
  const int nkb = (a.Sk + SCALE_ROWS - 1) / SCALE_ROWS;
  const float* ksc = a.k_scale + (int64_t)(b * a.Hkv + kvh) * nkb;
  const float* vsc = a.v_scale + (int64_t)(b * a.Hkv + kvh) * nkb;

  const int q0 = qt * BQ;
  const int qrow = q0 + w * 32 + n;
  const TilePlan plan = plan_rows(q0, min(q0 + BQ, a.Sq), a.Sq, a.Sk, BC, CAUSAL);
  // this wave's rows: the tiles it visits and the first one that needs a mask
  const int w0 = q0 + w * 32;
  const TilePlan wplan = plan_rows(w0, max(min(w0 + 32, a.Sq), w0 + 1), a.Sq, a.Sk, BC, CAUSAL);
  // keys at or past klim are invisible to this lane's query (tail; causal band)
  const int klim = CAUSAL ? min(a.Sk, qrow + (a.Sk - a.Sq) + 1) : a.Sk;
  const float dq = qrow < a.Sq ? a.q_scale[(int64_t)(b * a.Hq + h) * nqb + qrow / SCALE_ROWS] : 0.f;
  // score factor without the K descale; a negative score scale is moved into Q (sign
  // flip of the bf16 operand) so that the factor is >= 0
  const float c_q = fabsf(a.scale_log2) * dq;
  const uint32_t qsign = a.scale_log2 < 0.f ? 0x80008000u : 0u;

  // Q^T fragments (bf16 B operand): lane column = query, slots = d 16kc+8g .. +8.
  bf16x8 qf[D / 16];
#pragma unroll
  for (int kc = 0; kc < D / 16; ++kc) {
    u32x2 raw = {0u, 0u};
    if (qrow < a.Sq) raw = *reinterpret_cast<const u32x2*>(qb + (int64_t)qrow * D + 16 * kc + 8 * grp);
    u32x4 wide = e4m3x8_to_bf16(raw.x, raw.y);
    wide.x ^= qsign;
    wide.y ^= qsign;
    wide.z ^= qsign;
    wide.w ^= qsign;
    qf[kc] = as_v8<bf16x8>(wide);
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = f32x16{};
  float m_i = -INFINITY;
  float l_i = 0.f;
  float s_v = 1.f;   // V descale the accumulator is expressed in

  u32x4 kreg[K_LOADS];
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vb, (uint32_t)a.Sk * D);   // keys past S_k read 0

  // K(t) into registers (widened by store_tile); V(t) straight into its stage's LDS: load
  // r of wave w fills LDS chunks idx = r NT + 64 w + lane, i.e. (row idx / CPR, chunk
  // idx % CPR), from the row's key and swizzled chunk.
  auto load_tile = [&](int t, int stage) {
    const int k0 = t * BC;
#pragma unroll
    for (int r = 0; r < K_LOADS; ++r) {
      const int idx = r * NT + tid;
      const int row = idx / (D / 16);
      const int c16 = idx % (D / 16);
      const int key = k0 + row;
      u32x4 val = {0u, 0u, 0u, 0u};
      if (idx < BC * D / 16 && key < a.Sk) val = ld_global_16(kb + (int64_t)key * D + c16 * 16);
      kreg[r] = val;
    }
    const uint32_t vdst = lds_offset(lds + stage * L::STAGE + L::K_BYTES);
#pragma unroll
    for (int r = 0; r < V_LOADS; ++r) {
      const int idx0 = r * NT + w * kWave;   // wave-uniform
      if (idx0 < BC * CPR) {
        const int idx = idx0 + lane;
        const int row = idx / CPR, pos = idx % CPR;
        lds_load_16(vrs, (uint32_t)(v_row_key(row) * D + (pos ^ v_swz<D>(row)) * 16),
                    (uint32_t)(__builtin_amdgcn_readfirstlane(t) * BC * D),
                    __builtin_amdgcn_readfirstlane(vdst + idx0 * 16));
      }
    }
  };

  auto store_tile = [&](int stage) {
    uint8_t* ks = lds + stage * L::STAGE;
#pragma unroll
    for (int r = 0; r < K_LOADS; ++r) {
      const int idx = r * NT + tid;
      if (idx < BC * D / 16) {
        const int row = idx / (D / 16);
        const int c16 = idx % (D / 16);
        bf16* kd = reinterpret_cast<bf16*>(ks) + row * L::KSTR + c16 * 16;
        st_lds_16(kd, e4m3x8_to_bf16(kreg[r].x, kreg[r].y));
        st_lds_16(kd + 8, e4m3x8_to_bf16(kreg[r].z, kreg[r].w));
      }
    }
  };

  // Software pipeline (as in the 16-bit forward): step t issues the score product of
  // tile t+1 chunk by chunk between the exponentials of tile t, so that each chunk's
  // vector work runs while the matrix core works on independent products; then the
  // accumulator rescale and the P V product of tile t, the staging of tile t+2, and the
  // row max of tile t+1.  Tiles live in kStages LDS stages: step t reads K(t+1) and
  // V(t) and writes tile t+2 into the stage tile t-1 held, so one barrier per step
  // publishes the writes and frees the next stage.  Every element goes through the same
  // arithmetic in the same order as a tile-at-a-time schedule.
  constexpr int KC = D / 16;                 // contraction chunks of the score product
  constexpr int NCH = D == 128 ? 8 : 4;     // pipeline chunks per tile (one or two score chunks)
  constexpr int KPC = KC / NCH;              // score chunks per pipeline chunk
  constexpr int PPC = 16 / NCH;              // exponential pairs per pipeline chunk
  static_assert(KPC * NCH == KC, "the score chunks split evenly");

  // The tile whose probabilities come next: its score factor, the frame m its values
  // u = 2^8 exp2(x - m) are taken in, and the factor that moves l into that frame.
  float p_csc = 0.f, p_moff = 0.f, p_alpha = 1.f, p_mnew = -INFINITY;

  auto qk_part = [&](f32x16 (&sc)[2], int stage, int kc0, int kc1) {
    const bf16* kbf = reinterpret_cast<const bf16*>(lds + stage * L::STAGE);
#pragma unroll
    for (int kc = kc0; kc < kc1; ++kc) {
#pragma unroll
      for (int kbk = 0; kbk < 2; ++kbk) {
        const bf16x8 av = as_v8<bf16x8>(ld_lds_16(kbf + (kbk * 32 + n) * L::KSTR + 16 * kc + 8 * grp));
        sc[kbk] = Elem<bf16>::mfma(av, qf[kc], kc == 0 ? f32x16{} : sc[kbk]);
      }
      if ((kc & 1) == 1) __builtin_amdgcn_sched_barrier(0);   // bound the reads in flight
    }
  };

  // Descales before the row max: x = csc * s with csc = scale log2(e) dQ dK.  The max is
  // taken on the raw accumulators (csc >= 0: descales are positive and a negative score
  // scale is moved into Q), so x enters only through one FMA in the exponentials.
  // MASKED sets the invisible scores to -inf first (only the tiles the plan marks).
  auto prepare = [&](f32x16 (&sc)[2], int t, bool masked) {
    const float dk = ksc[(t * BC) / SCALE_ROWS];
    if (masked) {
      // visibility of register i of key block kbk: its key offset against this lane's
      // limit (the per-register offsets are constants, one compare each)
      const int lim = klim - t * BC - 4 * grp;
#pragma unroll
      for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[kbk][i] = (kbk * 32 + 8 * (i >> 2) + (i & 3)) < lim ? sc[kbk][i] : -INFINITY;
    }
    float r0 = vmax(sc[0][0], sc[0][1]), r1 = vmax(sc[0][2], sc[0][3]);
#pragma unroll
    for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
      for (int i = (kbk == 0 ? 4 : 0); i < 16; i += 4) {
        r0 = vmax(r0, vmax(sc[kbk][i], sc[kbk][i + 1]));
        r1 = vmax(r1, vmax(sc[kbk][i + 2], sc[kbk][i + 3]));
      }
    const float mr = vmax(r0, r1);
    const float csc = c_q * dk;
    const float mx = max_pair32(mr == -INFINITY ? -INFINITY : mr * csc);
    const float m_new = fmaxf(m_i, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    p_alpha = fast_exp2(m_i - m_use);
    p_moff = m_use - 8.f;                    // u = 2^8 exp2(x - m)
    p_csc = csc;
    p_mnew = m_new;
  };

  // Exponential pairs PPC c .. PPC (c+1) - 1 of tile t (pair p: key block p / 8,
  // registers 2 (p % 8) and + 1), their sums in rs0 (even registers) and rs1 (odd).
  auto exp_part = [&](auto masked_tag, f32x16 (&sc)[2], int t, int c, float& rs0, float& rs1) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int lim = klim - t * BC - 4 * grp;
#pragma unroll
    for (int pr = PPC * c; pr < PPC * (c + 1); ++pr) {
      const int kbk = pr >> 3, i = 2 * (pr & 7);
      // masked cells give u = 0 by selection (a zero descale or scale makes csc = 0,
      // and fma(-inf, 0, .) would be NaN)
      float u0 = fast_exp2(fmaf(sc[kbk][i], p_csc, -p_moff));
      float u1 = fast_exp2(fmaf(sc[kbk][i + 1], p_csc, -p_moff));
      if constexpr (MASKED) {
        u0 = (kbk * 32 + 8 * (i >> 2) + (i & 3)) < lim ? u0 : 0.f;
        u1 = (kbk * 32 + 8 * ((i + 1) >> 2) + ((i + 1) & 3)) < lim ? u1 : 0.f;
      }
      sc[kbk][i] = u0;
      sc[kbk][i + 1] = u1;
      rs0 += u0;
      rs1 += u1;
    }
  };

  // The running state moves to tile t's frame, then O takes tile t's P V product.
  auto finish = [&](f32x16 (&sc)[2], int t, int stage, float rs0, float rs1) {
    l_i = p_alpha * l_i + (rs0 + rs1);
    m_i = p_mnew;
    const float dv = vsc[(t * BC) / SCALE_ROWS];
    // The accumulator is kept in units of the current V descale s_v: moving to a tile
    // with descale dv (and a moved max) multiplies it by alpha s_v / dv, skipped when
    // that is 1 in every lane (same scale block, unmoved max).  A zero V descale (an
    // all-zero value block) makes the tile's values zero: the accumulator keeps its
    // frame and the tile adds nothing (dv is the same for every lane of the workgroup).
    const bool v_zero = !(dv != 0.f);
    const float beta = v_zero ? p_alpha : p_alpha * (s_v / dv);
    if (!v_zero) s_v = dv;
    if (wave_any(beta != 1.f)) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= beta;
      }
    }
    if (v_zero) return;
    // P^T as the fp8 B operand: slot j = register (j % 16) of key block j / 16.
    i32x8 pb;
#pragma unroll
    for (int wd = 0; wd < 8; ++wd) {
      const int kbk = wd >> 2;
      const int i0 = 4 * (wd & 3);
      int v = __builtin_amdgcn_cvt_pk_fp8_f32(sc[kbk][i0], sc[kbk][i0 + 1], 0, false);
      v = __builtin_amdgcn_cvt_pk_fp8_f32(sc[kbk][i0 + 2], sc[kbk][i0 + 3], v, true);
      pb[wd] = v;
    }
    // V^T (d row 32 db + n, slots 8m .. 8m+7 = LDS rows 16m + 8 grp .. +7) by transpose
    // reads: lane s of a 16-lane group addresses row s / 2 of the 8, half s % 2 of the
    // d chunk 2 db + (n / 16)
    const uint8_t* vs = lds + stage * L::STAGE + L::K_BYTES;
    const int s16 = lane & 15;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int cch = 2 * db + (n >> 4);
      i32x8 av;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int row = 16 * m + 8 * grp + (s16 >> 1);
        const u32x2 r = tr8_read(vs + row * D + ((cch ^ v_swz<D>(row)) * 16) + 8 * (s16 & 1));
        av[2 * m] = (int)r.x;
        av[2 * m + 1] = (int)r.y;
      }
      o[db] = mfma_fp8(av, pb, o[db]);
    }
  };

  // One step: tile t is in `cur` (scored, prepared), tile t+1 is scored into `nxt`.  A
  // wave whose rows see nothing of a tile (causal band) skips its work; every wave
  // still stages and passes the barrier.
  const int nt = plan.n_visit;
  const int wn = wplan.n_visit;
  auto step = [&](int t, f32x16 (&cur)[2], f32x16 (&nxt)[2]) {
    const bool has_new = t + 2 < nt;
    if (has_new) load_tile(t + 2, (t + 2) % kStages);
    const bool has_cur = t < wn, has_nxt = t + 1 < wn;
    const int s_cur = t % kStages, s_nxt = (t + 1) % kStages;
    float rs0 = 0.f, rs1 = 0.f;
    const bool masked = t >= wplan.first_masked;
    if (has_cur && has_nxt) {
      if (masked) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          qk_part(nxt, s_nxt, c * KPC, (c + 1) * KPC);
          exp_part(std::true_type{}, cur, t, c, rs0, rs1);
        }
      } else {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          qk_part(nxt, s_nxt, c * KPC, (c + 1) * KPC);
          exp_part(std::false_type{}, cur, t, c, rs0, rs1);
        }
      }
    } else if (has_cur) {
      if (masked) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) exp_part(std::true_type{}, cur, t, c, rs0, rs1);
      } else {
#pragma unroll
        for (int c = 0; c < NCH; ++c) exp_part(std::false_type{}, cur, t, c, rs0, rs1);
      }
    } else if (has_nxt) {
      qk_part(nxt, s_nxt, 0, KC);
    }
    if (has_cur) finish(cur, t, s_cur, rs0, rs1);
    if (has_new) store_tile((t + 2) % kStages);
    if (has_nxt) prepare(nxt, t + 1, t + 1 >= wplan.first_masked);
    wait_vmcnt<0>();                         // this thread's direct V loads have landed
    __syncthreads();
  };

  if (nt > 0) {
    load_tile(0, 0);
    store_tile(0);
  }
  if (nt > 1) {
    load_tile(1, 1);
    store_tile(1);
  }
  wait_vmcnt<0>();
  __syncthreads();
  f32x16 sa[2], sb[2];
  if (wn > 0) {
    qk_part(sa, 0, 0, KC);
    prepare(sa, 0, 0 >= wplan.first_masked);
  }
  for (int t = 0; t < nt; t += 2) {
    step(t, sa, sb);
    if (t + 1 < nt) step(t + 1, sb, sa);
  }

  const float l_tot = l_i + __shfl_xor(l_i, 32);
  const bool empty = (m_i == -INFINITY) || !(l_tot > 0.f);
  const float inv = empty ? 0.f : s_v / l_tot;
  if (qrow < a.Sq) {
    const int64_t orow = (int64_t)(b * a.Hq + h) * a.Sq + qrow;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int col = db * 32 + 8 * r4 + 4 * grp;
        if (OF32) {
          f32x4 v4 = {o[db][4 * r4] * inv, o[db][4 * r4 + 1] * inv, o[db][4 * r4 + 2] * inv, o[db][4 * r4 + 3] * inv};
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.o) + orow * D + col) = v4;
        } else {
          u32x2 pk;
          pk.x = Elem<bf16>::pack2(o[db][4 * r4] * inv, o[db][4 * r4 + 1] * inv);
          pk.y = Elem<bf16>::pack2(o[db][4 * r4 + 2] * inv, o[db][4 * r4 + 3] * inv);
          *reinterpret_cast<u32x2*>(reinterpret_cast<bf16*>(a.o) + orow * D + col) = pk;
        }
      }
    }
    if (a.lse != nullptr && grp == 0)
      a.lse[orow] = empty ? -INFINITY : (m_i + __log2f(l_tot) - 8.f) * ATTN_LN2;
  }
}

template <int D, int NW>
hipError_t launch_fp8(const Fp8Args& a0, hipStream_t stream) {
  Fp8Args a = a0;
  a.nqt = (a.Sq + NW * 32 - 1) / (NW * 32);
  const dim3 grid((unsigned)(a.nqt * a.B * a.Hq));
  if (a.o_f32)
    hipLaunchKernelGGL((fp8_fwd_kernel<D, NW, true>), grid, dim3(NW * kWave), 0, stream, a);
  else
    hipLaunchKernelGGL((fp8_fwd_kernel<D, NW, false>), grid, dim3(NW * kWave), 0, stream, a);
  return hipGetLastError();
}

template <int D, int NW>
hipError_t launch_fp8_c(const Fp8Args& a, hipStream_t stream) {
  return launch_fp8<D, NW>(a, stream);
}

}  // namespace

int attn_fp8_tile_keys() { return BC; }

// Eight waves (256 query rows) per workgroup when that still gives every compute unit a
// workgroup: each staged K/V tile (E4M3 widening, V transpose) then serves twice the
// rows ([4,16,8192,128]: 2.93 -> 2.37 ms); four otherwise.
hipError_t attn_launch_fwd_fp8(const Fp8Args& a, hipStream_t stream) {
  const int64_t wgs256 = (int64_t)((a.Sq + 255) / 256) * a.B * a.Hq;
  if (a.d == 64) return wgs256 >= 256 ? launch_fp8_c<64, 8>(a, stream) : launch_fp8_c<64, 4>(a, stream);
  return wgs256 >= 256 ? launch_fp8_c<128, 8>(a, stream) : launch_fp8_c<128, 4>(a, stream);
}

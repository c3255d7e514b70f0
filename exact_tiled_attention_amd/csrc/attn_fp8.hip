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
// V^T is stored in LDS with the keys of each d row permuted so that the 32 keys a lane
// group needs for one 64-key contraction are 32 contiguous bytes: key k lives at byte
// 32 * ((k >> 2) & 1) + ((k >> 3) << 2) + (k & 3) of its row.
#include <type_traits>

#include "attn_device.h"
#include "attn_launch.h"
#include "tile_plan.h"

namespace {

constexpr int kWave = 64;
constexpr int BC = 64;
constexpr int SCALE_ROWS = 128;

typedef __attribute__((ext_vector_type(8))) int i32x8;

template <int D>
struct Fp8Lds {
  static constexpr int KSTR = D + 8;      // bf16 elements per K row (widened from E4M3)
  static constexpr int VSTR = BC + 16;    // bytes per V^T row (E4M3)
  static constexpr int K_BYTES = BC * KSTR * 2;
  static constexpr int V_BYTES = D * VSTR;
  static constexpr int STAGE = K_BYTES + V_BYTES;
};

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

__device__ inline int vt_pos(int k) { return 32 * ((k >> 2) & 1) + ((k >> 3) << 2) + (k & 3); }

template <int D, int NW, bool OF32>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(2))) void fp8_fwd_kernel(Fp8Args a) {
  // causal masking is a runtime flag: the plans and the per-lane key limit below carry it
  const bool CAUSAL = a.causal != 0;
  typedef Fp8Lds<D> L;
  constexpr int NT = NW * kWave;
  constexpr int BQ = NW * 32;
  constexpr int K_LOADS = (BC * D / 16 + NT - 1) / NT;     // 16-byte K chunks per thread
  constexpr int V_BLOCKS = (BC / 4) * (D / 16);            // 4-key x 16-d byte blocks

  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * L::STAGE];

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
  u32x4 vreg[4];

  auto load_tile = [&](int t) {
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
    if (tid < V_BLOCKS) {
      const int kq = tid / (D / 16);
      const int dc = tid % (D / 16);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int key = k0 + 4 * kq + s;
        u32x4 val = {0u, 0u, 0u, 0u};
        if (key < a.Sk) val = ld_global_16(vb + (int64_t)key * D + dc * 16);
        vreg[s] = val;
      }
    }
  };

  auto store_tile = [&](int stage) {
    uint8_t* ks = lds + stage * L::STAGE;
    uint8_t* vs = ks + L::K_BYTES;
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
    if (tid < V_BLOCKS) {
      const int kq = tid / (D / 16);
      const int dc = tid % (D / 16);
      const int pos = vt_pos(4 * kq);
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        // 4 keys x 4 d bytes -> 4 dwords, each holding the 4 keys of one d column
        const uint32_t r0 = vreg[0][wd], r1 = vreg[1][wd], r2 = vreg[2][wd], r3 = vreg[3][wd];
        const uint32_t lo01 = __builtin_amdgcn_perm(r1, r0, 0x05010400u);
        const uint32_t lo23 = __builtin_amdgcn_perm(r3, r2, 0x05010400u);
        const uint32_t hi01 = __builtin_amdgcn_perm(r1, r0, 0x07030602u);
        const uint32_t hi23 = __builtin_amdgcn_perm(r3, r2, 0x07030602u);
        const uint32_t c0 = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);
        const uint32_t c1 = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);
        const uint32_t c2 = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
        const uint32_t c3 = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
        const int d0 = dc * 16 + 4 * wd;
        *reinterpret_cast<uint32_t*>(vs + (d0 + 0) * L::VSTR + pos) = c0;
        *reinterpret_cast<uint32_t*>(vs + (d0 + 1) * L::VSTR + pos) = c1;
        *reinterpret_cast<uint32_t*>(vs + (d0 + 2) * L::VSTR + pos) = c2;
        *reinterpret_cast<uint32_t*>(vs + (d0 + 3) * L::VSTR + pos) = c3;
      }
    }
  };

  // One K/V tile.  MASKED applies the key-tail mask (only the tiles the plan marks).
  auto compute_tile = [&](auto masked_tag, int t, int stage) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const uint8_t* ks = lds + stage * L::STAGE;
    const uint8_t* vs = ks + L::K_BYTES;
    const float dk = ksc[(t * BC) / SCALE_ROWS];
    const float dv = vsc[(t * BC) / SCALE_ROWS];
    f32x16 s[2];
    const bf16* kbf = reinterpret_cast<const bf16*>(ks);
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) {
#pragma unroll
      for (int kbk = 0; kbk < 2; ++kbk) {
        const bf16x8 av = as_v8<bf16x8>(ld_lds_16(kbf + (kbk * 32 + n) * L::KSTR + 16 * kc + 8 * grp));
        s[kbk] = Elem<bf16>::mfma(av, qf[kc], kc == 0 ? f32x16{} : s[kbk]);
      }
      if ((kc & 1) == 1) __builtin_amdgcn_sched_barrier(0);   // bound the reads in flight
    }
    // Descales before the row max: x = csc * s with csc = scale log2(e) dQ dK.  The max
    // is taken on the raw accumulators (csc >= 0: descales are positive and a negative
    // score scale is moved into Q), so x enters only through one FMA below.
    const float csc = c_q * dk;
    // visibility of register i of key block kbk: its key offset against this lane's
    // limit (the per-register offsets are constants, one compare each)
    const int lim = klim - t * BC - 4 * grp;
    auto vis = [&](int kbk, int i) { return !MASKED || (kbk * 32 + 8 * (i >> 2) + (i & 3)) < lim; };
    if constexpr (MASKED) {
#pragma unroll
      for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kbk][i] = vis(kbk, i) ? s[kbk][i] : -INFINITY;
    }
    float r0 = vmax(s[0][0], s[0][1]), r1 = vmax(s[0][2], s[0][3]);
#pragma unroll
    for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
      for (int i = (kbk == 0 ? 4 : 0); i < 16; i += 4) {
        r0 = vmax(r0, vmax(s[kbk][i], s[kbk][i + 1]));
        r1 = vmax(r1, vmax(s[kbk][i + 2], s[kbk][i + 3]));
      }
    const float mr = vmax(r0, r1);
    const float mx = max_pair32(mr == -INFINITY ? -INFINITY : mr * csc);
    const float m_new = fmaxf(m_i, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_i - m_use);
    const float m_off = m_use - 8.f;                 // u = 2^8 exp2(x - m)
    float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
    for (int kbk = 0; kbk < 2; ++kbk) {
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        // masked cells give u = 0 by selection (a zero descale or scale makes csc = 0,
        // and fma(-inf, 0, .) would be NaN)
        float u0 = fast_exp2(fmaf(s[kbk][i], csc, -m_off));
        float u1 = fast_exp2(fmaf(s[kbk][i + 1], csc, -m_off));
        if constexpr (MASKED) {
          u0 = vis(kbk, i) ? u0 : 0.f;
          u1 = vis(kbk, i + 1) ? u1 : 0.f;
        }
        s[kbk][i] = u0;
        s[kbk][i + 1] = u1;
        rs0 += u0;
        rs1 += u1;
      }
    }
    l_i = alpha * l_i + (rs0 + rs1);
    m_i = m_new;
    // The accumulator is kept in units of the current V descale s_v: moving to a tile
    // with descale dv (and a moved max) multiplies it by alpha s_v / dv, skipped when
    // that is 1 in every lane (same scale block, unmoved max).  A zero V descale (an
    // all-zero value block) makes the tile's values zero: the accumulator keeps its
    // frame and the tile adds nothing (dv is the same for every lane of the workgroup).
    const bool v_zero = !(dv != 0.f);
    const float beta = v_zero ? alpha : alpha * (s_v / dv);
    if (!v_zero) s_v = dv;
    if (wave_any(beta != 1.f)) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= beta;
      }
    }
    // A zero-valued tile adds nothing in the current frame (dv is the same in every lane).
    if (v_zero) return;
    // P^T as the fp8 B operand: slot j = register (j % 16) of key block j / 16.
    i32x8 pb;
#pragma unroll
    for (int wd = 0; wd < 8; ++wd) {
      const int kbk = wd >> 2;
      const int i0 = 4 * (wd & 3);
      int v = __builtin_amdgcn_cvt_pk_fp8_f32(s[kbk][i0], s[kbk][i0 + 1], 0, false);
      v = __builtin_amdgcn_cvt_pk_fp8_f32(s[kbk][i0 + 2], s[kbk][i0 + 3], v, true);
      pb[wd] = v;
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const uint8_t* vr = vs + (db * 32 + n) * L::VSTR + 32 * grp;
      const u32x4 lo = ld_lds_16(vr), hi = ld_lds_16(vr + 16);
      const i32x8 av = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      o[db] = mfma_fp8(av, pb, o[db]);
    }
  };

  const int nt = plan.n_visit;
  if (nt > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();
  for (int t = 0; t < nt; ++t) {
    const int stage = t & 1;
    if (t + 1 < nt) load_tile(t + 1);
    // a wave whose rows see nothing of tile t (causal band) skips it; every wave still
    // stages and passes the barrier
    if (t < wplan.n_visit) {
      if (t >= wplan.first_masked)
        compute_tile(std::true_type{}, t, stage);
      else
        compute_tile(std::false_type{}, t, stage);
    }
    if (t + 1 < nt) store_tile(stage ^ 1);
    __syncthreads();
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

// attn_decode.hip -- split-KV decode with an exact merge of partial states (gfx950).
//
// Decode has one query row per (sequence, query head), so the query-tile axis of the
// prefill grid collapses; the K/V axis is split into chunks instead and each chunk
// produces a partial state that a second pass merges ("M4.4 - FlashAttention-2 Work
// Partitioning and the Decode Boundary", section 0x01, the Flash-Decoding work axis;
// "M4.3 - IO-Aware Attention ...", sections 0x08B-0x08F: partial (m, l, u) states of
// disjoint key sets merge exactly, in any order, once they share one max frame).
//
// Pass 1 (split): one workgroup per (chunk, batch item, K/V head, head pass).  The
// chunk is read from HBM exactly once for the G query heads of the pass.  The work is
// a handful of dot products per key, far too thin for the matrix cores, and the
// kernel is bound by HBM bandwidth, so it stays on the vector ALUs:
//   * lane (row group rg, column chunk c8) loads 16 contiguous bytes of a key row, so
//     every wave-wide load covers whole rows (LPR lanes per row, RPI rows per load);
//   * q.k partial dots use v_dot2 on packed 16-bit pairs, then a DPP butterfly
//     (quad_perm, half-mirror, mirror) sums the LPR lanes of a row;
//   * p.V runs as v_dot2 over pairs of keys after an in-register interleave of V;
//   * each wave keeps (m, l, u) for its keys; the four waves merge through LDS and
//     write one partial per (chunk, query head).
// Pass 2 (merge): one wave per (batch item, query head) folds the partials in one
// max frame, O = u / l, LSE = m + ln l (all in base 2 internally).
#include "attn_device.h"
#include "attn_launch.h"

namespace {

constexpr int kThreads = 256;
#ifndef ATTN_DECODE_SUB
#define ATTN_DECODE_SUB 64
#endif
constexpr int kSub = ATTN_DECODE_SUB;   // keys per wave per sub-tile

template <typename T> struct Dot2;
template <> struct Dot2<f16> {
  static __device__ inline float dot(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
  }
};
template <> struct Dot2<bf16> {
  static __device__ inline float dot(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
  }
};

template <int CTRL> __device__ inline float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over the LPR consecutive lanes of a row group (LPR = 8 or 16); every lane of the
// group receives the total.
template <int LPR> __device__ inline float row_group_sum(float x) {
  x += dpp_mov<0xB1>(x);    // quad_perm [1,0,3,2]
  x += dpp_mov<0x4E>(x);    // quad_perm [2,3,0,1]
  x += dpp_mov<0x141>(x);   // row_half_mirror: pairs the two quads of each 8 lanes
  if (LPR == 16) x += dpp_mov<0x140>(x);   // row_mirror: pairs the two halves of 16
  return x;
}

// Combine across row groups (lanes LPR, 2 LPR, ... apart).
template <int LPR> __device__ inline float across_groups_max(float x) {
#pragma unroll
  for (int s = LPR; s < 64; s <<= 1) x = fmaxf(x, __shfl_xor(x, s));
  return x;
}
template <int LPR> __device__ inline float across_groups_sum(float x) {
#pragma unroll
  for (int s = LPR; s < 64; s <<= 1) x += __shfl_xor(x, s);
  return x;
}

template <typename T, int D, int G>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeArgs a) {
  constexpr int LPR = D / 8;          // lanes per key row (16 bytes each)
  constexpr int RPI = 64 / LPR;       // key rows per wave-wide load
  constexpr int NI = kSub / RPI;      // rows per lane per sub-tile
  typedef Dot2<T> DT;

  __shared__ float s_m[4][G];
  __shared__ float s_l[4][G];
  __shared__ float s_u[4][G][D];

  const int c = blockIdx.x;
  const int bkv = blockIdx.y;
  const int b = bkv / a.Hkv;
  const int kvh = bkv - b * a.Hkv;
  const int h0 = kvh * a.group + blockIdx.z * G;   // first query head of this pass

  int len = a.seqlens[b];
  len = len < 0 ? 0 : (len > a.Smax ? a.Smax : len);
  const int kbeg = c * a.chunk;
  if (kbeg >= len) return;                          // whole workgroup: no barrier reached
  const int kend = min(kbeg + a.chunk, len);

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int rg = lane / LPR;
  const int c8 = lane % LPR;

  const T* __restrict__ kbase = reinterpret_cast<const T*>(a.k) + ((int64_t)(b * a.Hkv + kvh) * a.Smax) * D;
  const T* __restrict__ vbase = reinterpret_cast<const T*>(a.v) + ((int64_t)(b * a.Hkv + kvh) * a.Smax) * D;
  const T* __restrict__ qbase = reinterpret_cast<const T*>(a.q) + ((int64_t)b * a.Hq + h0) * D;

  u32x4 qv[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) qv[hh] = ld_global_16(qbase + (int64_t)hh * D + 8 * c8);

  float m[G], l[G], u[G][8];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) u[hh][j] = 0.f;
  }

  for (int base = kbeg + kSub * w; base < kend; base += 4 * kSub) {
    u32x4 kr[NI], vr[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int key = base + rg + RPI * i;
      u32x4 zk = {0u, 0u, 0u, 0u};
      u32x4 zv = {0u, 0u, 0u, 0u};
      if (key < kend) {
        zk = ld_global_16(kbase + (int64_t)key * D + 8 * c8);
        zv = ld_global_16(vbase + (int64_t)key * D + 8 * c8);
      }
      kr[i] = zk;
      vr[i] = zv;
    }
    // Interleave V by key pairs: vp[i/2][2*dw+e] packs (V[i][d], V[i+1][d]).
    uint32_t vp[NI / 2][8];
#pragma unroll
    for (int i = 0; i < NI; i += 2) {
#pragma unroll
      for (int dw = 0; dw < 4; ++dw) {
        vp[i / 2][2 * dw] = pack_lo(vr[i][dw], vr[i + 1][dw]);
        vp[i / 2][2 * dw + 1] = pack_hi(vr[i][dw], vr[i + 1][dw]);
      }
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float s[NI];
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        float acc = 0.f;
#pragma unroll
        for (int dw = 0; dw < 4; ++dw) acc = DT::dot(qv[hh][dw], kr[i][dw], acc);
        acc = row_group_sum<LPR>(acc);
        const int key = base + rg + RPI * i;
        const float x = key < kend ? acc * a.scale_log2 : -INFINITY;
        s[i] = x;
        mx = fmaxf(mx, x);
      }
      mx = across_groups_max<LPR>(mx);
      const float m_new = fmaxf(m[hh], mx);          // finite: key `base` is valid
      const float alpha = fast_exp2(m[hh] - m_new);
      float rs = 0.f;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        s[i] = fast_exp2(s[i] - m_new);
        rs += s[i];
      }
      l[hh] = alpha * l[hh] + rs;
      m[hh] = m_new;
#pragma unroll
      for (int j = 0; j < 8; ++j) u[hh][j] *= alpha;
#pragma unroll
      for (int i = 0; i < NI; i += 2) {
        const uint32_t pp = Elem<T>::pack2(s[i], s[i + 1]);
#pragma unroll
        for (int j = 0; j < 8; ++j) u[hh][j] = DT::dot(pp, vp[i / 2][j], u[hh][j]);
      }
    }
  }

  // Sum each wave's per-lane shares over its row groups, then merge the four waves.
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const float lt = across_groups_sum<LPR>(l[hh]);
#pragma unroll
    for (int j = 0; j < 8; ++j) u[hh][j] = across_groups_sum<LPR>(u[hh][j]);
    if (lane == 0) {
      s_m[w][hh] = m[hh];
      s_l[w][hh] = lt;
    }
    if (rg == 0) {
#pragma unroll
      for (int j = 0; j < 8; ++j) s_u[w][hh][8 * c8 + j] = u[hh][j];
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int hh = idx / D;
    const int d = idx - hh * D;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, s_m[ww][hh]);
    float L = 0.f, U = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float mw = s_m[ww][hh];
      if (mw != -INFINITY) {                  // a wave with no keys is the identity
        const float f = fast_exp2(mw - M);
        L += f * s_l[ww][hh];
        U += f * s_u[ww][hh][d];
      }
    }
    const int64_t part = ((int64_t)b * a.Hq + h0 + hh) * a.nchunk + c;
    a.part_u[part * D + d] = U;
    if (d == 0) {
      a.part_ml[2 * part] = M;
      a.part_ml[2 * part + 1] = L;
    }
  }
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void decode_merge_kernel(DecodeArgs a) {
  constexpr int PER = D / 64;   // d values per lane
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);   // (b, query head)
  const int lane = threadIdx.x & 63;
  if (row >= a.B * a.Hq) return;
  const int b = row / a.Hq;
  int len = a.seqlens[b];
  len = len < 0 ? 0 : (len > a.Smax ? a.Smax : len);
  const int nch = (len + a.chunk - 1) / a.chunk;
  const float* ml = a.part_ml + (int64_t)row * a.nchunk * 2;
  const float* pu = a.part_u + (int64_t)row * a.nchunk * D;

  float M = -INFINITY;
  for (int cc = lane; cc < nch; cc += 64) M = fmaxf(M, ml[2 * cc]);
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) M = fmaxf(M, __shfl_xor(M, s));

  // Fold the partials in batches of 8 so that eight chunks' loads are in flight
  // together (the fold itself is a short dependent chain).
  constexpr int BATCH = 8;
  float L = 0.f;
  float U[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) U[j] = 0.f;
  for (int c0 = 0; c0 < nch; c0 += BATCH) {
    float mv[BATCH], lv[BATCH], uv[BATCH][PER];
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      const int cc = min(c0 + j, nch - 1);
      mv[j] = ml[2 * cc];
      lv[j] = ml[2 * cc + 1];
#pragma unroll
      for (int q = 0; q < PER; ++q) uv[j][q] = pu[(int64_t)cc * D + lane + 64 * q];
    }
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      const float f = (c0 + j < nch) ? fast_exp2(mv[j] - M) : 0.f;
      L += f * lv[j];
#pragma unroll
      for (int q = 0; q < PER; ++q) U[q] += f * uv[j][q];
    }
  }
  const bool empty = nch == 0 || !(L > 0.f);
  const float inv = empty ? 0.f : 1.f / L;
  T* o = reinterpret_cast<T*>(a.o) + (int64_t)row * D;
#pragma unroll
  for (int j = 0; j < PER; ++j) o[lane + 64 * j] = Elem<T>::from_f(U[j] * inv);
  if (a.lse != nullptr && lane == 0) a.lse[row] = empty ? -INFINITY : (M + __log2f(L)) * ATTN_LN2;
}

template <typename T, int D, int G>
hipError_t launch_g(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)a.nchunk, (unsigned)(a.B * a.Hkv), (unsigned)(a.group / G));
  hipLaunchKernelGGL((decode_split_kernel<T, D, G>), grid, dim3(kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid2((unsigned)((a.B * a.Hq + 3) / 4));
  hipLaunchKernelGGL((decode_merge_kernel<T, D>), grid2, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t stream) {
  if (a.group % 4 == 0) return launch_g<T, D, 4>(a, stream);
  if (a.group % 2 == 0) return launch_g<T, D, 2>(a, stream);
  return launch_g<T, D, 1>(a, stream);
}

template <typename T>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  if (a.d == 64) return launch_d<T, 64>(a, stream);
  return launch_d<T, 128>(a, stream);
}

}  // namespace

hipError_t attn_launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.dtype_bf16) return launch_t<bf16>(a, stream);
  return launch_t<f16>(a, stream);
}

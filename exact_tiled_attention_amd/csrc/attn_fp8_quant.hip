// attn_fp8_quant.hip -- E4M3 quantisation of Q/K/V with optional incoherent processing.
//
// "M4.6 - FlashAttention-3/4 Hardware Pipelines ...", section 0x06: per-block descales
// (one per 128 rows of one (batch, head)) or one per tensor, and for Q and K the
// optional right transform R = diag(s) H / sqrt(d) (random signs s, Sylvester Hadamard
// H; orthogonal, so (Q R)(K R)^T = Q K^T before quantisation; V is not transformed).
//
// Sixteen lanes hold one row of d values (8 per lane for d = 128, 4 for d = 64); the
// Walsh-Hadamard butterflies run inside a lane for element distances below the lane's
// share and across lanes (shuffles) above it, in Sylvester order: the pair (i, i + len)
// becomes (a + b, a - b).
//   pass 1: transform, block amax -> descale (block mode) or raw amax (tensor mode);
//   pass 2 (tensor mode): one workgroup reduces the amaxes and writes every descale;
//   pass 3: the same transform (identical float32 arithmetic), x / descale clamped to
//           +-448, rounded to E4M3 by the hardware conversion (nearest even).
#include "../../include/attn.h"
#include "attn_device.h"
#include "attn_launch.h"

namespace {

constexpr int kQT = 256;       // threads per workgroup
constexpr int kQRows = 128;    // rows per descale block
constexpr float kE4M3Max = 448.f;

// Load this lane's EPL values of a row (16 lanes per row), apply signs and the
// normalised Walsh-Hadamard transform when HAD.
template <typename T, int D, bool HAD>
__device__ inline void row_values(const T* row, const float* signs, int l16, float (&x)[D / 16]) {
  constexpr int EPL = D / 16;
  const T* p = row + EPL * l16;
  if constexpr (EPL == 8) {
    const u32x4 raw = ld_global_16(p);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      x[2 * w] = Elem<T>::to_f(__builtin_bit_cast(T, (uint16_t)(raw[w] & 0xFFFF)));
      x[2 * w + 1] = Elem<T>::to_f(__builtin_bit_cast(T, (uint16_t)(raw[w] >> 16)));
    }
  } else {
    const u32x2 raw = *reinterpret_cast<const u32x2*>(p);
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      x[2 * w] = Elem<T>::to_f(__builtin_bit_cast(T, (uint16_t)(raw[w] & 0xFFFF)));
      x[2 * w + 1] = Elem<T>::to_f(__builtin_bit_cast(T, (uint16_t)(raw[w] >> 16)));
    }
  }
  if constexpr (HAD) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) x[e] *= signs[EPL * l16 + e];
    // element distances 1 .. EPL/2 inside the lane
#pragma unroll
    for (int len = 1; len < EPL; len <<= 1)
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if ((i & len) == 0) {
          const float a = x[i], b = x[i + len];
          x[i] = a + b;
          x[i + len] = a - b;
        }
    // distances EPL .. D/2 across the 16 lanes of the row
#pragma unroll
    for (int lm = 1; lm < 16; lm <<= 1) {
      const bool upper = (l16 & lm) != 0;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const float o = __shfl_xor(x[i], lm);
        x[i] = upper ? o - x[i] : x[i] + o;
      }
    }
    const float norm = 1.f / __builtin_sqrtf((float)D);
#pragma unroll
    for (int i = 0; i < EPL; ++i) x[i] *= norm;
  }
}

template <typename T, int D, bool HAD>
__global__ __launch_bounds__(kQT) void quant_amax_kernel(QuantArgs a) {
  constexpr int EPL = D / 16;
  const int blk = blockIdx.x, bh = blockIdx.y;
  const int l16 = threadIdx.x & 15;
  const int r0 = threadIdx.x >> 4;          // 16 rows per pass
  const T* base = reinterpret_cast<const T*>(a.x) + (int64_t)bh * a.S * D;
  float m = 0.f;
  for (int r = r0; r < kQRows; r += kQT / 16) {
    const int row = blk * kQRows + r;
    if (row < a.S) {                          // uniform over the row's 16 lanes
      float x[EPL];
      row_values<T, D, HAD>(base + (int64_t)row * D, a.signs, l16, x);
#pragma unroll
      for (int i = 0; i < EPL; ++i) m = fmaxf(m, fabsf(x[i]));
    }
  }
  __shared__ float red[kQT / 64];
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) m = fmaxf(m, __shfl_xor(m, s));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = red[0];
#pragma unroll
    for (int w = 1; w < kQT / 64; ++w) t = fmaxf(t, red[w]);
    const int64_t idx = (int64_t)bh * a.nblk + blk;
    a.descale[idx] = a.per_tensor ? t : (t > 0.f ? t / kE4M3Max : 1.f);
  }
}

// one workgroup: amax over every block, then every descale
__global__ __launch_bounds__(kQT) void quant_tensor_kernel(QuantArgs a, int64_t n) {
  float m = 0.f;
  for (int64_t i = threadIdx.x; i < n; i += kQT) m = fmaxf(m, a.descale[i]);
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) m = fmaxf(m, __shfl_xor(m, s));
  __shared__ float red[kQT / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  float t = red[0];
#pragma unroll
  for (int w = 1; w < kQT / 64; ++w) t = fmaxf(t, red[w]);
  const float desc = t > 0.f ? t / kE4M3Max : 1.f;
  for (int64_t i = threadIdx.x; i < n; i += kQT) a.descale[i] = desc;
}

template <typename T, int D, bool HAD>
__global__ __launch_bounds__(kQT) void quant_encode_kernel(QuantArgs a) {
  constexpr int EPL = D / 16;
  const int blk = blockIdx.x, bh = blockIdx.y;
  const int l16 = threadIdx.x & 15;
  const int r0 = threadIdx.x >> 4;
  const T* base = reinterpret_cast<const T*>(a.x) + (int64_t)bh * a.S * D;
  uint8_t* out = a.codes + (int64_t)bh * a.S * D;
  const float desc = a.descale[(int64_t)bh * a.nblk + blk];
  for (int r = r0; r < kQRows; r += kQT / 16) {
    const int row = blk * kQRows + r;
    if (row >= a.S) break;
    float x[EPL];
    row_values<T, D, HAD>(base + (int64_t)row * D, a.signs, l16, x);
    uint32_t w[EPL / 4];
#pragma unroll
    for (int i = 0; i < EPL / 4; ++i) {
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = fminf(fmaxf(x[4 * i + e] / desc, -kE4M3Max), kE4M3Max);
      int pk = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
      pk = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], pk, true);
      w[i] = (uint32_t)pk;
    }
    uint8_t* dst = out + (int64_t)row * D + EPL * l16;
    if constexpr (EPL == 8)
      *reinterpret_cast<u32x2*>(dst) = u32x2{w[0], w[1]};
    else
      *reinterpret_cast<uint32_t*>(dst) = w[0];
  }
}

template <typename T, int D, bool HAD>
hipError_t launch_q(const QuantArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)a.nblk, (unsigned)(a.B * a.H));
  hipLaunchKernelGGL((quant_amax_kernel<T, D, HAD>), grid, dim3(kQT), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.per_tensor) {
    hipLaunchKernelGGL(quant_tensor_kernel, dim3(1), dim3(kQT), 0, stream, a, (int64_t)a.B * a.H * a.nblk);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((quant_encode_kernel<T, D, HAD>), grid, dim3(kQT), 0, stream, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_q_t(const QuantArgs& a, hipStream_t stream) {
  const bool had = a.signs != nullptr;
  if (a.d == 64) return had ? launch_q<T, 64, true>(a, stream) : launch_q<T, 64, false>(a, stream);
  return had ? launch_q<T, 128, true>(a, stream) : launch_q<T, 128, false>(a, stream);
}

}  // namespace

hipError_t attn_launch_fp8_quantize(const QuantArgs& a, hipStream_t stream) {
  if (a.dtype_bf16) return launch_q_t<bf16>(a, stream);
  return launch_q_t<f16>(a, stream);
}

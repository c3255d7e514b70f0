// attn_device.h -- gfx950 device helpers: element types, MFMA wrappers, lane layouts.
//
// Matrix-core layout used throughout (v_mfma_f32_32x32x16_{f16,bf16}, wave64):
//   A operand (32 x 16, M x K): lane l holds row  m = l % 32 and 8 contraction slots
//   B operand (16 x 32, K x N): lane l holds column n = l % 32 and the same 8 slots
//   C/D       (32 x 32)       : lane l holds column n = l % 32, register i holds row
//                               m = 8 * (i / 4) + 4 * (l / 32) + (i % 4).
// The contraction slots of lane l are the 8 values of lane group g = l / 32; A and B
// pair slot-for-slot, so any consistent assignment of contraction indices to
// (g, slot) is a valid product.  The kernels choose that assignment per product.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 f16;
typedef __bf16 bf16;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

#define ATTN_LOG2E 1.4426950408889634f
#define ATTN_LN2 0.6931471805599453f

// Element traits: 8-wide operand vector and conversions.
template <typename T> struct Elem;
template <> struct Elem<f16> {
  typedef f16x8 v8;
  static __device__ inline float to_f(f16 x) { return (float)x; }
  static __device__ inline f16 from_f(float x) { return (f16)x; }
  static __device__ inline uint32_t pack2(float a, float b) {
    f16x2 h;
    h.x = (f16)a;
    h.y = (f16)b;
    return __builtin_bit_cast(uint32_t, h);
  }
  static __device__ inline f32x16 mfma(const v8& a, const v8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};
template <> struct Elem<bf16> {
  typedef bf16x8 v8;
  static __device__ inline float to_f(bf16 x) { return (float)x; }
  static __device__ inline bf16 from_f(float x) { return (bf16)x; }
  static __device__ inline uint32_t pack2(float a, float b) {
    bf16x2 h;
    h.x = (bf16)a;
    h.y = (bf16)b;
    return __builtin_bit_cast(uint32_t, h);
  }
  static __device__ inline f32x16 mfma(const v8& a, const v8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <typename V> __device__ inline V as_v8(const u32x4& u) { return __builtin_bit_cast(V, u); }

__device__ inline u32x4 ld_global_16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ inline void st_global_16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }

__device__ inline u32x4 ld_lds_16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ inline u32x2 ld_lds_8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }
__device__ inline void st_lds_16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ inline void st_lds_8(void* p, const u32x2& v) { *reinterpret_cast<u32x2*>(p) = v; }

__device__ inline float wave_max_xor32(float x) { return fmaxf(x, __shfl_xor(x, 32)); }
__device__ inline float wave_sum_xor32(float x) { return x + __shfl_xor(x, 32); }

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Software exp2 on the FMA pipe ("M4.6 - FlashAttention-3/4 Hardware Pipelines",
// section 0x09): x = n + f with n = floor(x) and f in [0, 1); 2^f from the degree-3
// polynomial that minimises the maximum relative error on [0, 1] (coefficients fitted
// for this library by the Remez exchange, 7.5e-5), scaled by 2^n through the exponent.
// Arguments below -150 (and -inf) give 0; a NaN argument gives 0 as well.
__device__ inline float soft_exp2(float x) {
  x = fmaxf(x, -150.f);
  const float n = __builtin_floorf(x);
  const float f = x - n;
  float p = fmaf(0.07802452147006989f, f, 0.22606715559959412f);
  p = fmaf(p, f, 0.6958335638046265f);
  p = fmaf(p, f, 0.9999251961708069f);
  return __builtin_ldexpf(p, (int)n);
}

// 16-bit lane interleave helpers for the register transpose of 4 rows x 8 columns.
// lo16(a) | lo16(b) << 16  and  hi16(a) | hi16(b) << 16.
__device__ inline uint32_t pack_lo(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ inline uint32_t pack_hi(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

// Raw buffer resource over [base, base + bytes): loads at or past `bytes` return 0,
// which replaces per-element tail predicates with the hardware range check.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ inline u32x4 buf_load_16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0));
}
// Streaming form: the non-temporal hint, for data read exactly once.
__device__ inline u32x4 buf_load_16_stream(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 2));
}
__device__ inline u32x2 buf_load_8(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)byte_off, 0, 0));
}

// 32-bit LDS byte address of a pointer into __shared__ memory.
__device__ inline uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Direct buffer -> LDS load of 16 bytes per lane from byte voff + soff of the buffer:
// lane l's bytes land at LDS byte address dst + 16 l (soff and dst wave-uniform);
// out-of-range lanes write zeros.  Issued as an asm statement so that the compiler does
// not add its own (full) vmcnt waits before LDS reads of the ring: the kernels wait
// explicitly with wait_vmcnt.  The statement sets M0, which the kernels' compiled code
// does not otherwise use.
__device__ inline void lds_load_16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint32_t dst) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(r), "s"(soff), "s"(dst)
               : "memory", "m0");
#pragma clang diagnostic pop
}

// Wait until at most N vector memory operations of this wave are outstanding
// (s_waitcnt vmcnt(N); the other counters are not waited on).
template <int N> __device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// True in every lane when the predicate holds in at least one active lane.
__device__ inline bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

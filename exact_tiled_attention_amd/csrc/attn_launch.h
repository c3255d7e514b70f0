// attn_launch.h -- internal launcher interface between the C ABI layer and the kernels.
// Argument checking happens in attn_api.cpp before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "attn_philox.h"

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, Hq, Hkv, Sq, Sk, d;
  int group;          // Hq / Hkv
  int causal;
  int dtype_bf16;     // 1: bf16, 0: fp16
  float scale_log2;   // scale * log2(e)
  int nqt;            // query tiles (filled by the launcher)
  // Packed variable-length layout (null cu_q: the padded [B, H, S, d] layout).  Q/O
  // token-major [total_q, Hq, d], K/V [total_k, Hkv, d], LSE [Hq, total_q]; B is the
  // number of sequences, Sq / Sk the longest ones.
  const int* cu_q;
  const int* cu_k;
  int total_q, total_k;
  int dropout;        // 1: apply dropout with `drop` (padded layout only)
  DropParams drop;
  int exp_emulated;   // 0, 2 or 4 of every 8 exponentials by soft_exp2 (padded, no dropout)
};

struct Fp8Args {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  const float* q_scale;
  const float* k_scale;
  const float* v_scale;
  void* o;
  float* lse;
  int B, Hq, Hkv, Sq, Sk, d;
  int group;
  int causal;
  int o_f32;          // 1: float32 output, 0: bf16 output
  float scale_log2;
  int nqt;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dO;
  void* dq;
  void* dk;
  void* dv;
  float* dq_acc;      // [B,Hq,Sq,d] float32 workspace
  float* delta;       // [B,Hq,Sq]  float32 workspace (D rows, pre-scaled)
  int B, Hq, Hkv, Sq, Sk, d;
  int group;
  int causal;
  int dtype_bf16;
  int grad_type;      // attn_dtype_t of dq/dk/dv
  float scale;
  float scale_log2;
  // deterministic mode: dQ from the query-owner kernel over dq_splits contiguous key
  // ranges, partials [dq_splits][B,Hq,Sq,d] float32 (when dq_splits > 1) reduced in a
  // fixed binary tree; no atomics anywhere
  int deterministic;
  int dq_splits;
  float* dq_part;
  int dropout;        // 1: regenerate the forward's dropout decisions from `drop`
  DropParams drop;
  // fp8 operands: q, k, v are E4M3 codes with float32 descales [B, H, ceil(S/128)];
  // o and dO are bf16 (dtype_bf16 = 1)
  int fp8;
  const float* q_scale;
  const float* k_scale;
  const float* v_scale;
  // owners running on exact fp16 copies of bf16 operands: the factors that undo the
  // copies' powers of two (section 5 of the backward); null otherwise
  const float* f16_fac;
};

// Deterministic mode with bf16 operands: workspace of the exact fp16 copies (host side,
// read by the preparation kernels only).  amax: [5][kBwdAmaxBlocks] per-block maxima of
// q, k, v, dO, o, then the 4 exponents (int) and kBwdFacs factors (float); copy: the
// fp16 copies of q, k, v, dO.
struct BwdF16Ws {
  uint32_t* amax;
  void* copy[4];
};
constexpr int kBwdAmaxBlocks = 512;
constexpr int kBwdFacs = 7;
// bytes of BwdF16Ws::amax (maxima, exponents, factors)
constexpr size_t kBwdAmaxBytes = (5 * kBwdAmaxBlocks + 4 + kBwdFacs) * sizeof(uint32_t);

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const int* seqlens;
  void* o;
  float* lse;
  float* part_ml;     // [B*Hq, nchunk, 2] float32 (m in base 2, l)
  float* part_u;      // [B*Hq, nchunk, d] float32
  int B, Hq, Hkv, Smax, d, chunk, nchunk;
  int group;
  int dtype_bf16;
  float scale_log2;
  // paged pool (block_table != nullptr): k, v [num_pages, Hkv, 1 << page_shift, d];
  // block_table [B, max_pages]; Smax = max_pages << page_shift
  const int* block_table;
  int max_pages, num_pages, page_shift;
};

struct QuantArgs {
  const void* x;          // [B, H, S, d] element type
  const float* signs;     // [d] +-1, or null: no transform
  uint8_t* codes;         // [B, H, S, d] E4M3
  float* descale;         // [B, H, nblk] float32
  int B, H, S, d, nblk;
  int per_tensor;
  int dtype_bf16;
};

hipError_t attn_launch_fwd(const FwdArgs& a, hipStream_t stream);
hipError_t attn_launch_exp2_soft(const float* x, float* y, int64_t n, hipStream_t stream);
hipError_t attn_launch_fp8_quantize(const QuantArgs& a, hipStream_t stream);
hipError_t attn_launch_fwd_fp8(const Fp8Args& a, hipStream_t stream);
int attn_fp8_tile_keys();
hipError_t attn_launch_bwd(const BwdArgs& a, const BwdF16Ws* f16, hipStream_t stream);
hipError_t attn_launch_decode(const DecodeArgs& a, hipStream_t stream);
// device address of the current GPU's decode scratch (ATTN_DECODE_NOALLOC_SCRATCH_BYTES)
hipError_t attn_decode_scratch(void** ptr);

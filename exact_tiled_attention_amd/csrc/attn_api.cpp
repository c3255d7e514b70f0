// attn_api.cpp -- the C ABI of libattn: argument checks (pure host, before any HIP
// call), workspace sizing and dispatch to the kernel launchers.
#include <math.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "../../include/attn.h"
#include "attn_launch.h"
#include "tile_plan.h"

namespace {

constexpr int kMaxSeq = 1 << 20;
constexpr int kMaxBH = 1 << 16;

int check_dims(int B, int Hq, int Hkv, int Sq, int Sk, int d, bool allow_sk0) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Sq <= 0) return ATTN_ERR_SHAPE;
  if (Sk < 0 || (!allow_sk0 && Sk == 0)) return ATTN_ERR_SHAPE;
  if (Sq > kMaxSeq || Sk > kMaxSeq) return ATTN_ERR_SHAPE;
  if ((int64_t)B * Hq > kMaxBH) return ATTN_ERR_SHAPE;
  if (Hq % Hkv != 0) return ATTN_ERR_GQA;
  if (d != 64 && d != 128) return ATTN_ERR_HEADDIM;
  return ATTN_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Deterministic-mode workspace: D rows | dq_splits float32 dQ partials (dq_splits > 1) |
// per-block maxima and exponents | fp16 copies of q, dO, k, v (used for bf16 operands).
// Returns the bytes needed; with a workspace, points a's fields into it.
size_t det_layout(int B, int Hq, int Hkv, int Sq, int Sk, int d, int dq_splits, void* ws, bool bf16_ops,
                  BwdArgs* a, BwdF16Ws* cw) {
  const size_t rows = (size_t)B * Hq * Sq, krows = (size_t)B * Hkv * Sk;
  const size_t o_part = align256(rows * sizeof(float));
  const size_t o_amax = o_part + (dq_splits > 1 ? align256((size_t)dq_splits * rows * d * sizeof(float)) : 0);
  const size_t o_q = o_amax + align256(kBwdAmaxBytes);
  const size_t qbytes = align256(rows * d * 2), kbytes = align256(krows * d * 2);
  const size_t o_do = o_q + qbytes, o_k = o_do + qbytes, o_v = o_k + kbytes;
  if (a != nullptr) {
    char* w = (char*)ws;
    a->delta = (float*)w;
    a->dq_part = dq_splits > 1 ? (float*)(w + o_part) : nullptr;
    if (bf16_ops) {
      cw->amax = (uint32_t*)(w + o_amax);
      cw->copy[0] = w + o_q;
      cw->copy[1] = w + o_k;
      cw->copy[2] = w + o_v;
      cw->copy[3] = w + o_do;
    }
  }
  return o_v + kbytes;
}

// attn_bwd's dQ form by key length: the column owner's atomic adds below kBwdSplitKeys
// keys, the query-row owner (the deterministic form) from there on.  Measured on MI355X,
// bf16, float32 gradients: the atomic form is 6-16 % faster at 256-512 keys, 6-9 %
// slower at 1024, 26-40 % slower at 2048-8192 keys (each 128-key column block adds one
// float32 pass over the dQ accumulator, performed past the L2).
constexpr int kBwdSplitKeys = 1024;

int decode_chunks(int Smax, int chunk) { return (Smax + chunk - 1) / chunk; }

}  // namespace

extern "C" {

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "invalid or too large tensor size";
    case ATTN_ERR_GQA: return "H_q is not a multiple of H_kv";
    case ATTN_ERR_HEADDIM: return "unsupported head dimension";
    case ATTN_ERR_DTYPE: return "unsupported element type";
    case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case ATTN_ERR_HIP: return "HIP launch or runtime error";
    case ATTN_ERR_ARG: return "argument out of range";
    default: return "unknown status";
  }
}

int attn_tile_plan(int q_begin, int q_end, int Sq, int Sk, int block_k, int causal,
                   int* n_visit, int* first_masked) {
  if (n_visit == nullptr || first_masked == nullptr) return ATTN_ERR_NULL;
  if (block_k <= 0 || Sq <= 0 || Sk < 0 || q_begin < 0 || q_end <= q_begin || q_end > Sq)
    return ATTN_ERR_ARG;
  const TilePlan p = plan_rows(q_begin, q_end, Sq, Sk, block_k, causal != 0);
  *n_visit = p.n_visit;
  *first_masked = p.first_masked;
  return ATTN_OK;
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int Hq, int Hkv, int Sq, int Sk, int d, float scale, int causal,
             attn_dtype_t dtype, void* stream) {
  if (q == nullptr || o == nullptr) return ATTN_ERR_NULL;
  if (Sk > 0 && (k == nullptr || v == nullptr)) return ATTN_ERR_NULL;
  int st = check_dims(B, Hq, Hkv, Sq, Sk, d, true);
  if (st != ATTN_OK) return st;
  if (dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
  if (!isfinite(scale)) return ATTN_ERR_ARG;
  FwdArgs a = {};
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Sq = Sq; a.Sk = Sk; a.d = d;
  a.group = Hq / Hkv;
  a.causal = causal != 0;
  a.dtype_bf16 = dtype == ATTN_BF16;
  a.scale_log2 = scale * 1.4426950408889634f;
  return hip_status(attn_launch_fwd(a, (hipStream_t)stream));
}

int attn_fwd_exp_emulated(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int Hq, int Hkv, int Sq, int Sk, int d, float scale, int causal,
                          attn_dtype_t dtype, int emulated_per_8, void* stream) {
  if (emulated_per_8 != 0 && emulated_per_8 != 2 && emulated_per_8 != 4) return ATTN_ERR_ARG;
  if (q == nullptr || o == nullptr) return ATTN_ERR_NULL;
  if (Sk > 0 && (k == nullptr || v == nullptr)) return ATTN_ERR_NULL;
  int st = check_dims(B, Hq, Hkv, Sq, Sk, d, true);
  if (st != ATTN_OK) return st;
  if (dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
  if (!isfinite(scale)) return ATTN_ERR_ARG;
  FwdArgs a = {};
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Sq = Sq; a.Sk = Sk; a.d = d;
  a.group = Hq / Hkv;
  a.causal = causal != 0;
  a.dtype_bf16 = dtype == ATTN_BF16;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.exp_emulated = emulated_per_8;
  return hip_status(attn_launch_fwd(a, (hipStream_t)stream));
}

int attn_exp2_soft(const float* x, float* y, long long n, void* stream) {
  if (n < 0 || n > (1LL << 31)) return ATTN_ERR_SHAPE;
  if (n > 0 && (x == nullptr || y == nullptr)) return ATTN_ERR_NULL;
  return hip_status(attn_launch_exp2_soft(x, y, (int64_t)n, (hipStream_t)stream));
}

// Dropout parameters from (p, seed, offset); p must be in [0, 1).
bool make_drop(float p, unsigned long long seed, unsigned offset, DropParams* dp) {
  if (!(p >= 0.f && p < 1.f)) return false;
  const double t = floor((double)p * 4294967296.0);
  dp->thresh = (uint32_t)(t > 4294967295.0 ? 4294967295.0 : t);
  dp->seed_lo = (uint32_t)(seed & 0xFFFFFFFFull);
  dp->seed_hi = (uint32_t)(seed >> 32);
  dp->offset = offset;
  dp->rp = 1.f / (1.f - p);
  return true;
}

int attn_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int Hq, int Hkv, int Sq, int Sk, int d, float scale, int causal,
                     float dropout_p, unsigned long long seed, unsigned offset,
                     attn_dtype_t dtype, void* stream) {
  if (q == nullptr || o == nullptr) return ATTN_ERR_NULL;
  if (Sk > 0 && (k == nullptr || v == nullptr)) return ATTN_ERR_NULL;
  int st = check_dims(B, Hq, Hkv, Sq, Sk, d, true);
  if (st != ATTN_OK) return st;
  if (dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
  if (!isfinite(scale)) return ATTN_ERR_ARG;
  FwdArgs a = {};
  if (!make_drop(dropout_p, seed, offset, &a.drop)) return ATTN_ERR_ARG;
  a.dropout = 1;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Sq = Sq; a.Sk = Sk; a.d = d;
  a.group = Hq / Hkv;
  a.causal = causal != 0;
  a.dtype_bf16 = dtype == ATTN_BF16;
  a.scale_log2 = scale * 1.4426950408889634f;
  return hip_status(attn_launch_fwd(a, (hipStream_t)stream));
}

int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int Hq, int Hkv,
                    int max_seqlen_q, int max_seqlen_k, int total_q, int total_k, int d,
                    float scale, int causal, attn_dtype_t dtype, void* stream) {
  if (cu_seqlens_q == nullptr || cu_seqlens_k == nullptr) return ATTN_ERR_NULL;
  if (total_q > 0 && (q == nullptr || o == nullptr)) return ATTN_ERR_NULL;
  if (total_k > 0 && (k == nullptr || v == nullptr)) return ATTN_ERR_NULL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || total_q < 0 ||
      total_k < 0)
    return ATTN_ERR_SHAPE;
  if (max_seqlen_q > kMaxSeq || max_seqlen_k > kMaxSeq || (int64_t)B * Hq > kMaxBH)
    return ATTN_ERR_SHAPE;
  if (Hq % Hkv != 0) return ATTN_ERR_GQA;
  if (d != 64 && d != 128) return ATTN_ERR_HEADDIM;
  if (dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
  if (!isfinite(scale)) return ATTN_ERR_ARG;
  // one sequence's rows (token stride H d), with a tile of tail rows past its end,
  // must span less than 2 GiB: the kernels form 32-bit signed row offsets
  if (((int64_t)max_seqlen_q + 256) * Hq * d * 2 >= ((int64_t)1 << 31) ||
      ((int64_t)max_seqlen_k + 256) * Hkv * d * 2 >= ((int64_t)1 << 31))
    return ATTN_ERR_SHAPE;
  if (total_q == 0 || max_seqlen_q == 0) return ATTN_OK;   // no query row: nothing to write
  FwdArgs a = {};
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Sq = max_seqlen_q; a.Sk = max_seqlen_k; a.d = d;
  a.group = Hq / Hkv;
  a.causal = causal != 0;
  a.dtype_bf16 = dtype == ATTN_BF16;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.total_q = total_q;
  a.total_k = total_k;
  return hip_status(attn_launch_fwd(a, (hipStream_t)stream));
}

int attn_fp8_kv_tile(void) { return attn_fp8_tile_keys(); }

int attn_fp8_quantize(const void* x, attn_dtype_t dtype, int B, int H, int S, int d,
                      const float* signs, int per_tensor, unsigned char* codes, float* descale,
                      void* stream) {
  if (x == nullptr || codes == nullptr || descale == nullptr) return ATTN_ERR_NULL;
  if (B <= 0 || H <= 0 || S <= 0 || S > kMaxSeq || (int64_t)B * H > 65535) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_HEADDIM;
  if (dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
  QuantArgs a = {};
  a.x = x; a.signs = signs; a.codes = codes; a.descale = descale;
  a.B = B; a.H = H; a.S = S; a.d = d;
  a.nblk = (S + 127) / 128;
  a.per_tensor = per_tensor != 0;
  a.dtype_bf16 = dtype == ATTN_BF16;
  return hip_status(attn_launch_fp8_quantize(a, (hipStream_t)stream));
}

int attn_fwd_fp8(const void* q8, const void* k8, const void* v8,
                 const float* q_scale, const float* k_scale, const float* v_scale,
                 void* o, float* lse, int B, int Hq, int Hkv, int Sq, int Sk, int d,
                 float scale, int causal, attn_dtype_t o_dtype, void* stream) {
  if (q8 == nullptr || k8 == nullptr || v8 == nullptr || q_scale == nullptr ||
      k_scale == nullptr || v_scale == nullptr || o == nullptr)
    return ATTN_ERR_NULL;
  int st = check_dims(B, Hq, Hkv, Sq, Sk, d, false);
  if (st != ATTN_OK) return st;
  if (o_dtype != ATTN_BF16 && o_dtype != ATTN_F32) return ATTN_ERR_DTYPE;
  if (!isfinite(scale)) return ATTN_ERR_ARG;
  Fp8Args a = {};
  a.q = (const uint8_t*)q8; a.k = (const uint8_t*)k8; a.v = (const uint8_t*)v8;
  a.q_scale = q_scale; a.k_scale = k_scale; a.v_scale = v_scale;
  a.o = o; a.lse = lse;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Sq = Sq; a.Sk = Sk; a.d = d;
  a.group = Hq / Hkv;
  a.causal = causal != 0;
  a.o_f32 = o_dtype == ATTN_F32;
  a.scale_log2 = scale * 1.4426950408889634f;
  return hip_status(attn_launch_fwd_fp8(a, (hipStream_t)stream));
}

size_t attn_bwd_workspace_size(int B, int Hq, int Hkv, int Sq, int Sk, int d) {
  if (check_dims(B, Hq, Hkv, Sq, Sk, d, false) != ATTN_OK) return 0;
  const size_t rows = (size_t)B * Hq * Sq;
  const size_t atomic = align256(rows * d * sizeof(float)) + align256(rows * sizeof(float));
  const size_t split = det_layout(B, Hq, Hkv, Sq, Sk, d, 1, nullptr, false, nullptr, nullptr);
  return atomic > split ? atomic : split;
}

}  // extern "C"

namespace {

// attn_bwd (split = true: the form by key length) and attn_bwd_atomic
int bwd_16bit(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO,
              void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq, int Sk, int d, float scale,
              int causal, attn_dtype_t dtype, attn_dtype_t grad_dtype, void* workspace, size_t workspace_bytes,
              void* stream, bool split) {
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || lse == nullptr ||
      dO == nullptr || dq == nullptr || dk == nullptr || dv == nullptr)
    return ATTN_ERR_NULL;
  int st = check_dims(B, Hq, Hkv, Sq, Sk, d, false);
  if (st != ATTN_OK) return st;
  if (dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
  if (grad_dtype != ATTN_F32 && grad_dtype != ATTN_BF16 && grad_dtype != ATTN_F16)
    return ATTN_ERR_DTYPE;
  if (!isfinite(scale)) return ATTN_ERR_ARG;
  if ((int64_t)B * Hkv > 65535) return ATTN_ERR_SHAPE;   // one grid row per (b, kv head)
  const size_t need = attn_bwd_workspace_size(B, Hq, Hkv, Sq, Sk, d);
  if (workspace == nullptr || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  const size_t rows = (size_t)B * Hq * Sq;
  BwdArgs a = {};
  BwdF16Ws cw = {};
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse; a.dO = dO;
  a.dq = dq; a.dk = dk; a.dv = dv;
  if (split && Sk >= kBwdSplitKeys) {
    det_layout(B, Hq, Hkv, Sq, Sk, d, 1, workspace, dtype == ATTN_BF16, &a, &cw);
    a.deterministic = 1;
    a.dq_splits = 1;
  } else {
    a.dq_acc = (float*)workspace;
    a.delta = (float*)((char*)workspace + align256(rows * d * sizeof(float)));
  }
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Sq = Sq; a.Sk = Sk; a.d = d;
  a.group = Hq / Hkv;
  a.causal = causal != 0;
  a.dtype_bf16 = dtype == ATTN_BF16;
  a.grad_type = (int)grad_dtype;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  return hip_status(attn_launch_bwd(a, &cw, (hipStream_t)stream));
}

}  // namespace

extern "C" {

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dO, void* dq, void* dk, void* dv,
             int B, int Hq, int Hkv, int Sq, int Sk, int d, float scale, int causal,
             attn_dtype_t dtype, attn_dtype_t grad_dtype,
             void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_16bit(q, k, v, o, lse, dO, dq, dk, dv, B, Hq, Hkv, Sq, Sk, d, scale, causal, dtype, grad_dtype,
                   workspace, workspace_bytes, stream, true);
}

int attn_bwd_atomic(const void* q, const void* k, const void* v, const void* o, const float* lse,
                    const void* dO, void* dq, void* dk, void* dv,
                    int B, int Hq, int Hkv, int Sq, int Sk, int d, float scale, int causal,
                    attn_dtype_t dtype, attn_dtype_t grad_dtype,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_16bit(q, k, v, o, lse, dO, dq, dk, dv, B, Hq, Hkv, Sq, Sk, d, scale, causal, dtype, grad_dtype,
                   workspace, workspace_bytes, stream, false);
}

int attn_bwd_fp8(const void* q8, const void* k8, const void* v8, const float* q_scale, const float* k_scale,
                 const float* v_scale, const void* o, const float* lse, const void* dO, void* dq, void* dk,
                 void* dv, int B, int Hq, int Hkv, int Sq, int Sk, int d, float scale, int causal,
                 attn_dtype_t grad_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (q8 == nullptr || k8 == nullptr || v8 == nullptr || q_scale == nullptr || k_scale == nullptr ||
      v_scale == nullptr || o == nullptr || lse == nullptr || dO == nullptr || dq == nullptr ||
      dk == nullptr || dv == nullptr)
    return ATTN_ERR_NULL;
  int st = check_dims(B, Hq, Hkv, Sq, Sk, d, false);
  if (st != ATTN_OK) return st;
  if (grad_dtype != ATTN_F32 && grad_dtype != ATTN_BF16 && grad_dtype != ATTN_F16) return ATTN_ERR_DTYPE;
  if (!isfinite(scale)) return ATTN_ERR_ARG;
  if ((int64_t)B * Hkv > 65535) return ATTN_ERR_SHAPE;   // one grid row per (b, kv head)
  const size_t need = attn_bwd_workspace_size(B, Hq, Hkv, Sq, Sk, d);
  if (workspace == nullptr || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  const size_t rows = (size_t)B * Hq * Sq;
  BwdArgs a = {};
  BwdF16Ws cw = {};
  a.q = q8; a.k = k8; a.v = v8; a.o = o; a.lse = lse; a.dO = dO;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.dq_acc = (float*)workspace;
  a.delta = (float*)((char*)workspace + align256(rows * d * sizeof(float)));
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Sq = Sq; a.Sk = Sk; a.d = d;
  a.group = Hq / Hkv;
  a.causal = causal != 0;
  a.dtype_bf16 = 1;            // o and dO are bf16
  a.grad_type = (int)grad_dtype;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.fp8 = 1;
  a.q_scale = q_scale; a.k_scale = k_scale; a.v_scale = v_scale;
  return hip_status(attn_launch_bwd(a, &cw, (hipStream_t)stream));
}

size_t attn_bwd_deterministic_workspace_size(int B, int Hq, int Hkv, int Sq, int Sk, int d,
                                             int dq_splits) {
  if (check_dims(B, Hq, Hkv, Sq, Sk, d, false) != ATTN_OK) return 0;
  if (dq_splits < 1 || dq_splits > 16 || (dq_splits & (dq_splits - 1)) != 0) return 0;
  return det_layout(B, Hq, Hkv, Sq, Sk, d, dq_splits, nullptr, false, nullptr, nullptr);
}

int attn_bwd_deterministic(const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dO, void* dq, void* dk, void* dv,
                           int B, int Hq, int Hkv, int Sq, int Sk, int d, float scale, int causal,
                           attn_dtype_t dtype, attn_dtype_t grad_dtype, int dq_splits,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || lse == nullptr ||
      dO == nullptr || dq == nullptr || dk == nullptr || dv == nullptr)
    return ATTN_ERR_NULL;
  int st = check_dims(B, Hq, Hkv, Sq, Sk, d, false);
  if (st != ATTN_OK) return st;
  if (dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
  if (grad_dtype != ATTN_F32 && grad_dtype != ATTN_BF16 && grad_dtype != ATTN_F16)
    return ATTN_ERR_DTYPE;
  if (!isfinite(scale)) return ATTN_ERR_ARG;
  if (dq_splits < 1 || dq_splits > 16 || (dq_splits & (dq_splits - 1)) != 0) return ATTN_ERR_ARG;
  if ((int64_t)B * Hkv > 65535) return ATTN_ERR_SHAPE;
  const size_t need = attn_bwd_deterministic_workspace_size(B, Hq, Hkv, Sq, Sk, d, dq_splits);
  if (workspace == nullptr || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  BwdArgs a = {};
  BwdF16Ws cw = {};
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse; a.dO = dO;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.dq_acc = nullptr;
  det_layout(B, Hq, Hkv, Sq, Sk, d, dq_splits, workspace, dtype == ATTN_BF16, &a, &cw);
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Sq = Sq; a.Sk = Sk; a.d = d;
  a.group = Hq / Hkv;
  a.causal = causal != 0;
  a.dtype_bf16 = dtype == ATTN_BF16;
  a.grad_type = (int)grad_dtype;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.deterministic = 1;
  a.dq_splits = dq_splits;
  return hip_status(attn_launch_bwd(a, &cw, (hipStream_t)stream));
}

int attn_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     const void* dO, void* dq, void* dk, void* dv,
                     int B, int Hq, int Hkv, int Sq, int Sk, int d, float scale, int causal,
                     float dropout_p, unsigned long long seed, unsigned offset,
                     attn_dtype_t dtype, attn_dtype_t grad_dtype, int deterministic, int dq_splits,
                     void* workspace, size_t workspace_bytes, void* stream) {
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || lse == nullptr ||
      dO == nullptr || dq == nullptr || dk == nullptr || dv == nullptr)
    return ATTN_ERR_NULL;
  int st = check_dims(B, Hq, Hkv, Sq, Sk, d, false);
  if (st != ATTN_OK) return st;
  if (dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
  if (grad_dtype != ATTN_F32 && grad_dtype != ATTN_BF16 && grad_dtype != ATTN_F16)
    return ATTN_ERR_DTYPE;
  if (!isfinite(scale)) return ATTN_ERR_ARG;
  if ((int64_t)B * Hkv > 65535) return ATTN_ERR_SHAPE;
  BwdArgs a = {};
  BwdF16Ws cw = {};
  if (!make_drop(dropout_p, seed, offset, &a.drop)) return ATTN_ERR_ARG;
  a.dropout = 1;
  const size_t rows = (size_t)B * Hq * Sq;
  if (deterministic) {
    if (dq_splits < 1 || dq_splits > 16 || (dq_splits & (dq_splits - 1)) != 0) return ATTN_ERR_ARG;
    const size_t need = attn_bwd_deterministic_workspace_size(B, Hq, Hkv, Sq, Sk, d, dq_splits);
    if (workspace == nullptr || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
    a.dq_acc = nullptr;
    det_layout(B, Hq, Hkv, Sq, Sk, d, dq_splits, workspace, dtype == ATTN_BF16, &a, &cw);
    a.deterministic = 1;
    a.dq_splits = dq_splits;
  } else {
    // attn_bwd's form: atomic dQ below kBwdSplitKeys keys, the query-row owner from there
    const size_t need = attn_bwd_workspace_size(B, Hq, Hkv, Sq, Sk, d);
    if (workspace == nullptr || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
    if (Sk >= kBwdSplitKeys) {
      det_layout(B, Hq, Hkv, Sq, Sk, d, 1, workspace, dtype == ATTN_BF16, &a, &cw);
      a.deterministic = 1;
      a.dq_splits = 1;
    } else {
      a.dq_acc = (float*)workspace;
      a.delta = (float*)((char*)workspace + align256(rows * d * sizeof(float)));
    }
  }
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse; a.dO = dO;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Sq = Sq; a.Sk = Sk; a.d = d;
  a.group = Hq / Hkv;
  a.causal = causal != 0;
  a.dtype_bf16 = dtype == ATTN_BF16;
  a.grad_type = (int)grad_dtype;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  return hip_status(attn_launch_bwd(a, &cw, (hipStream_t)stream));
}

int attn_decode_pick_chunk(int B, int Hq, int Smax) {
  if (B <= 0 || Hq <= 0 || Smax <= 0) return 256;
  // Larger chunks write fewer partial states and launch fewer workgroups; keep at least
  // 16384 (query head, chunk) pairs at full length so that the grid still fills the
  // chip.  Multiples of 768 keys: chunks of 1024, 2048 and 4096 keys (power-of-two
  // strides between the concurrently read chunks of a head) measured 15-40 % slower.
  for (int c : {1536, 768}) {
    if ((int64_t)B * Hq * decode_chunks(Smax, c) >= 16384) return c;
  }
  return 256;
}

size_t attn_decode_workspace_size(int B, int Hq, int Smax, int d, int chunk) {
  if (B <= 0 || Hq <= 0 || Smax <= 0 || Smax > kMaxSeq || (int64_t)B * Hq > kMaxBH) return 0;
  if ((d != 64 && d != 128) || chunk <= 0 || chunk % 64 != 0) return 0;
  const size_t parts = (size_t)B * Hq * decode_chunks(Smax, chunk);
  return align256(parts * 2 * sizeof(float)) + align256(parts * d * sizeof(float));
}

}  // extern "C"

namespace {

// Argument checks of the contiguous-cache decode (pure host arithmetic).
int check_decode(const void* q, const void* k_cache, const void* v_cache, const int* seqlens_k, void* o,
                 int B, int Hq, int Hkv, int Smax, int d, float scale, int chunk, attn_dtype_t dtype) {
  if (q == nullptr || k_cache == nullptr || v_cache == nullptr || seqlens_k == nullptr ||
      o == nullptr)
    return ATTN_ERR_NULL;
  int st = check_dims(B, Hq, Hkv, 1, Smax, d, false);
  if (st != ATTN_OK) return st;
  if (dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
  if (chunk <= 0 || chunk % 64 != 0 || chunk > 4096 || !isfinite(scale)) return ATTN_ERR_ARG;
  if ((int64_t)B * Hkv > 65535) return ATTN_ERR_SHAPE;   // one grid row per (b, kv head)
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_decode_splitkv(const void* q, const void* k_cache, const void* v_cache,
                        const int* seqlens_k, void* o, float* lse,
                        int B, int Hq, int Hkv, int Smax, int d, float scale, int chunk,
                        attn_dtype_t dtype, void* workspace, size_t workspace_bytes,
                        void* stream) {
  const int st = check_decode(q, k_cache, v_cache, seqlens_k, o, B, Hq, Hkv, Smax, d, scale, chunk, dtype);
  if (st != ATTN_OK) return st;
  const size_t need = attn_decode_workspace_size(B, Hq, Smax, d, chunk);
  if (workspace == nullptr || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  DecodeArgs a = {};
  a.q = q; a.k = k_cache; a.v = v_cache; a.seqlens = seqlens_k; a.o = o; a.lse = lse;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Smax = Smax; a.d = d; a.chunk = chunk;
  a.nchunk = decode_chunks(Smax, chunk);
  const size_t parts = (size_t)B * Hq * a.nchunk;
  a.part_ml = (float*)workspace;
  a.part_u = (float*)((char*)workspace + align256(parts * 2 * sizeof(float)));
  a.group = Hq / Hkv;
  a.dtype_bf16 = dtype == ATTN_BF16;
  a.scale_log2 = scale * 1.4426950408889634f;
  return hip_status(attn_launch_decode(a, (hipStream_t)stream));
}

int attn_decode_splitkv_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                const int* seqlens_k, void* o, float* lse,
                                int B, int Hq, int Hkv, int Smax, int d, float scale, int chunk,
                                attn_dtype_t dtype, void* stream) {
  const int st = check_decode(q, k_cache, v_cache, seqlens_k, o, B, Hq, Hkv, Smax, d, scale, chunk, dtype);
  if (st != ATTN_OK) return st;
  const size_t need = attn_decode_workspace_size(B, Hq, Smax, d, chunk);
  if (need == 0 || need > (size_t)ATTN_DECODE_NOALLOC_SCRATCH_BYTES) return ATTN_ERR_WORKSPACE;
  void* ws = nullptr;
  if (attn_decode_scratch(&ws) != hipSuccess) return ATTN_ERR_HIP;
  // the split pass writes every partial the merge reads: nothing needs clearing
  return attn_decode_splitkv(q, k_cache, v_cache, seqlens_k, o, lse, B, Hq, Hkv, Smax, d, scale, chunk, dtype,
                             ws, need, stream);
}

int attn_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                      const int* block_table, const int* seqlens_k, void* o, float* lse,
                      int B, int Hq, int Hkv, int num_pages, int page_size, int max_pages, int d,
                      float scale, int chunk, attn_dtype_t dtype, void* workspace,
                      size_t workspace_bytes, void* stream) {
  if (q == nullptr || k_pages == nullptr || v_pages == nullptr || block_table == nullptr ||
      seqlens_k == nullptr || o == nullptr)
    return ATTN_ERR_NULL;
  if (page_size < 64 || page_size > 4096 || (page_size & (page_size - 1)) != 0) return ATTN_ERR_ARG;
  if (num_pages <= 0 || max_pages <= 0 || (int64_t)max_pages * page_size > kMaxSeq) return ATTN_ERR_SHAPE;
  const int Smax = max_pages * page_size;
  int st = check_dims(B, Hq, Hkv, 1, Smax, d, false);
  if (st != ATTN_OK) return st;
  if (dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
  if (chunk <= 0 || chunk % 64 != 0 || chunk > 4096 || !isfinite(scale)) return ATTN_ERR_ARG;
  if ((int64_t)B * Hkv > 65535) return ATTN_ERR_SHAPE;
  const size_t need = attn_decode_workspace_size(B, Hq, Smax, d, chunk);
  if (workspace == nullptr || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  DecodeArgs a = {};
  a.q = q; a.k = k_pages; a.v = v_pages; a.seqlens = seqlens_k; a.o = o; a.lse = lse;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Smax = Smax; a.d = d; a.chunk = chunk;
  a.nchunk = decode_chunks(Smax, chunk);
  const size_t parts = (size_t)B * Hq * a.nchunk;
  a.part_ml = (float*)workspace;
  a.part_u = (float*)((char*)workspace + align256(parts * 2 * sizeof(float)));
  a.group = Hq / Hkv;
  a.dtype_bf16 = dtype == ATTN_BF16;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.block_table = block_table;
  a.max_pages = max_pages;
  a.num_pages = num_pages;
  int sh = 0;
  while ((1 << sh) < page_size) ++sh;
  a.page_shift = sh;
  return hip_status(attn_launch_decode(a, (hipStream_t)stream));
}

}  // extern "C"

/*
 * attn.h -- C ABI of libattn, exact tiled attention for AMD Instinct MI355X (gfx950).
 *
 * Operation (all entry points): exact dense attention
 *     O = softmax(scale * Q K^T + mask) V,   LSE = log-sum-exp of each masked score row
 * computed tile by tile without materialising the [S_q, S_k] score or probability
 * matrices ("M4.3 - IO-Aware Attention and FlashAttention-1", sections 0x08-0x09;
 * "M4.4 - FlashAttention-2 Work Partitioning and the Decode Boundary", sections
 * 0x02-0x03).
 *
 * Conventions shared by every call
 *   - Tensors are contiguous row-major [B, H, S, d] ("BHSD") in device memory owned
 *     by the caller.  The library never allocates or frees device memory: scratch is
 *     passed in as a workspace whose size the matching *_workspace_size() returns
 *     (attn_decode_splitkv_noalloc uses a fixed library-owned device array instead).
 *   - Query head h reads K/V head h / (H_q / H_kv); H_q must be a multiple of H_kv
 *     (M4.4, section 0x06A).  Output and LSE are indexed by query head.
 *   - causal != 0 makes cell (i, k) visible iff k <= i + (S_k - S_q), the bottom-right
 *     alignment (M4.4, section 0x05.1F).  A query row with no visible key (only
 *     possible when S_q > S_k) gets O = 0 and LSE = -inf and adds no gradient.
 *   - LSE is natural-log, float32, [B, H_q, S_q].
 *   - Supported head dimension d: 64 and 128.  Supported element types: ATTN_F16 and
 *     ATTN_BF16 (ATTN_FP8_E4M3 only through attn_fwd_fp8).
 *   - Every call checks its arguments on the host before any HIP call and returns a
 *     negative status without touching the GPU when they are invalid.  Valid calls
 *     are asynchronous on `stream` (a hipStream_t; NULL = the default stream); the
 *     results are ready after the stream is synchronised.  A failed launch returns
 *     ATTN_ERR_HIP.  The library keeps no state between calls (except the per-GPU
 *     scratch of attn_decode_splitkv_noalloc).
 *   - Sizes are int (each dimension and each product used for indexing must fit the
 *     64-bit offsets the kernels use; S_q, S_k <= 2^20, B*H <= 2^16 are enforced).
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_F16 = 0,
  ATTN_BF16 = 1,
  ATTN_F32 = 2,
  ATTN_FP8_E4M3 = 3
} attn_dtype_t;

enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = -1,      /* a required pointer is NULL                              */
  ATTN_ERR_SHAPE = -2,     /* a size is <= 0 (or S_k < 0), or exceeds the limits above */
  ATTN_ERR_GQA = -3,       /* H_q is not a multiple of H_kv                            */
  ATTN_ERR_HEADDIM = -4,   /* d is not 64 or 128                                       */
  ATTN_ERR_DTYPE = -5,     /* unsupported element / output / gradient type            */
  ATTN_ERR_WORKSPACE = -6, /* workspace missing or smaller than *_workspace_size()     */
  ATTN_ERR_HIP = -7,       /* a HIP launch or runtime call failed                      */
  ATTN_ERR_ARG = -8        /* another argument is out of its range (chunk, scale)      */
};

/* Human-readable text for a status code (static storage, never NULL). */
const char* attn_status_string(int status);

/*
 * attn_fwd -- tiled forward with saved log-sum-exp.
 * "M4.4 - FlashAttention-2 Work Partitioning and the Decode Boundary", section 0x03
 * (Algorithm 1: one owner per query tile streams K/V tiles, carries (m, l, u) on chip,
 * normalises once and commits O and LSE once) and section 0x02D (O = u / l,
 * LSE = m + log l).
 *
 *   q   [B, Hq,  Sq, d]  element type `dtype`          (in)
 *   k,v [B, Hkv, Sk, d]  element type `dtype`          (in)
 *   o   [B, Hq,  Sq, d]  element type `dtype`          (out)
 *   lse [B, Hq,  Sq]     float32, natural log          (out; may be NULL to skip)
 *   scale: the score multiplier (1/sqrt(d) is the usual value); must be finite.
 *   Sk = 0 is allowed: every row is empty (O = 0, LSE = -inf).
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int Hq, int Hkv, int Sq, int Sk, int d, float scale, int causal,
             attn_dtype_t dtype, void* stream);

/*
 * attn_fwd_exp_emulated -- attn_fwd with part of the softmax exponentials computed in
 * software on the FMA pipe instead of the hardware exponential ("M4.6 - FlashAttention-
 * 3/4 Hardware Pipelines ...", section 0x09: exp-throughput relief).  The software
 * exp2 reduces x = n + f (n = floor(x), f in [0, 1)), evaluates a degree-3 polynomial
 * for 2^f whose coefficients minimise the maximum relative error on [0, 1] (7.5e-5;
 * fitted for this library by the Remez exchange) and scales by 2^n; see attn_exp2_soft.
 * The result differs from attn_fwd by that error on the emulated probabilities.
 *
 *   Arguments as attn_fwd, plus emulated_per_8: 0, 2 or 4 of every 8 exponentials of a
 *   key chunk are emulated (else ATTN_ERR_ARG); 0 is attn_fwd exactly.
 */
int attn_fwd_exp_emulated(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int Hq, int Hkv, int Sq, int Sk, int d, float scale, int causal,
                          attn_dtype_t dtype, int emulated_per_8, void* stream);

/*
 * attn_exp2_soft -- the software exp2 of attn_fwd_exp_emulated, element by element:
 * y[i] = soft_exp2(x[i]) in float32 (fused multiply-adds in Horner order; arguments
 * at or below -150, -inf included, give 0; results below 2^-126 may be flushed to 0).  x, y: device float32 [n], 0 <= n <= 2^31 (else
 * ATTN_ERR_SHAPE); asynchronous on `stream`.
 */
int attn_exp2_soft(const float* x, float* y, long long n, void* stream);

/*
 * attn_fwd_dropout -- attn_fwd with attention dropout on the probabilities.
 * "M4.4 - FlashAttention-2 ...", section 0x03I and "M4.3 - IO-Aware Attention ...",
 * section 0x0DF: the maximum, the denominator and the LSE stay those of the undropped
 * softmax; each probability element is kept or dropped before P V and the kept ones
 * are scaled by 1 / (1 - dropout_p); the decisions are a pure function of the
 * element's coordinates so attn_bwd_dropout regenerates them.  Element (b, h, query
 * row i, key j) takes word j % 4 of Philox4x32-10 (counter (j / 4, i, b Hq + h,
 * offset), key (seed mod 2^32, seed / 2^32)) and is kept iff the word is at least
 * floor(dropout_p 2^32).
 *
 *   Arguments as attn_fwd, plus dropout_p in [0, 1) (else ATTN_ERR_ARG), the 64-bit
 *   seed and a 32-bit offset (e.g. a step counter: a new offset draws new decisions).
 */
int attn_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int Hq, int Hkv, int Sq, int Sk, int d, float scale, int causal,
                     float dropout_p, unsigned long long seed, unsigned offset,
                     attn_dtype_t dtype, void* stream);

/*
 * attn_fwd_varlen -- the forward of attn_fwd on packed variable-length sequences.
 * "M4.4 - FlashAttention-2 Work Partitioning and the Decode Boundary", sections 0x04B
 * (a packed launch covers the longest sequence; workgroups past a sequence's rows
 * return at entry) and 0x06F (each packed sequence has its own query and key extents,
 * causal alignment and tile classes; heads map as in attn_fwd).
 *
 *   q   [total_q, Hq,  d]  token-major, element type `dtype`                 (in)
 *   k,v [total_k, Hkv, d]  token-major, element type `dtype`                 (in)
 *   o   [total_q, Hq,  d]  element type `dtype`                              (out)
 *   lse [Hq, total_q]      float32, natural log                    (out; may be NULL)
 *   cu_seqlens_q, cu_seqlens_k: device int32 [B+1], nondecreasing, starting at 0;
 *       sequence b owns query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and keys
 *       cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1                                (in)
 *   max_seqlen_q / max_seqlen_k: upper bounds of the per-sequence lengths (they size
 *       the launch); total_q / total_k: rows of q and k.  Lengths beyond the bounds
 *       or offsets beyond the totals are clamped: inconsistent metadata may give wrong
 *       rows, never an access outside the tensors.
 *   causal: bottom-right alignment per sequence (delta = S_k,b - S_q,b).
 *   A sequence with no keys gives O = 0, LSE = -inf on its rows.  One sequence's rows
 *   must span less than 2 GiB ((max_seqlen + 256) * H * d * 2 bytes: 32-bit signed row
 *   offsets, including a tile of rows past the end), else ATTN_ERR_SHAPE.
 */
int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int Hq, int Hkv,
                    int max_seqlen_q, int max_seqlen_k, int total_q, int total_k, int d,
                    float scale, int causal, attn_dtype_t dtype, void* stream);

/*
 * attn_fp8_quantize -- E4M3 codes and descales for attn_fwd_fp8, with optional
 * incoherent processing.  "M4.6 - FlashAttention-3/4 Hardware Pipelines ...", section
 * 0x06: scales per 128-row block of one (batch, head), or one per tensor (the
 * granularity ablation); for Q and K the optional right transform R = diag(signs) H /
 * sqrt(d) with the Sylvester Hadamard H (orthogonal: (Q R)(K R)^T = Q K^T before
 * quantisation; give Q and K the same signs and do not transform V).
 *
 *   x [B, H, S, d] element type `dtype` (ATTN_F16 / ATTN_BF16), d = 64 or 128   (in)
 *   signs: device float32 [d] of +-1, or NULL for no transform                   (in)
 *   per_tensor: 0: descale = amax(block) / 448 per (b, h, 128-row block) (1 for an
 *       all-zero block); 1: one descale from the amax of the whole tensor, written to
 *       every entry
 *   codes [B, H, S, d] E4M3FN bytes = round-to-nearest-even of (x R) / descale,
 *       clamped to +-448                                                          (out)
 *   descale [B, H, ceil(S / 128)] float32                                         (out)
 */
int attn_fp8_quantize(const void* x, attn_dtype_t dtype, int B, int H, int S, int d,
                      const float* signs, int per_tensor, unsigned char* codes, float* descale,
                      void* stream);

/*
 * attn_fwd_fp8 -- forward on E4M3FN operands with per-block descales.
 * "M4.6 - FlashAttention-3/4 Hardware Pipelines", section 0x06 ("Derive Where Every
 * Scale Must Enter"; "Why The Source Raises Softmax Probabilities By 2^8"):
 *   S = scale * dQ_i * dK_j * (Q8 K8_j^T) before the row max;  u = 2^8 exp(S - m);
 *   P8 = E4M3(u) (round to nearest even) feeds the P V product;  l sums unrounded u;
 *   o += dV_j * (P8 V8_j) per K/V tile;  O = o / l;  LSE = m + ln l - 8 ln 2.
 *
 *   q8 [B,Hq,Sq,d], k8/v8 [B,Hkv,Sk,d]: E4M3FN bytes (OCP encoding, max 448)   (in)
 *   q_scale [B,Hq,ceil(Sq/128)], k_scale/v_scale [B,Hkv,ceil(Sk/128)]: float32
 *       descales, one per 128-row block of the row axis                        (in)
 *   o   [B,Hq,Sq,d]: o_dtype ATTN_BF16 or ATTN_F32                             (out)
 *   lse [B,Hq,Sq] float32 (may be NULL)                                        (out)
 *   d = 64 or 128; causal as attn_fwd (bottom-right; masked cells get u = 0).  K/V
 *   tiles of attn_fp8_kv_tile() keys are visited in ascending order, which fixes the
 *   frame in which each probability is rounded.  A zero descale (an all-zero block)
 *   or a zero scale is valid: a zero value descale makes its tile add nothing.
 */
int attn_fwd_fp8(const void* q8, const void* k8, const void* v8,
                 const float* q_scale, const float* k_scale, const float* v_scale,
                 void* o, float* lse, int B, int Hq, int Hkv, int Sq, int Sk, int d,
                 float scale, int causal, attn_dtype_t o_dtype, void* stream);

/* K/V tile width (keys) of the fp8 forward's streaming loop. */
int attn_fp8_kv_tile(void);

/*
 * attn_bwd -- backward of attn_fwd from its saved O and LSE.
 * "M4.4 - FlashAttention-2 ...", section 0x06.1 (Algorithm 2): D = rowsum(dO * O);
 * each workgroup owns one K/V column tile of one K/V head, recomputes
 * P = exp(scale Q K^T - LSE) tile by tile for every query head of the group,
 * forms dS = P * (dP - D), keeps dK/dV in registers (the group sum over the query
 * heads sharing the K/V head is done in the owner, section 0x06E).  dQ has two forms
 * (section 0x06.1F and the ownership table of section 0x06.1G), chosen by key length:
 *   Sk < 1024: the column owner adds its dQ contributions to a float32 accumulator
 *       with atomics and a last pass scales and converts dQ (attn_bwd_atomic);
 *   Sk >= 1024: a query-row owner recomputes P and dS and writes dQ directly, exactly
 *       as attn_bwd_deterministic with dq_splits = 1 (each 128-key column tile's
 *       atomic adds are one float32 pass over the dQ accumulator, performed past the
 *       L2; from about 1024 keys on they cost more than the recomputation).
 *
 *   q,o,dO [B,Hq,Sq,d] and k,v [B,Hkv,Sk,d]: element type `dtype`              (in)
 *   lse [B,Hq,Sq] float32 as written by attn_fwd                              (in)
 *   dq [B,Hq,Sq,d], dk/dv [B,Hkv,Sk,d]: element type `grad_dtype`
 *       (ATTN_F32, ATTN_BF16 or ATTN_F16)                                      (out)
 *   workspace: >= attn_bwd_workspace_size(...) bytes of device memory, any
 *       content on entry (enough for either form: the float32 dQ accumulator and D
 *       rows, or the deterministic form's D rows and fp16 copies)            (scratch)
 *   Requires Sk >= 1.  Results of the atomic form are not bitwise repeatable.
 */
size_t attn_bwd_workspace_size(int B, int Hq, int Hkv, int Sq, int Sk, int d);
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dO, void* dq, void* dk, void* dv,
             int B, int Hq, int Hkv, int Sq, int Sk, int d, float scale, int causal,
             attn_dtype_t dtype, attn_dtype_t grad_dtype,
             void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_bwd_atomic -- attn_bwd with the column owner's atomic dQ at every key length
 * ("M4.4 - FlashAttention-2 ...", section 0x06.1, Algorithm 2 and section 0x06.1F).
 * Arguments and workspace as attn_bwd.
 */
int attn_bwd_atomic(const void* q, const void* k, const void* v, const void* o, const float* lse,
                    const void* dO, void* dq, void* dk, void* dv,
                    int B, int Hq, int Hkv, int Sq, int Sk, int d, float scale, int causal,
                    attn_dtype_t dtype, attn_dtype_t grad_dtype,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_bwd_fp8 -- backward of attention on E4M3 operands with per-block descales: the
 * gradients with respect to the dequantised operands Q_d = dQ Q8, K_d = dK K8,
 * V_d = dV V8 (one float32 descale per 128-row block, as attn_fwd_fp8 takes them) of
 * O = softmax(scale Q_d K_d^T + mask) V_d, by the FA2 split of attn_bwd ("M4.4 -
 * FlashAttention-2 ...", section 0x06.1, Algorithm 2): P = exp(scale Q_d K_d^T - LSE)
 * recomputed from the caller's LSE, D = rowsum(dO * O) from the caller's O, dV = P^T dO,
 * dP = dO V_d^T, dS = P (dP - D), dQ = scale dS K_d, dK = scale dS^T Q_d.  The pages
 * leave FP8 training to future work ("M4.6 - FlashAttention-3/4 Hardware Pipelines",
 * section 0x06, after its accuracy table), so no quantisation enters the backward: the
 * E4M3 values are widened exactly to bf16 for the matrix products (float32
 * accumulation), the descales enter per tile in float32, and the probabilities and dS
 * enter dV, dK and dQ as hi + lo bf16 pairs as in attn_bwd.  With O and LSE of the exact
 * forward on the dequantised operands these are the exact gradients; with the outputs of
 * attn_fwd_fp8 (whose probabilities are rounded to E4M3) its quantisation error reaches
 * the gradients through D.
 *
 *   q8 [B,Hq,Sq,d], k8/v8 [B,Hkv,Sk,d]: E4M3FN bytes; *_scale as attn_fwd_fp8      (in)
 *   o, dO [B,Hq,Sq,d] bf16; lse [B,Hq,Sq] float32 (natural log)                   (in)
 *   dq [B,Hq,Sq,d], dk/dv [B,Hkv,Sk,d]: grad_dtype (ATTN_F32, ATTN_BF16, ATTN_F16) (out)
 *   workspace: >= attn_bwd_workspace_size(...) bytes (float32 dQ accumulator + D)
 *   d = 64 or 128; causal as attn_fwd; dQ is accumulated with atomics as in attn_bwd.
 */
int attn_bwd_fp8(const void* q8, const void* k8, const void* v8, const float* q_scale, const float* k_scale,
                 const float* v_scale, const void* o, const float* lse, const void* dO, void* dq, void* dk,
                 void* dv, int B, int Hq, int Hkv, int Sq, int Sk, int d, float scale, int causal,
                 attn_dtype_t grad_dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_bwd_deterministic -- attn_bwd with bitwise-repeatable results (no atomics).
 * "M4.4 - FlashAttention-2 ...", section 0x06.1F (atomic dQ accumulation has no fixed
 * order; the alternative materialises one partial per producer and reduces the
 * partials in a fixed tree) and section 0x06.1G with its ownership table (a query-row
 * owner makes dQ_i a direct output).  dK and dV come from the column owner as in
 * attn_bwd (register sums in a fixed order, one write each).  dQ comes from a
 * query-row owner that recomputes P and dS and walks the key tiles in ascending order:
 * with dq_splits = 1 it writes dQ directly; with dq_splits = 2, 4, 8 or 16 the key
 * tiles are cut into that many contiguous ranges, each writes a float32 partial, and
 * the partials are summed in a fixed binary tree.  The recomputation costs two more
 * matrix products per tile than attn_bwd's atomic dQ.
 * bf16 operands: q, k, v and dO are first copied into the workspace as fp16 values
 * scaled by one power of two per tensor, chosen from the tensor's largest magnitude (and
 * o's, for v) so that it lands in [4, 8); a bf16 value scaled so is an fp16 value unless
 * it falls below fp16's normal range (2^-14 after scaling), so the copies are exact
 * there.  Both owners then run on the copies with fp16 products: P and dS enter dV, dK
 * and dQ as single fp16 operands (relative rounding 2^-12) where attn_bwd uses bf16 hi +
 * lo pairs, and the scales are undone in float32 at the end.  The exponents are clamped
 * to [-60, 60].
 *
 *   Arguments as attn_bwd, plus dq_splits (1, 2, 4, 8 or 16; else ATTN_ERR_ARG).
 *   workspace: >= attn_bwd_deterministic_workspace_size(..., dq_splits) bytes
 *       (D rows, the dq_splits partials when dq_splits > 1, the fp16 copies of q, dO,
 *       k, v and their exponents; the size does not depend on the dtype)    (scratch)
 */
size_t attn_bwd_deterministic_workspace_size(int B, int Hq, int Hkv, int Sq, int Sk, int d,
                                             int dq_splits);
int attn_bwd_deterministic(const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dO, void* dq, void* dk, void* dv,
                           int B, int Hq, int Hkv, int Sq, int Sk, int d, float scale, int causal,
                           attn_dtype_t dtype, attn_dtype_t grad_dtype, int dq_splits,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_bwd_dropout -- backward of attn_fwd_dropout (same dropout_p, seed and offset).
 * "M4.4 - FlashAttention-2 ...", section 0x03I (the backward regenerates the forward's
 * decisions; D = rowsum(dO * O) with the dropped O) and "M4.3 - IO-Aware Attention ...",
 * section 0x0DF (coordinate-stable replay).  With Z = keep / (1 - p) per element:
 * dV = (P Z)^T dO, dS = P (Z dP - D), dQ = scale dS K, dK = scale dS^T Q.
 *
 *   Arguments as attn_bwd, plus dropout_p, seed, offset as given to attn_fwd_dropout,
 *   deterministic (0: dQ in attn_bwd's form for the key length, workspace
 *   attn_bwd_workspace_size; 1: as attn_bwd_deterministic with dq_splits, workspace
 *   attn_bwd_deterministic_workspace_size).
 */
int attn_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     const void* dO, void* dq, void* dk, void* dv,
                     int B, int Hq, int Hkv, int Sq, int Sk, int d, float scale, int causal,
                     float dropout_p, unsigned long long seed, unsigned offset,
                     attn_dtype_t dtype, attn_dtype_t grad_dtype, int deterministic, int dq_splits,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_decode_splitkv -- one new query per sequence against a K/V cache.
 * "M4.4 - FlashAttention-2 ...", section 0x01 (Flash-Decoding splits the K/V axis
 * into chunks, then reduces over chunks) and "M4.3 - IO-Aware Attention ...",
 * sections 0x08B-0x08F (partial (m, l, u) states merge exactly in any order).
 * Pass 1: one workgroup per (chunk, b, kv head) reads its K/V chunk once for all
 * H_q/H_kv query heads of the group and writes one partial (m, l, u) per query head.
 * Pass 2: per (b, query head) the partials are merged in one max frame, O = u / l,
 * LSE = m + ln l.
 *
 *   q [B,Hq,1,d]; k_cache, v_cache [B,Hkv,Smax,d]: element type `dtype`        (in)
 *   seqlens_k: device int32[B], 0 <= seqlens_k[b] <= Smax; sequence b attends to
 *       keys [0, seqlens_k[b]) (a length of 0 gives O = 0, LSE = -inf)          (in)
 *   o [B,Hq,1,d] element type `dtype`; lse [B,Hq,1] float32 (may be NULL)      (out)
 *   chunk: keys per split, a positive multiple of 64, at most 4096;
 *       attn_decode_pick_chunk gives the library's choice for a shape.
 *   workspace: >= attn_decode_workspace_size(B, Hq, Smax, d, chunk) bytes     (scratch)
 */
size_t attn_decode_workspace_size(int B, int Hq, int Smax, int d, int chunk);
/* attn_decode_pick_chunk -- the split size this library uses by default for B
 * sequences of up to Smax keys and Hq query heads: the largest of 1536, 768 keys that
 * still gives at least 16384 (query head, chunk) pairs at full length, else 256.  Pure
 * host arithmetic; never fails (256 for non-positive arguments). */
int attn_decode_pick_chunk(int B, int Hq, int Smax);
int attn_decode_splitkv(const void* q, const void* k_cache, const void* v_cache,
                        const int* seqlens_k, void* o, float* lse,
                        int B, int Hq, int Hkv, int Smax, int d, float scale, int chunk,
                        attn_dtype_t dtype, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * attn_decode_splitkv_noalloc -- attn_decode_splitkv without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  The partial states go to a
 * library-owned device array of ATTN_DECODE_NOALLOC_SCRATCH_BYTES per GPU (created
 * when the library's code object is loaded on that GPU, kept until the process
 * ends); the call itself allocates and frees nothing.  Its device address is looked
 * up once per GPU on the first call there.
 *
 *   Arguments as attn_decode_splitkv without workspace / workspace_bytes.
 *   ATTN_ERR_WORKSPACE when attn_decode_workspace_size(B, Hq, Smax, d, chunk) exceeds
 *   ATTN_DECODE_NOALLOC_SCRATCH_BYTES (a larger chunk needs fewer partials).
 *   Every call on one GPU shares that GPU's array: calls that overlap on one GPU
 *   (several streams or host threads at once) race and must be serialised by the
 *   caller.  The array keeps the last call's partials; nothing in it needs to start
 *   at zero, since the split pass writes every partial the merge pass reads.
 */
#define ATTN_DECODE_NOALLOC_SCRATCH_BYTES (64u << 20)
int attn_decode_splitkv_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                const int* seqlens_k, void* o, float* lse,
                                int B, int Hq, int Hkv, int Smax, int d, float scale, int chunk,
                                attn_dtype_t dtype, void* stream);

/*
 * attn_decode_paged -- attn_decode_splitkv over a paged K/V pool.
 * "M4.6 - FlashAttention-3/4 Hardware Pipelines ...", section 0x03 (a paged source
 * supplies a logical K/V block from a physical page named by a page index; masking a
 * tail score does not by itself make the page read safe), with the split and merge of
 * attn_decode_splitkv ("M4.4 - FlashAttention-2 ...", section 0x00A defers paged-cache
 * addressing of split-KV decode to a later article, so its layout here is this
 * library's reading).  Key j of sequence b is row j % P of page block_table[b, j / P].
 *
 *   q [B,Hq,1,d]; k_pages, v_pages [num_pages, Hkv, P, d]: element type `dtype`  (in)
 *   block_table: device int32 [B, max_pages]; entries in [0, num_pages); only the
 *       first ceil(seqlens_k[b] / P) entries of row b are read; an entry outside
 *       the pool is clamped into it (wrong rows, never an access outside the pool) (in)
 *   seqlens_k: device int32 [B], clamped to [0, max_pages * P]                   (in)
 *   page_size P: a power of two, 64 <= P <= 4096 (else ATTN_ERR_ARG); rows of a page
 *       past the sequence length are never read (they may hold anything).
 *   o [B,Hq,1,d] element type `dtype`; lse [B,Hq,1] float32 (may be NULL)        (out)
 *   chunk: as for attn_decode_splitkv.
 *   workspace: >= attn_decode_workspace_size(B, Hq, max_pages * P, d, chunk) bytes
 */
int attn_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                      const int* block_table, const int* seqlens_k, void* o, float* lse,
                      int B, int Hq, int Hkv, int num_pages, int page_size, int max_pages, int d,
                      float scale, int chunk, attn_dtype_t dtype, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * attn_tile_plan -- host-side view of the causal / tail tile iterator the kernels use.
 * For query rows [q_begin, q_end) against S_k keys in tiles of `block_k`, writes the
 * number of key tiles visited in ascending order (*n_visit) and the index of the
 * first visited tile that needs an element mask (*first_masked; == *n_visit when none
 * does).  Classification follows "M4.4 - FlashAttention-2 ...", section 0x05.1B
 * (skipped iff k0 > q_end - 1 + delta, fully visible iff k1 - 1 <= q_begin + delta,
 * delta = S_k - S_q).  Pure host code; returns ATTN_ERR_ARG / ATTN_ERR_NULL on bad
 * arguments.
 */
int attn_tile_plan(int q_begin, int q_end, int Sq, int Sk, int block_k, int causal,
                   int* n_visit, int* first_masked);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */

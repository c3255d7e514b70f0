// attn_decode.hip -- split-KV decode with an exact merge of partial states (gfx950).
//
// Decode has one query row per (sequence, query head), so the query-tile axis of the
// prefill grid collapses; the K/V axis is split into chunks instead and each chunk
// produces a partial state that a second pass merges ("M4.4 - FlashAttention-2 Work
// Partitioning and the Decode Boundary", section 0x01, the Flash-Decoding work axis;
// "M4.3 - IO-Aware Attention ...", sections 0x08B-0x08F: partial (m, l, u) states of
// disjoint key sets merge exactly, in any order, once they share one max frame).
//
// Pass 1 (split): one workgroup per (chunk, batch item, K/V head, head pass); the
// chunk is read from HBM exactly once for the G <= 16 query heads of the pass.  Each
// wave takes 64 keys of the chunk per pass (32 for short chunks, see kShortChunk) and
// runs both products on the 16x16x32 matrix core, with the G query heads as the N
// dimension (only G of its 16 columns
// carry data; the matrix core has the headroom, and the products stay off the vector
// ALUs, which keeps the kernel bound by HBM):
//   * every HBM load is a wave-wide 1 KiB of whole K or V rows with the streaming
//     (non-temporal) hint, the pattern that reads fastest; K and V then pass through
//     the wave's own LDS region (no workgroup barrier), K first;
//   * scores S^T = K Q^T: the K fragments (16 keys x 32 d) are read from LDS as the
//     A operand;
//   * the accumulator layout puts one head per lane column and 4 keys per lane, so
//     the probabilities become the A operand of O = P V without moving;
//   * V is read back transposed with ds_read_b64_tr_b16 as the B operand.
// The four waves then merge their (m, l, u) through LDS and write one partial per
// (chunk, query head).
// Pass 2 (merge): one wave per (batch item, query head) folds the partials in one
// max frame, O = u / l, LSE = m + ln l (all in base 2 internally).
#include "attn_device.h"
#include "attn_launch.h"
#include "../../include/attn.h"

#include <mutex>

// Partial states of attn_decode_splitkv_noalloc, for callers that cannot allocate: a
// file-scope device array (one copy per GPU the library runs on, alive until the
// process ends).  Host code never passes `scratch` itself to a kernel (on the host the
// name is only a stand-in); it uses the device address that attn_decode_scratch()
// looks up once per device with hipGetSymbolAddress.
static __device__ __align__(256) uint8_t scratch[ATTN_DECODE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kThreads = 256;
// Keys per wave per pass: 64, or 32 for chunks of up to 512 keys (half the staging
// registers and LDS, three waves per SIMD instead of two, so that more short chunks'
// first loads are in flight at once: 0.799 -> 0.791 ms at 256-key chunks on the
// [64 x 32 heads, 8 K/V heads, d 128] decode; at 1536-key chunks 64 keys are faster,
// 0.677 against 0.695 ms).
constexpr int kShortChunk = 512;

typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

template <typename T> struct Mfma16;
template <> struct Mfma16<f16> {
  static __device__ inline f32x4 run(const u32x4& a, const u32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};
template <> struct Mfma16<bf16> {
  static __device__ inline f32x4 run(const u32x4& a, const u32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

// 16x16x32 layouts (wave64): A lane l = row l%16, contraction slots from group l/16;
// B lane l = column l%16, same slots; C lane l = column l%16, rows 4(l/16) .. +3.

// K and V rows pass through the wave's LDS region with their 16-byte chunks
// XOR-swizzled (chunk p of row r at position p ^ swz(r)):
//  * K: the A-fragment read takes one chunk of 16 consecutive rows per 16-lane group;
//  * V: one 32-lane pass of the transpose read takes 8 rows x 2 chunks;
// both swizzles put those accesses on distinct banks.
template <int D> __device__ inline int swz_k(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D> __device__ inline int swz_v(int r) { return D == 128 ? 2 * (r & 7) : 2 * ((r >> 1) & 3); }

// PG: K/V come from a paged pool [num_pages, Hkv, P, D] through the block table
// (logical page i of sequence b is physical page block_table[b, i]); otherwise from
// contiguous caches [B, Hkv, Smax, D].
template <typename T, int D, int G, bool PG, int kSub>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kSub == 32 ? 3 : 2))) void decode_split_kernel(DecodeArgs a) {
  constexpr int DC = D / 32;          // contraction chunks of the score product
  constexpr int DB = D / 16;          // 16-wide d blocks of the output
  constexpr int KT = kSub / 16;       // 16-key score tiles per pass
  constexpr int CPR = D / 8;          // 16-byte chunks per V row
  constexpr int VLD = kSub * CPR / 64;   // V chunks staged per lane per pass
  static_assert(G >= 1 && G <= 16, "heads per pass");
  static_assert(kSub == 32 || kSub == 64, "keys per pass");
  typedef Mfma16<T> MF;

  __shared__ __attribute__((aligned(16))) uint8_t s_v[4][kSub * D * 2];
  __shared__ float s_m[4][G];
  __shared__ float s_l[4][G];
  __shared__ float s_u[4][G][D];

  const int c = blockIdx.x;
  const int bkv = blockIdx.y;
  const int b = bkv / a.Hkv;
  const int kvh = bkv - b * a.Hkv;
  const int h0 = kvh * a.group + blockIdx.z * G;   // first query head of this pass

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int kbeg = c * a.chunk;

  // Paged: physical page of the logical page holding key x (the table index clamped
  // into the row, the entry into the pool: a bad entry reads wrong rows, in bounds).
  // The wave's first lookup is issued before the length is known, so that the two
  // loads overlap; each later one is issued a pass ahead.
  auto page_of = [&](int x) {
    const int lp = min(x >> a.page_shift, a.max_pages - 1);
    return min(max(a.block_table[(int64_t)b * a.max_pages + lp], 0), a.num_pages - 1);
  };
  int pg_next = 0;
  if constexpr (PG) pg_next = page_of(kbeg + kSub * w);
  int len = a.seqlens[b];
  if constexpr (PG) asm volatile("" : : "s"(pg_next), "s"(len));   // both lookups before the length test
  len = len < 0 ? 0 : (len > a.Smax ? a.Smax : len);
  if (kbeg >= len) return;                          // whole workgroup: no barrier reached
  const int kend = min(kbeg + a.chunk, len);

  const int n = lane & 15;
  const int g = lane >> 4;

  // loads past the sequence's length return zero (the buffer range check)
  const int64_t head_row0 = PG ? 0 : (int64_t)(b * a.Hkv + kvh) * a.Smax;
  const T* kbase = reinterpret_cast<const T*>(a.k) + head_row0 * D;
  const T* vbase = reinterpret_cast<const T*>(a.v) + head_row0 * D;
  __amdgpu_buffer_rsrc_t kr = make_rsrc(kbase, (uint32_t)len * D * 2);
  __amdgpu_buffer_rsrc_t vr = make_rsrc(vbase, (uint32_t)len * D * 2);
  const T* qbase = reinterpret_cast<const T*>(a.q) + ((int64_t)b * a.Hq + h0) * D;
  uint8_t* vt = s_v[w];

  // Q^T as the B operand: column n = head h0 + n (zero for n >= G), slots d 32dc + 8g.
  u32x4 qf[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) {
    qf[dc] = u32x4{0u, 0u, 0u, 0u};
    if (n < G) qf[dc] = ld_global_16(qbase + (int64_t)n * D + 32 * dc + 8 * g);
  }

  // Running state: m (base 2) per head column n (equal on the four lane groups), the
  // lane's share of l, and the output rows 4g .. 4g+3 (heads) at d = 16db + n.
  float m_i = -INFINITY, l_i = 0.f;
  f32x4 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int base = kbeg + kSub * w; base < kend; base += 4 * kSub) {
    // All of the pass's loads first, each wave-wide load 1 KiB of whole rows with the
    // streaming hint (every byte is read once); K then V go through the wave's LDS
    // region, K first.
    // Paged: the pass's kSub keys lie in one page (P is a power of two >= 64 and base a
    // multiple of kSub); its rows of this head are contiguous.  The resource covers the
    // page rows below the sequence length, so rows past it read as zero as above.
    int row0 = base;
    if constexpr (PG) {
      const int pg = pg_next;
      const int in_page = base & ((1 << a.page_shift) - 1);
      const int64_t prow = ((int64_t)pg * a.Hkv + kvh) * (1 << a.page_shift) + in_page;
      const uint32_t bytes = (uint32_t)min(kSub, len - base) * D * 2;
      kr = make_rsrc(reinterpret_cast<const T*>(a.k) + prow * D, bytes);
      vr = make_rsrc(reinterpret_cast<const T*>(a.v) + prow * D, bytes);
      row0 = 0;
    }
    u32x4 kv[VLD], vv[VLD];
#pragma unroll
    for (int r = 0; r < VLD; ++r) {
      const int idx = r * 64 + lane;
      kv[r] = buf_load_16_stream(kr, (uint32_t)((row0 + idx / CPR) * D + 8 * (idx % CPR)) * 2);
    }
#pragma unroll
    for (int r = 0; r < VLD; ++r) {
      const int idx = r * 64 + lane;
      vv[r] = buf_load_16_stream(vr, (uint32_t)((row0 + idx / CPR) * D + 8 * (idx % CPR)) * 2);
    }
    if constexpr (PG) {
      if (base + 4 * kSub < kend) pg_next = page_of(base + 4 * kSub);
    }
#pragma unroll
    for (int r = 0; r < VLD; ++r) {
      const int idx = r * 64 + lane;
      const int row = idx / CPR;
      st_lds_16(vt + row * D * 2 + (((idx % CPR) ^ swz_k<D>(row)) * 16), kv[r]);
    }
    // K fragment (tile kt, contraction chunk dc): row 16kt + n, chunk 4dc + g.
    u32x4 kf[KT][DC];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        const int row = 16 * kt + n;
        kf[kt][dc] = ld_lds_16(vt + row * D * 2 + (((4 * dc + g) ^ swz_k<D>(row)) * 16));
      }
#pragma unroll
    for (int r = 0; r < VLD; ++r) {
      const int idx = r * 64 + lane;
      const int row = idx / CPR;
      st_lds_16(vt + row * D * 2 + (((idx % CPR) ^ swz_v<D>(row)) * 16), vv[r]);
    }

    // Scores: tile kt, lane (g, n) holds keys base + 16kt + 4g + i for head n.
    f32x4 sc[KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      sc[kt] = MF::run(kf[kt][0], qf[0], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int dc = 1; dc < DC; ++dc) sc[kt] = MF::run(kf[kt][dc], qf[dc], sc[kt]);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = base + 16 * kt + 4 * g + i;
        const float x = key < kend ? sc[kt][i] * a.scale_log2 : -INFINITY;
        sc[kt][i] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_i, mx);              // finite: key `base` is valid
    const float alpha = fast_exp2(m_i - m_new);
    m_i = m_new;
    // P as the A operand of O = P V: row n = head, slots 0..3 = keys 32j + 4g + i,
    // slots 4..7 = keys 32j + 16 + 4g + i.
    u32x4 pa[KT / 2];
    float rs = 0.f;
#pragma unroll
    for (int j = 0; j < KT / 2; ++j) {
      float e[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        e[i] = fast_exp2(sc[2 * j][i] - m_new);
        e[4 + i] = fast_exp2(sc[2 * j + 1][i] - m_new);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) rs += e[i];
      pa[j] = u32x4{Elem<T>::pack2(e[0], e[1]), Elem<T>::pack2(e[2], e[3]), Elem<T>::pack2(e[4], e[5]),
                    Elem<T>::pack2(e[6], e[7])};
    }
    l_i = alpha * l_i + rs;
    // Output rows are heads 4g + i; their alpha lives in the lanes of column 4g + i.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float ai = __shfl(alpha, 4 * g + i);
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db][i] *= ai;
    }
    // V^T fragments by transpose reads: the 16-lane group g reads the 4 keys x 16 d
    // block at keys 32j + 4g (+16 for slots 4..7), d = 16db; lane s of the group
    // addresses key row s/4, d columns 4(s%4) .. +3.
#pragma unroll
    for (int j = 0; j < KT / 2; ++j) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int col = 16 * db + 4 * (n & 3);
        const int r0 = 32 * j + 4 * g + (n >> 2);
        const int r1 = r0 + 16;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(vt + r0 * D * 2 + (((col >> 3) ^ swz_v<D>(r0)) * 16) + (col & 7) * 2));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(vt + r1 * D * 2 + (((col >> 3) ^ swz_v<D>(r1)) * 16) + (col & 7) * 2));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
        const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
        o[db] = MF::run(pa[j], u32x4{l2.x, l2.y, h2.x, h2.y}, o[db]);
      }
    }
  }

  // l: sum the four lane groups' shares.  Then merge the four waves through LDS.
  const float lt = l_i + __shfl_xor(l_i, 16);
  const float l_tot = lt + __shfl_xor(lt, 32);
  if (g == 0 && n < G) {
    s_m[w][n] = m_i;
    s_l[w][n] = l_tot;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hh = 4 * g + i;
    if (hh < G) {
#pragma unroll
      for (int db = 0; db < DB; ++db) s_u[w][hh][16 * db + n] = o[db][i];
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
  const bool paged = a.block_table != nullptr;
  if (a.chunk <= kShortChunk) {
    if (paged)
      hipLaunchKernelGGL((decode_split_kernel<T, D, G, true, 32>), grid, dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_split_kernel<T, D, G, false, 32>), grid, dim3(kThreads), 0, stream, a);
  } else {
    if (paged)
      hipLaunchKernelGGL((decode_split_kernel<T, D, G, true, 64>), grid, dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_split_kernel<T, D, G, false, 64>), grid, dim3(kThreads), 0, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid2((unsigned)((a.B * a.Hq + 3) / 4));
  hipLaunchKernelGGL((decode_merge_kernel<T, D>), grid2, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

// Heads per pass: the largest of 16, 8, 4, 2, 1 that divides the group.
template <typename T, int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t stream) {
  if (a.group % 16 == 0) return launch_g<T, D, 16>(a, stream);
  if (a.group % 8 == 0) return launch_g<T, D, 8>(a, stream);
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

// Device address of this GPU's `scratch` (the current device), looked up on the first
// call per device and kept; later calls return the kept address.
hipError_t attn_decode_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

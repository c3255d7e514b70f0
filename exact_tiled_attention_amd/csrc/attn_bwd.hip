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
// Wave layout of the main kernel (4 waves, BKV = 128 keys, wave w owns keys
// 32w .. 32w+31 of the tile).  S and dP are computed un-transposed on the 32x32x16
// matrix core with the query rows as M and the wave's keys as N, so each lane holds
// ONE key and 16 query rows of it: exactly the A-operand shape that dV += P^T dO and
// dK += dS^T Q need, with no data movement.  Their B operands (dO and Q with the
// query index as the contraction) come from the row-major staged tiles through
// ds_read_b64_tr_b16 (one column of 4 consecutive rows per lane).  dQ needs dS with
// queries as rows: dS goes to LDS key-major (8-byte writes of 4 queries) and comes
// back through the same transpose read; each wave then forms one (query block, d
// block) of dS K over all 128 keys.  Staged rows are unpadded, their 16-byte chunks
// XOR-swizzled so that both the 16-byte fragment reads and the transpose reads of a
// tile hit distinct banks.
#include <type_traits>

#include "../../include/attn.h"
#include "attn_device.h"
#include "attn_launch.h"
#include "tile_plan.h"

namespace {

constexpr int kWave = 64;
constexpr int kNT = 256;
constexpr int kBKV = 128;

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
    float* dq = a.dq_acc + row * D + 8 * c8;
    const u32x4 z = {0u, 0u, 0u, 0u};
    st_global_16(dq, z);
    st_global_16(dq + 4, z);
  }
  // sum over the LPR lanes of the row (LPR = 8 or 16 consecutive lanes)
#pragma unroll
  for (int s = 1; s < LPR; s <<= 1) acc += __shfl_xor(acc, s);
  if (row < rows && c8 == 0) a.delta[row] = acc;
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

// Pack 8 floats into 8 element values (hi) and, for bf16, the 8 residuals x - hi (lo).
template <typename T>
__device__ inline void split_pack8(const f32x16& x, int off, u32x4& hi, u32x4& lo) {
  float r[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = x[off + j];
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

// ---------------------------------------------------------------------------------
// 2. main column-owner kernel
//
// Chunk swizzle of the staged Q / dO rows (chunk p of row r at p ^ swz(r)):
//  * 16-byte fragment reads: 16 consecutive rows, one chunk -> 16 distinct banks groups;
//  * transpose reads: 4 consecutive rows x 4 consecutive chunks -> 16 distinct groups.
template <int D> __device__ inline int swz_q(int r) {
  if constexpr (D == 128) return 4 * (r & 3) + ((r >> 2) & 3);
  const int k = (r >> 1) & 7;   // rows of 128 bytes: pairs of rows share a 256-byte bank span
  return (k >> 1) | ((k & 1) << 2);
}

template <int D, int BQ>
struct BwdLds {
  static constexpr int ROWB = D * 2;          // staged row bytes
  static constexpr int Q = 0;                 // byte offsets
  static constexpr int DO = Q + BQ * ROWB;
  static constexpr int DST = DO + BQ * ROWB;  // dS^T [key][query], 16-bit
  static constexpr int KSTR = kBKV + 8;       // K^T [d][key] stride (elements)
  static constexpr int KT = DST + kBKV * BQ * 2;
  static constexpr int BYTES = KT + D * KSTR * 2;
};

typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ inline u32x2 tr_read(const uint8_t* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p));
}

template <typename T, typename G, int D, bool CAUSAL>
__global__ __launch_bounds__(kNT) void bwd_main_kernel(BwdArgs a) {
  typedef Elem<T> E;
  typedef typename E::v8 V8;
  constexpr int BQ = (D == 128) ? 32 : 64;
  constexpr int MB = BQ / 32;               // query blocks of 32 per tile
  constexpr int KC = D / 16;                // contraction chunks over d
  constexpr int QC = BQ / 16;               // contraction chunks over queries
  constexpr int DB = D / 32;                // d blocks of 32
  constexpr int CPR = D / 8;                // 16-byte chunks per staged row
  constexpr int SCH = BQ * CPR / (kNT / 2); // chunks per staging thread (Q or dO)
  typedef BwdLds<D, BQ> L;
  static_assert(SCH * (kNT / 2) == BQ * CPR, "staging chunks split evenly");

  __shared__ __attribute__((aligned(16))) uint8_t lds[L::BYTES];
  __shared__ __attribute__((aligned(16))) float s_lse[BQ];
  __shared__ __attribute__((aligned(16))) float s_del[BQ];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int n = lane & 31;
  const int grp = lane >> 5;
  const int s16 = lane & 15;
  const int hsel = (lane >> 4) & 1;          // 16-lane group within the 32-lane half

  const int jt = blockIdx.x;                 // key tile
  const int bkv = blockIdx.y;
  const int b = bkv / a.Hkv;
  const int kvh = bkv - b * a.Hkv;
  const int k0 = jt * kBKV;
  const int k1 = min(k0 + kBKV, a.Sk);
  const bool key_tail = (k0 + kBKV) > a.Sk;
  const int delta = a.Sk - a.Sq;

  const T* kbase = reinterpret_cast<const T*>(a.k) + ((int64_t)(b * a.Hkv + kvh) * a.Sk) * D;
  const T* vbase = reinterpret_cast<const T*>(a.v) + ((int64_t)(b * a.Hkv + kvh) * a.Sk) * D;

  // This wave's 32 keys as MFMA B operands (lane column = key, slots = d 16kc+8g..).
  const int mykey = k0 + 32 * w + n;
  V8 kf[KC], vf[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    u32x4 rk = {0u, 0u, 0u, 0u}, rv = {0u, 0u, 0u, 0u};
    if (mykey < a.Sk) {
      rk = ld_global_16(kbase + (int64_t)mykey * D + 16 * kc + 8 * grp);
      rv = ld_global_16(vbase + (int64_t)mykey * D + 16 * kc + 8 * grp);
    }
    kf[kc] = as_v8<V8>(rk);
    vf[kc] = as_v8<V8>(rv);
  }
  // K^T of the whole tile into LDS ([d][key]) for the dQ product: 4-key x 8-d blocks.
  {
    T* kt = reinterpret_cast<T*>(lds + L::KT);
    for (int blk = tid; blk < (kBKV / 4) * (D / 8); blk += kNT) {
      const int kq = blk / (D / 8);
      const int dc = blk % (D / 8);
      u32x4 r[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int key = k0 + 4 * kq + s;
        r[s] = u32x4{0u, 0u, 0u, 0u};
        if (key < a.Sk) r[s] = ld_global_16(kbase + (int64_t)key * D + dc * 8);
      }
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        u32x2 ev, od;
        ev.x = pack_lo(r[0][wd], r[1][wd]);
        ev.y = pack_lo(r[2][wd], r[3][wd]);
        od.x = pack_hi(r[0][wd], r[1][wd]);
        od.y = pack_hi(r[2][wd], r[3][wd]);
        st_lds_8(kt + (dc * 8 + 2 * wd) * L::KSTR + 4 * kq, ev);
        st_lds_8(kt + (dc * 8 + 2 * wd + 1) * L::KSTR + 4 * kq, od);
      }
    }
  }

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) {
    dk[i] = f32x16{};
    dv[i] = f32x16{};
  }

  const ColPlan cp = plan_cols(k0, k1, a.Sq, a.Sk, BQ, CAUSAL);
  const int nq = cp.n_qtiles - cp.first_qtile;
  const int nsteps = nq * a.group;

  // Staging: the first half of the threads stages Q, the second dO; chunk idx =
  // r * 128 + (tid % 128) of the tile is (row idx / CPR, chunk idx % CPR).
  const bool stage_do = tid >= kNT / 2;
  const int st_t = tid % (kNT / 2);
  u32x4 sreg[SCH];
  float slse = 0.f, sdel = 0.f;

  auto step_coords = [&](int step, int& h, int& qt) {
    h = kvh * a.group + step / nq;
    qt = cp.first_qtile + step % nq;
  };
  auto prefetch = [&](int step) {
    int h, qt;
    step_coords(step, h, qt);
    const T* src = reinterpret_cast<const T*>(stage_do ? a.dO : a.q) + ((int64_t)(b * a.Hq + h) * a.Sq) * D;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(src, (uint32_t)a.Sq * D * 2);
#pragma unroll
    for (int r = 0; r < SCH; ++r) {
      const int idx = r * (kNT / 2) + st_t;
      sreg[r] = buf_load_16(rs, (uint32_t)((qt * BQ + idx / CPR) * D + 8 * (idx % CPR)) * 2);
    }
    if (tid < BQ) {
      const int qr = qt * BQ + tid;
      const int64_t ri = (int64_t)(b * a.Hq + h) * a.Sq + qr;
      slse = qr < a.Sq ? a.lse[ri] * ATTN_LOG2E : 0.f;
      sdel = qr < a.Sq ? a.delta[ri] : 0.f;
    }
  };
  auto store_stage = [&]() {
    uint8_t* dst = lds + (stage_do ? L::DO : L::Q);
#pragma unroll
    for (int r = 0; r < SCH; ++r) {
      const int idx = r * (kNT / 2) + st_t;
      const int row = idx / CPR;
      st_lds_16(dst + row * L::ROWB + (((idx % CPR) ^ swz_q<D>(row)) * 16), sreg[r]);
    }
    if (tid < BQ) {
      s_lse[tid] = slse;
      s_del[tid] = sdel;
    }
  };

  // One step: S / dP for the wave's keys, P and dS, the dV / dK products, dS^T to LDS.
  // MASKED applies the element mask (tails and the causal band).
  auto compute = [&](auto masked_tag, int qt) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const uint8_t* sq = lds + L::Q;
    const uint8_t* sdo = lds + L::DO;
    f32x16 s[MB], dp[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const int row = 32 * mb + n;
        const int off = row * L::ROWB + (((2 * kc + grp) ^ swz_q<D>(row)) * 16);
        const V8 aq = as_v8<V8>(ld_lds_16(sq + off));
        const V8 ad = as_v8<V8>(ld_lds_16(sdo + off));
        s[mb] = E::mfma(aq, kf[kc], kc == 0 ? f32x16{} : s[mb]);
        dp[mb] = E::mfma(ad, vf[kc], kc == 0 ? f32x16{} : dp[mb]);
      }
    }
    // P = exp2(S log2e scale - LSE log2e); dS = P (dP - D).
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int qb = 32 * mb + 8 * r4 + 4 * grp;       // local query of regs 4r4..4r4+3
        const f32x4 lv = *reinterpret_cast<const f32x4*>(&s_lse[qb]);
        const f32x4 dl = *reinterpret_cast<const f32x4*>(&s_del[qb]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * r4 + e;
          float pv = fast_exp2(fmaf(s[mb][i], a.scale_log2, -lv[e]));
          if constexpr (MASKED) {
            const int qr = qt * BQ + qb + e;
            const bool vis = qr < a.Sq && mykey < a.Sk && (!CAUSAL || mykey <= qr + delta);
            pv = vis ? pv : 0.f;
          }
          s[mb][i] = pv;
          dp[mb][i] = pv * (dp[mb][i] - dl[e]);
        }
      }
    }
    // dV += P^T dO, dK += dS^T Q: A = this lane's key row, slots = queries
    // 16c + 8(j/4) + 4g + j%4 (registers 8(c%2) + j of query block c/2); B by
    // transpose reads of the staged tiles: the 16-lane group reads 4 queries x 16 d
    // (rows 16c + 4g, +8 for slots 4..7), lane s addressing row s/4, d 4(s%4).
    // With bf16 elements P and dS enter as hi + lo pairs of bf16 values (x = hi + lo
    // to about 16 significant bits), so these two sums keep float32-like precision.
#pragma unroll
    for (int c = 0; c < QC; ++c) {
      const int mb = c >> 1;
      const int hb = (c & 1) * 8;
      u32x4 pp, ss, pl, sl;
      split_pack8<T>(s[mb], hb, pp, pl);
      split_pack8<T>(dp[mb], hb, ss, sl);
      const int r0 = 16 * c + 4 * grp + (s16 >> 2);
      const int r1 = r0 + 8;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int col = 32 * db + 16 * hsel + 4 * (s16 & 3);
        const int o0 = r0 * L::ROWB + (((col >> 3) ^ swz_q<D>(r0)) * 16) + (col & 7) * 2;
        const int o1 = r1 * L::ROWB + (((col >> 3) ^ swz_q<D>(r1)) * 16) + (col & 7) * 2;
        const u32x2 olo = tr_read(sdo + o0), ohi = tr_read(sdo + o1);
        const u32x2 qlo = tr_read(sq + o0), qhi = tr_read(sq + o1);
        const V8 ob = as_v8<V8>(u32x4{olo.x, olo.y, ohi.x, ohi.y});
        const V8 qb4 = as_v8<V8>(u32x4{qlo.x, qlo.y, qhi.x, qhi.y});
        dv[db] = E::mfma(as_v8<V8>(pp), ob, dv[db]);
        dk[db] = E::mfma(as_v8<V8>(ss), qb4, dk[db]);
        if (kSplit<T>) {
          dv[db] = E::mfma(as_v8<V8>(pl), ob, dv[db]);
          dk[db] = E::mfma(as_v8<V8>(sl), qb4, dk[db]);
        }
      }
    }
    // dS^T -> LDS [key][query]: registers 4r4 .. 4r4+3 are 4 consecutive queries.
    uint8_t* dst = lds + L::DST;
    const int krow = 32 * w + n;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        u32x2 pk;
        pk.x = E::pack2(dp[mb][4 * r4 + 0], dp[mb][4 * r4 + 1]);
        pk.y = E::pack2(dp[mb][4 * r4 + 2], dp[mb][4 * r4 + 3]);
        st_lds_8(dst + (krow * BQ + 32 * mb + 8 * r4 + 4 * grp) * 2, pk);
      }
  };

  if (nsteps > 0) prefetch(0);
  for (int step = 0; step < nsteps; ++step) {
    int h, qt;
    step_coords(step, h, qt);
    // The previous step's reads of the staged tiles ended before its barrier (B), and
    // this step's dS^T writes come after barrier (A): one barrier pair per step.
    store_stage();
    __syncthreads();                                          // (A) stage visible
    if (step + 1 < nsteps) prefetch(step + 1);

    const bool masked = key_tail || qt < cp.nomask_qtile || (qt + 1) * BQ > a.Sq;
    if (masked)
      compute(std::true_type{}, qt);
    else
      compute(std::false_type{}, qt);
    __syncthreads();                                          // (B) dS^T visible
    // dQ_acc += dS K: wave w takes query block mb and d block db; contraction over the
    // 128 keys, slots = keys 16kc + 8g + j; A = dS by transpose reads of dS^T (the
    // 16-lane group reads 4 keys x 16 queries), B = K^T rows; result lane = d
    // column, regs = queries.
    {
      constexpr int NBLK = MB * DB;                          // (query block, d block) pairs
      const uint8_t* dstl = lds + L::DST;
      const T* kt = reinterpret_cast<const T*>(lds + L::KT);
      float* dqb = a.dq_acc + ((int64_t)(b * a.Hq + h) * a.Sq) * D;
      for (int blk = w; blk < NBLK; blk += 4) {
        const int mb = blk / DB;
        const int db = blk % DB;
        f32x16 acc = f32x16{};
        const int qcol = 32 * mb + 16 * hsel + 4 * (s16 & 3);
#pragma unroll
        for (int kc = 0; kc < kBKV / 16; ++kc) {
          const int kr0 = 16 * kc + 8 * grp + (s16 >> 2);
          const u32x2 lo = tr_read(dstl + (kr0 * BQ + qcol) * 2);
          const u32x2 hi = tr_read(dstl + ((kr0 + 4) * BQ + qcol) * 2);
          const V8 av = as_v8<V8>(u32x4{lo.x, lo.y, hi.x, hi.y});
          const V8 bv = as_v8<V8>(ld_lds_16(kt + (32 * db + n) * L::KSTR + 16 * kc + 8 * grp));
          acc = E::mfma(av, bv, acc);
        }
        const int dcol = 32 * db + n;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int qr = qt * BQ + 32 * mb + 8 * (i >> 2) + 4 * grp + (i & 3);
          if (qr < a.Sq) unsafeAtomicAdd(dqb + (int64_t)qr * D + dcol, acc[i]);
        }
      }
    }
  }

  // dK = scale * sum dS^T Q, dV = sum P^T dO; lane = d column, regs = keys.
  G* dkb = reinterpret_cast<G*>(a.dk) + ((int64_t)(b * a.Hkv + kvh) * a.Sk) * D;
  G* dvb = reinterpret_cast<G*>(a.dv) + ((int64_t)(b * a.Hkv + kvh) * a.Sk) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int dcol = 32 * db + n;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = k0 + 32 * w + 8 * (i >> 2) + 4 * grp + (i & 3);
      if (key < a.Sk) {
        store_grad<G>(dkb + (int64_t)key * D + dcol, dk[db][i] * a.scale);
        store_grad<G>(dvb + (int64_t)key * D + dcol, dv[db][i]);
      }
    }
  }
}

template <typename T, typename G, int D>
hipError_t launch_bwd_tg(const BwdArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.B * a.Hq * a.Sq;
  constexpr int RPB = kNT / (D / 8);
  hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(kNT), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((a.Sk + kBKV - 1) / kBKV), (unsigned)(a.B * a.Hkv));
  if (a.causal)
    hipLaunchKernelGGL((bwd_main_kernel<T, G, D, true>), grid, dim3(kNT), 0, stream, a);
  else
    hipLaunchKernelGGL((bwd_main_kernel<T, G, D, false>), grid, dim3(kNT), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n4 = rows * D / 4;
  hipLaunchKernelGGL((bwd_convert_kernel<G>), dim3((unsigned)((n4 + kNT - 1) / kNT)), dim3(kNT), 0, stream, a, n4);
  return hipGetLastError();
}

template <typename T, typename G>
hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t stream) {
  if (a.d == 64) return launch_bwd_tg<T, G, 64>(a, stream);
  return launch_bwd_tg<T, G, 128>(a, stream);
}

template <typename T>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t stream) {
  if (a.grad_type == ATTN_F32) return launch_bwd_d<T, float>(a, stream);
  if (a.grad_type == ATTN_BF16) return launch_bwd_d<T, bf16>(a, stream);
  return launch_bwd_d<T, f16>(a, stream);
}

}  // namespace

hipError_t attn_launch_bwd(const BwdArgs& a, hipStream_t stream) {
  if (a.dtype_bf16) return launch_bwd_t<bf16>(a, stream);
  return launch_bwd_t<f16>(a, stream);
}

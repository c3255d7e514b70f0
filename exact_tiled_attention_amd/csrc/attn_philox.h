// attn_philox.h -- Philox4x32-10 counter-based generator for dropout decisions.
//
// Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC 2011):
// ten rounds of two 32x32 -> 64-bit products by fixed multipliers, the high halves
// mixed with the other two counter words and the key, the key advanced by two Weyl
// constants between rounds.  The output is a pure function of (counter, key), which is
// what lets the backward regenerate the forward's decisions from element coordinates
// ("M4.4 - FlashAttention-2 ...", section 0x03I; "M4.3 - IO-Aware Attention ...",
// section 0x0DF).
//
// Coordinate map used by the kernels: element (b, h, query row i, key j) of a call with
// seed s and offset f takes word j % 4 of Philox(counter = (j / 4, i, b H_q + h, f),
// key = (s mod 2^32, s div 2^32)); it is kept iff the word >= floor(p 2^32).
#pragma once

#include <stdint.h>

#include "attn_device.h"

__device__ inline u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                      uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    // three-input exclusive or (v_bitop3_b32, truth table 0x96)
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, (unsigned char)0x96);
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, (unsigned char)0x96);
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
  }
  return u32x4{c0, c1, c2, c3};
}

// Per-call dropout parameters (all uniform).
struct DropParams {
  uint32_t thresh;    // words below are dropped: floor(p 2^32)
  uint32_t seed_lo, seed_hi;
  uint32_t offset;
  float rp;           // 1 / (1 - p)
};

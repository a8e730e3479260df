// fa_philox.h -- the counter-based generator behind in-kernel dropout.
//
// Philox4x32 with 10 rounds (Salmon, Moraes, Dror, Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC'11): per round, two 32 x 32 -> 64-bit
// products of counter words 0 and 2 with fixed multipliers; the high halves
// are XORed with the other two words and the round key, the words are
// permuted, and the key advances by a Weyl increment between rounds. On
// gfx950 each product is one v_mad_u64_u32 and each three-way XOR one
// v_bitop3_b32; the key is wave-uniform, so the key schedule stays in
// scalar registers.
//
// Dropout use: one call with counter (j / 8, i, b * Hq + h, offset) serves
// keys 8 (j / 8) .. 8 (j / 8) + 7 of query row i; key 8 g + e takes the
// 16-bit half (e & 1) of word (e >> 1), and is kept iff that uniform is
// below the threshold T (1 .. 65535).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_internal.h"

namespace fa {

struct Philox4 {
  uint32_t w[4];
};

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                                 uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)c0 * 0xD2511F53u;
    const uint64_t p1 = (uint64_t)c2 * 0xCD9E8D57u;
    // three-input XOR in one v_bitop3_b32 (truth table 0x96)
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return Philox4{{c0, c1, c2, c3}};
}

// The generator output for key group g (keys 8 g .. 8 g + 7) of row i of
// head bh under the problem's seed and offset.
__device__ __forceinline__ Philox4 drop_bits(const Problem& p, uint32_t g, uint32_t i,
                                             uint32_t bh) {
  return philox4x32_10(g, i, bh, p.drop_off, p.seed_lo, p.seed_hi);
}

// Is key 8 g + e kept? (thr <= 65535; the high half compares as a whole
// word: (w >> 16) < thr  <=>  w < thr * 65536.)
__device__ __forceinline__ bool drop_keep(const Philox4& x, int e, uint32_t thr) {
  const uint32_t w = x.w[e >> 1];
  return (e & 1) ? (w < (thr << 16)) : ((uint16_t)w < (uint16_t)thr);
}

// Zero the dropped entries of one run of 8 consecutive keys held in
// registers v[r0 .. r0 + 7] (key 8 g + e in v[r0 + e]).
template <typename V>
__device__ __forceinline__ void drop_run8(V& v, int r0, const Philox4& x, uint32_t thr) {
#pragma unroll
  for (int e = 0; e < 8; ++e) v[r0 + e] = drop_keep(x, e, thr) ? v[r0 + e] : 0.f;
}

// 8 keep bits of one call: bit e = key 8 g + e kept.
__device__ __forceinline__ uint32_t drop_byte(const Philox4& x, uint32_t thr) {
  uint32_t b = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) b |= drop_keep(x, e, thr) ? (1u << e) : 0u;
  return b;
}

// Transpose of an 8 x 8 bit matrix (twice, one per byte of a 16-bit value)
// across the 8 lanes of each aligned lane group: on entry lane e holds bit c
// of row e (byte 0) and of row 8 + e (byte 1); on exit lane c holds bit r =
// entry (row r, column c) for r = 0 .. 15. Three butterfly stages exchange
// the off-diagonal blocks of size 4, 2 and 1 with partner lane ^ k.
__device__ __forceinline__ uint32_t transpose8x8x2(uint32_t v) {
  const int lane = __lane_id();
#pragma unroll
  for (int k = 4; k >= 1; k >>= 1) {
    const uint32_t hi = k == 4 ? 0xF0F0u : k == 2 ? 0xCCCCu : 0xAAAAu;
    const uint32_t par = (uint32_t)__shfl_xor((int)v, k);
    v = (lane & k) ? ((v & hi) | ((par & hi) >> k)) : ((v & ~hi & 0xFFFFu) | ((par & ~hi & 0xFFFFu) << k));
  }
  return v;
}

}  // namespace fa

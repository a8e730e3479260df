// fa_stage.h -- cooperative global -> LDS staging of K/V/Q/dO tiles.
//
// A tile is ROWS consecutive sequence rows of one head, D elements each.
// Rows at or past `nvalid` are filled with zeros (never read from memory).
// 256 threads cooperate; every global access is a 16-byte vector load, and
// consecutive threads read consecutive 16-byte pieces of a row.
#pragma once

#include "fa_device.h"

namespace fa {

union Chunk {
  uint4 v;
  uint32_t d[4];
};

// Row-major copy: dst[r * PITCH + c] = src[(row0 + r) * stride + c].
template <typename T, int D, int ROWS, int PITCH>
__device__ __forceinline__ void stage_rows(const T* __restrict__ src, int64_t stride, int row0,
                                           int nvalid, T* dst, int tid) {
  constexpr int EPC = Traits<T>::EPC;
  constexpr int CPR = D / EPC;  // chunks per row
  constexpr int CHUNKS = ROWS * CPR;
  static_assert(CHUNKS % 256 == 0 || CHUNKS < 256, "tile/thread mismatch");
#pragma unroll
  for (int c = tid; c < CHUNKS; c += 256) {
    const int r = c / CPR, col = (c % CPR) * EPC;
    const int row = row0 + r;
    const uint4 x = ld16(src, (int64_t)row * stride + col, row < nvalid);
    *reinterpret_cast<uint4*>(dst + r * PITCH + col) = x;
  }
}

// Transposed copy: dst[c * PITCH + r] = src[(row0 + r) * stride + c].
// Each thread takes 4 consecutive rows x one 16-byte column piece and writes
// 4 rows of each of its columns as one 8-byte (bf16) or 16-byte (fp32) store.
template <typename T, int D, int ROWS, int PITCH>
__device__ __forceinline__ void stage_cols(const T* __restrict__ src, int64_t stride, int row0,
                                           int nvalid, T* dst, int tid) {
  constexpr int EPC = Traits<T>::EPC;
  constexpr int CPR = D / EPC;
  constexpr int GROUPS = (ROWS / 4) * CPR;
  static_assert(ROWS % 4 == 0, "rows in groups of 4");
#pragma unroll
  for (int g = tid; g < GROUPS; g += 256) {
    const int rg = g / CPR, colc = g % CPR;
    Chunk x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = row0 + 4 * rg + i;
      x[i].v = ld16(src, (int64_t)row * stride + colc * EPC, row < nvalid);
    }
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sh = (e & 1) * 16;
        uint32_t v0 = (x[0].d[e >> 1] >> sh) & 0xffffu, v1 = (x[1].d[e >> 1] >> sh) & 0xffffu;
        uint32_t v2 = (x[2].d[e >> 1] >> sh) & 0xffffu, v3 = (x[3].d[e >> 1] >> sh) & 0xffffu;
        *reinterpret_cast<uint2*>(dst + (colc * 8 + e) * PITCH + 4 * rg) =
            make_uint2(v0 | (v1 << 16), v2 | (v3 << 16));
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        *reinterpret_cast<uint4*>(dst + (colc * 4 + e) * PITCH + 4 * rg) =
            make_uint4(x[0].d[e], x[1].d[e], x[2].d[e], x[3].d[e]);
      }
    }
  }
}

// MFMA operand of one lane: KC/2 consecutive elements at p (16 bytes for bf16).
template <typename T>
__device__ __forceinline__ typename Traits<T>::Frag frag(const T* p) {
  if constexpr (sizeof(T) == 2) {
    return *reinterpret_cast<const bf16x8*>(p);
  } else {
    return *p;
  }
}

// Same, from global memory, zero when !ok.
template <typename T>
__device__ __forceinline__ typename Traits<T>::Frag frag_g(const T* p, bool ok) {
  if constexpr (sizeof(T) == 2) {
    if (!ok) {
      bf16x8 z;
#pragma unroll
      for (int e = 0; e < 8; ++e) z[e] = (bf16)0.f;
      return z;
    }
    return *reinterpret_cast<const bf16x8*>(p);
  } else {
    return ok ? *p : 0.f;
  }
}

}  // namespace fa

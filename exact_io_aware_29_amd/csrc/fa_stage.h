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

namespace fa {

// ------------------------------------------------------------------------
// Register-staged K/V tiles for the bf16 kernels (software prefetch).
//
// A tile of ROWS rows x D bf16 is fetched into registers with 16-byte
// loads while the previous tile is being computed, then written to LDS in
// one of two layouts:
//   * row-major with a 16-byte pad per row (pitch D + 8), read as MFMA A
//     operands of 8 consecutive head-dim elements;
//   * transposed (element (row, t) at [t][row]) with a 16-byte pad per
//     transposed row and its 8-row chunks XOR-swizzled by tswz(t), read as A
//     operands of 8 consecutive sequence rows. gfx950's LDS has 64 four-byte
//     banks; a 16-byte read is served 16 lanes at a time and an 8-byte write
//     32 lanes at a time. Readers take 16 consecutive t at one chunk index,
//     which the pad alone spreads over all banks (tswz is constant over
//     them); writers take 8 column chunks x 2 row-chunk values x 2 halves,
//     and tswz, built from bits 4.. of t, spreads those over all banks too.
// ------------------------------------------------------------------------

template <int D, int ROWS>
struct TileGeom {
  static constexpr int CPR = D / 8;                // 16-byte chunks per row
  static constexpr int NCH = ROWS * CPR / 256;     // row-major chunks per thread
  static constexpr int NGR = (ROWS / 4) * CPR / 256;  // 4-row groups per thread
  static constexpr int RPITCH = D + 8;             // row-major pitch (elements)
  static constexpr int TPITCH = ROWS + 8;          // transposed pitch (elements)
  static_assert(ROWS * CPR % 256 == 0 && (ROWS / 4) * CPR % 256 == 0, "tile/thread mismatch");
};

// Chunk swizzle of transposed row t for a tile of ROWS sequence rows. With
// 128 rows the writers' two row-chunk values differ in bit 0, so the
// swizzle uses bits 1..2; with 64 rows they share one chunk and bits 0..2
// are free.
template <int ROWS>
__device__ __forceinline__ int tswz(int t) {
  if constexpr (ROWS == 128) {
    return ((t >> 4) & 3) << 1;
  } else {
    static_assert(ROWS == 64, "transposed tiles hold 64 or 128 rows");
    return (t >> 4) & 7;
  }
}

// Element offset of the 16-byte chunk holding rows 8*kc .. 8*kc+7 of
// transposed row t.
template <int ROWS, int TPITCH>
__device__ __forceinline__ int tposn(int t, int kc) {
  return t * TPITCH + 8 * (kc ^ tswz<ROWS>(t));
}

// Thread -> (4-row group, 16-byte column chunk) for the transposing copy:
// eight consecutive lanes take the eight column chunks of a 128-byte row
// segment (coalesced global loads); the next lane bits select neighbouring
// row groups (and, with 16 chunks per row, the other half of the row).
template <int CPR>
__device__ __forceinline__ void tmap(int g, int& rg, int& colc) {
  if constexpr (CPR == 8) {
    colc = g & 7;
    rg = g >> 3;
  } else {
    colc = (g & 7) | (((g >> 4) & 1) << 3);
    rg = ((g >> 3) & 1) | ((g >> 5) << 1);
  }
}

template <int D, int ROWS>
struct RowRegs {
  uint4 c[TileGeom<D, ROWS>::NCH];
};
template <int D, int ROWS>
struct ColRegs {
  uint4 c[TileGeom<D, ROWS>::NGR][4];
};

template <int D, int ROWS>
__device__ __forceinline__ void load_rows(RowRegs<D, ROWS>& r, const bf16* __restrict__ src,
                                          int64_t stride, int row0, int nvalid, int tid) {
  using G = TileGeom<D, ROWS>;
  const bool full = row0 + ROWS <= nvalid;
#pragma unroll
  for (int i = 0; i < G::NCH; ++i) {
    const int c = tid + 256 * i;
    const int row = row0 + c / G::CPR, col = (c % G::CPR) * 8;
    r.c[i] = ld16(src, (int64_t)row * stride + col, full || row < nvalid);
  }
}

template <int D, int ROWS>
__device__ __forceinline__ void store_rows(const RowRegs<D, ROWS>& r, bf16* dst, int tid) {
  using G = TileGeom<D, ROWS>;
#pragma unroll
  for (int i = 0; i < G::NCH; ++i) {
    const int c = tid + 256 * i;
    *reinterpret_cast<uint4*>(dst + (c / G::CPR) * G::RPITCH + (c % G::CPR) * 8) = r.c[i];
  }
}

template <int D, int ROWS>
__device__ __forceinline__ void load_cols(ColRegs<D, ROWS>& r, const bf16* __restrict__ src,
                                          int64_t stride, int row0, int nvalid, int tid) {
  using G = TileGeom<D, ROWS>;
  const bool full = row0 + ROWS <= nvalid;
#pragma unroll
  for (int i = 0; i < G::NGR; ++i) {
    int rg, colc;
    tmap<G::CPR>(tid + 256 * i, rg, colc);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = row0 + 4 * rg + j;
      r.c[i][j] = ld16(src, (int64_t)row * stride + colc * 8, full || row < nvalid);
    }
  }
}

template <int D, int ROWS>
__device__ __forceinline__ void store_cols(const ColRegs<D, ROWS>& r, bf16* dst, int tid) {
  using G = TileGeom<D, ROWS>;
  static_assert(ROWS >= 64, "the chunk swizzle needs >= 8 chunks per transposed row");
#pragma unroll
  for (int i = 0; i < G::NGR; ++i) {
    int rg, colc;
    tmap<G::CPR>(tid + 256 * i, rg, colc);
    Chunk x[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j].v = r.c[i][j];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int sh = (e & 1) * 16;
      const uint32_t v0 = (x[0].d[e >> 1] >> sh) & 0xffffu, v1 = (x[1].d[e >> 1] >> sh) & 0xffffu;
      const uint32_t v2 = (x[2].d[e >> 1] >> sh) & 0xffffu, v3 = (x[3].d[e >> 1] >> sh) & 0xffffu;
      const int t = colc * 8 + e;
      *reinterpret_cast<uint2*>(dst + tposn<ROWS, G::TPITCH>(t, rg >> 1) + 4 * (rg & 1)) =
          make_uint2(v0 | (v1 << 16), v2 | (v3 << 16));
    }
  }
}

// Row-major store of registers fetched with the transposing thread map.
template <int D, int ROWS>
__device__ __forceinline__ void store_rows_t(const ColRegs<D, ROWS>& r, bf16* dst, int tid) {
  using G = TileGeom<D, ROWS>;
#pragma unroll
  for (int i = 0; i < G::NGR; ++i) {
    int rg, colc;
    tmap<G::CPR>(tid + 256 * i, rg, colc);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<uint4*>(dst + (4 * rg + j) * G::RPITCH + colc * 8) = r.c[i][j];
  }
}

}  // namespace fa

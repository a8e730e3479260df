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
// DMA-staged tiles (bf16 kernels).
//
// Tiles of ROWS sequence rows x D bf16 live in LDS row-major and unpadded;
// the sixteen-byte chunk c of row r sits at chunk position c ^ swz(r). They
// are filled by buffer loads that write LDS directly (64 lanes x 16 bytes =
// one contiguous KiB per wave instruction), so a lane's global source is
// chosen to be the chunk that belongs at its LDS position. Buffer loads
// return zero beyond the tensor's last row, which zero-fills tail tiles
// without predication.
//
// Operands are read back in two ways (both bank-conflict free on gfx950's
// 64 LDS banks with this swizzle, as measured):
//   * 16-byte reads of 8 consecutive head-dim elements of one row (MFMA
//     A operands whose rows are sequence rows);
//   * ds_read_b64_tr_b16 transposing reads, which give each lane 4
//     consecutive sequence rows of one head-dim column (MFMA A operands
//     whose rows are head-dim indices). Within each 16-lane group, output
//     lane i receives element i % 4 of the 8 bytes loaded by group lane
//     4 e + i / 4, for e = 0..3; loader lane 4 e + a therefore reads row
//     base + e at columns 4 a .. 4 a + 3 of a 16-column slice.
// ------------------------------------------------------------------------

typedef __amdgpu_buffer_rsrc_t Rsrc;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
#define FA_LDS __attribute__((address_space(3)))

// Raw buffer over [base, base + nbytes); the dword-3 constant selects the
// plain 32-bit data format used for untyped buffer access on this chip.
__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes,
                                           0x00020000);
}

// Byte extent of a resource over the first `rows` rows of one head (row
// pitch `sb` bytes, `rb` bytes of data per row). The range check covers the
// sum of the lane and scalar offsets, so every read at or past row `rows`
// returns zero: key rows past a sequence's valid length are never fetched,
// whatever their memory holds. The host guarantees that no row offset of a
// visited tile reaches 2^32 (no wrap back into the range) and that the row
// pitch is at least `rb` (rows do not overlap).
__device__ __forceinline__ uint32_t rows_extent(int rows, int sb, int rb) {
  return rows > 0 ? (uint32_t)(rows - 1) * (uint32_t)sb + (uint32_t)rb : 0u;
}

// SW selects the chunk swizzle by the reads that the tile serves. LDS has
// 64 banks of 4 bytes; the lanes served in one cycle must hit distinct
// banks. Measured on gfx950 (bank-conflict counters over 68 candidate
// swizzles): a 16-byte read serves together the 16 lanes with equal lane
// bit 5 and equal parity of lane bits 2..4; an 8-byte transposing read
// serves each 32-lane half together.
//   SW = 0, the 32x32 products' reads (rows in swap_bits23 order, chunk
//           pairs per lane half; transposing reads of 4-row groups);
//   SW = 1, the 16x16x32 products: row reads of 16 rows x 4 consecutive
//           chunks (lane i + 16 g: row i, chunk 4 c + g) and transposing
//           reads of 8 rows x a chunk pair (2 k, 2 k + 1). At d = 128, an
//           XOR swizzle S makes both conflict-free iff S^-1(1) has bits 2
//           and 3 set; this S maps row 12 to 1. At d = 64 (two rows per
//           bank period, row bit 0 picks the bank half) S(r) = r AND 6
//           does.
// Either swizzle depends on a row's low 4 bits only.
template <int D, int ROWS, int SW = 0>
struct SwzTile {
  static constexpr int RB = 2 * D;            // bytes per row
  static constexpr int CPR = D / 8;           // 16-byte chunks per row
  static constexpr int BYTES = ROWS * RB;
  static constexpr int NLD = BYTES / (256 * 16);  // DMA loads per thread
  static_assert(BYTES % (256 * 16) == 0, "tile must be a whole number of workgroup loads");
  static_assert(ROWS % 16 == 0, "operand fetch works on 16-row groups");
  static_assert(SW == 0 || D == 128 || D == 64, "16x16x32 swizzles for d = 64 and 128");
  __device__ static __forceinline__ int swz(int r) {
    if constexpr (SW == 1 && D == 64) {
      return r & 6;
    } else if constexpr (SW == 1) {
      return (((r & 7) << 1) | ((r >> 3) & 1)) ^ (r & 8);
    } else if constexpr (D == 64) {
      return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
    } else {
      return ((r & 3) << 2) | ((r >> 2) & 3);
    }
  }
  __device__ static __forceinline__ int off(int r, int c) { return r * RB + 16 * (c ^ swz(r)); }
};

// Per-lane global byte offsets (relative to the tile's first row) of the
// DMA loads that fill one tile of type T when NW waves share the work;
// computed once per kernel. Wave w's load i fills LDS kibibyte i * NW + w
// of the tile.
template <class T, int NL, int NW = 4>
__device__ __forceinline__ void dma_offsets_t(int (&voff)[NL], int stride_bytes, int w, int lane) {
  static_assert(NL * NW * 1024 == T::BYTES, "one offset per DMA load");
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int p = (i * NW + w) * 64 + lane;  // 16-byte LDS position
    const int r = p / T::CPR, pc = p % T::CPR;
    voff[i] = (int)((uint32_t)r * (uint32_t)stride_bytes + 16u * (uint32_t)(pc ^ T::swz(r)));
  }
}

template <int D, int ROWS, int NL, int NW = 4>
__device__ __forceinline__ void dma_offsets(int (&voff)[NL], int stride_bytes, int w, int lane) {
  dma_offsets_t<SwzTile<D, ROWS>, NL, NW>(voff, stride_bytes, w, lane);
}

// Cache-policy bits of a buffer load (gfx950): non-temporal, for data
// that is read once (evicted first rather than kept for reuse).
constexpr int kCpolNonTemporal = 2;

// CPOL: the loads' cache-policy bits (0 = default, for tiles that other
// workgroups read again from L2; kCpolNonTemporal for a stream read once).
template <int D, int ROWS, int NW = 4, int CPOL = 0>
__device__ __forceinline__ void dma_tile(Rsrc rs, const int* voff, uint32_t soff, char* tile,
                                         int w) {
  using T = SwzTile<D, ROWS>;
  constexpr int NL = T::BYTES / (NW * 1024);
#pragma unroll
  for (int i = 0; i < NL; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (FA_LDS void*)(tile + (i * NW + w) * 1024), 16,
                                             voff[i], soff, 0, CPOL);
}

// This wave's DMA loads have landed in LDS.
__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Debug build (FA_PARANOID_BARRIERS=1): a workgroup barrier before every
// refill of an LDS stage (every wave has finished reading it), and a full
// wait plus barrier right after the refill is issued (it has landed for
// every wave before anything else runs). Results must be bit-identical to
// the release build, which overlaps the refill with the reads of the other
// stage and relies on restrict-qualified stage pointers to keep the two
// apart. In the release build both calls compile to nothing.
#ifndef FA_PARANOID_BARRIERS
#define FA_PARANOID_BARRIERS 0
#endif
__device__ __forceinline__ void paranoid_before_fill() {
  if (FA_PARANOID_BARRIERS) __syncthreads();
}
__device__ __forceinline__ void paranoid_after_fill() {
  if (FA_PARANOID_BARRIERS) {
    wait_dma();
    __syncthreads();
  }
}

// Lane index of a wave64, computed by an opaque mbcnt pair: the compiler
// cannot hoist or share it, so values derived from it in a loop are rebuilt
// there instead of being kept live (or spilled) across iterations.
__device__ __forceinline__ int fresh_lane_id() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// 16-byte row operand at byte offset `off` of an LDS tile.
__device__ __forceinline__ bf16x8 lds_row(const char* tile, int off) {
  return *reinterpret_cast<const bf16x8*>(tile + off);
}

// Transposed operand: two transposing reads (slots 0-3 and 4-7).
__device__ __forceinline__ bf16x8 lds_tr(const char* tile, int off0, int off1) {
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(tile + off0));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(tile + off1));
  const i16x8 c = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, c);
}

// Lane offsets for the row operand of a 32-row MFMA block whose rows are
// loaded in swap_bits23 order: chunk 2 kk + h of row swap_bits23(lane % 32).
template <int D, int ROWS, int NK>
__device__ __forceinline__ void row_offsets(int (&off)[NK], int lr, int hh) {
  static_assert(NK == D / 16, "one offset per 16-wide head-dim step");
  using T = SwzTile<D, ROWS>;
  const int r = swap_bits23(lr);
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) off[kk] = T::off(r, 2 * kk + hh);
}

// Lane offsets for the transposed operand: output lane l (row = head-dim
// index 32 db + l % 32) gets sequence rows 16 c + 8 h + 4 j + 0..3 (slots
// 4 j .. 4 j + 3). As a loader, lane l of 16-lane group g reads row
// 8 h + 4 j + (q >> 2) at head-dim 32 db + 16 (g & 1) + 4 (q & 3).
// The sixteen-row base 16 c (+ 32 t) is added as an immediate.
template <int D, int ROWS, int NB>
__device__ __forceinline__ void tr_offsets(int (&off)[NB][2], int lane) {
  static_assert(NB == D / 32, "one offset pair per 32-row head-dim block");
  using T = SwzTile<D, ROWS>;
  const int g = lane >> 4, q = lane & 15, hh = lane >> 5;
#pragma unroll
  for (int db = 0; db < NB; ++db)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = 8 * hh + 4 * j + (q >> 2);
      const int d = 32 * db + 16 * (g & 1) + 4 * (q & 3);
      off[db][j] = r * T::RB + 16 * ((d >> 3) ^ T::swz(r)) + 2 * (d & 7);
    }
}

}  // namespace fa

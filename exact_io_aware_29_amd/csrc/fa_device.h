// fa_device.h -- device-side building blocks shared by the gfx950 kernels.
//
// Matrix-core conventions (CDNA 32x32 MFMA, wave64):
//   D[i][j] = sum_k A[i][k] B[k][j] over one 32 x 32 output block.
//   A operand: lane l supplies row i = l % 32, B operand: column j = l % 32;
//   both take their K slice from lane half h = l / 32 in the same slot order,
//   so any consistent slot -> k assignment contracts correctly.
//   C/D: lane l holds column j = l % 32; register r holds row
//   i = 8 * (r / 4) + 4 * h + r % 4.
//
// Row permutation. When a 32-row operand is loaded with MFMA row i taking
// physical row swap_bits23(i), register r of lane half h of the result
// belongs to physical row 16 * (r / 8) + 8 * h + r % 8. Each lane then owns
// two runs of 8 consecutive physical rows (registers 0..7 and 8..15), which
// is exactly the K-slot layout the next product needs: the registers can be
// rounded to bf16 and fed straight back as a B operand, and the matching A
// operand is one 16-byte read of 8 consecutive rows from a transposed tile.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_internal.h"

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kInf = __builtin_inff();

// Element-type traits: K extent of one MFMA and elements per 16-byte chunk.
template <typename T> struct Traits;
template <> struct Traits<bf16> {
  static constexpr int KC = 16;
  static constexpr int EPC = 8;
  typedef bf16x8 Frag;
};
template <> struct Traits<float> {
  static constexpr int KC = 2;
  static constexpr int EPC = 4;
  typedef float Frag;
};

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// 16x16x32 product. Per lane l (i = l mod 16, g = l / 16): A supplies row
// i and B column i, both with K slots 8 g .. 8 g + 7; the result holds
// column i, rows 4 g .. 4 g + 3 (registers 0..3).
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// All-reduces over the four lanes i, i + 16, i + 32, i + 48 (one column
// of a 16x16 result). v_permlane16_swap exchanges the odd 16-lane groups of
// its first operand with the even groups of its second, v_permlane32_swap
// the upper half of the first with the lower half of the second.
//
// Maximum of a and of b at once: the 16-lane swap of (a, b) leaves a's
// pair maxima in lane groups 0 and 2 and b's in groups 1 and 3, the
// 32-lane swap completes both, and a last 16-lane swap of that result with
// itself returns a's maximum in its first output and b's in its second.
__device__ __forceinline__ void quad_max2(float a, float b, float& ma, float& mb) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  float x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  ma = __uint_as_float(r[0]);
  mb = __uint_as_float(r[1]);
}
// Sum: each swap applied to (x, x) returns x of the lane and of its
// partner, in some order.
__device__ __forceinline__ float quad_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ int swap_bits23(int i) {
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

// Physical row (0..31) of register r in lane half h after a swap_bits23 load.
__device__ __forceinline__ int perm_row(int r, int h) {
  return 16 * (r >> 3) + 8 * h + (r & 7);
}

// Output row (0..31) of register r in lane half h for an unpermuted product.
__device__ __forceinline__ int c_row(int r, int h) {
  return 8 * (r >> 2) + 4 * h + (r & 3);
}

// All-reduce across the two lane halves (lane l and lane l ^ 32).
// v_permlane32_swap exchanges the upper half of its first operand with the
// lower half of its second; applied to (x, x) it leaves x[l % 32] in one
// result and x[l % 32 + 32] in the other, in every lane.
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Tree reductions of one accumulator block. The maximum uses three-input
// maxima (v_max3_f32): 8 operations in a dependency chain of depth 3; the
// sum is pairwise: 15 operations, depth 4 instead of 15.
__device__ __forceinline__ float tree_max16(const f32x16& s) {
  float a[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) a[i] = fmaxf(fmaxf(s[3 * i], s[3 * i + 1]), s[3 * i + 2]);
  return fmaxf(fmaxf(fmaxf(a[0], a[1]), a[2]), fmaxf(fmaxf(a[3], a[4]), s[15]));
}
__device__ __forceinline__ float tree_sum16(const f32x16& s) {
  float a[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = s[i] + s[i + 8];
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = a[i] + a[i + 4];
  return (a[0] + a[2]) + (a[1] + a[3]);
}

// True in every lane if `pred` holds in any active lane of the wave.
__device__ __forceinline__ bool wave_any(bool pred) { return __any(pred); }

// Debug build with per-workgroup timelines (FA_TIMELINE=1, libfa_timeline.so;
// nothing else loads it). Thread 0 of each workgroup stores 64-bit stamps
// into a device array of its kernel: the 100 MHz real-time counter at fixed
// points (entry, each block's start, its first tile or step ready, the end
// of its tile loop, exit), the XCD / CU it runs on, and the block's tile
// count. Only the first kTlWorkgroups workgroups of a launch record. In the
// release build every stamp compiles to nothing.
#ifndef FA_TIMELINE
#define FA_TIMELINE 0
#endif
constexpr int kTlWorkgroups = 1 << 16;
constexpr int kTlSlots = 16;  // words per workgroup
// Word layout: 0 entry, 1 (XCC_ID << 32 | HW_ID), 10 exit; for block r of
// the workgroup (r = 0, 1): 2 + 4r start, 3 + 4r first tile ready, 4 + 4r
// tile loop done, 5 + 4r (block index << 16 | tiles or steps).
#if FA_TIMELINE
#define FA_TL(buf, slot, value)                                                   \
  do {                                                                           \
    if (threadIdx.x == 0 && blockIdx.x < (unsigned)kTlWorkgroups)                \
      (buf)[(size_t)blockIdx.x * kTlSlots + (slot)] = (unsigned long long)(value); \
  } while (0)
#else
#define FA_TL(buf, slot, value) \
  do {                          \
  } while (0)
#endif
__device__ __forceinline__ unsigned long long tl_now() { return __builtin_amdgcn_s_memrealtime(); }
__device__ __forceinline__ unsigned long long tl_where() {
  return (unsigned long long)(unsigned)__builtin_amdgcn_s_getreg((31 << 11) | 4) |
         ((unsigned long long)(unsigned)__builtin_amdgcn_s_getreg((31 << 11) | 20) << 32);
}

// Workgroup index -> logical index. Workgroups are handed to the 8 XCDs of
// the chip round-robin (w % 8); this bijection gives each XCD a contiguous
// range of logical indices, so the Q blocks of one head (adjacent logical
// indices) share that XCD's L2 when they stream the same K/V tiles.
__device__ __forceinline__ int xcd_remap(int w, int total) {
  const int xcd = w & 7, idx = w >> 3;
  const int base = total >> 3, rem = total & 7;
  return xcd * base + (xcd < rem ? xcd : rem) + idx;
}

__device__ __forceinline__ bf16x8 pack8(const f32x16& s, int c) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (bf16)s[8 * c + e];
  return r;
}

__device__ __forceinline__ uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

// 16-byte global load, zero when !ok (the address is not formed then).
template <typename T>
__device__ __forceinline__ uint4 ld16(const T* base, int64_t off, bool ok) {
  return ok ? *reinterpret_cast<const uint4*>(base + off) : zero4();
}

// Number of valid keys of batch entry b.
__device__ __forceinline__ int valid_keys(const int32_t* seqlens, int b, int n) {
  if (!seqlens) return n;
  int L = seqlens[b];
  return L < 0 ? 0 : (L > n ? n : L);
}

// Present 128 x 128 blocks along one line (a row or a column) of a block
// mask, looked up 64 blocks at a time: lane l tests block base + l, and one
// wave ballot gathers the 64 answers, which stay cached for the following
// lookups. A run of absent blocks then costs one vector load per 64 blocks
// instead of one dependent load per tile (at N = 65536 a sparse row would
// otherwise take about a thousand serial loads to find its ten blocks).
// Every call is made by a full wave with wave-uniform arguments, so the
// window lives in scalar registers.
struct MaskLine {
  const uint8_t* p;  // the line's first block; null when there is no mask
  int64_t step;      // bytes from one block of the line to the next
  int n;             // blocks on the line
  int base;          // first block of the cached window
  uint64_t bits;     // bit i: block base + i is present

  __device__ __forceinline__ MaskLine(const uint8_t* first, int64_t stride, int nblocks)
      : p(first), step(stride), n(nblocks), base(-64), bits(0) {}

  // First present block at or after blk, or n if none is; blk itself when
  // there is no mask.
  __device__ __forceinline__ int next(int blk) {
    if (p == nullptr) return blk;
    while (blk < n) {
      if (blk < base || blk >= base + 64) {
        // A scalar window address plus a 32-bit lane offset (lane * step <
        // 2^31: the block-mask pitch is limited to 2^24 bytes), with the lane
        // index made on the spot, so the reload holds few vector registers.
        base = blk;
        const uint8_t* w = p + (int64_t)base * step;
        int ln;
        asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
        const bool on = base + ln < n && w[(uint32_t)ln * (uint32_t)step] != 0;
        bits = __builtin_amdgcn_ballot_w64(on);
      }
      const uint64_t m = bits >> (blk - base);
      if (m != 0) return blk + __builtin_ctzll(m);
      blk = base + 64;
    }
    return n;
  }

  // First tile index >= t (tiles of BC keys or rows along the line) whose
  // block is present, or a value >= tend if none is before tend.
  template <int BC>
  __device__ __forceinline__ int next_tile(int t, int tend) {
    static_assert(BC <= 128 && 128 % BC == 0, "tiles subdivide a mask block");
    if (t >= tend) return t;
    const int b0 = (t * BC) >> 7;
    const int blk = next(b0);
    return blk == b0 ? t : min(tend, blk * (128 / BC));
  }
};

// Mask row of the query block starting at row q0 (a multiple of 128).
__device__ __forceinline__ MaskLine mask_row(const uint8_t* bm, int ld, int nlb, int q0) {
  return MaskLine(bm ? bm + (int64_t)(q0 >> 7) * ld : nullptr, 1, nlb);
}

__device__ __forceinline__ void log_tile(uint32_t* log, int64_t row_word0, int kcol) {
  const int kb = kcol >> 7;
  atomicOr(log + row_word0 + (kb >> 5), 1u << (kb & 31));
}

}  // namespace fa

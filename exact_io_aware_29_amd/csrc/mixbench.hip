// mixbench.hip -- instruction-mix ceiling of the matrix-core kernels.
//
// Times a wave-tile of 64 v_mfma_f32_16x16x32_bf16 products interleaved
// evenly with E v_exp_f32 and F other fp32 VALU operations (fused
// multiply-adds), and optionally R 16-byte LDS reads that feed the first R
// products' A operands and T transposing 8-byte LDS reads that, two by two,
// feed the next T / 2 products' A operands, at two waves
// per SIMD on every SIMD (512 workgroups of 256 threads, the attention
// kernels' occupancy), with no barriers or memory traffic. A kernel whose
// main loop issues that mix per 64 products cannot run faster than this on
// the same board: the time is the bound set by the instruction mix alone,
// under the board's power limit (operands are pseudo-random bf16 and change
// from one product to the next, as real operands do).
//
// Measurement only: the attention library does not use this code.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kM = 64;        // products per wave-tile
constexpr int kLds = 65536;   // LDS bytes per workgroup (two per CU fit)
// LDS levels: none; 16 row reads + 32 transposing reads per tile (the
// forward's pattern); 24 + 32 (the dK/dV step's pattern).
constexpr int kLdsR[3] = {0, 16, 24};
constexpr int kLdsT[3] = {0, 32, 32};

__device__ inline uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

__device__ inline __bf16 rnd_bf16(uint32_t key) {
  return (__bf16)((float)(mix32(key) & 0xffffu) * (1.f / 65536.f) - 0.5f);
}

// Scheduling groups: product m, then its share of the E + F VALU operations.
template <int E, int F, int m>
__device__ __forceinline__ void groups() {
  if constexpr (m < kM) {
    constexpr int n = E * (m + 1) / kM - E * m / kM + F * (m + 1) / kM - F * m / kM;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (n > 0) __builtin_amdgcn_sched_group_barrier(0x002, n, 0);
    groups<E, F, m + 1>();
  }
}

template <int E, int F, int L>
__global__ __launch_bounds__(256, 2) void mix_kernel(int iters, float* sink) {
  constexpr int R = kLdsR[L], T = kLdsT[L];
  // Highest byte read: 15 KiB (base) + 63 * 512 + 1 KiB < kLds (R, T <= 64).
  static_assert(R + T / 2 <= kM && R <= 64 && T <= 64, "reads feed distinct products");
  __shared__ __attribute__((aligned(1024))) char smem[L ? kLds : 16];
  const int tid = threadIdx.x, lane = tid & 63;
  if constexpr (L != 0) {
    for (int i = tid; i < kLds / 4; i += 256)
      reinterpret_cast<uint32_t*>(smem)[i] = mix32((uint32_t)i) & 0x3f7f3f7fu;  // finite bf16 pairs
    __syncthreads();
  }
  const uint32_t seed = blockIdx.x * 256u + (uint32_t)tid;
  bf16x8 a[4], b[4];
  for (int j = 0; j < 4; ++j)
    for (int e = 0; e < 8; ++e) {
      a[j][e] = rnd_bf16(seed * 64u + 8u * j + e);
      b[j][e] = rnd_bf16(0x9e3779b9u + seed * 64u + 8u * j + e);
    }
  f32x4 d[8] = {};
  float x[8], y[16];
  for (int i = 0; i < 8; ++i) x[i] = 0.001f * (float)(lane + i);
  for (int i = 0; i < 16; ++i) y[i] = 0.002f * (float)(lane - i);
  for (int it = 0; it < iters; ++it) {
    const int base = ((it * 5) & 15) * 1024;  // loop-variant: reads are not hoisted
    int ec = 0, fc = 0;
#pragma unroll
    for (int m = 0; m < kM; ++m) {
      // A operand: a 16-byte row read (first R products), two transposing
      // reads (next T / 2 products, as the kernels' transposed operands), or
      // a register.
      bf16x8 am = a[m & 3];
      if (m < R) {
        am = *reinterpret_cast<const bf16x8*>(smem + base + 512 * m + 16 * lane);
      } else if (m < R + T / 2) {
        typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
        const int t = 2 * (m - R);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(smem + base + 512 * t + 8 * lane));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(smem + base + 512 * (t + 1) + 8 * lane));
        am = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
      d[m & 7] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am, b[(m >> 2) & 3], d[m & 7], 0, 0, 0);
      const int e1 = E * (m + 1) / kM, f1 = F * (m + 1) / kM;
#pragma unroll
      for (; ec < e1; ++ec) x[ec & 7] = __builtin_amdgcn_exp2f(-x[ec & 7]);
#pragma unroll
      for (; fc < f1; ++fc) y[fc & 15] = fmaf(y[fc & 15], 0.999f, 0.0001f);
    }
    groups<E, F, 0>();
  }
  float s = 0.f;
  for (int i = 0; i < 8; ++i)
    for (int j = 0; j < 4; ++j) s += d[i][j];
  for (int i = 0; i < 8; ++i) s += x[i];
  for (int i = 0; i < 16; ++i) s += y[i];
  if (s == 12345.f) sink[tid] = s;  // never true; keeps every result live
}

typedef void (*MixFn)(int, float*);

template <int E, int F, int L>
void launch(int iters, float* sink) {
  hipLaunchKernelGGL((mix_kernel<E, F, L>), dim3(512), dim3(256), 0, 0, iters, sink);
}

#define FA_MIX_ROW(E, L)                                                                 \
  {launch<E, 0, L>, launch<E, 32, L>, launch<E, 64, L>, launch<E, 96, L>, launch<E, 128, L>, \
   launch<E, 160, L>}
#define FA_MIX_PLANE(L) \
  {FA_MIX_ROW(0, L), FA_MIX_ROW(8, L), FA_MIX_ROW(16, L), FA_MIX_ROW(24, L), FA_MIX_ROW(32, L)}
const MixFn kTable[3][5][6] = {FA_MIX_PLANE(0), FA_MIX_PLANE(1), FA_MIX_PLANE(2)};
#undef FA_MIX_PLANE
#undef FA_MIX_ROW

}  // namespace

extern "C" {

// Grid of the measured mixes: E = 8 * ei (ei = 0..4) exponentials and
// F = 32 * fi (fi = 0..5) other VALU operations per 64 products, at LDS
// level li = 0..2 with row_reads[li] 16-byte and tr_reads[li] transposing
// 8-byte reads per tile (either array may be null).
int fa_mixbench_grid(int* n_e, int* n_f, int* n_lds, int* row_reads, int* tr_reads) {
  *n_e = 5;
  *n_f = 6;
  *n_lds = 3;
  for (int i = 0; i < 3; ++i) {
    if (row_reads) row_reads[i] = kLdsR[i];
    if (tr_reads) tr_reads[i] = kLdsT[i];
  }
  return 0;
}

// Best of `reps` timed launches of `iters` wave-tiles per wave for grid
// point (ei, fi, li), after one short warm-up launch; writes the
// milliseconds. Returns 0, -1 for an index outside the grid or a bad count,
// or the HIP error code.
int fa_mixbench(int ei, int fi, int li, int iters, int reps, float* ms) {
  if (ei < 0 || ei >= 5 || fi < 0 || fi >= 6 || li < 0 || li >= 3 || iters <= 0 || reps <= 0 ||
      ms == nullptr)
    return -1;
  float* sink = nullptr;
  hipError_t e = hipMalloc(&sink, 256 * sizeof(float));
  if (e != hipSuccess) return (int)e;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  float best = 1e30f;
  e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  if (e == hipSuccess) {
    kTable[li][ei][fi](8, sink);
    e = hipDeviceSynchronize();
  }
  for (int r = 0; r < reps && e == hipSuccess; ++r) {
    e = hipEventRecord(e0, 0);
    if (e != hipSuccess) break;
    kTable[li][ei][fi](iters, sink);
    e = hipGetLastError();
    if (e == hipSuccess) e = hipEventRecord(e1, 0);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    float t = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&t, e0, e1);
    if (e == hipSuccess && t < best) best = t;
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  (void)hipFree(sink);
  if (e != hipSuccess) return (int)e;
  *ms = best;
  return 0;
}

}  // extern "C"

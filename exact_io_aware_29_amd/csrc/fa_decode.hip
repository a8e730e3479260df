// fa_decode.hip -- decode attention: one query row per head against a long
// key/value cache, split over the keys.
//
// In decoding the score matrix is a single row per head, so nothing N x N
// is ever formed and the work is bound by reading the K/V cache from HBM
// once (the synthesis page, section 3 item 4). Parallelism comes from
// splitting the keys: one workgroup per (batch, key/value head, block of
// up to 16 query heads of its group, key split) computes a normalised
// partial output and its log-sum-exp over its keys, and a combine kernel
// merges the splits with the softmax merge rule (the tutorial page,
// exercise 2): with m = max_s lse_s and w_s = 2^(lse_s - m),
// O = sum_s w_s O_s / sum_s w_s and LSE = m + log2(sum_s w_s) (base 2 here,
// natural log on output).
//
// Inside a workgroup each wave takes 16 of every 64 keys. The query heads
// of a GQA group share the K/V tiles: S^T = K Q^T is one 16x16x32 matrix
// product per 32 head-dim columns (keys x query heads), and the result
// registers are exactly the B operand of the 16x16x16 product
// O^T += V^T P^T, whose A operand is a transposing LDS read of the V tile.
// The four waves' partials are merged through LDS at the end.
#include "fa_stage.h"

namespace fa {

__device__ __forceinline__ f32x4 mfma16k32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16k16(i16x4 a, i16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

template <int D>
struct DecCfg {
  static constexpr int BC = 64;       // keys per tile: 16 per wave
  static constexpr int NKK = D / 32;  // 16x16x32 products per score block
  static constexpr int NDB = D / 16;  // 16-row blocks of O^T
  using T = SwzTile<D, BC>;
  static constexpr float kLag = 8.f;  // lazy rescale threshold (log2 units)
};

// 16-lane reductions across the four lane groups (lanes c, c+16, c+32, c+48).
__device__ __forceinline__ float group_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float group_sum(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

template <int D>
__global__ __launch_bounds__(256, 2) void decode_split_kernel(DecodeArgs a) {
  using C = DecCfg<D>;
  using T = typename C::T;
  __shared__ __attribute__((aligned(1024))) char smem[2][2 * T::BYTES];

  const Problem& p = a.p;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, g = lane >> 4;

  int u = blockIdx.x;
  const int s = u % a.splits;
  u /= a.splits;
  const int hb = u % a.hblocks;
  u /= a.hblocks;
  const int hk = u % p.Hkv, b = u / p.Hkv;

  const int L = __builtin_amdgcn_readfirstlane(valid_keys(p.seqlens, b, p.N));
  const int k_lo = s * a.split_len;
  const int k_hi = min(k_lo + a.split_len, L);
  const int ntiles = k_hi > k_lo ? (k_hi - k_lo + C::BC - 1) / C::BC : 0;

  // This lane's query column is head hk * G + 16 hb + col of the group.
  const int gi = 16 * hb + col;
  const bool qok = gi < p.G;
  const int h = hk * p.G + (qok ? gi : 0);
  bf16x8 qf[C::NKK];
  {
    const bf16* qrow = static_cast<const bf16*>(a.q) + b * a.sq.b + h * a.sq.h + 8 * g;
#pragma unroll
    for (int kk = 0; kk < C::NKK; ++kk) qf[kk] = frag_g(qrow + 32 * kk, qok);
  }

  const int ksb = 2 * (int)a.sk.n, vsb = 2 * (int)a.sv.n;
  // The cache rows past the valid length L read as zero, whatever their
  // memory holds (a cache is often allocated uninitialised).
  const Rsrc krs = make_rsrc(static_cast<const bf16*>(a.k) + b * a.sk.b + hk * a.sk.h,
                             rows_extent(L, ksb, 2 * D));
  const Rsrc vrs = make_rsrc(static_cast<const bf16*>(a.v) + b * a.sv.b + hk * a.sv.h,
                             rows_extent(L, vsb, 2 * D));
  int kvo[T::NLD], vvo[T::NLD];
  dma_offsets<D, C::BC>(kvo, ksb, w, lane);
  dma_offsets<D, C::BC>(vvo, vsb, w, lane);
  // A operand of S^T (K rows 16 w + col, head-dim chunk 4 kk + g) and of
  // O^T (V^T: loader lane 4 e + q of group g reads key row 16 w + 4 g + e at
  // head-dim 16 db + 4 q, which the transposing read hands to output lane
  // 4 q + 0..3 as keys 4 g + 0..3).
  int koff[C::NKK], voff[C::NDB];
#pragma unroll
  for (int kk = 0; kk < C::NKK; ++kk) koff[kk] = T::off(16 * w + col, 4 * kk + g);
  {
    const int r = 16 * w + 4 * g + (col >> 2);
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      const int d = 16 * db + 4 * (col & 3);
      voff[db] = r * T::RB + 16 * ((d >> 3) ^ T::swz(r)) + 2 * (d & 7);
    }
  }

  f32x4 acc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) acc[db] = f32x4{};
  float m_ref = -kInf;  // exponent reference of this query column (log2 units)
  float l_run = 0.f;    // this lane's share of the column's exp-sum
  const float sl2 = p.scale_l2;

  auto issue = [&](int t, char* stage) {
    const uint32_t row0 = (uint32_t)(k_lo + t * C::BC);
    // Every cache row is read once: non-temporal loads (5.46 -> 5.84 TB/s
    // at B16 H32/KV8 with 16K-32K cached keys).
    dma_tile<D, C::BC, 4, kCpolNonTemporal>(krs, kvo, row0 * ksb, stage, w);
    dma_tile<D, C::BC, 4, kCpolNonTemporal>(vrs, vvo, row0 * vsb, stage + T::BYTES, w);
  };
  if (ntiles > 0) issue(0, smem[0]);
  wait_dma();
  __syncthreads();

  // One tile read from `ks` while the next lands in `fill` (restrict: the
  // reads do not wait for that DMA; the explicit wait and barrier end it).
  auto tile = [&](int t, const char* __restrict__ ks, char* __restrict__ fill) {
    const char* vs = ks + T::BYTES;
    if (t + 1 < ntiles) {
      paranoid_before_fill();
      issue(t + 1, fill);
      paranoid_after_fill();
    }
    f32x4 sc = f32x4{};
#pragma unroll
    for (int kk = 0; kk < C::NKK; ++kk) sc = mfma16k32(lds_row(ks, koff[kk]), qf[kk], sc);
    const int key0 = k_lo + t * C::BC + 16 * w + 4 * g;  // this lane's keys: key0 + r
    if (__builtin_expect(k_lo + (t + 1) * C::BC > k_hi, false)) {
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[r] = key0 + r < k_hi ? sc[r] : -kInf;
    }
    const float mx = group_max(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]))) * sl2;
    if (wave_any(mx > m_ref + C::kLag)) {
      const float m_new = fmaxf(m_ref, mx);
      const float alpha = m_new == -kInf ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) acc[db] *= alpha;
    }
    const float m_use = m_ref == -kInf ? 0.f : m_ref;
    i16x4 pb;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float e = __builtin_amdgcn_exp2f(fmaf(sc[r], sl2, -m_use));
      l_run += e;
      pb[r] = __builtin_bit_cast(short, (bf16)e);
    }
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
      acc[db] = mfma16k16(__builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(vs + voff[db])),
                          pb, acc[db]);
    if (t + 1 < ntiles) {
      wait_dma();
      __syncthreads();
    }
  };
  for (int t = 0; t < ntiles; ++t) tile(t, smem[t & 1], smem[(t & 1) ^ 1]);

  // Merge the four waves' partials through LDS: per wave, the column
  // statistics (m, l) and O~ (16 columns x D).
  __syncthreads();
  float* const stat = reinterpret_cast<float*>(smem[0]);  // [4 waves][2][16]
  float* const ot = stat + 4 * 2 * 16;                    // [4 waves][16][D]
  const float l_tot = group_sum(l_run);
  if (g == 0) {
    stat[(w * 2 + 0) * 16 + col] = m_ref;
    stat[(w * 2 + 1) * 16 + col] = l_tot;
  }
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) ot[(w * 16 + col) * D + 16 * db + 4 * g + r] = acc[db][r];
  __syncthreads();
  const int64_t out_row0 = ((int64_t)b * p.Hq + hk * p.G + 16 * hb) ;  // head of column 0
  for (int idx = tid; idx < 16 * D; idx += 256) {
    const int c = idx / D, d = idx - c * D;
    if (16 * hb + c >= p.G) continue;
    float mw[4], mstar = -kInf;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      mw[ww] = stat[(ww * 2 + 0) * 16 + c];
      mstar = fmaxf(mstar, mw[ww]);
    }
    float wsum = 0.f, o = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float f = mw[ww] == -kInf ? 0.f : __builtin_amdgcn_exp2f(mw[ww] - mstar);
      wsum += f * stat[(ww * 2 + 1) * 16 + c];
      o += f * ot[(ww * 16 + c) * D + d];
    }
    const float on = wsum > 0.f ? o / wsum : 0.f;
    const float lse2 = wsum > 0.f ? mstar + __log2f(wsum) : -kInf;
    const int64_t row = out_row0 + c;  // (b, head) linear index
    if (a.splits == 1) {
      const int hh = hk * p.G + 16 * hb + c;
      char* obase = static_cast<char*>(a.o);
      const int64_t oe = b * a.so.b + hh * a.so.h + d;
      if (a.o_fp32)
        reinterpret_cast<float*>(obase)[oe] = on;
      else
        reinterpret_cast<bf16*>(obase)[oe] = (bf16)on;
      if (d == 0) a.lse[row] = lse2 == -kInf ? -kInf : lse2 * kLn2;
    } else {
      a.ws_o[(row * a.splits + s) * D + d] = on;
      if (d == 0) a.ws_lse[row * a.splits + s] = lse2;
    }
  }
}

// Merge of the splits of one (batch, query head): 64 lanes, D / 64 columns
// each.
template <int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(DecodeArgs a) {
  const Problem& p = a.p;
  const int64_t row = blockIdx.x;  // b * Hq + h
  const int b = (int)(row / p.Hq), h = (int)(row - (int64_t)b * p.Hq);
  const float* ls = a.ws_lse + row * a.splits;
  float m = -kInf;
  for (int s = 0; s < a.splits; ++s) m = fmaxf(m, ls[s]);
  const float mref = m == -kInf ? 0.f : m;  // every split empty: all weights 0
  float wsum = 0.f;
  float o[D / 64] = {};
  // Splits in batches of 8 whose loads are independent, so their latencies
  // overlap instead of adding up one split after another.
  for (int s0 = 0; s0 < a.splits; s0 += 8) {
    float f[8], x[8][D / 64];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int s = s0 + u;
      const float l = s < a.splits ? ls[s] : -kInf;
      const bool ok = l != -kInf;  // an empty split's partial is never read
      f[u] = ok ? __builtin_amdgcn_exp2f(l - mref) : 0.f;
      const float* os = a.ws_o + (row * a.splits + (ok ? s : 0)) * D;
#pragma unroll
      for (int j = 0; j < D / 64; ++j) x[u][j] = ok ? os[threadIdx.x + 64 * j] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      wsum += f[u];
#pragma unroll
      for (int j = 0; j < D / 64; ++j) o[j] = fmaf(f[u], x[u][j], o[j]);
    }
  }
  char* obase = static_cast<char*>(a.o);
#pragma unroll
  for (int j = 0; j < D / 64; ++j) {
    const float v = wsum > 0.f ? o[j] / wsum : 0.f;
    const int64_t oe = b * a.so.b + h * a.so.h + threadIdx.x + 64 * j;
    if (a.o_fp32)
      reinterpret_cast<float*>(obase)[oe] = v;
    else
      reinterpret_cast<bf16*>(obase)[oe] = (bf16)v;
  }
  if (threadIdx.x == 0) a.lse[row] = wsum > 0.f ? (m + __log2f(wsum)) * kLn2 : -kInf;
}

template <int D>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t st) {
  const int64_t grid = (int64_t)a.p.B * a.p.Hkv * a.hblocks * a.splits;
  hipLaunchKernelGGL((decode_split_kernel<D>), dim3((unsigned)grid), dim3(256), 0, st, a);
  if (a.splits > 1)
    hipLaunchKernelGGL((decode_combine_kernel<D>), dim3((unsigned)((int64_t)a.p.B * a.p.Hq)),
                       dim3(64), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int head_dim, hipStream_t st) {
  return head_dim == 64 ? launch_decode_t<64>(a, st) : launch_decode_t<128>(a, st);
}

}  // namespace fa

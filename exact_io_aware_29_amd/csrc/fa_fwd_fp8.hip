// fa_fwd_fp8.hip -- FP8 (OCP e4m3) attention forward for gfx950.
//
// FlashAttention-3 carries the tiled forward to FP8 inputs (cross-paper
// synthesis page, section 2: FP8 with incoherent processing), and
// SageAttention quantises P V to FP8 (same section); the result is no longer
// exact attention. Here Q, K and V arrive as e4m3 codes with per-tensor
// descale factors, and the structure is the bf16 forward's (Q-outer loop,
// one workgroup of 4 waves per 128 query rows, K/V tiles double-buffered in
// LDS by buffer-load DMA, lazy online softmax in fp32, normalisation at the
// end) with both products on the gfx950 matrix core's 32 x 32 x 64 FP8
// instruction:
//
//   S^T = K_j Q_i^T     A = K rows (one 64-wide head-dim block per product),
//                       B = this lane's Q row, kept in registers
//   P~  = 2^(S c - m)   fp32, then rounded to e4m3 (P~ <= 2^8 < 448)
//   O^T += V_j^T P~^T   A = V^T by transposing 8-bit LDS reads, B = P~
//
// The matrix core pairs A-lane (m + 32 h) byte b with B-lane (n + 32 h) byte
// b, so the k order inside a lane is free as long as both operands share it.
// Byte j of this lane's P~ operand is the score register 16 t + r (key
// 32 t + c_row(r, h) of the 64-key tile), and the V^T operand is read so that
// its byte j holds that same key: each 8-byte transposing read gives a
// 16-lane group one head-dim column per lane for 8 keys (lane i takes byte
// i % 8 of the 8 bytes that group lane 2 j + i / 8 loads).
//
// The row sum l comes from the fp32 P~, so the only rounding beyond fp32 is
// that of P~ in the numerator.
#include "fa_stage.h"

namespace fa {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

// Tile of ROWS rows x D one-byte elements in LDS: row-major, unpadded, the
// 16-byte chunk c of row r at chunk position c ^ swz(r). This swizzle keeps
// both the 16-byte row reads of the K operand and the 8-byte transposing
// reads of the V operand free of bank conflicts (64 banks, modelled for both
// head dims).
template <int D, int ROWS>
struct Tile8 {
  static constexpr int RB = D;         // bytes per row
  static constexpr int CPR = D / 16;   // 16-byte chunks per row
  static constexpr int BYTES = ROWS * RB;
  static constexpr int NLD = BYTES / (256 * 16);  // DMA loads per thread
  static_assert(BYTES % (256 * 16) == 0, "tile must be a whole number of workgroup loads");
  __device__ static __forceinline__ int swz(int r) {
    return ((r >> 2) ^ ((r & 3) << 1)) & (CPR - 1);
  }
  __device__ static __forceinline__ int off(int r, int c) { return r * RB + 16 * (c ^ swz(r)); }
};

template <int D>
struct Fwd8 {
  static constexpr int BR = 128;  // query rows per workgroup (4 waves x 32)
  static constexpr int BC = 64;   // keys per tile: one 64-deep PV product
  static constexpr int NSUB = 2;  // 32-key sub-tiles of S^T
  static constexpr int NKD = D / 64;
  static constexpr int NDB = D / 32;
  using T = Tile8<D, BC>;
  static constexpr float kLag = 8.f;  // P~ <= 2^8, inside e4m3's range
};

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  // format 0 (e4m3) for both operands, unit block scales (E8M0 127 = 2^0)
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Byte offsets (relative to the tile's first row) of this lane's DMA loads.
template <typename T>
__device__ __forceinline__ void dma_offsets8(int (&voff)[T::NLD], int stride_bytes, int w,
                                             int lane) {
#pragma unroll
  for (int i = 0; i < T::NLD; ++i) {
    const int p = (i * 4 + w) * 64 + lane;  // 16-byte LDS position
    const int r = p / T::CPR, pc = p % T::CPR;
    voff[i] = r * stride_bytes + 16 * (pc ^ T::swz(r));
  }
}

template <typename T>
__device__ __forceinline__ void dma_tile8(Rsrc rs, const int (&voff)[T::NLD], uint32_t soff,
                                          char* tile, int w) {
#pragma unroll
  for (int i = 0; i < T::NLD; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (FA_LDS void*)(tile + (i * 4 + w) * 1024), 16,
                                             voff[i], soff, 0, 0);
}

template <int D>
__global__ __launch_bounds__(256, 2) void fwd_kernel_fp8(FwdArgs a) {
  using C = Fwd8<D>;
  using T = typename C::T;
  // Two stages of (K tile | V tile).
  __shared__ __attribute__((aligned(1024))) char smem[2][2 * T::BYTES];

  const Problem& p = a.p;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, hh = lane >> 5;

  const int nqb = (p.N + C::BR - 1) / C::BR;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int head_lin = L / nqb;
  const int qbi = L - head_lin * nqb;
  const int qb = p.causal ? nqb - 1 - qbi : qbi;  // causal: longest rows first
  const int b = head_lin / p.Hq, h = head_lin - b * p.Hq, hk = h / p.G;
  const int q0 = qb * C::BR;
  const int my_q = q0 + 32 * w + lr;

  const int ksb = (int)a.sk.n, vsb = (int)a.sv.n;  // row strides in bytes
  const int kvalid = __builtin_amdgcn_readfirstlane(valid_keys(p.seqlens, b, p.N));
  const Rsrc krs = make_rsrc(static_cast<const uint8_t*>(a.k) + b * a.sk.b + hk * a.sk.h,
                             rows_extent(kvalid, ksb, D));
  const Rsrc vrs = make_rsrc(static_cast<const uint8_t*>(a.v) + b * a.sv.b + hk * a.sv.h,
                             rows_extent(kvalid, vsb, D));
  const int kend = min(p.causal ? min(kvalid, q0 + C::BR) : kvalid, q0 + C::BR + p.wr);
  const int ntiles = (kend + C::BC - 1) / C::BC;
  const int kfirst = max(0, q0 - p.wl) / C::BC;

  // This lane's Q row as the B operand: bytes 64 kd + 32 hh .. + 31.
  i32x8 qf[C::NKD];
  {
    const bool ok = my_q < p.N;
    const uint8_t* qrow = static_cast<const uint8_t*>(a.q) + b * a.sq.b + h * a.sq.h +
                          (int64_t)(ok ? my_q : 0) * a.sq.n + 32 * hh;
#pragma unroll
    for (int kd = 0; kd < C::NKD; ++kd) {
      const uint4 lo = ok ? *reinterpret_cast<const uint4*>(qrow + 64 * kd) : zero4();
      const uint4 hi = ok ? *reinterpret_cast<const uint4*>(qrow + 64 * kd + 16) : zero4();
      qf[kd] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                     (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
  }

  int kvo[T::NLD], vvo[T::NLD];
  dma_offsets8<T>(kvo, ksb, w, lane);
  dma_offsets8<T>(vvo, vsb, w, lane);
  // K operand: key row lr of a sub-tile (the swizzle depends on the row
  // modulo 32 only, so sub-tile t adds 32 t rows as an immediate), chunks
  // 4 kd + 2 hh and 4 kd + 2 hh + 1.
  int koff[C::NKD][2];
#pragma unroll
  for (int kd = 0; kd < C::NKD; ++kd)
#pragma unroll
    for (int x = 0; x < 2; ++x) koff[kd][x] = T::off(lr, 4 * kd + 2 * hh + x);
  // V^T operand, read q (0..3) of head-dim block db: this lane loads 8 bytes
  // of key 16 q + 4 (g / 2) + {0,1,2,3,8,9,10,11}[e] at head-dim
  // 32 db + 16 (g % 2) + 8 bb (g = lane / 16, e = (lane % 16) / 2,
  // bb = lane % 2). The swizzle then depends on q only through q % 2; q / 2
  // adds 32 rows.
  int toff[C::NDB][2];
  {
    const int g = lane >> 4, e = (lane & 15) >> 1, bb = lane & 1;
    const int kofs = 8 * (e >> 2) + (e & 3);
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int qq = 0; qq < 2; ++qq)
        toff[db][qq] = T::off(16 * qq + 4 * (g >> 1) + kofs, 2 * db + (g & 1)) + 8 * bb;
  }

  f32x16 acc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) acc[db] = f32x16{};
  float m_ref = -kInf;  // exponent reference of this lane's row (log2 units)
  float l_run = 0.f;    // this lane half's share of the row's exp-sum
  const float sl2 = p.scale_l2 * a.qk_descale;
  const int64_t log_row =
      a.log ? (((int64_t)b * p.Hq + h) * p.nlb + (q0 >> 7)) * p.logw : 0;

  MaskLine mrow = mask_row(p.bm, p.bm_ld, p.nlb, q0);
  auto next_visit = [&](int kt) { return mrow.next_tile<C::BC>(kt, ntiles); };
  auto issue = [&](int kt, char* stage) {
    dma_tile8<T>(krs, kvo, (uint32_t)(kt * C::BC) * ksb, stage, w);
    dma_tile8<T>(vrs, vvo, (uint32_t)(kt * C::BC) * vsb, stage + T::BYTES, w);
  };

  int kt = next_visit(kfirst);
  if (kt < ntiles) {
    issue(kt, smem[0]);
    wait_dma();
    __syncthreads();
  }
  auto tile = [&](const char* __restrict__ Ks, char* __restrict__ fill) {
    const char* Vs = Ks + T::BYTES;
    const int key0 = kt * C::BC;
    const int nxt = next_visit(kt + 1);
    if (nxt < ntiles) {  // lands while this tile is computed
      paranoid_before_fill();
      issue(nxt, fill);
      paranoid_after_fill();
    }
    if (a.log && tid == 0) log_tile(a.log, log_row, key0);
    const bool need_mask = (p.causal && key0 + C::BC - 1 > q0) || (key0 + C::BC > kvalid) ||
                           (key0 < q0 + C::BR - 1 - p.wl) || (key0 + C::BC - 1 > q0 + p.wr);

    f32x16 s[C::NSUB];
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int t = 0; t < C::NSUB; ++t) s[t] = f32x16{};
#pragma unroll
    for (int kd = 0; kd < C::NKD; ++kd)
#pragma unroll
      for (int t = 0; t < C::NSUB; ++t) {
        const char* kp = Ks + 32 * t * T::RB;
        const uint4 lo = *reinterpret_cast<const uint4*>(kp + koff[kd][0]);
        const uint4 hi = *reinterpret_cast<const uint4*>(kp + koff[kd][1]);
        const i32x8 ka = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                          (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        s[t] = mfma_fp8(ka, qf[kd], s[t]);
      }
    __builtin_amdgcn_s_setprio(0);
    if (__builtin_expect(need_mask, false)) {  // boundary tiles only
      // Register r of sub-tile t holds key key0 + 32 t + c_row(r, hh); it is
      // seen iff my_q - wl <= key <= my_q + hi (hi = 0 under the causal
      // mask, else the right window edge) and key < kvalid.
      const unsigned hi = p.causal ? 0u : (unsigned)p.wr;
      const unsigned span = (unsigned)p.wl + hi;
      const unsigned base = (unsigned)(key0 + 4 * hh + p.wl) - (unsigned)my_q;
#pragma unroll
      for (int t = 0; t < C::NSUB; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 32 * t + c_row(r, hh);
          const bool kill =
              (base + (unsigned)(32 * t + c_row(r, 0)) > span) | (key >= kvalid);
          s[t][r] = kill ? -kInf : s[t][r];  // branch-free select
        }
    }
    float mx = fmaxf(tree_max16(s[0]), tree_max16(s[1]));
    mx = half_max(mx) * sl2;
    if (wave_any(mx > m_ref + C::kLag)) {
      const float m_new = fmaxf(m_ref, mx);
      const float alpha = m_new == -kInf ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
    }
    const float m_use = m_ref == -kInf ? 0.f : m_ref;
    // P~ (fp32) into the row sum, then rounded to e4m3: byte 16 t + r of the
    // B operand is register r of sub-tile t.
    i32x8 pf;
#pragma unroll
    for (int t = 0; t < C::NSUB; ++t) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[t][r] = __builtin_amdgcn_exp2f(fmaf(s[t][r], sl2, -m_use));
      l_run += tree_sum16(s[t]);
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        int v = __builtin_amdgcn_cvt_pk_fp8_f32(s[t][4 * q4], s[t][4 * q4 + 1], 0, false);
        v = __builtin_amdgcn_cvt_pk_fp8_f32(s[t][4 * q4 + 2], s[t][4 * q4 + 3], v, true);
        pf[4 * t + q4] = v;
      }
    }
    // O^T += V^T P~^T: four transposing reads give this lane the 32 keys of
    // its P~ bytes at head-dim 32 db + lane % 32.
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      i32x8 va;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (FA_LDS i32x2*)(Vs + toff[db][q & 1] + (q >> 1) * 32 * T::RB));
        va[2 * q] = x[0];
        va[2 * q + 1] = x[1];
      }
      acc[db] = mfma_fp8(va, pf, acc[db]);
    }
    __builtin_amdgcn_s_setprio(0);
    if (nxt < ntiles) {
      wait_dma();
      __syncthreads();  // next tile landed everywhere; this tile is no longer read
    }
    kt = nxt;
  };
  // Unrolled by two: each copy reads its stage at a fixed LDS address.
  while (kt < ntiles) {
    tile(smem[0], smem[1]);
    if (kt >= ntiles) break;
    tile(smem[1], smem[0]);
  }

  const float l_tot = half_sum(l_run);
  const float inv = l_tot > 0.f ? a.v_descale / l_tot : 0.f;
  if (my_q < p.N) {
    char* obase = static_cast<char*>(a.o);
    const int64_t orow = b * a.so.b + h * a.so.h + (int64_t)my_q * a.so.n;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * hh;  // c_row(4 g, hh)
        const float v0 = acc[db][4 * g] * inv, v1 = acc[db][4 * g + 1] * inv;
        const float v2 = acc[db][4 * g + 2] * inv, v3 = acc[db][4 * g + 3] * inv;
        if (a.o_fp32) {
          *reinterpret_cast<float4*>(obase + (orow + d0) * 4) = make_float4(v0, v1, v2, v3);
        } else {
          bf16x4 pk;
          pk[0] = (bf16)v0;
          pk[1] = (bf16)v1;
          pk[2] = (bf16)v2;
          pk[3] = (bf16)v3;
          *reinterpret_cast<bf16x4*>(obase + (orow + d0) * 2) = pk;
        }
      }
    if (hh == 0) {
      const float lse = l_tot > 0.f ? (m_ref + __log2f(l_tot)) * kLn2 : -kInf;
      a.lse[((int64_t)b * p.Hq + h) * p.N + my_q] = lse;
    }
  }
}

hipError_t launch_fwd_fp8(const FwdArgs& a, int head_dim, hipStream_t s) {
  const int64_t nqb = (a.p.N + 127) / 128;
  const int64_t grid = nqb * a.p.Hq * a.p.B;
  if (head_dim == 64)
    hipLaunchKernelGGL(fwd_kernel_fp8<64>, dim3((unsigned)grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(fwd_kernel_fp8<128>, dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace fa

// fa_bwd.hip -- recomputation backward for gfx950 (bf16 inputs).
//
// The forward kept only O and LSE = m + ln l per row (FlashAttention
// deep-reading report, zako-mio, sections 2.5 and 3.3: no N x N matrix is
// stored; S and P are rebuilt on chip from Q, K and the row statistic).
// Three kernels, in stream order:
//
//   bwd_pre   D_i = dO_i . O_i                       (memory-bound row dots)
//   bwd_dkdv  one workgroup per 128 keys of one K/V head, 32 keys per wave;
//             for every query head of the group and every visited block of
//             query rows:  S = Q K^T,  P = 2^(S scale log2e - LSE log2e),
//             dP = dO V^T,  dS = P (dP - D),
//             dV^T += dO^T P,  dK^T += Q^T dS        (fp32 in registers)
//   bwd_dq    one workgroup per 128 query rows, 32 rows per wave; for every
//             visited K/V tile: S^T = K Q^T, dP^T = V dO^T, dS^T as above,
//             dQ^T += K^T dS^T
//
// D_i = sum_j P_ij dP_ij equals dO_i . O_i because O_i = sum_j P_ij V_j;
// computing it from the stored O costs one pass over O and dO instead of a
// second reduction per tile. All gradients stay in fp32 registers for the
// whole key (or query) block and are written once; there are no atomics.
#include "fa_stage.h"

namespace fa {

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// ----------------------------------------------------------------- D = rowsum(dO * O)

template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdArgs a) {
  constexpr int TPR = D / 8;  // lanes per row, 8 elements each
  constexpr int RPB = 256 / TPR;
  const Problem& p = a.p;
  const int64_t rows = (int64_t)p.B * p.Hq * p.N;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  float acc = 0.f;
  if (row < rows) {
    const int64_t i = row % p.N;
    const int64_t bh = row / p.N;
    const int64_t h = bh % p.Hq, b = bh / p.Hq;
    Chunk g;
    g.v = *reinterpret_cast<const uint4*>(static_cast<const bf16*>(a.dout) + b * a.sdo.b +
                                          h * a.sdo.h + i * a.sdo.n + part * 8);
    if (a.o_fp32) {
      const float* op = static_cast<const float*>(a.o) + b * a.so.b + h * a.so.h + i * a.so.n + part * 8;
      const float4 o0 = *reinterpret_cast<const float4*>(op);
      const float4 o1 = *reinterpret_cast<const float4*>(op + 4);
      acc = bf16_lo(g.d[0]) * o0.x + bf16_hi(g.d[0]) * o0.y + bf16_lo(g.d[1]) * o0.z +
            bf16_hi(g.d[1]) * o0.w + bf16_lo(g.d[2]) * o1.x + bf16_hi(g.d[2]) * o1.y +
            bf16_lo(g.d[3]) * o1.z + bf16_hi(g.d[3]) * o1.w;
    } else {
      Chunk o;
      o.v = *reinterpret_cast<const uint4*>(static_cast<const bf16*>(a.o) + b * a.so.b +
                                            h * a.so.h + i * a.so.n + part * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc += bf16_lo(g.d[e]) * bf16_lo(o.d[e]) + bf16_hi(g.d[e]) * bf16_hi(o.d[e]);
    }
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (part == 0 && row < rows) a.dvec[row] = acc;
}

// LSE in base-2 units; an empty row (LSE = -inf) becomes +inf so that every
// rebuilt probability of that row is 2^-inf = 0.
__device__ __forceinline__ float lse2_of(float lse) {
  return lse == -kInf ? kInf : lse * kLog2e;
}

// ----------------------------------------------------------------- dK, dV

template <int D>
struct DkdvCfg {
  static constexpr int BK = 128;       // keys per workgroup (4 waves x 32)
  static constexpr int BQ = 8192 / D;  // query rows staged per step
  static constexpr int NQS = BQ / 32;
  static constexpr int NKK = D / 16;
  static constexpr int NDB = D / 32;
  using G = TileGeom<D, BQ>;
};

template <int D>
__global__ __launch_bounds__(256, D == 64 ? 2 : 1) void bwd_dkdv_kernel(BwdArgs a) {
  using C = DkdvCfg<D>;
  using G = typename C::G;
  __shared__ __attribute__((aligned(16))) bf16 Qs[C::BQ * G::RPITCH];
  __shared__ __attribute__((aligned(16))) bf16 dOs[C::BQ * G::RPITCH];
  __shared__ __attribute__((aligned(16))) bf16 Qt[D * G::TPITCH];
  __shared__ __attribute__((aligned(16))) bf16 dOt[D * G::TPITCH];
  __shared__ __attribute__((aligned(16))) float lse_s[C::BQ];
  __shared__ __attribute__((aligned(16))) float dvec_s[C::BQ];

  const Problem& p = a.p;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 31, hh = lane >> 5;
  const int nkb = (p.N + C::BK - 1) / C::BK;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int head_lin = L / nkb;
  const int kb = L - head_lin * nkb;  // causal: low key blocks carry the most rows
  const int b = head_lin / p.Hkv, hk = head_lin - b * p.Hkv;
  const int k0 = kb * C::BK;
  const int my_k = k0 + 32 * w + lr;
  const float sl2 = p.scale_l2;

  const bf16* Kp = static_cast<const bf16*>(a.k) + b * a.sk.b + hk * a.sk.h;
  const bf16* Vp = static_cast<const bf16*>(a.v) + b * a.sv.b + hk * a.sv.h;

  // This lane's key as the B operand of S = Q K^T and dP = dO V^T.
  bf16x8 kf[C::NKK], vf[C::NKK];
  {
    const bool ok = my_k < p.N;
    const int64_t r = ok ? my_k : 0;
#pragma unroll
    for (int kk = 0; kk < C::NKK; ++kk) {
      kf[kk] = frag_g(Kp + r * a.sk.n + 16 * kk + 8 * hh, ok);
      vf[kk] = frag_g(Vp + r * a.sv.n + 16 * kk + 8 * hh, ok);
    }
  }

  f32x16 dkt[C::NDB], dvt[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) {
    dkt[db] = f32x16{};
    dvt[db] = f32x16{};
  }

  const int kvalid = valid_keys(p.seqlens, b, p.N);
  if (k0 < kvalid) {  // else every key of the block is masked: dK = dV = 0
    // Steps run over (query head of the group) x (query block); rows above
    // the diagonal see none of these keys under the causal mask.
    const int qfirst = p.causal ? k0 / C::BQ : 0;
    const int nq = (p.N + C::BQ - 1) / C::BQ - qfirst;
    const int nsteps = p.G * nq;
    auto next_step = [&](int st) {
      while (st < nsteps && !block_on(p.bm, p.bm_ld, (qfirst + st % nq) * C::BQ, k0)) ++st;
      return st;
    };
    const int arow = swap_bits23(lr) * G::RPITCH + 8 * hh;
    int trow[C::NDB], tsw[C::NDB];
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      trow[db] = (32 * db + lr) * G::TPITCH;
      tsw[db] = tswz<C::BQ>(32 * db + lr);
    }

    ColRegs<D, C::BQ> qreg, doreg;
    float lse_r = 0.f, dvec_r = 0.f;
    auto fetch = [&](int st) {
      const int h = hk * p.G + st / nq;
      const int q0b = (qfirst + st % nq) * C::BQ;
      load_cols<D, C::BQ>(qreg, static_cast<const bf16*>(a.q) + b * a.sq.b + h * a.sq.h, a.sq.n,
                          q0b, p.N, tid);
      load_cols<D, C::BQ>(doreg, static_cast<const bf16*>(a.dout) + b * a.sdo.b + h * a.sdo.h,
                          a.sdo.n, q0b, p.N, tid);
      if (tid < C::BQ) {
        const int qi = q0b + tid;
        const int64_t off = ((int64_t)b * p.Hq + h) * p.N + qi;
        lse_r = qi < p.N ? lse2_of(a.lse[off]) : kInf;
        dvec_r = qi < p.N ? a.dvec[off] : 0.f;
      }
    };
    auto stage = [&]() {
      store_rows_t<D, C::BQ>(qreg, Qs, tid);
      store_cols<D, C::BQ>(qreg, Qt, tid);
      store_rows_t<D, C::BQ>(doreg, dOs, tid);
      store_cols<D, C::BQ>(doreg, dOt, tid);
      if (tid < C::BQ) {
        lse_s[tid] = lse_r;
        dvec_s[tid] = dvec_r;
      }
    };

    int st = next_step(0);
    if (st < nsteps) {
      fetch(st);
      stage();
      __syncthreads();
    }
    while (st < nsteps) {
      const int h = hk * p.G + st / nq;
      const int q0b = (qfirst + st % nq) * C::BQ;
      const int nx = next_step(st + 1);
      if (nx < nsteps) fetch(nx);  // in flight during this step
      if (a.log_kv && tid == 0)
        log_tile(a.log_kv, (((int64_t)b * p.Hq + h) * p.nlb + (q0b >> 7)) * p.logw, k0);
      const bool need_mask = (p.causal && k0 + C::BK - 1 > q0b) || (k0 + C::BK > kvalid);

#pragma unroll
      for (int u = 0; u < C::NQS; ++u) {
        // Skip query sub-tiles that lie entirely above this wave's keys.
        if (p.causal && q0b + 32 * u + 31 < k0 + 32 * w) continue;
        f32x16 s = f32x16{}, dp = f32x16{};
        const int ao = 32 * u * G::RPITCH + arow;
#pragma unroll
        for (int kk = 0; kk < C::NKK; ++kk) {
          s = mfma(frag<bf16>(Qs + ao + 16 * kk), kf[kk], s);
          dp = mfma(frag<bf16>(dOs + ao + 16 * kk), vf[kk], dp);
        }
        // Register r holds query row 32u + perm_row(r, hh) of this step.
        const f32x4* l4 = reinterpret_cast<const f32x4*>(lse_s + 32 * u + 8 * hh);
        const f32x4* d4 = reinterpret_cast<const f32x4*>(dvec_s + 32 * u + 8 * hh);
        f32x4 lv[4] = {l4[0], l4[1], l4[4], l4[5]};
        f32x4 dv4[4] = {d4[0], d4[1], d4[4], d4[5]};
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float pv = __builtin_amdgcn_exp2f(fmaf(s[r], sl2, -lv[r >> 2][r & 3]));
          if (need_mask) {
            const int qi = q0b + 32 * u + perm_row(r, hh);
            if ((p.causal && my_k > qi) || my_k >= kvalid) pv = 0.f;
          }
          s[r] = pv;
          dp[r] = pv * (dp[r] - dv4[r >> 2][r & 3]);
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const bf16x8 pf = pack8(s, c);
          const bf16x8 dsf = pack8(dp, c);
          const int kc = 4 * u + 2 * c + hh;
#pragma unroll
          for (int db = 0; db < C::NDB; ++db) {
            const int to = trow[db] + 8 * (kc ^ tsw[db]);
            dvt[db] = mfma(frag<bf16>(dOt + to), pf, dvt[db]);
            dkt[db] = mfma(frag<bf16>(Qt + to), dsf, dkt[db]);
          }
        }
      }
      if (nx < nsteps) {
        __syncthreads();
        stage();
        __syncthreads();
      }
      st = nx;
    }
  }

  if (my_k < p.N) {
    bf16* dkp = static_cast<bf16*>(a.dk) + b * a.sdk.b + hk * a.sdk.h + (int64_t)my_k * a.sdk.n;
    bf16* dvp = static_cast<bf16*>(a.dv) + b * a.sdv.b + hk * a.sdv.h + (int64_t)my_k * a.sdv.n;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * hh;
        bf16x4 kq, vq;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kq[e] = (bf16)(dkt[db][4 * g + e] * p.scale);
          vq[e] = (bf16)dvt[db][4 * g + e];
        }
        *reinterpret_cast<bf16x4*>(dkp + d0) = kq;
        *reinterpret_cast<bf16x4*>(dvp + d0) = vq;
      }
  }
}

// ----------------------------------------------------------------- dQ

template <int D>
struct DqCfg {
  static constexpr int BR = 128;       // query rows per workgroup
  static constexpr int BC = 8192 / D;  // keys per tile (128 or 64)
  static constexpr int NSUB = BC / 32;
  static constexpr int NKK = D / 16;
  static constexpr int NDB = D / 32;
  using G = TileGeom<D, BC>;
};

template <int D>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(BwdArgs a) {
  using C = DqCfg<D>;
  using G = typename C::G;
  __shared__ __attribute__((aligned(16))) bf16 Ks[C::BC * G::RPITCH];
  __shared__ __attribute__((aligned(16))) bf16 Vs[C::BC * G::RPITCH];
  __shared__ __attribute__((aligned(16))) bf16 Kt[D * G::TPITCH];

  const Problem& p = a.p;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 31, hh = lane >> 5;
  const int nqb = (p.N + C::BR - 1) / C::BR;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int head_lin = L / nqb;
  const int qbi = L - head_lin * nqb;
  const int qb = p.causal ? nqb - 1 - qbi : qbi;
  const int b = head_lin / p.Hq, h = head_lin - b * p.Hq, hk = h / p.G;
  const int q0 = qb * C::BR;
  const int my_q = q0 + 32 * w + lr;
  const float sl2 = p.scale_l2;

  const bf16* Kp = static_cast<const bf16*>(a.k) + b * a.sk.b + hk * a.sk.h;
  const bf16* Vp = static_cast<const bf16*>(a.v) + b * a.sv.b + hk * a.sv.h;

  const bool qok = my_q < p.N;
  bf16x8 qf[C::NKK], dof[C::NKK];
  {
    const int64_t r = qok ? my_q : 0;
    const bf16* Qp = static_cast<const bf16*>(a.q) + b * a.sq.b + h * a.sq.h + r * a.sq.n + 8 * hh;
    const bf16* dOp = static_cast<const bf16*>(a.dout) + b * a.sdo.b + h * a.sdo.h + r * a.sdo.n + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < C::NKK; ++kk) {
      qf[kk] = frag_g(Qp + 16 * kk, qok);
      dof[kk] = frag_g(dOp + 16 * kk, qok);
    }
  }
  const int64_t rowstat = ((int64_t)b * p.Hq + h) * p.N + (qok ? my_q : 0);
  const float lse2 = qok ? lse2_of(a.lse[rowstat]) : kInf;
  const float dq_d = qok ? a.dvec[rowstat] : 0.f;

  f32x16 acc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) acc[db] = f32x16{};

  const int kvalid = valid_keys(p.seqlens, b, p.N);
  const int kend = p.causal ? min(kvalid, q0 + C::BR) : kvalid;
  const int ntiles = (kend + C::BC - 1) / C::BC;
  const int64_t log_row =
      a.log_q ? (((int64_t)b * p.Hq + h) * p.nlb + (q0 >> 7)) * p.logw : 0;
  auto next_visit = [&](int kt) {
    while (kt < ntiles && !block_on(p.bm, p.bm_ld, q0, kt * C::BC)) ++kt;
    return kt;
  };
  const int arow = swap_bits23(lr) * G::RPITCH + 8 * hh;
  int trow[C::NDB], tsw[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) {
    trow[db] = (32 * db + lr) * G::TPITCH;
    tsw[db] = tswz<C::BC>(32 * db + lr);
  }

  ColRegs<D, C::BC> kreg, vreg;
  auto stage = [&]() {
    store_rows_t<D, C::BC>(kreg, Ks, tid);
    store_cols<D, C::BC>(kreg, Kt, tid);
    store_rows_t<D, C::BC>(vreg, Vs, tid);
  };
  int kt = next_visit(0);
  if (kt < ntiles) {
    load_cols<D, C::BC>(kreg, Kp, a.sk.n, kt * C::BC, p.N, tid);
    load_cols<D, C::BC>(vreg, Vp, a.sv.n, kt * C::BC, p.N, tid);
    stage();
    __syncthreads();
  }
  while (kt < ntiles) {
    const int key0 = kt * C::BC;
    const int nxt = next_visit(kt + 1);
    if (nxt < ntiles) {
      load_cols<D, C::BC>(kreg, Kp, a.sk.n, nxt * C::BC, p.N, tid);
      load_cols<D, C::BC>(vreg, Vp, a.sv.n, nxt * C::BC, p.N, tid);
    }
    if (a.log_q && tid == 0) log_tile(a.log_q, log_row, key0);
    const bool need_mask = (p.causal && key0 + C::BC - 1 > q0) || (key0 + C::BC > kvalid);
#pragma unroll
    for (int t = 0; t < C::NSUB; ++t) {
      const int sk0 = key0 + 32 * t;
      if ((p.causal && sk0 > q0 + 32 * w + 31) || sk0 >= kvalid) continue;
      f32x16 st = f32x16{}, dpt = f32x16{};
      const int ao = 32 * t * G::RPITCH + arow;
#pragma unroll
      for (int kk = 0; kk < C::NKK; ++kk) {
        st = mfma(frag<bf16>(Ks + ao + 16 * kk), qf[kk], st);
        dpt = mfma(frag<bf16>(Vs + ao + 16 * kk), dof[kk], dpt);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pv = __builtin_amdgcn_exp2f(fmaf(st[r], sl2, -lse2));
        if (need_mask) {
          const int key = key0 + 32 * t + perm_row(r, hh);
          if ((p.causal && key > my_q) || key >= kvalid) pv = 0.f;
        }
        dpt[r] = pv * (dpt[r] - dq_d);
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const bf16x8 dsf = pack8(dpt, c);
        const int kc = 4 * t + 2 * c + hh;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
          acc[db] = mfma(frag<bf16>(Kt + trow[db] + 8 * (kc ^ tsw[db])), dsf, acc[db]);
      }
    }
    if (nxt < ntiles) {
      __syncthreads();
      stage();
      __syncthreads();
    }
    kt = nxt;
  }

  if (qok) {
    bf16* dqp = static_cast<bf16*>(a.dq) + b * a.sdq.b + h * a.sdq.h + (int64_t)my_q * a.sdq.n;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (bf16)(acc[db][4 * g + e] * p.scale);
        *reinterpret_cast<bf16x4*>(dqp + 32 * db + 8 * g + 4 * hh) = v;
      }
  }
}

// ----------------------------------------------------------------- launchers

hipError_t launch_bwd_pre(const BwdArgs& a, int head_dim, hipStream_t s) {
  const int64_t rows = (int64_t)a.p.B * a.p.Hq * a.p.N;
  const int rpb = 256 / (head_dim / 8);
  const int64_t grid = (rows + rpb - 1) / rpb;
  if (head_dim == 64)
    hipLaunchKernelGGL(bwd_pre_kernel<64>, dim3((unsigned)grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(bwd_pre_kernel<128>, dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const BwdArgs& a, int head_dim, hipStream_t s) {
  const int64_t grid = (int64_t)((a.p.N + 127) / 128) * a.p.Hkv * a.p.B;
  if (head_dim == 64)
    hipLaunchKernelGGL(bwd_dkdv_kernel<64>, dim3((unsigned)grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(bwd_dkdv_kernel<128>, dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const BwdArgs& a, int head_dim, hipStream_t s) {
  const int64_t grid = (int64_t)((a.p.N + 127) / 128) * a.p.Hq * a.p.B;
  if (head_dim == 64)
    hipLaunchKernelGGL(bwd_dq_kernel<64>, dim3((unsigned)grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(bwd_dq_kernel<128>, dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace fa

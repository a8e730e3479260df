// fa_bwd.hip -- recomputation backward for gfx950 (bf16 inputs).
//
// The forward kept only O and LSE = m + ln l per row (FlashAttention
// deep-reading report, zako-mio, sections 2.5 and 3.3: no N x N matrix is
// stored; S and P are rebuilt on chip from Q, K and the row statistic).
// Two kernels, in stream order:
//
//   bwd_dq    one workgroup per 128 query rows, 32 rows per wave; first the
//             row statistics D_i = dO_i . O_i and LSE_i log2e of its rows
//             (stored for the next kernel), then for every visited K/V
//             tile: S^T = K Q^T, dP^T = V dO^T, dS^T = P (dP - D),
//             dQ^T += K^T dS^T                      (fp32 in registers)
//   bwd_dkdv  one workgroup per 128 keys of one K/V head, 32 keys per wave;
//             for every query head of the group and every visited block of
//             query rows:  S = Q K^T,  P = 2^(S scale log2e - LSE log2e),
//             dP = dO V^T,  dS = P (dP - D),
//             dV^T += dO^T P,  dK^T += Q^T dS        (fp32 in registers)
//
// D_i = sum_j P_ij dP_ij equals dO_i . O_i because O_i = sum_j P_ij V_j;
// computing it from the stored O costs one read of O instead of a second
// reduction per tile, and the dQ kernel, which already holds the row's dO,
// does it in its prologue. All gradients stay in fp32 registers for the
// whole key (or query) block and are written once; there are no atomics.
#include "fa_philox.h"
#include "fa_stage.h"

namespace fa {

// ----------------------------------------------------------------- row statistics

// LSE in base-2 units; an empty row (LSE = -inf) becomes +inf so that every
// rebuilt probability of that row is 2^-inf = 0.
__device__ __forceinline__ float lse2_of(float lse) {
  return lse == -kInf ? kInf : lse * kLog2e;
}

// A row value as the starting accumulator of a product chain. The output
// of a 32 x 32 product keeps 16 rows per lane, so subtracting a per-row
// value there would need those 16 values in every lane (eight 16-byte LDS
// reads per sub-tile for LSE and D). Instead one extra product broadcasts
// it: lane i of the A operand holds its row's value c split exactly into
// three bf16 terms (two truncations, then the rounded rest: c to within
// 2^-23 |c|) in K slots 0..2, and a constant B operand with -1 in those
// slots makes every output of row i equal to -c. Lane half 0 carries one
// value (row LSE) and lane half 1 another (row D), which the two B
// constants select: K slots 0..2 are lane half 0's, slots 8..10 half 1's.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
struct f32x4x4 {
  f32x4 v[4];
};

__device__ __forceinline__ bf16x8 split3_frag(float c) {
  const uint32_t hi = __float_as_uint(c) & 0xffff0000u;
  const float r1 = c - __uint_as_float(hi);
  const uint32_t mid = __float_as_uint(r1) & 0xffff0000u;
  const float lo = r1 - __uint_as_float(mid);
  u32x4 w;
  w[0] = (hi >> 16) | mid;
  w[1] = (uint32_t)__builtin_bit_cast(uint16_t, (bf16)lo);
  w[2] = 0u;
  w[3] = 0u;
  return __builtin_bit_cast(bf16x8, w);
}

// -1 in K slots 0..2 of lane half `half`, zero elsewhere.
__device__ __forceinline__ bf16x8 neg_ones_frag(int hh, int half) {
  u32x4 w;
  w[0] = hh == half ? 0xBF80BF80u : 0u;
  w[1] = hh == half ? 0x0000BF80u : 0u;
  w[2] = 0u;
  w[3] = 0u;
  return __builtin_bit_cast(bf16x8, w);
}

// ----------------------------------------------------------------- dK, dV

template <int D>
struct DkdvCfg {
  static constexpr int BK = 128;  // keys per workgroup (4 waves x 32)
  // At d=128 the dK and dV accumulators alone take 128 registers; the
  // kernel keeps two waves per SIMD by staging 32 query rows per step (one
  // sub-tile at a time) and reading V's operand fragments from an LDS copy of
  // the workgroup's V block instead of holding them in registers.
  static constexpr bool VLDS = D == 128;
  static constexpr int BQ = D == 64 ? 128 : 32;  // query rows staged per step
  static constexpr int NQS = BQ / 32;
  static constexpr int NG = D == 64 ? 2 : 1;     // sub-tiles per straight-line group
  static constexpr int FB = D == 64 ? 4 : 2;     // operand fragments fetched per batch
  static constexpr int NKK = D / 16;
  static constexpr int NDB = D / 32;
  // Row statistics enter as chain starts (one product per chain) instead of
  // per-register LDS reads: at d=64, 31 fewer LDS reads per step against 8
  // more products; at d=128 (one sub-tile per step) the saving is 7 reads
  // and the extra registers would spill.
  static constexpr bool FOLD = D == 64;
  using T = SwzTile<D, BQ>;
  using VT = SwzTile<D, BK>;
  // One stage: Q tile | dO tile | log2-domain LSE of its rows | D of its
  // rows. The row statistics arrive by dword DMA, 64 rows per wave load.
  static constexpr int NRC = (BQ + 63) / 64;  // 64-row loads per statistic
  static constexpr int LSE_OFF = 2 * T::BYTES;
  static constexpr int DVEC_OFF = LSE_OFF + 256 * NRC;
  static constexpr int STAGE = DVEC_OFF + 256 * NRC;
  // LDS: two stages, then (VLDS) the V block of the workgroup's keys.
  static constexpr int VOFF = 2 * STAGE;
  static constexpr int LDS_BYTES = VOFF + (VLDS ? VT::BYTES : 0);
  static_assert(STAGE % 256 == 0, "stages keep the 256-byte bank period");
};

// MASK: the general variant, with the block-mask scan and (d=128) the
// per-wave band skip compiled in, for launches with a block mask, a sliding
// window or dropout (dropout launches allocate registers better with it: the
// d=64 pair does not spill, against 2 spills without). Launches with none of
// them use the lean variant, which keeps its register allocation.
template <int D, bool DROP, int NREP, bool MASK>
__global__ __launch_bounds__(256, 2) void bwd_dkdv_kernel(BwdArgs a) {
  using C = DkdvCfg<D>;
  using T = typename C::T;
  // Two stages of (Q tile | dO tile | row statistics), filled while the
  // other is read, and at d=128 the V block. One LDS object: every access
  // goes through a restrict-qualified pointer into it, so alias information
  // can separate the stage being read from the one being filled.
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];

  const Problem& p = a.p;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, hh = lane >> 5;
  const int nkb = (p.N + C::BK - 1) / C::BK;
  // Causal (NREP = 2): a workgroup takes key block i and then block
  // nkb - 1 - i, so that every workgroup sees about the same number of
  // query rows (the heaviest block first). NREP = 1: one block, in order of
  // decreasing work under the causal mask (low key blocks carry the most
  // rows).
  static_assert(NREP == 1 || NREP == 2, "one block or a pair");
  const int nunit = NREP == 2 ? (nkb + 1) / 2 : nkb;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int head_lin = L / nunit;
  const int ui = L - head_lin * nunit;
  const int b = head_lin / p.Hkv, hk = head_lin - b * p.Hkv;
  for (int rep = 0; rep < NREP; ++rep) {
    const int kb = rep == 0 ? ui : nkb - 1 - ui;
    if (rep == 1) {
      if (kb == ui) break;  // the middle block of an odd count
      __syncthreads();  // the first block's last step and V block are no longer read
    }
    const int k0 = kb * C::BK;
    const int my_k = k0 + 32 * w + lr;
    const float sl2 = p.scale_l2;
    const bool causal = p.causal != 0;

    const bf16* Kp = static_cast<const bf16*>(a.k) + b * a.sk.b + hk * a.sk.h;
    const bf16* Vp = static_cast<const bf16*>(a.v) + b * a.sv.b + hk * a.sv.h;

    // This lane's key as the B operand of S = Q K^T and dP = dO V^T (V from
    // LDS at d=128). Keys past the valid length are zero, whatever their
    // memory holds: their P is 0, and their dK and dV come out 0.
    const int kvalid = __builtin_amdgcn_readfirstlane(valid_keys(p.seqlens, b, p.N));
    bf16x8 kf[C::NKK], vf[C::VLDS ? 1 : C::NKK];
    {
      const bool ok = my_k < kvalid;
      const int64_t r = ok ? my_k : 0;
  #pragma unroll
      for (int kk = 0; kk < C::NKK; ++kk) {
        kf[kk] = frag_g(Kp + r * a.sk.n + 16 * kk + 8 * hh, ok);
        if constexpr (!C::VLDS) vf[kk] = frag_g(Vp + r * a.sv.n + 16 * kk + 8 * hh, ok);
      }
    }

    f32x16 dkt[C::NDB], dvt[C::NDB];
  #pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      dkt[db] = f32x16{};
      dvt[db] = f32x16{};
    }

    if (k0 < kvalid) {  // else every key of the block is masked: dK = dV = 0
      // Steps run over (query head of the group) x (query block), limited to
      // the rows that can see a key of this block: from the causal diagonal or
      // the right window edge, up to the left window edge.
      const int qfirst = max(p.causal ? k0 : 0, k0 - p.wr) / C::BQ;
      const int qend = min(p.N, k0 + C::BK + p.wl);
      const int nq = max(0, (qend + C::BQ - 1) / C::BQ - qfirst);
      const int nsteps = p.G * nq;
      // Steps whose rows meet a present block of this key block's mask
      // column; the column is the same for every query head of the group.
      MaskLine mcol(MASK ? p.bm + (k0 >> 7) : nullptr, p.bm_ld, p.nlb);
      auto next_step = [&](int st) {
        if (MASK && p.bm != nullptr) {
          while (st < nsteps) {
            const int g = st / nq, j = st - g * nq;
            const int j2 = mcol.next_tile<C::BQ>(qfirst + j, qfirst + nq) - qfirst;
            if (j2 < nq) return g * nq + j2;
            st = (g + 1) * nq;  // none left in this head's rows: the next head
          }
          return nsteps;
        } else {
          return st;
        }
      };
      // Step sidx -> (query head, first row). Without a mask: query blocks
      // from the last one down, heads of the group innermost, so that the
      // workgroups of one key/value head start on the same Q and dO tiles
      // and share them through L2. With a mask: heads outer, blocks upward
      // (the order of the mask scan).
      auto step_unit = [&](int sidx, int& h, int& q0b) {
        if (MASK && p.bm != nullptr) {
          h = hk * p.G + sidx / nq;
          q0b = (qfirst + sidx % nq) * C::BQ;
        } else {
          const int jd = p.G == 1 ? sidx : sidx / p.G;
          h = hk * p.G + (sidx - jd * p.G);
          q0b = (qfirst + nq - 1 - jd) * C::BQ;
        }
      };
      const int qsb = 2 * (int)a.sq.n, dsb = 2 * (int)a.sdo.n;
      int qvo[T::NLD], dvo[T::NLD];
      if constexpr (!C::VLDS) {
        dma_offsets<D, C::BQ>(qvo, qsb, w, lane);
        dma_offsets<D, C::BQ>(dvo, dsb, w, lane);
      }
      static_assert(2 * C::NRC <= 4, "one wave per 64-row statistics load");
      int roff_k[C::VLDS ? 1 : C::NKK], troff[C::NDB][2];
      if constexpr (C::VLDS) {
        // Only step 0's row offset stays live; the others are rebuilt per
        // step (chunk 2 kk + hh of a swizzled row = step 0's offset XOR 32 kk).
        roff_k[0] = T::off(swap_bits23(lr), hh);
      } else {
        row_offsets<D, C::BQ>(roff_k, lr, hh);
      }
      tr_offsets<D, C::BQ>(troff, lane);

      // Q and dO tiles of a step and the LSE / D values of its rows all arrive
      // by DMA into the stage; rows past the sequence read as zero, and with
      // their Q and dO rows zero they add nothing to dK or dV.
      auto issue = [&](int sidx, char* stage) {
        int h, q0b;
        step_unit(sidx, h, q0b);
        const Rsrc qrs = make_rsrc(static_cast<const bf16*>(a.q) + b * a.sq.b + h * a.sq.h,
                                   rows_extent(p.N, qsb, 2 * D));
        const Rsrc drs = make_rsrc(static_cast<const bf16*>(a.dout) + b * a.sdo.b + h * a.sdo.h,
                                   rows_extent(p.N, dsb, 2 * D));
        // Registers are at their limit with the V block in LDS: rebuild the
        // DMA offsets for this step from a lane index read afresh (an opaque
        // mbcnt, so neither it nor the offsets are hoisted out of the loop and
        // kept live, and nothing is reloaded from scratch, which would wait on
        // the DMA just issued).
        const int ln = C::VLDS ? fresh_lane_id() : lane;
        if constexpr (C::VLDS) {
          dma_offsets<D, C::BQ>(qvo, qsb, w, ln);
          dma_offsets<D, C::BQ>(dvo, dsb, w, ln);
        }
        dma_tile<D, C::BQ>(qrs, qvo, (uint32_t)q0b * qsb, stage, w);
        dma_tile<D, C::BQ>(drs, dvo, (uint32_t)q0b * dsb, stage + T::BYTES, w);
        if (w < 2 * C::NRC) {  // wave-uniform: one 64-row load of LSE or D
          const int64_t row0 = ((int64_t)b * p.Hq + h) * p.N;
          const bool is_d = w >= C::NRC;
          const int c = is_d ? w - C::NRC : w;
          const Rsrc rs = make_rsrc((is_d ? a.dvec : a.lse2) + row0, (uint32_t)p.N * 4);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rs, (FA_LDS void*)(stage + (is_d ? C::DVEC_OFF : C::LSE_OFF) + 256 * c), 4, 4 * ln,
              (uint32_t)(q0b + 64 * c) * 4, 0, 0);
        }
      };

      const int vb0 = C::VT::off(32 * w + lr, hh);
      if constexpr (C::VLDS) {
        using VT = typename C::VT;
        static_assert((VT::RB & (VT::RB - 1)) == 0 && VT::CPR * 16 == VT::RB,
                      "chunk field below a power-of-two row pitch");
        int vvo[VT::NLD];
        const int vsb = 2 * (int)a.sv.n;
        dma_offsets<D, C::BK>(vvo, vsb, w, lane);
        const Rsrc vrs = make_rsrc(Vp, rows_extent(kvalid, vsb, 2 * D));
        dma_tile<D, C::BK>(vrs, vvo, (uint32_t)k0 * vsb, smem + C::VOFF, w);
      }

      int sidx = next_step(0);
      if (sidx < nsteps) issue(sidx, smem);
      wait_dma();  // the V block (if staged) and the first step
      __syncthreads();
      // One step reading stage `Qs` while the next lands in `fill`
      // (restrict-qualified: these reads never wait for that DMA).
      auto step = [&](const char* __restrict__ Qs, char* __restrict__ fill,
                      const char* __restrict__ Vb) {
        const char* dOs = Qs + T::BYTES;
        int h, q0b;
        step_unit(sidx, h, q0b);
        // B-operand offsets of this lane's key row in the V block. The chunk
        // field of a swizzled offset lies below the row pitch, so head-dim
        // step kk (chunk 2 kk + hh) is step 0's offset XOR 32 kk; rebuilt each
        // step from one live register (all eight kept live across the loop
        // would push a row offset out to scratch).
        int vboff[C::VLDS ? C::NKK : 1], roff[C::NKK];
        if constexpr (C::VLDS) {
          int v0 = vb0, r0 = roff_k[0];
          asm volatile("" : "+v"(v0), "+v"(r0));
  #pragma unroll
          for (int kk = 0; kk < C::NKK; ++kk) {
            vboff[kk] = v0 ^ (32 * kk);
            roff[kk] = r0 ^ (32 * kk);
          }
        } else {
  #pragma unroll
          for (int kk = 0; kk < C::NKK; ++kk) roff[kk] = roff_k[kk];
        }
        const int nx = next_step(sidx + 1);
        if (nx < nsteps) {  // lands during this step
          paranoid_before_fill();
          issue(nx, fill);
          paranoid_after_fill();
        }
        // Dropout keep bits of this lane's key for every row of the step, made
        // before the score products so that the generator's temporaries never
        // share the registers with the S and dP accumulators (the empty asm
        // with a memory clobber keeps the block ahead of the LDS reads). The 8
        // lanes that share a key group (lane % 8 = key % 8) each run the
        // generator for two rows of a sub-tile (perm_row(e, hh) and
        // perm_row(8 + e, hh), e = lane % 8); a bit transpose across those
        // lanes hands every lane bit r = row perm_row(r, hh).
        uint32_t dbits[DROP ? C::NQS : 1];
        if constexpr (DROP) {
          const int ln = fresh_lane_id();
          const int e = ln & 7, hl = ln >> 5;
          const uint32_t kg = (uint32_t)(k0 + 32 * w + (ln & 24)) >> 3;
          const uint32_t bh = (uint32_t)(b * p.Hq + h);
  #pragma unroll
          for (int u = 0; u < C::NQS; ++u) {
            const uint32_t row0 = (uint32_t)(q0b + 32 * u + 8 * hl + e);
            const uint32_t lo = drop_byte(drop_bits(p, kg, row0, bh), p.drop_thr);
            const uint32_t hi = drop_byte(drop_bits(p, kg, row0 + 16, bh), p.drop_thr);
            dbits[u] = transpose8x8x2(lo | (hi << 8));
            asm volatile("" : "+v"(dbits[u]) : : "memory");
          }
        }
        if (a.log_kv && tid == 0)
          log_tile(a.log_kv, (((int64_t)b * p.Hq + h) * p.nlb + (q0b >> 7)) * p.logw, k0);
        const bool need_mask = (p.causal && k0 + C::BK - 1 > q0b) || (k0 + C::BK > kvalid) ||
                               (q0b + C::BQ - 1 > k0 + p.wl) || (q0b < k0 + C::BK - 1 - p.wr);

        // Straight-line step (no per-sub-tile branches): all S and dP products,
        // one uniform mask block, then P / dS and the dV, dK products, so the
        // compiler can overlap one sub-tile's exponentials with another's
        // matrix products.
        // FOLD: row statistics as chain starts. Lane half 0 reads LSE log2e /
        // (scale log2e) of its A-operand row (clamped: an empty row's +inf
        // becomes a finite value whose probabilities still underflow to 0),
        // half 1 the row's D. S then starts at -LSE / scale and dP at -D
        // (without dropout; with it dP starts at 0 and D is applied per
        // element). Otherwise the 16 per-register values are read from LDS.
        const float* stat_row = reinterpret_cast<const float*>(
                                    Qs + ((lane >> 5) ? C::DVEC_OFF : C::LSE_OFF)) +
                                swap_bits23(lr);
        const float stat_mul = hh ? 1.f : 1.f / sl2;
        auto row_stats = [&](int off, int u) {  // the 16 values of sub-tile u
          const f32x4* v4 = reinterpret_cast<const f32x4*>(Qs + off) + 8 * u + 2 * hh;
          return f32x4x4{v4[0], v4[1], v4[4], v4[5]};
        };
  #pragma unroll
        for (int g0 = 0; g0 < C::NQS; g0 += C::NG) {
          // d=128: when no row of the step sees any of this wave's 32 keys
          // (rows above the keys under the causal mask, or outside the band),
          // the wave's P is exactly 0 and the step adds nothing to dK or dV;
          // it is skipped (causal: 6 of the 16 wave-steps of the diagonal
          // block). Causal pairs test the diagonal, one-block launches of the
          // general variant without dropout the band; d=64, whose paired
          // dropout kernel would spill with it, has no test.
          if (D == 128 &&
              (NREP == 2 ? q0b + 32 * (g0 + C::NG) - 1 < k0 + 32 * w
                         : MASK && !DROP &&
                               (q0b + 32 * (g0 + C::NG) - 1 + (causal ? 0 : p.wr) < k0 + 32 * w ||
                                q0b + 32 * g0 - p.wl > k0 + 32 * w + 31)))
            continue;
          f32x16 s[C::NG], dp[C::NG];
  #pragma unroll
          for (int uu = 0; uu < C::NG; ++uu) {
            if constexpr (C::FOLD) {
              const bf16x8 cf = split3_frag(fminf(stat_row[32 * (g0 + uu)] * stat_mul, 1e30f));
              s[uu] = mfma(cf, neg_ones_frag(hh, 0), f32x16{});
              dp[uu] = DROP ? f32x16{} : mfma(cf, neg_ones_frag(hh, 1), f32x16{});
            } else {
              s[uu] = f32x16{};
              dp[uu] = f32x16{};
            }
            const char* qp = Qs + 32 * (g0 + uu) * T::RB;
            const char* dop = dOs + 32 * (g0 + uu) * T::RB;
  #pragma unroll
            for (int k4 = 0; k4 < C::NKK; k4 += C::FB) {
              bf16x8 qa[C::FB], da[C::FB], va[C::FB];
  #pragma unroll
              for (int i = 0; i < C::FB; ++i) {
                qa[i] = lds_row(qp, roff[k4 + i]);
                da[i] = lds_row(dop, roff[k4 + i]);
                if constexpr (C::VLDS) va[i] = lds_row(Vb, vboff[k4 + i]);
                else va[i] = vf[k4 + i];
              }
  #pragma unroll
              for (int i = 0; i < C::FB; ++i) {
                s[uu] = mfma(qa[i], kf[k4 + i], s[uu]);
                dp[uu] = mfma(da[i], va[i], dp[uu]);
              }
            }
          }
          // Register r of sub-tile u holds query row 32u + perm_row(r, hh).
  #pragma unroll
          for (int uu = 0; uu < C::NG; ++uu) {
            if constexpr (C::FOLD) {
  #pragma unroll
              for (int r = 0; r < 16; ++r) s[uu][r] = __builtin_amdgcn_exp2f(s[uu][r] * sl2);
            } else {
              const f32x4x4 lv = row_stats(C::LSE_OFF, g0 + uu);
  #pragma unroll
              for (int r = 0; r < 16; ++r)
                s[uu][r] = __builtin_amdgcn_exp2f(fmaf(s[uu][r], sl2, -lv.v[r >> 2][r & 3]));
            }
          }
          if (__builtin_expect(need_mask, false)) {  // boundary tiles only
            // Row qi sees key my_k iff qi - wl <= my_k <= qi + hi (hi = 0 under
            // the causal mask, else the right window edge), i.e. iff
            // qi - my_k + hi lies in [0, wl + hi]: one unsigned compare per
            // element against a per-lane base (exact in 32-bit wrap-around for
            // N <= 2^30).
            // (The lane terms come from a fresh lane index: this rarely taken
            // block would otherwise hold them live, or reload them from
            // scratch, across the whole loop.)
            const int ln = fresh_lane_id();
            const int kl = k0 + 32 * w + (ln & 31);  // = my_k
            const bool kpad = kl >= kvalid;
            const unsigned hi = causal ? 0u : (unsigned)p.wr;
            const unsigned span = (unsigned)p.wl + hi;
            const unsigned base = (unsigned)(q0b + 8 * (ln >> 5)) + hi - (unsigned)kl;
  #pragma unroll
            for (int uu = 0; uu < C::NG; ++uu)
  #pragma unroll
              for (int r = 0; r < 16; ++r) {
                const unsigned t = base + (unsigned)(32 * (g0 + uu) + perm_row(r, 0));
                s[uu][r] = (kpad | (t > span)) ? 0.f : s[uu][r];  // branch-free select
              }
          }
  #pragma unroll
          for (int uu = 0; uu < C::NG; ++uu) {
            if constexpr (DROP) {
              const f32x4x4 dv = row_stats(C::DVEC_OFF, g0 + uu);
              const uint32_t bits = dbits[g0 + uu];
  #pragma unroll
              for (int r = 0; r < 16; ++r) {
                // All-ones / all-zero mask from keep bit r; P o Z is one AND.
                int m = __builtin_amdgcn_sbfe((int)bits, r, 1);
                asm("" : "+v"(m));  // opaque: keeps the AND (not a compare + select)
                const float pz = __int_as_float(__float_as_int(s[uu][r]) & m);
                // dS' = P (Z dP~ - q D) = (P o Z) dP~ - P (q D)  (the D row
                // vector holds q D); P o Z also feeds dV.
                dp[uu][r] = fmaf(pz, dp[uu][r], -s[uu][r] * dv.v[r >> 2][r & 3]);
                s[uu][r] = pz;
              }
            } else if constexpr (C::FOLD) {
  #pragma unroll
              for (int r = 0; r < 16; ++r) dp[uu][r] = s[uu][r] * dp[uu][r];  // dP started at -D
            } else {
              const f32x4x4 dv = row_stats(C::DVEC_OFF, g0 + uu);
  #pragma unroll
              for (int r = 0; r < 16; ++r) dp[uu][r] = s[uu][r] * (dp[uu][r] - dv.v[r >> 2][r & 3]);
            }
  #pragma unroll
            for (int c = 0; c < 2; ++c) {
              const bf16x8 pf = pack8(s[uu], c);
              const bf16x8 dsf = pack8(dp[uu], c);
              const int rb = (32 * (g0 + uu) + 16 * c) * T::RB;
  #pragma unroll
              for (int db = 0; db < C::NDB; ++db) {
                dvt[db] = mfma(lds_tr(dOs + rb, troff[db][0], troff[db][1]), pf, dvt[db]);
                dkt[db] = mfma(lds_tr(Qs + rb, troff[db][0], troff[db][1]), dsf, dkt[db]);
              }
            }
          }
        }
        if (nx < nsteps) {
          wait_dma();
          __syncthreads();
        }
        sidx = nx;
      };
      for (int st = 0; sidx < nsteps; st ^= 1)
        step(smem + st * C::STAGE, smem + (st ^ 1) * C::STAGE, smem + C::VOFF);
    }

    // Under dropout both products carry the 1 / q of the kept probabilities.
    const float vscale = DROP ? p.drop_scale : 1.f;
    const float kscale = p.scale * vscale;
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
            kq[e] = (bf16)(dkt[db][4 * g + e] * kscale);
            vq[e] = (bf16)(dvt[db][4 * g + e] * vscale);
          }
          *reinterpret_cast<bf16x4*>(dkp + d0) = kq;
          *reinterpret_cast<bf16x4*>(dvp + d0) = vq;
        }
    }
  }  // key blocks of this workgroup
}

// ------------------------------------------------- dK, dV, 16x16x32 products
//
// The dK/dV pass without a block mask or dropout (causal, key padding and
// sliding windows allowed) at d=128 on the
// 16x16x32 matrix instruction. Per wave two 16-key blocks (keys
// k0 + 32 w + 16 kb + i), per step two 16-row query blocks:
//   S = Q K^T    (A: query rows from the stage, B: the lane's key rows)
//   dP = dO V^T  (A: dO rows, B: V rows from the workgroup's V block)
// A lane then holds, for key column i, query rows 4 g .. 4 g + 3 of both
// query blocks: with block 0 in K slots 0-3 and block 1 in slots 4-7 that
// is the B operand of
//   dV^T += dO^T P,   dK^T += Q^T dS   (A: two transposing reads, 4 rows each)
// the slot order of the forward's P V product. The row statistics of those
// four rows are one 16-byte LDS read per query block.
#if FA_TIMELINE
// Timeline stamps of the 16x16x32 dQ and dK/dV kernels (debug build).
__device__ unsigned long long fa_tl_dq[kTlWorkgroups * kTlSlots];
__device__ unsigned long long fa_tl_dkdv[kTlWorkgroups * kTlSlots];
#endif

template <int D, int NW>
struct DkdvM {
  // Keys per workgroup: NW waves x 2 blocks of 16. Query rows per step: 32
  // with 4 waves (two workgroups per CU hold two stages and the V block);
  // 64 with 8 waves (one workgroup per CU, still two waves per SIMD), as two
  // 32-row sub-blocks per barrier, which halves the barriers and the Q / dO
  // DMA per product.
  static constexpr int BK = 32 * NW;
  static constexpr int BQ = NW == 8 ? 64 : 32;
  static constexpr int NSB = BQ / 32;
  static constexpr int NDC = D / 32;
  static constexpr int NDB = D / 16;
  using T = SwzTile<D, BQ, 1>;
  using VT = SwzTile<D, BK, 1>;
  static constexpr int QNL = T::BYTES / (NW * 1024);   // DMA loads per thread, Q or dO tile
  static constexpr int VNL = VT::BYTES / (NW * 1024);  // DMA loads per thread, V block
  // One stage: Q tile | dO tile | LSE log2e of 64 rows | D of 64 rows (one
  // dword DMA per lane; at BQ = 32 the next step's 32 rows come along).
  static constexpr int LSE_OFF = 2 * T::BYTES;
  static constexpr int DVEC_OFF = LSE_OFF + 256;
  static constexpr int STAGE = DVEC_OFF + 256;
  static constexpr int VOFF = 2 * STAGE;
  static constexpr int LDS_BYTES = VOFF + VT::BYTES;
  static_assert(STAGE % 256 == 0, "stages keep the 256-byte bank period");
  static_assert(T::RB == VT::RB, "Q, dO and V rows share lane offsets");
};

template <int D, int NREP, int NW>
__global__ __launch_bounds__(64 * NW, NW == 8 ? 1 : 2) void bwd_dkdv_kernel_m16(BwdArgs a) {
  using C = DkdvM<D, NW>;
  using T = typename C::T;
  using VT = typename C::VT;
  static_assert(D == 128, "the XOR offset identities below assume 16 chunks per row");
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];

  const Problem& p = a.p;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int nkb = (p.N + C::BK - 1) / C::BK;
  // Key blocks as in the 32x32 kernel: causal pairs i and nkb - 1 - i.
  static_assert(NREP == 1 || NREP == 2, "one block or a pair");
  const int nunit = NREP == 2 ? (nkb + 1) / 2 : nkb;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int head_lin = L / nunit;
  const int ui = L - head_lin * nunit;
  const int b = head_lin / p.Hkv, hk = head_lin - b * p.Hkv;
  const float sl2 = p.scale_l2;
  const bool causal = p.causal != 0;
  const int kvalid = __builtin_amdgcn_readfirstlane(valid_keys(p.seqlens, b, p.N));
  FA_TL(fa_tl_dkdv, 0, tl_now());
  FA_TL(fa_tl_dkdv, 1, tl_where());
  const int qsb = 2 * (int)a.sq.n, dsb = 2 * (int)a.sdo.n, vsb = 2 * (int)a.sv.n;

  for (int rep = 0; rep < NREP; ++rep) {
    const int kb = rep == 0 ? ui : nkb - 1 - ui;
    if (rep == 1) {
      if (kb == ui) break;  // the middle block of an odd count
      __syncthreads();  // the first block's last step and V block are no longer read
    }
    const int k0 = kb * C::BK;
    const int kw0 = k0 + 32 * w;  // first key of this wave
    const bf16* Kp = static_cast<const bf16*>(a.k) + b * a.sk.b + hk * a.sk.h;
    const bf16* Vp = static_cast<const bf16*>(a.v) + b * a.sv.b + hk * a.sv.h;

    // The lane's keys kw0 + 16 kk + li as B operands (head-dim chunk dc,
    // slots 8 lg .. 8 lg + 7); keys past the valid length are zero.
    bf16x8 kf[2][C::NDC];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int key = kw0 + 16 * kk + li;
      const bool ok = key < kvalid;
      const bf16* kr = Kp + (int64_t)(ok ? key : 0) * a.sk.n + 8 * lg;
#pragma unroll
      for (int dc = 0; dc < C::NDC; ++dc) kf[kk][dc] = frag_g(kr + 32 * dc, ok);
    }
    f32x4 dkt[C::NDB][2], dvt[C::NDB][2];
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) dkt[db][kk] = dvt[db][kk] = f32x4{};

    if (k0 < kvalid) {  // else every key of the block is masked: dK = dV = 0
      // Steps: (query head of the group) x (32-row query block), from the
      // causal diagonal down; query blocks from the last one, heads of the
      // group innermost.
      // Rows that can see a key of this block: from the causal diagonal or
      // the right window edge, up to the left window edge.
      const int qfirst = max(causal ? k0 : 0, k0 - p.wr) / C::BQ;
      const int qend = min(p.N, k0 + C::BK + p.wl);
      const int nq = max(0, (qend + C::BQ - 1) / C::BQ - qfirst);
      const int nsteps = p.G * nq;
      auto step_unit = [&](int sidx, int& h, int& q0b) {
        const int jd = p.G == 1 ? sidx : sidx / p.G;
        h = hk * p.G + (sidx - jd * p.G);
        q0b = (qfirst + nq - 1 - jd) * C::BQ;
      };
      auto issue = [&](int sidx, char* stage) {
        int h, q0b;
        step_unit(sidx, h, q0b);
        // DMA offsets rebuilt from a fresh lane index (not kept live across
        // the loop: registers are at their limit).
        const int ln = fresh_lane_id();
        int qvo[C::QNL], dvo[C::QNL];
        dma_offsets_t<T, C::QNL, NW>(qvo, qsb, w, ln);
        dma_offsets_t<T, C::QNL, NW>(dvo, dsb, w, ln);
        const Rsrc qrs = make_rsrc(static_cast<const bf16*>(a.q) + b * a.sq.b + h * a.sq.h,
                                   rows_extent(p.N, qsb, 2 * D));
        const Rsrc drs = make_rsrc(static_cast<const bf16*>(a.dout) + b * a.sdo.b + h * a.sdo.h,
                                   rows_extent(p.N, dsb, 2 * D));
        dma_tile<D, C::BQ, NW>(qrs, qvo, (uint32_t)q0b * qsb, stage, w);
        dma_tile<D, C::BQ, NW>(drs, dvo, (uint32_t)q0b * dsb, stage + T::BYTES, w);
        if (w < 2) {  // wave-uniform: wave 0 loads LSE, wave 1 D
          const int64_t row0 = ((int64_t)b * p.Hq + h) * p.N;
          const Rsrc rs = make_rsrc((w ? a.dvec : a.lse2) + row0, (uint32_t)p.N * 4);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rs, (FA_LDS void*)(stage + (w ? C::DVEC_OFF : C::LSE_OFF)), 4, 4 * ln,
              (uint32_t)q0b * 4, 0, 0);
        }
      };
      {
        int vvo[C::VNL];
        dma_offsets_t<VT, C::VNL, NW>(vvo, vsb, w, lane);
        const Rsrc vrs = make_rsrc(Vp, rows_extent(kvalid, vsb, 2 * D));
        dma_tile<D, C::BK, NW>(vrs, vvo, (uint32_t)k0 * vsb, smem + C::VOFF, w);
      }
      // Row operands (query, dO and V rows 16 x + li, chunk 4 dc + lg; the
      // swizzle depends on a row's low 4 bits only, so the 16-row block
      // base is an immediate) and transposed operands (loader lane 4 e + a
      // of group lg reads query row 4 lg + e (+ 16) at head-dim 16 db + 4 a).
      // The swizzle XORs the chunk index, so chunk 4 dc + lg lies at the
      // dc = 0 offset XOR 64 dc, and head-dim block db at the db = 0 offset
      // XOR 32 db: one register each stays live, the rest are rebuilt per
      // step.
      const int roff0 = T::off(li, lg);
      int toff0;
      {
        const int rr = 4 * lg + (li >> 2), aa = li & 3;
        const int d = 4 * aa;
        toff0 = rr * T::RB + 16 * ((d >> 3) ^ T::swz(rr)) + 2 * (d & 7);
      }

      FA_TL(fa_tl_dkdv, 2 + 4 * rep, tl_now());
      int sidx = 0;
      if (sidx < nsteps) issue(sidx, smem);
      wait_dma();  // the V block and the first step
      __syncthreads();
      FA_TL(fa_tl_dkdv, 3 + 4 * rep, tl_now());
      auto step = [&](const char* __restrict__ Qs, char* __restrict__ fill,
                      const char* __restrict__ Vb) {
        const char* dOs = Qs + T::BYTES;
        int h, q0b;
        step_unit(sidx, h, q0b);
        const int nx = sidx + 1;
        if (nx < nsteps) {  // lands during this step
          paranoid_before_fill();
          issue(nx, fill);
          paranoid_after_fill();
        }
        if (a.log_kv && tid == 0) {
          // Every 128-key block of the workgroup that a row of the step sees.
          const int64_t row_word0 = (((int64_t)b * p.Hq + h) * p.nlb + (q0b >> 7)) * p.logw;
          const int hi = causal ? 0 : p.wr;
          for (int kc = k0; kc < k0 + C::BK && kc < kvalid; kc += 128)
            if (kc <= q0b + C::BQ - 1 + hi && kc + 127 >= q0b - p.wl)
              log_tile(a.log_kv, row_word0, kc);
        }
        // (Causal pairs never carry a window: its terms compile into the
        // one-block instances only.)
        const bool need_mask =
            (causal && k0 + C::BK - 1 > q0b) || (k0 + C::BK > kvalid) ||
            (NREP == 1 && ((q0b + C::BQ - 1 > k0 + p.wl) || (q0b < k0 + C::BK - 1 - p.wr)));
        const char* Vw = Vb + 32 * w * VT::RB;
        // 32-row sub-blocks of the step, one after the other (a loop, not
        // unrolled: two unrolled copies would overlap and spill).
#pragma unroll 1
        for (int sb = 0; sb < C::NSB; ++sb) {
        const int qs0 = q0b + 32 * sb;
        const char* Qsb = Qs + 32 * sb * T::RB;
        const char* dOsb = dOs + 32 * sb * T::RB;
        // When no row of the sub-block sees a key of the wave (above the
        // causal diagonal, outside the band) its P is exactly 0 and it adds
        // nothing to dK or dV.
        const bool wave_off = NREP == 2 ? qs0 + 31 < kw0
                                        : qs0 + 31 + (causal ? 0 : p.wr) < kw0 ||
                                              qs0 - p.wl > kw0 + 31;
        if (!wave_off) {
          int roff[C::NDC], toff[C::NDB];
          {
            int r0 = roff0, t0 = toff0;
            asm volatile("" : "+v"(r0), "+v"(t0));
#pragma unroll
            for (int dc = 0; dc < C::NDC; ++dc) roff[dc] = r0 ^ (64 * dc);
#pragma unroll
            for (int db = 0; db < C::NDB; ++db) toff[db] = t0 ^ (32 * db);
          }
          f32x4 s[2][2], dp[2][2];  // [query block][key block]
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) s[rb][kk] = dp[rb][kk] = f32x4{};
          __builtin_amdgcn_s_setprio(1);
#pragma unroll
          for (int dc = 0; dc < C::NDC; ++dc) {
            bf16x8 qa[2], da[2], va[2];
#pragma unroll
            for (int x = 0; x < 2; ++x) {
              qa[x] = lds_row(Qsb + 16 * x * T::RB, roff[dc]);
              da[x] = lds_row(dOsb + 16 * x * T::RB, roff[dc]);
              va[x] = lds_row(Vw + 16 * x * VT::RB, roff[dc]);
            }
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
              for (int kk = 0; kk < 2; ++kk) {
                s[rb][kk] = mfma16(qa[rb], kf[kk][dc], s[rb][kk]);
                dp[rb][kk] = mfma16(da[rb], va[kk], dp[rb][kk]);
              }
          }
          {
            // One chunk's six reads ahead of its eight products.
            __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
            for (int i = 0; i < C::NDC - 1; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
              __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
              __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
              __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
          }
          __builtin_amdgcn_s_setprio(0);
          // LSE log2e and D of rows qs0 + 16 rb + 4 lg + r, r = 0..3.
          f32x4 l4[2], d4[2];
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            l4[rb] = *reinterpret_cast<const f32x4*>(Qs + C::LSE_OFF + 4 * (32 * sb + 16 * rb + 4 * lg));
            d4[rb] = *reinterpret_cast<const f32x4*>(Qs + C::DVEC_OFF + 4 * (32 * sb + 16 * rb + 4 * lg));
          }
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
              for (int r = 0; r < 4; ++r)
                s[rb][kk][r] = __builtin_amdgcn_exp2f(fmaf(s[rb][kk][r], sl2, -l4[rb][r]));
          if (__builtin_expect(need_mask, false)) {
            const unsigned span = (unsigned)p.wl + (causal ? 0u : (unsigned)p.wr);
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
              for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                  const int key = kw0 + 16 * kk + li;
                  const int row = qs0 + 16 * rb + 4 * lg + r;
                  // Row i sees key j iff i - wl <= j <= i + hi (hi = 0 under
                  // the causal mask, else the right window edge), j < kvalid.
                  const bool kill = key >= kvalid || (NREP == 2 ? key > row
                                                                : (unsigned)(key - row + p.wl) > span);
                  s[rb][kk][r] = kill ? 0.f : s[rb][kk][r];
                }
          }
          bf16x8 pf[2], dsf[2];
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                pf[kk][4 * rb + r] = (bf16)s[rb][kk][r];
                dsf[kk][4 * rb + r] = (bf16)(s[rb][kk][r] * (dp[rb][kk][r] - d4[rb][r]));
              }
          __builtin_amdgcn_s_setprio(1);
#pragma unroll
          for (int db = 0; db < C::NDB; ++db) {
            const bf16x8 dot = lds_tr(dOsb, toff[db], toff[db] + 16 * T::RB);
            const bf16x8 qt = lds_tr(Qsb, toff[db], toff[db] + 16 * T::RB);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
              dvt[db][kk] = mfma16(dot, pf[kk], dvt[db][kk]);
              dkt[db][kk] = mfma16(qt, dsf[kk], dkt[db][kk]);
            }
          }
          {
            // Two head-dim blocks of reads ahead of their products.
            __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
            for (int i = 0; i < C::NDB - 2; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
              __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
          }
          __builtin_amdgcn_s_setprio(0);
        }  // !wave_off
        }  // sub-blocks
        if (nx < nsteps) {
          wait_dma();
          __syncthreads();
        }
        sidx = nx;
      };
      for (int st = 0; sidx < nsteps; st ^= 1)
        step(smem + st * C::STAGE, smem + (st ^ 1) * C::STAGE, smem + C::VOFF);
      FA_TL(fa_tl_dkdv, 4 + 4 * rep, tl_now());
      FA_TL(fa_tl_dkdv, 5 + 4 * rep, ((unsigned long long)kb << 16) | (unsigned)nsteps);
    }

    // Register e of block (db, kk) is head-dim 16 db + 4 lg + e of key
    // kw0 + 16 kk + li.
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int key = kw0 + 16 * kk + li;
      if (key < p.N) {
        bf16* dkp = static_cast<bf16*>(a.dk) + b * a.sdk.b + hk * a.sdk.h + (int64_t)key * a.sdk.n;
        bf16* dvp = static_cast<bf16*>(a.dv) + b * a.sdv.b + hk * a.sdv.h + (int64_t)key * a.sdv.n;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
          bf16x4 kq, vq;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            kq[e] = (bf16)(dkt[db][kk][e] * p.scale);
            vq[e] = (bf16)dvt[db][kk][e];
          }
          *reinterpret_cast<bf16x4*>(dkp + 16 * db + 4 * lg) = kq;
          *reinterpret_cast<bf16x4*>(dvp + 16 * db + 4 * lg) = vq;
        }
      }
    }
  }  // key blocks of this workgroup
  FA_TL(fa_tl_dkdv, 10, tl_now());
}

// ----------------------------------------------------------------- dQ

template <int D>
struct DqCfg {
  static constexpr int BR = 128;  // query rows per workgroup
  static constexpr int BC = 64;   // keys per tile
  static constexpr int NSUB = BC / 32;
  static constexpr int NKK = D / 16;
  static constexpr int NDB = D / 32;
  using T = SwzTile<D, BC>;
};

// MASK as in the dK/dV kernel.
template <int D, bool DROP, int NREP, bool MASK>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(BwdArgs a) {
  using C = DqCfg<D>;
  using T = typename C::T;
  // Two stages of (K tile | V tile); K^T operands come from the K tile
  // through transposing reads.
  __shared__ __attribute__((aligned(1024))) char smem[2][2 * T::BYTES];

  const Problem& p = a.p;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, hh = lane >> 5;
  const int nqb = (p.N + C::BR - 1) / C::BR;
  // NREP = 2 (causal, no left window edge): query blocks nqb - 1 - i and i in
  // one workgroup, heaviest first, as in the forward.
  static_assert(NREP == 1 || NREP == 2, "one block or a pair");
  const int nunit = NREP == 2 ? (nqb + 1) / 2 : nqb;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int head_lin = L / nunit;
  const int ui = L - head_lin * nunit;
  const int b = head_lin / p.Hq, h = head_lin - b * p.Hq, hk = h / p.G;
  const float sl2 = p.scale_l2;
  const bool causal = p.causal != 0;

  // Keys past the valid length read as zero, whatever their memory holds.
  const int kvalid = __builtin_amdgcn_readfirstlane(valid_keys(p.seqlens, b, p.N));
  const int ksb = 2 * (int)a.sk.n, vsb = 2 * (int)a.sv.n;
  const Rsrc krs = make_rsrc(static_cast<const bf16*>(a.k) + b * a.sk.b + hk * a.sk.h,
                             rows_extent(kvalid, ksb, 2 * D));
  const Rsrc vrs = make_rsrc(static_cast<const bf16*>(a.v) + b * a.sv.b + hk * a.sv.h,
                             rows_extent(kvalid, vsb, 2 * D));
  for (int rep = 0; rep < NREP; ++rep) {
    const int qb = NREP == 2 ? (rep == 0 ? nqb - 1 - ui : ui) : (causal ? nqb - 1 - ui : ui);
    if (rep == 1) {
      if (qb == nqb - 1 - ui) break;  // the middle block of an odd count
      __syncthreads();  // the first block's last tile is no longer read
    }
    const int q0 = qb * C::BR;
    const int my_q = q0 + 32 * w + lr;

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
    // Row statistics of this lane's row, computed here and stored for the
    // dK/dV kernel, which runs after this one: D = dO . O (the two lane halves
    // hold interleaved halves of the row), q D under dropout (with
    // dP = (Z / q) o dO V^T, dS = P o (dP - D) = (1 / q) P o (Z o dO V^T - q D),
    // and the 1 / q joins the final scales), and the LSE in base-2 units
    // (+inf for a row with no allowed key, so that every rebuilt probability
    // of it is 2^-inf = 0).
    const int64_t rowstat = ((int64_t)b * p.Hq + h) * p.N + (qok ? my_q : 0);
    float dpart = 0.f;
    if (qok) {
      const int64_t orow = b * a.so.b + h * a.so.h + (int64_t)my_q * a.so.n + 8 * hh;
#pragma unroll
      for (int kk = 0; kk < C::NKK; ++kk) {
        float o8[8];
        if (a.o_fp32) {
          const float* op = static_cast<const float*>(a.o) + orow + 16 * kk;
          const float4 x0 = *reinterpret_cast<const float4*>(op);
          const float4 x1 = *reinterpret_cast<const float4*>(op + 4);
          o8[0] = x0.x; o8[1] = x0.y; o8[2] = x0.z; o8[3] = x0.w;
          o8[4] = x1.x; o8[5] = x1.y; o8[6] = x1.z; o8[7] = x1.w;
        } else {
          const bf16x8 x = *reinterpret_cast<const bf16x8*>(static_cast<const bf16*>(a.o) + orow + 16 * kk);
#pragma unroll
          for (int e = 0; e < 8; ++e) o8[e] = (float)x[e];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) dpart = fmaf((float)dof[kk][e], o8[e], dpart);
      }
    }
    const float dsum = half_sum(dpart);
    const float dq_d = p.drop ? dsum * p.drop_q : dsum;
    const float lse2 = qok ? lse2_of(a.lse[rowstat]) : kInf;
    if (qok && hh == 0) {
      a.dvec[rowstat] = dq_d;
      a.lse2[rowstat] = lse2;
    }
    // Without dropout every dP^T chain starts at -D (one value per lane: the
    // lane's query row), set by one product from these two operands, so that
    // dS = P dP needs no subtraction.
    const bf16x8 d_split = split3_frag(dq_d), d_neg = neg_ones_frag(hh, 0);

    int kvo[T::NLD], vvo[T::NLD];
    dma_offsets<D, C::BC>(kvo, ksb, w, lane);
    dma_offsets<D, C::BC>(vvo, vsb, w, lane);
    int roff[C::NKK], troff[C::NDB][2];
    row_offsets<D, C::BC>(roff, lr, hh);
    tr_offsets<D, C::BC>(troff, lane);

    f32x16 acc[C::NDB];
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) acc[db] = f32x16{};

    const int kend = min(p.causal ? min(kvalid, q0 + C::BR) : kvalid, q0 + C::BR + p.wr);
    const int ntiles = (kend + C::BC - 1) / C::BC;
    const int64_t log_row =
        a.log_q ? (((int64_t)b * p.Hq + h) * p.nlb + (q0 >> 7)) * p.logw : 0;
    MaskLine mrow = mask_row(MASK ? p.bm : nullptr, p.bm_ld, p.nlb, q0);
    // The tile index is wave-uniform; saying so keeps the DMA offsets in
    // scalar registers (otherwise each buffer load may be wrapped in a
    // read-first-lane loop).
    auto next_visit = [&](int kt) {
      return __builtin_amdgcn_readfirstlane(MASK ? mrow.next_tile<C::BC>(kt, ntiles) : kt);
    };
    auto issue = [&](int kt, char* stage) {
      dma_tile<D, C::BC>(krs, kvo, (uint32_t)(kt * C::BC) * ksb, stage, w);
      dma_tile<D, C::BC>(vrs, vvo, (uint32_t)(kt * C::BC) * vsb, stage + T::BYTES, w);
    };

    int kt = next_visit(max(0, q0 - p.wl) / C::BC);
    if (kt < ntiles) {
      issue(kt, smem[0]);
      wait_dma();
      __syncthreads();
    }
    // One key tile read from stage `Ks` while the next lands in `fill`
    // (restrict-qualified: these reads never wait for that DMA).
    auto tile = [&](const char* __restrict__ Ks, char* __restrict__ fill) {
      const char* Vs = Ks + T::BYTES;
      const int key0 = kt * C::BC;
      const int nxt = next_visit(kt + 1);
      if (nxt < ntiles) {
        paranoid_before_fill();
        issue(nxt, fill);
        paranoid_after_fill();
      }
      if (a.log_q && tid == 0) log_tile(a.log_q, log_row, key0);
      const bool need_mask = (p.causal && key0 + C::BC - 1 > q0) || (key0 + C::BC > kvalid) ||
                             (key0 < q0 + C::BR - 1 - p.wl) || (key0 + C::BC - 1 > q0 + p.wr);
      // A wave whose 32 rows see no key of a 32-key sub-tile (above the
      // causal diagonal, outside the band) skips it: its P would be 0 and so
      // would its dS, leaving dQ bit-identical. Causal pairs test the
      // diagonal, one-block launches of the general variant without dropout
      // the band; the rest compile no test.
      const int r0 = q0 + 32 * w;
#pragma unroll
      for (int t = 0; t < C::NSUB; ++t) {
        if (NREP == 2 ? key0 + 32 * t > r0 + 31
                      : MASK && !DROP && (key0 + 32 * t > r0 + 31 + (causal ? 0 : p.wr) ||
                                          key0 + 32 * t + 31 < r0 - p.wl))
          continue;
        f32x16 st = f32x16{}, dpt = DROP ? f32x16{} : mfma(d_neg, d_split, f32x16{});
        const char* kp = Ks + 32 * t * T::RB;
        const char* vp = Vs + 32 * t * T::RB;
        // Raised priority while this wave feeds the matrix pipe, so that the
        // other wave on the SIMD fills the VALU between its products.
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int k4 = 0; k4 < C::NKK; k4 += 4) {
          bf16x8 ka[4], va[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            ka[i] = lds_row(kp, roff[k4 + i]);
            va[i] = lds_row(vp, roff[k4 + i]);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            st = mfma(ka[i], qf[k4 + i], st);
            dpt = mfma(va[i], dof[k4 + i], dpt);
          }
        }
        __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int r = 0; r < 16; ++r) st[r] = __builtin_amdgcn_exp2f(fmaf(st[r], sl2, -lse2));
        if (__builtin_expect(need_mask, false)) {  // boundary tiles only
          // Key j is seen iff my_q - wl <= j <= my_q + hi (hi = 0 under the
          // causal mask, else the right window edge) and j < kvalid; the band
          // test is one unsigned compare of j - my_q + wl against wl + hi.
          const unsigned hi = causal ? 0u : (unsigned)p.wr;
          const unsigned span = (unsigned)p.wl + hi;
          const unsigned base = (unsigned)(key0 + 32 * t + 8 * hh + p.wl) - (unsigned)my_q;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + 32 * t + perm_row(r, hh);
            const bool kill = (base + (unsigned)perm_row(r, 0) > span) | (key >= kvalid);
            st[r] = kill ? 0.f : st[r];  // branch-free select
          }
        }
        if constexpr (DROP) {  // dP~ of dropped entries is zero (dq_d holds q D)
#pragma unroll
          for (int c = 0; c < 2; ++c)
            drop_run8(dpt, 8 * c,
                      drop_bits(p, (uint32_t)(key0 + 32 * t + 16 * c + 8 * hh) >> 3,
                                (uint32_t)my_q, (uint32_t)(b * p.Hq + h)),
                      p.drop_thr);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) dpt[r] = st[r] * (DROP ? dpt[r] - dq_d : dpt[r]);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const bf16x8 dsf = pack8(dpt, c);
          const char* ktp = Ks + (32 * t + 16 * c) * T::RB;
#pragma unroll
          for (int db = 0; db < C::NDB; ++db)
            acc[db] = mfma(lds_tr(ktp, troff[db][0], troff[db][1]), dsf, acc[db]);
        }
        __builtin_amdgcn_s_setprio(0);
      }
      if (nxt < ntiles) {
        wait_dma();
        __syncthreads();
      }
      kt = nxt;
    };
    for (int st = 0; kt < ntiles; st ^= 1) tile(smem[st], smem[st ^ 1]);

    const float qscale = DROP ? p.scale * p.drop_scale : p.scale;
    if (qok) {
      bf16* dqp = static_cast<bf16*>(a.dq) + b * a.sdq.b + h * a.sdq.h + (int64_t)my_q * a.sdq.n;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          bf16x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (bf16)(acc[db][4 * g + e] * qscale);
          *reinterpret_cast<bf16x4*>(dqp + 32 * db + 8 * g + 4 * hh) = v;
        }
    }
  }  // query blocks of this workgroup
}

// ------------------------------------------------- dQ, 16x16x32 products
//
// The dQ pass without a block mask or dropout (causal, key padding and
// sliding windows allowed) on the
// 16x16x32 matrix instruction (less energy per flop than 32x32x16 under the
// board's power limit; see the forward's 16x16x32 kernel for the layouts).
// Per wave two 16-row blocks; per 64-key tile four 16-key blocks:
//   S^T = K Q^T,  dP^T - D = V dO^T (started at -D),  P = 2^(S c - LSE2),
//   dS^T = P (dP^T - D),  dQ^T += K^T dS^T   (K^T from transposing reads)
// Each lane's accumulator registers of a 16x16 block all belong to the
// lane's query row, so the dP^T chains start at that row's -D directly.
template <int D, int NW>
struct DqM {
  // Query rows per workgroup: NW waves x 32. Keys per tile: 64 with 4 waves
  // (two workgroups per CU); 128 with 8 waves (one workgroup per CU, still
  // two waves per SIMD), which halves the barriers and the K/V DMA per
  // product.
  static constexpr int BR = 32 * NW;
  static constexpr int BC = NW == 8 ? 128 : 64;
  static constexpr int NKB = BC / 16;
  static constexpr int NH = BC / 32;  // 32-key halves per tile
  static constexpr int NDC = D / 32;
  static constexpr int NDB = D / 16;
  using T = SwzTile<D, BC, 1>;
  static constexpr int KNL = T::BYTES / (NW * 1024);  // DMA loads per thread, K or V tile
};

template <int D, int NREP, int NW>
__global__ __launch_bounds__(64 * NW, NW == 8 ? 1 : 2) void bwd_dq_kernel_m16(BwdArgs a) {
  using C = DqM<D, NW>;
  using T = typename C::T;
  __shared__ __attribute__((aligned(1024))) char smem[2][2 * T::BYTES];

  const Problem& p = a.p;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int nqb = (p.N + C::BR - 1) / C::BR;
  static_assert(NREP == 1 || NREP == 2, "one block or a pair");
  const int nunit = NREP == 2 ? (nqb + 1) / 2 : nqb;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int head_lin = L / nunit;
  const int ui = L - head_lin * nunit;
  const int b = head_lin / p.Hq, h = head_lin - b * p.Hq, hk = h / p.G;
  const float sl2 = p.scale_l2;
  FA_TL(fa_tl_dq, 0, tl_now());
  FA_TL(fa_tl_dq, 1, tl_where());
  const bool causal = p.causal != 0;

  const int kvalid = __builtin_amdgcn_readfirstlane(valid_keys(p.seqlens, b, p.N));
  const int ksb = 2 * (int)a.sk.n, vsb = 2 * (int)a.sv.n;
  const Rsrc krs = make_rsrc(static_cast<const bf16*>(a.k) + b * a.sk.b + hk * a.sk.h,
                             rows_extent(kvalid, ksb, 2 * D));
  const Rsrc vrs = make_rsrc(static_cast<const bf16*>(a.v) + b * a.sv.b + hk * a.sv.h,
                             rows_extent(kvalid, vsb, 2 * D));
  for (int rep = 0; rep < NREP; ++rep) {
    const int qb = NREP == 2 ? (rep == 0 ? nqb - 1 - ui : ui) : (causal ? nqb - 1 - ui : ui);
    if (rep == 1) {
      if (qb == nqb - 1 - ui) break;  // the middle block of an odd count
      __syncthreads();  // the first block's last tile is no longer read
    }
    const int q0 = qb * C::BR;
    const int r0 = q0 + 32 * w;

    // The lane's rows r0 + li and r0 + 16 + li: Q and dO as B operands
    // (head-dim chunk dc, slots 8 lg .. 8 lg + 7), and their statistics.
    bf16x8 qf[2][C::NDC], dof[2][C::NDC];
    float dneg[2], lse2[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int row = r0 + 16 * rb + li;
      const bool ok = row < p.N;
      const int64_t r = ok ? row : 0;
      const bf16* Qp = static_cast<const bf16*>(a.q) + b * a.sq.b + h * a.sq.h + r * a.sq.n + 8 * lg;
      const bf16* dOp = static_cast<const bf16*>(a.dout) + b * a.sdo.b + h * a.sdo.h + r * a.sdo.n + 8 * lg;
#pragma unroll
      for (int dc = 0; dc < C::NDC; ++dc) {
        qf[rb][dc] = frag_g(Qp + 32 * dc, ok);
        dof[rb][dc] = frag_g(dOp + 32 * dc, ok);
      }
      // D = dO . O over the row (the four lanes of the row hold interleaved
      // quarters of it), and the LSE in base-2 units (+inf for an empty row);
      // both stored for the dK/dV kernel.
      float dpart = 0.f;
      if (ok) {
        const int64_t orow = b * a.so.b + h * a.so.h + (int64_t)row * a.so.n + 8 * lg;
#pragma unroll
        for (int dc = 0; dc < C::NDC; ++dc) {
          float o8[8];
          if (a.o_fp32) {
            const float* op = static_cast<const float*>(a.o) + orow + 32 * dc;
            const float4 x0 = *reinterpret_cast<const float4*>(op);
            const float4 x1 = *reinterpret_cast<const float4*>(op + 4);
            o8[0] = x0.x; o8[1] = x0.y; o8[2] = x0.z; o8[3] = x0.w;
            o8[4] = x1.x; o8[5] = x1.y; o8[6] = x1.z; o8[7] = x1.w;
          } else {
            const bf16x8 x = *reinterpret_cast<const bf16x8*>(static_cast<const bf16*>(a.o) + orow + 32 * dc);
#pragma unroll
            for (int e = 0; e < 8; ++e) o8[e] = (float)x[e];
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) dpart = fmaf((float)dof[rb][dc][e], o8[e], dpart);
        }
      }
      const float dsum = quad_sum(dpart);
      const int64_t rowstat = ((int64_t)b * p.Hq + h) * p.N + r;
      lse2[rb] = ok ? lse2_of(a.lse[rowstat]) : kInf;
      dneg[rb] = -dsum;
      if (ok && lg == 0) {
        a.dvec[rowstat] = dsum;
        a.lse2[rowstat] = lse2[rb];
      }
    }

    int kvo[C::KNL], vvo[C::KNL];
    dma_offsets_t<T, C::KNL, NW>(kvo, ksb, w, lane);
    dma_offsets_t<T, C::KNL, NW>(vvo, vsb, w, lane);
    // Row operands (K and V rows 16 kb + li, chunk 4 dc + lg) and K^T
    // operands (transposing reads: key row 4 lg + e (+ 16, + 32 c) at
    // head-dim 16 db + 4 a for loader lane 4 e + a), as in the forward.
    int roff[C::NDC], toff[C::NDB];
#pragma unroll
    for (int dc = 0; dc < C::NDC; ++dc) roff[dc] = T::off(li, 4 * dc + lg);
    {
      const int rr = 4 * lg + (li >> 2), aa = li & 3;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        const int d = 16 * db + 4 * aa;
        toff[db] = rr * T::RB + 16 * ((d >> 3) ^ T::swz(rr)) + 2 * (d & 7);
      }
    }

    f32x4 acc[C::NDB][2];
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) acc[db][0] = acc[db][1] = f32x4{};

    // Keys any row of the block may see (causal / padding / right window
    // edge bound the end, the left window edge the start).
    const int kend = min(causal ? min(kvalid, q0 + C::BR) : kvalid, q0 + C::BR + p.wr);
    const int ntiles = (kend + C::BC - 1) / C::BC;
    const int64_t log_row0 = (((int64_t)b * p.Hq + h) * p.nlb + (q0 >> 7)) * p.logw;
    auto issue = [&](int kt, char* stage) {
      dma_tile<D, C::BC, NW>(krs, kvo, (uint32_t)(kt * C::BC) * ksb, stage, w);
      dma_tile<D, C::BC, NW>(vrs, vvo, (uint32_t)(kt * C::BC) * vsb, stage + T::BYTES, w);
    };
    FA_TL(fa_tl_dq, 2 + 4 * rep, tl_now());
    int kt = max(0, q0 - p.wl) / C::BC;
    if (kt < ntiles) {
      issue(kt, smem[0]);
      wait_dma();
      __syncthreads();
    }
    FA_TL(fa_tl_dq, 3 + 4 * rep, tl_now());
    auto tile = [&](const char* __restrict__ Ks, char* __restrict__ fill) {
      const char* Vs = Ks + T::BYTES;
      const int key0 = kt * C::BC;
      const int nxt = kt + 1;
      if (nxt < ntiles) {
        paranoid_before_fill();
        issue(nxt, fill);
        paranoid_after_fill();
      }
      if (a.log_q && tid == 0) {
        // Each 128-row block of the workgroup that sees a key of the tile:
        // rows i of the block and keys j of the tile with i - wl <= j <=
        // i + hi (hi = 0 under the causal mask, else the right window edge).
        const int hi = causal ? 0 : p.wr;
        for (int j = 0; j < C::BR / 128 && (q0 >> 7) + j < p.nlb; ++j) {
          const int qj = q0 + 128 * j;
          if (key0 <= qj + 127 + hi && key0 + C::BC - 1 >= qj - p.wl)
            log_tile(a.log_q, log_row0 + (int64_t)j * p.logw, key0);
        }
      }
      const bool need_mask =
          (causal && key0 + C::BC - 1 > q0) || (key0 + C::BC > kvalid) ||
          (NREP == 1 && ((key0 < q0 + C::BR - 1 - p.wl) || (key0 + C::BC - 1 > q0 + p.wr)));
      // A wave whose rows see no key of the tile (above the causal diagonal,
      // outside the band) has P = 0 there and skips it (dQ bit-identical).
      const bool wave_off = NREP == 2 ? key0 > r0 + 31
                                      : key0 > r0 + 31 + (causal ? 0 : p.wr) ||
                                            key0 + C::BC - 1 < r0 - p.wl;
      if (!wave_off) {
        // 32-key halves, each S/dP -> P, dS -> dQ products, so that only
        // half of a 64-key block of S and dP is live at once; a causal-pair
        // wave skips a half whose keys all lie above its rows.
#pragma unroll
        for (int c = 0; c < C::NH; ++c) {
          if (NREP == 2 && C::NH > 2 && key0 + 32 * c > r0 + 31) continue;
          f32x4 s[2][2], dp[2][2];
#pragma unroll
          for (int hb = 0; hb < 2; ++hb)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
              s[hb][rb] = f32x4{};
              dp[hb][rb] = f32x4{dneg[rb], dneg[rb], dneg[rb], dneg[rb]};
            }
          __builtin_amdgcn_s_setprio(1);
#pragma unroll
          for (int dc = 0; dc < C::NDC; ++dc)
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
              const int kb = 2 * c + hb;
              const bf16x8 kf = lds_row(Ks + 16 * kb * T::RB, roff[dc]);
              const bf16x8 vf = lds_row(Vs + 16 * kb * T::RB, roff[dc]);
#pragma unroll
              for (int rb = 0; rb < 2; ++rb) {
                s[hb][rb] = mfma16(kf, qf[rb][dc], s[hb][rb]);
                dp[hb][rb] = mfma16(vf, dof[rb][dc], dp[hb][rb]);
              }
            }
          {
            // Two reads (K and V) two blocks ahead of their four products.
            constexpr int NR = C::NDC * 2;
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
            for (int i = 0; i < NR - 2; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
              __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
          }
          __builtin_amdgcn_s_setprio(0);
          // P = 2^(S c - LSE2); dS = P (dP - D). Register r of key block
          // 2 c + hb is key key0 + 32 c + 16 hb + 4 lg + r, of row
          // r0 + 16 rb + li.
#pragma unroll
          for (int hb = 0; hb < 2; ++hb)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
              for (int r = 0; r < 4; ++r)
                s[hb][rb][r] = __builtin_amdgcn_exp2f(fmaf(s[hb][rb][r], sl2, -lse2[rb]));
          if (__builtin_expect(need_mask, false)) {
            const unsigned span = (unsigned)p.wl + (causal ? 0u : (unsigned)p.wr);
#pragma unroll
            for (int hb = 0; hb < 2; ++hb)
#pragma unroll
              for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                  const int key = key0 + 32 * c + 16 * hb + 4 * lg + r;
                  const int row = r0 + 16 * rb + li;
                  // Row i sees key j iff i - wl <= j <= i + hi (hi = 0 under
                  // the causal mask, else the right window edge), j < kvalid.
                  const bool kill = key >= kvalid || (NREP == 2 ? key > row
                                                                : (unsigned)(key - row + p.wl) > span);
                  s[hb][rb][r] = kill ? 0.f : s[hb][rb][r];
                }
          }
          bf16x8 dsf[2];
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int hb = 0; hb < 2; ++hb)
#pragma unroll
              for (int r = 0; r < 4; ++r)
                dsf[rb][4 * hb + r] = (bf16)(s[hb][rb][r] * dp[hb][rb][r]);
          __builtin_amdgcn_s_setprio(1);
          const char* kp = Ks + 32 * c * T::RB;
#pragma unroll
          for (int db = 0; db < C::NDB; ++db) {
            const bf16x8 ktf = lds_tr(kp, toff[db], toff[db] + 16 * T::RB);
            acc[db][0] = mfma16(ktf, dsf[0], acc[db][0]);
            acc[db][1] = mfma16(ktf, dsf[1], acc[db][1]);
          }
          {
            __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
            for (int i = 0; i < C::NDB - 4; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
              __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
          }
          __builtin_amdgcn_s_setprio(0);
        }
      }  // !wave_off
      if (nxt < ntiles) {
        wait_dma();
        __syncthreads();
      }
      kt = nxt;
    };
    for (int st = 0; kt < ntiles; st ^= 1) tile(smem[st], smem[st ^ 1]);
    FA_TL(fa_tl_dq, 4 + 4 * rep, tl_now());
    FA_TL(fa_tl_dq, 5 + 4 * rep, ((unsigned long long)qb << 16) | (unsigned)ntiles);

#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int row = r0 + 16 * rb + li;
      if (row < p.N) {
        bf16* dqp = static_cast<bf16*>(a.dq) + b * a.sdq.b + h * a.sdq.h + (int64_t)row * a.sdq.n;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
          bf16x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (bf16)(acc[db][rb][e] * p.scale);
          *reinterpret_cast<bf16x4*>(dqp + 16 * db + 4 * lg) = v;
        }
      }
    }
  }  // query blocks of this workgroup
  FA_TL(fa_tl_dq, 10, tl_now());
}

// ----------------------------------------------------------------- launchers

#ifndef FA_DKDV_M16
#define FA_DKDV_M16 1
#endif
#ifndef FA_DKDV_M16_WAVES
#define FA_DKDV_M16_WAVES 8
#endif

hipError_t launch_bwd_dkdv(const BwdArgs& a, int head_dim, hipStream_t s) {
  const int64_t nkb = (a.p.N + 127) / 128;
  const dim3 blk(256);
  // Pairs of key blocks where the causal work shrinks with the block index.
  const bool pair = a.p.causal && a.p.wl >= a.p.N;
  const dim3 g((unsigned)((pair ? (nkb + 1) / 2 : nkb) * a.p.Hkv * a.p.B));
  const bool mask = a.p.bm != nullptr || a.p.drop || a.p.wl < a.p.N || a.p.wr < a.p.N;
#define FA_DKDV_LAUNCH(DD, DR)                                                           \
  do {                                                                                   \
    if (pair) {                                                                          \
      if (mask) hipLaunchKernelGGL((bwd_dkdv_kernel<DD, DR, 2, true>), g, blk, 0, s, a); \
      else hipLaunchKernelGGL((bwd_dkdv_kernel<DD, DR, 2, DR>), g, blk, 0, s, a);     \
    } else {                                                                             \
      if (mask) hipLaunchKernelGGL((bwd_dkdv_kernel<DD, DR, 1, true>), g, blk, 0, s, a); \
      else hipLaunchKernelGGL((bwd_dkdv_kernel<DD, DR, 1, DR>), g, blk, 0, s, a);     \
    }                                                                                    \
  } while (0)
  if (head_dim == 64) {
    if (a.p.drop) FA_DKDV_LAUNCH(64, true);
    else FA_DKDV_LAUNCH(64, false);
  } else if (a.p.bm == nullptr && !a.p.drop && FA_DKDV_M16) {
    // No block mask or dropout at d=128 (causal, key padding and windows
    // allowed): the 16x16x32 kernel, 8 waves and 256 keys per workgroup.
    constexpr int NW = FA_DKDV_M16_WAVES;
    const int64_t nkb8 = (a.p.N + 32 * NW - 1) / (32 * NW);
    const dim3 g8((unsigned)((pair ? (nkb8 + 1) / 2 : nkb8) * a.p.Hkv * a.p.B));
    if (pair) hipLaunchKernelGGL((bwd_dkdv_kernel_m16<128, 2, NW>), g8, dim3(64 * NW), 0, s, a);
    else hipLaunchKernelGGL((bwd_dkdv_kernel_m16<128, 1, NW>), g8, dim3(64 * NW), 0, s, a);
  } else {
    if (a.p.drop) FA_DKDV_LAUNCH(128, true);
    else FA_DKDV_LAUNCH(128, false);
  }
#undef FA_DKDV_LAUNCH
  return hipGetLastError();
}

#ifndef FA_DQ_M16
#define FA_DQ_M16 1
#endif
#ifndef FA_DQ_M16_D64
#define FA_DQ_M16_D64 1
#endif
#ifndef FA_DQ_M16_WIDE_N
#define FA_DQ_M16_WIDE_N 8192
#endif

hipError_t launch_bwd_dq(const BwdArgs& a, int head_dim, hipStream_t s) {
  const int64_t grid = (int64_t)((a.p.N + 127) / 128) * a.p.Hq * a.p.B;
  const dim3 blk(256);
  // Pairs of query blocks where the causal work grows with the block index.
  const bool pair = a.p.causal && a.p.wl >= a.p.N;
  const dim3 g((unsigned)(pair ? ((a.p.N + 127) / 128 + 1) / 2 * a.p.Hq * a.p.B : grid));
  const bool mask = a.p.bm != nullptr || a.p.drop || a.p.wl < a.p.N || a.p.wr < a.p.N;
#define FA_DQ_LAUNCH(DD, DR)                                                             \
  do {                                                                                   \
    if (pair) {                                                                          \
      if (mask) hipLaunchKernelGGL((bwd_dq_kernel<DD, DR, 2, true>), g, blk, 0, s, a);   \
      else hipLaunchKernelGGL((bwd_dq_kernel<DD, DR, 2, DR>), g, blk, 0, s, a);       \
    } else {                                                                             \
      if (mask) hipLaunchKernelGGL((bwd_dq_kernel<DD, DR, 1, true>), g, blk, 0, s, a);   \
      else hipLaunchKernelGGL((bwd_dq_kernel<DD, DR, 1, DR>), g, blk, 0, s, a);       \
    }                                                                                    \
  } while (0)
  if (a.p.bm == nullptr && !a.p.drop && FA_DQ_M16 && (head_dim == 128 || FA_DQ_M16_D64)) {
    // No block mask or dropout (causal, key padding and windows allowed):
    // the 16x16x32 kernel (4 waves at d=64, where 8 would lose a wave per
    // SIMD).
    if (head_dim == 64) {
      if (pair) hipLaunchKernelGGL((bwd_dq_kernel_m16<64, 2, 4>), g, blk, 0, s, a);
      else hipLaunchKernelGGL((bwd_dq_kernel_m16<64, 1, 4>), g, blk, 0, s, a);
    } else if (a.p.N >= FA_DQ_M16_WIDE_N && a.p.wl >= a.p.N && a.p.wr >= a.p.N) {
      // Long rows without a window: 256 query rows per workgroup. Below this
      // length the larger causal diagonal block costs more than the halved
      // barriers save (N = 4096: 0.668 -> 0.682 ms; N = 16384: 2.454 ->
      // 2.381 ms); under a window the band's edge blocks do (N = 8192,
      // 1023 keys back: 0.414 ms with 128 rows, 0.468 ms with 256).
      const int64_t nqb8 = (a.p.N + 255) / 256;
      const dim3 g8((unsigned)((pair ? (nqb8 + 1) / 2 : nqb8) * a.p.Hq * a.p.B));
      if (pair) hipLaunchKernelGGL((bwd_dq_kernel_m16<128, 2, 8>), g8, dim3(512), 0, s, a);
      else hipLaunchKernelGGL((bwd_dq_kernel_m16<128, 1, 8>), g8, dim3(512), 0, s, a);
    } else {
      if (pair) hipLaunchKernelGGL((bwd_dq_kernel_m16<128, 2, 4>), g, blk, 0, s, a);
      else hipLaunchKernelGGL((bwd_dq_kernel_m16<128, 1, 4>), g, blk, 0, s, a);
    }
  } else if (head_dim == 64) {
    if (a.p.drop) FA_DQ_LAUNCH(64, true);
    else FA_DQ_LAUNCH(64, false);
  } else {
    if (a.p.drop) FA_DQ_LAUNCH(128, true);
    else FA_DQ_LAUNCH(128, false);
  }
#undef FA_DQ_LAUNCH
  return hipGetLastError();
}

}  // namespace fa

#if FA_TIMELINE
// Debug build only (fa_timeline.h): copy or clear the dQ (which = 0) or
// dK/dV (which = 1) stamps.
extern "C" int fa_timeline_bwd_read(int which, void* dst, size_t words) {
  if (words > (size_t)fa::kTlWorkgroups * fa::kTlSlots || which < 0 || which > 1) return -1;
  return which ? (int)hipMemcpyFromSymbol(dst, HIP_SYMBOL(fa::fa_tl_dkdv), words * 8, 0,
                                          hipMemcpyDeviceToHost)
               : (int)hipMemcpyFromSymbol(dst, HIP_SYMBOL(fa::fa_tl_dq), words * 8, 0,
                                          hipMemcpyDeviceToHost);
}
extern "C" int fa_timeline_bwd_clear() {
  void* a = nullptr;
  void* b = nullptr;
  if (hipGetSymbolAddress(&a, HIP_SYMBOL(fa::fa_tl_dq)) != hipSuccess ||
      hipGetSymbolAddress(&b, HIP_SYMBOL(fa::fa_tl_dkdv)) != hipSuccess)
    return -1;
  const size_t bytes = (size_t)fa::kTlWorkgroups * fa::kTlSlots * 8;
  if (hipMemset(a, 0, bytes) != hipSuccess) return -1;
  return (int)hipMemset(b, 0, bytes);
}
#endif

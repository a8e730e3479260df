// fa_fwd.hip -- tiled exact-attention forward for gfx950.
//
// One workgroup (4 waves, 256 lanes) owns one block of 128 query rows of one
// (batch, head) -- the Q-outer loop order that FlashAttention-2 introduced
// (zhaifeiyue.github.io cross-paper synthesis, section 2: outer loop over Q,
// split-Q work partition between warps). Each wave owns 32 of the rows and
// streams every visited K/V tile of the head through LDS:
//
//   S^T = K_j Q_i^T            bf16 MFMA, fp32 accumulators (32 keys x 32 rows)
//   mask, row max m~, m_new = max(m, m~), alpha = 2^(m - m_new)
//   P~ = 2^(s * scale * log2 e - m_new),  l = alpha * l + rowsum(P~)
//   O^T = alpha * O^T + V_j^T P~^T   bf16 MFMA (P~ rounded to bf16)
//
// which is the incremental softmax of the FlashAttention deep-reading report
// (zako-mio), sections 2.4 and 3.2, in base 2, with the normalisation by l
// delayed to the end (FlashAttention-2's delayed rescaling). Computing the
// transposed scores makes every lane own a single query row: the row max is
// 16 in-register compares plus one exchange with the other lane half, the
// row sum needs no exchange until the epilogue, and the P~ registers are
// already in the B-operand layout of the PV product.
//
// Tiles with no allowed entry (causal upper triangle, keys past the valid
// length, absent block-mask blocks) are skipped before they are loaded;
// element masks are applied only on tiles that straddle a boundary.
//
// Dropout (zako-mio report, section 3.2: part of the fused kernel): after
// P~ has entered the row sum, dropped entries are zeroed before the PV
// product, and the final 1 / l also carries the 1 / q rescale. Each lane
// regenerates its row's keep bits with one Philox call per run of 8
// consecutive keys it holds; nothing is stored.
#include "fa_philox.h"
#include "fa_stage.h"

namespace fa {

template <typename T, int D>
struct FwdCfg {
  static constexpr bool kBf16 = sizeof(T) == 2;
  static constexpr int BR = 128;                                        // rows per workgroup
  static constexpr int BC = kBf16 ? (D == 64 ? 128 : 64) : (D == 64 ? 64 : 32);  // keys per tile
  static constexpr int KC = Traits<T>::KC;
  static constexpr int EPC = Traits<T>::EPC;
  static constexpr int NKK = D / KC;     // MFMAs along d per 32 x 32 score block
  static constexpr int NSUB = BC / 32;   // 32-key sub-tiles per tile
  static constexpr int NDB = D / 32;     // 32-wide d blocks of O^T
  static constexpr int KROW = D + EPC;   // K tile pitch (16-byte pad)
  static constexpr int VROW = BC + EPC;  // transposed V tile pitch (16-byte pad)
};

template <typename T, int D>
__global__ __launch_bounds__(256) void fwd_kernel(FwdArgs a) {
  using C = FwdCfg<T, D>;
  using Frag = typename Traits<T>::Frag;
  __shared__ __attribute__((aligned(16))) T Ks[C::BC * C::KROW];
  __shared__ __attribute__((aligned(16))) T Vt[D * C::VROW];

  const Problem& p = a.p;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 31, hh = lane >> 5;

  const int nqb = (p.N + C::BR - 1) / C::BR;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int head_lin = L / nqb;
  const int qbi = L - head_lin * nqb;
  const int qb = p.causal ? nqb - 1 - qbi : qbi;  // causal: longest rows first
  const int b = head_lin / p.Hq, h = head_lin - b * p.Hq, hk = h / p.G;
  const int q0 = qb * C::BR;
  const int my_q = q0 + 32 * w + lr;

  const T* Qp = static_cast<const T*>(a.q) + b * a.sq.b + h * a.sq.h;
  const T* Kp = static_cast<const T*>(a.k) + b * a.sk.b + hk * a.sk.h;
  const T* Vp = static_cast<const T*>(a.v) + b * a.sv.b + hk * a.sv.h;

  const int kvalid = valid_keys(p.seqlens, b, p.N);
  const int kend = min(p.causal ? min(kvalid, q0 + C::BR) : kvalid, q0 + C::BR + p.wr);
  const int ntiles = (kend + C::BC - 1) / C::BC;

  // This lane's query row as the B operand of S^T = K Q^T.
  Frag qf[C::NKK];
  {
    const bool ok = my_q < p.N;
    const T* qrow = Qp + (int64_t)(ok ? my_q : 0) * a.sq.n + hh * (C::KC / 2);
#pragma unroll
    for (int kk = 0; kk < C::NKK; ++kk) qf[kk] = frag_g(qrow + kk * C::KC, ok);
  }

  f32x16 acc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) acc[db] = f32x16{};
  float m_run = -kInf;  // running max of raw scores
  float l_run = 0.f;    // this lane half's share of the running exp-sum
  const float sl2 = p.scale_l2;
  const int64_t log_row =
      a.log ? (((int64_t)b * p.Hq + h) * p.nlb + (q0 >> 7)) * p.logw : 0;

  // Visited tiles only: the block-mask scan is uniform per workgroup.
  MaskLine mrow = mask_row(p.bm, p.bm_ld, p.nlb, q0);
  for (int kt = mrow.next_tile<C::BC>(max(0, q0 - p.wl) / C::BC, ntiles); kt < ntiles;
       kt = mrow.next_tile<C::BC>(kt + 1, ntiles)) {
    const int key0 = kt * C::BC;
    __syncthreads();
    stage_rows<T, D, C::BC, C::KROW>(Kp, a.sk.n, key0, kvalid, Ks, tid);
    stage_cols<T, D, C::BC, C::VROW>(Vp, a.sv.n, key0, kvalid, Vt, tid);
    __syncthreads();
    if (a.log && tid == 0) log_tile(a.log, log_row, key0);

    // S^T for this wave's 32 rows against the tile's keys.
    f32x16 s[C::NSUB];
#pragma unroll
    for (int t = 0; t < C::NSUB; ++t) {
      s[t] = f32x16{};
      const T* krow = Ks + (32 * t + swap_bits23(lr)) * C::KROW + hh * (C::KC / 2);
#pragma unroll
      for (int kk = 0; kk < C::NKK; ++kk) s[t] = mfma(frag<T>(krow + kk * C::KC), qf[kk], s[t]);
    }

    const bool need_mask = (p.causal && key0 + C::BC - 1 > q0) || (key0 + C::BC > kvalid) ||
                           (key0 < q0 + C::BR - 1 - p.wl) || (key0 + C::BC - 1 > q0 + p.wr);
    if (__builtin_expect(need_mask, false)) {  // boundary tiles only
      // Key j is seen iff my_q - wl <= j <= my_q + hi (hi = 0 under the
      // causal mask, else the right window edge) and j < kvalid; the band
      // test is one unsigned compare of j - my_q + wl against wl + hi.
      const unsigned hi = p.causal ? 0u : (unsigned)p.wr;
      const unsigned span = (unsigned)p.wl + hi;
      const unsigned base = (unsigned)(key0 + 8 * hh + p.wl) - (unsigned)my_q;
#pragma unroll
      for (int t = 0; t < C::NSUB; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 32 * t + perm_row(r, hh);
          const bool kill =
              (base + (unsigned)(32 * t + perm_row(r, 0)) > span) | (key >= kvalid);
          s[t][r] = kill ? -kInf : s[t][r];  // branch-free select
        }
    }

    float mx = -kInf;
#pragma unroll
    for (int t = 0; t < C::NSUB; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[t][r]);
    mx = half_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_ref = (m_new == -kInf) ? 0.f : m_new * sl2;
    const float alpha = __builtin_amdgcn_exp2f(m_run * sl2 - m_ref);
    m_run = m_new;

    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < C::NSUB; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = __builtin_amdgcn_exp2f(fmaf(s[t][r], sl2, -m_ref));
        s[t][r] = e;
        psum += e;
      }
    l_run = fmaf(l_run, alpha, psum);
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
    if (p.drop) {  // register r of sub-tile t is key key0 + 32 t + perm_row(r, hh)
#pragma unroll
      for (int t = 0; t < C::NSUB; ++t)
#pragma unroll
        for (int c = 0; c < 2; ++c)
          drop_run8(s[t], 8 * c,
                    drop_bits(p, (uint32_t)(key0 + 32 * t + 16 * c + 8 * hh) >> 3,
                              (uint32_t)my_q, (uint32_t)(b * p.Hq + h)),
                    p.drop_thr);
    }

    // O^T += V^T P~^T: the P~ registers are the B operand directly.
#pragma unroll
    for (int t = 0; t < C::NSUB; ++t) {
      if constexpr (C::kBf16) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const bf16x8 pf = pack8(s[t], c);
#pragma unroll
          for (int db = 0; db < C::NDB; ++db) {
            const T* vp = Vt + (32 * db + lr) * C::VROW + 32 * t + 16 * c + 8 * hh;
            acc[db] = mfma(frag<T>(vp), pf, acc[db]);
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
#pragma unroll
          for (int db = 0; db < C::NDB; ++db) {
            const float vf = Vt[(32 * db + lr) * C::VROW + 32 * t + perm_row(r, hh)];
            acc[db] = mfma(vf, s[t][r], acc[db]);
          }
        }
      }
    }
  }

  // Epilogue: O = O~ / l (times 1 / q under dropout), LSE = m * scale + ln l.
  const float l_tot = half_sum(l_run);
  const float inv = l_tot > 0.f ? (p.drop ? p.drop_scale : 1.f) / l_tot : 0.f;
  if (my_q < p.N) {
    char* obase = static_cast<char*>(a.o);
    const int64_t orow = b * a.so.b + h * a.so.h + (int64_t)my_q * a.so.n;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * hh;
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
      const float lse = l_tot > 0.f ? (m_run * sl2 + __log2f(l_tot)) * kLn2 : -kInf;
      a.lse[((int64_t)b * p.Hq + h) * p.N + my_q] = lse;
    }
  }
}

// ------------------------------------------------------------------ bf16

template <int D>
struct FwdB {
  static constexpr int BR = 128;                  // rows per workgroup (4 waves x 32)
  static constexpr int BC = 64;                   // keys per tile
  static constexpr int NKK = D / 16;
  static constexpr int NSUB = BC / 32;
  static constexpr int NDB = D / 32;
  using T = SwzTile<D, BC>;
  // Running maxima are allowed to lag the true row maximum by up to this
  // much (log2 units): P~ then stays below 2^8, which bf16 and the fp32 sums
  // hold exactly as well as values below 1, and the O rescale (one multiply
  // per accumulator) is only paid when a row's maximum really grows.
  static constexpr float kLag = 8.f;
};

// MASK: the general variant, with the block-mask scan and the per-wave band
// skip compiled in, for launches with a block mask, a sliding window or
// dropout. Launches with none of them use the lean variant, which keeps its
// register allocation. (Dropout launches take the general one even without a
// mask: their allocation is better with it, 128 VGPRs and four waves per SIMD
// at d=64 against 149 without.)
template <int D, bool DROP, int NREP, bool MASK>
__global__ __launch_bounds__(256, 2) void fwd_kernel_bf16(FwdArgs a) {
  using C = FwdB<D>;
  using T = typename C::T;
  // Two stages of (K tile | V tile), filled by DMA while the other is read.
  __shared__ __attribute__((aligned(1024))) char smem[2][2 * T::BYTES];

  const Problem& p = a.p;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, hh = lane >> 5;

  const int nqb = (p.N + C::BR - 1) / C::BR;
  // Causal (NREP = 2): a workgroup takes query block nqb - 1 - i and then
  // block i, so that every workgroup does about the same work (nqb + 1
  // blocks of keys per pair) and the per-block prologue and epilogue are
  // spread over twice the tiles; heaviest block first. NREP = 1: one block.
  static_assert(NREP == 1 || NREP == 2, "one block or a pair");
  const int nunit = NREP == 2 ? (nqb + 1) / 2 : nqb;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int head_lin = L / nunit;
  const int ui = L - head_lin * nunit;
  const int b = head_lin / p.Hq, h = head_lin - b * p.Hq, hk = h / p.G;

  const int kvalid = __builtin_amdgcn_readfirstlane(valid_keys(p.seqlens, b, p.N));
  const int ksb = 2 * (int)a.sk.n, vsb = 2 * (int)a.sv.n;  // row strides in bytes
  const Rsrc krs = make_rsrc(static_cast<const bf16*>(a.k) + b * a.sk.b + hk * a.sk.h,
                             rows_extent(kvalid, ksb, 2 * D));
  const Rsrc vrs = make_rsrc(static_cast<const bf16*>(a.v) + b * a.sv.b + hk * a.sv.h,
                             rows_extent(kvalid, vsb, 2 * D));
  for (int rep = 0; rep < NREP; ++rep) {
    const int qb = NREP == 2 ? (rep == 0 ? nqb - 1 - ui : ui) : ui;
    if (rep == 1) {
      if (qb == nqb - 1 - ui) break;  // the middle block of an odd count
      __syncthreads();  // the first block's last tile is no longer read
    }
    const int q0 = qb * C::BR;
    const int my_q = q0 + 32 * w + lr;
    // Keys any row of the block may see: causal / padding / right window edge
    // bound the end, the left window edge the start.
    const int kend = min(p.causal ? min(kvalid, q0 + C::BR) : kvalid, q0 + C::BR + p.wr);
    const int ntiles = (kend + C::BC - 1) / C::BC;
    const int kfirst = max(0, q0 - p.wl) / C::BC;

    bf16x8 qf[C::NKK];
    {
      const bool ok = my_q < p.N;
      const bf16* qrow = static_cast<const bf16*>(a.q) + b * a.sq.b + h * a.sq.h +
                         (int64_t)(ok ? my_q : 0) * a.sq.n + 8 * hh;
#pragma unroll
      for (int kk = 0; kk < C::NKK; ++kk) qf[kk] = frag_g(qrow + 16 * kk, ok);
    }

    int kvo[T::NLD], vvo[T::NLD];
    dma_offsets<D, C::BC>(kvo, ksb, w, lane);
    dma_offsets<D, C::BC>(vvo, vsb, w, lane);
    int roff[C::NKK], troff[C::NDB][2];
    row_offsets<D, C::BC>(roff, lr, hh);
    tr_offsets<D, C::BC>(troff, lane);

    f32x16 acc[C::NDB];
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) acc[db] = f32x16{};
    float m_ref = -kInf;  // exponent reference of this lane's row (log2 units)
    float l_run = 0.f;    // this lane half's share of the row's exp-sum
    const float sl2 = p.scale_l2;
    const int64_t log_row =
        a.log ? (((int64_t)b * p.Hq + h) * p.nlb + (q0 >> 7)) * p.logw : 0;

    MaskLine mrow = mask_row(MASK ? p.bm : nullptr, p.bm_ld, p.nlb, q0);
    auto next_visit = [&](int kt) { return MASK ? mrow.next_tile<C::BC>(kt, ntiles) : kt; };
    auto issue = [&](int kt, char* stage) {
      dma_tile<D, C::BC>(krs, kvo, (uint32_t)(kt * C::BC) * ksb, stage, w);
      dma_tile<D, C::BC>(vrs, vvo, (uint32_t)(kt * C::BC) * vsb, stage + T::BYTES, w);
    };

    int kt = next_visit(kfirst);
    if (kt < ntiles) {
      issue(kt, smem[0]);
      wait_dma();
      __syncthreads();
    }
    // One key tile, read from stage `Ks` while the next visited tile lands in
    // `fill`. The two restrict-qualified stages tell the compiler that these
    // reads never alias that DMA, so it does not make the transposing reads
    // wait for the DMA to land.
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

      // A wave whose 32 rows see no key of the tile (above the causal
      // diagonal, outside the band) skips it: every score would be -inf,
      // every P~ exactly 0, and m, l and O come out bit-identical. Causal
      // pairs test the diagonal; one-block launches of the general variant
      // without dropout test the band; the rest compile no test.
      const int r0 = q0 + 32 * w;
      const bool wave_off =
          NREP == 2 ? key0 > r0 + 31
                    : MASK && !DROP &&
                          (key0 > r0 + 31 + (p.causal ? 0 : p.wr) || key0 + C::BC - 1 < r0 - p.wl);
      if (!wave_off) {
      // One straight-line block per tile (no per-sub-tile branches), so the
      // compiler can overlap one sub-tile's exponentials with its neighbour's
      // matrix products: all S^T products, one max and lazy-rescale test for
      // the whole tile, then exp / pack / PV per sub-tile.
      f32x16 s[C::NSUB];
      // Raised priority while this wave feeds the matrix pipe, so that waves
      // sharing the SIMD fill the VALU between its products.
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int t = 0; t < C::NSUB; ++t) s[t] = f32x16{};
      // Head-dim steps outer, sub-tiles inner: the sub-tiles' accumulation
      // chains interleave.
#pragma unroll
      for (int kk = 0; kk < C::NKK; ++kk)
#pragma unroll
        for (int t = 0; t < C::NSUB; ++t)
          s[t] = mfma(lds_row(Ks + 32 * t * T::RB, roff[kk]), qf[kk], s[t]);
      {
        // Keep four operand fragments in flight ahead of the products.
        constexpr int NM = C::NSUB * C::NKK;
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int i = 0; i < NM - 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      }
      __builtin_amdgcn_s_setprio(0);
      if (__builtin_expect(need_mask, false)) {  // boundary tiles only
        // Key j is seen iff my_q - wl <= j <= my_q + hi (hi = 0 under the
        // causal mask, else the right window edge) and j < kvalid; the band
        // test is one unsigned compare of j - my_q + wl against wl + hi.
        const unsigned hi = p.causal ? 0u : (unsigned)p.wr;
        const unsigned span = (unsigned)p.wl + hi;
        const unsigned base = (unsigned)(key0 + 8 * hh + p.wl) - (unsigned)my_q;
#pragma unroll
        for (int t = 0; t < C::NSUB; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + 32 * t + perm_row(r, hh);
            const bool kill =
                (base + (unsigned)(32 * t + perm_row(r, 0)) > span) | (key >= kvalid);
            s[t][r] = kill ? -kInf : s[t][r];  // branch-free select
          }
      }
      float mx = tree_max16(s[0]);
#pragma unroll
      for (int t = 1; t < C::NSUB; ++t) mx = fmaxf(mx, tree_max16(s[t]));
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
#pragma unroll
      for (int t = 0; t < C::NSUB; ++t) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[t][r] = __builtin_amdgcn_exp2f(fmaf(s[t][r], sl2, -m_use));
        l_run += tree_sum16(s[t]);
        if constexpr (DROP) {  // zero dropped entries after they entered l
#pragma unroll
          for (int c = 0; c < 2; ++c)
            drop_run8(s[t], 8 * c,
                      drop_bits(p, (uint32_t)(key0 + 32 * t + 16 * c + 8 * hh) >> 3,
                                (uint32_t)my_q, (uint32_t)(b * p.Hq + h)),
                      p.drop_thr);
        }
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const bf16x8 pf = pack8(s[t], c);
          const char* vp = Vs + (32 * t + 16 * c) * T::RB;
#pragma unroll
          for (int db = 0; db < C::NDB; ++db)
            acc[db] = mfma(lds_tr(vp, troff[db][0], troff[db][1]), pf, acc[db]);
        }
        {
          // Transposing reads of four operands in flight ahead of the products.
          constexpr int NM = 2 * C::NDB;
          __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
          for (int i = 0; i < NM - 4; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        }
        __builtin_amdgcn_s_setprio(0);
      }
      }  // !wave_off
      if (nxt < ntiles) {
        wait_dma();
        __syncthreads();  // next tile landed everywhere; this tile is no longer read
      }
      kt = nxt;
    };
    // Unrolled by two so that each copy reads a stage at a fixed LDS address:
    // every operand address is then a lane offset plus an immediate.
    while (kt < ntiles) {
      tile(smem[0], smem[1]);
      if (kt >= ntiles) break;
      tile(smem[1], smem[0]);
    }

    const float l_tot = half_sum(l_run);
    const float inv = l_tot > 0.f ? (DROP ? p.drop_scale : 1.f) / l_tot : 0.f;
    if (my_q < p.N) {
      char* obase = static_cast<char*>(a.o);
      const int64_t orow = b * a.so.b + h * a.so.h + (int64_t)my_q * a.so.n;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = 32 * db + 8 * g + 4 * hh;
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
  }  // q-blocks of this workgroup
}

// ------------------------------------------------------ bf16, 16x16x32 MFMA
//
// The forward without a block mask or dropout (causal, key padding and
// sliding windows allowed) on the
// v_mfma_f32_16x16x32_bf16 matrix instruction. Under the board's power
// limit a 16x16x32 product costs less energy per flop than a 32x32x16 one
// (it moves a quarter of the accumulator registers for half the flops), and
// the clock the limit allows rises accordingly. The tiling and staging are
// those of fwd_kernel_bf16: 128 query rows per workgroup, 32 per wave (two
// 16-row blocks), K/V tiles of 64 keys (four 16-key blocks) double-buffered
// in LDS by DMA.
//
// Layout of one 16x16x32 product (per lane l, i = l mod 16, g = l / 16):
// A supplies row i with K slots 8 g .. 8 g + 7, B column i with the same K
// slots, and the result holds column i, rows 4 g .. 4 g + 3. So with
//   S^T = K Q^T   (A: key rows from LDS, B: the lane's query rows)
// a lane holds, for each of its two query rows, keys 4 g .. 4 g + 3 of each
// 16-key block; taking the key blocks 2 c and 2 c + 1 together, those eight
// values are exactly a B operand of
//   O^T += V^T P~^T   (A: V^T from two transposing reads of 4 keys each)
// so P~ never leaves the registers. A row's 16 values per tile are spread
// over the 4 lanes i, i + 16, i + 32, i + 48: the row maximum and the row
// sum finish with two lane swaps (permlane16 and permlane32).

#if FA_TIMELINE
// Timeline stamps of the 16x16x32 forward (debug build).
__device__ unsigned long long fa_tl_fwd[kTlWorkgroups * kTlSlots];
#endif

template <int D>
struct FwdM {
  static constexpr int BR = 128;    // rows per workgroup (4 waves x 2 blocks of 16)
  static constexpr int BC = 64;     // keys per tile (4 blocks of 16)
  static constexpr int NKB = BC / 16;
  static constexpr int NDC = D / 32;  // 32-wide head-dim chunks of the S products
  static constexpr int NDB = D / 16;  // 16-wide head-dim blocks of O^T
  using T = SwzTile<D, BC, 1>;
  static constexpr float kLag = 8.f;
};

template <int D, int NREP>
__global__ __launch_bounds__(256, 2) void fwd_kernel_m16(FwdArgs a) {
  using C = FwdM<D>;
  using T = typename C::T;
  __shared__ __attribute__((aligned(1024))) char smem[2][2 * T::BYTES];

  const Problem& p = a.p;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;

  const int nqb = (p.N + C::BR - 1) / C::BR;
  static_assert(NREP == 1 || NREP == 2, "one block or a pair");
  const int nunit = NREP == 2 ? (nqb + 1) / 2 : nqb;
  int head_lin, ui;
  if (NREP == 1 && a.order) {
    // Heaviest blocks first. Workgroup i runs on XCD i mod 8 and is that
    // XCD's (i / 8)-th workgroup. With the key/value heads (b * Hkv + hk) a
    // multiple of 8 in number, XCD x takes the heads congruent to x mod 8,
    // block level by block level, the G query heads of each together, so
    // each K/V head stays in one XCD's L2; otherwise workgroup i takes block
    // nqb - 1 - i / heads of query head i mod heads.
    const int ng = p.B * p.Hkv;
    if ((ng & 7) == 0) {
      const unsigned per = (unsigned)(ng >> 3) * (unsigned)p.G;  // items per level per XCD
      const unsigned j = blockIdx.x >> 3;
      const unsigned r = j % per;
      const int grp = (int)(blockIdx.x & 7) + 8 * (int)(r / (unsigned)p.G);
      head_lin = grp * p.G + (int)(r % (unsigned)p.G);
      ui = nqb - 1 - (int)(j / per);
    } else {
      const int nh = p.Hq * p.B;
      head_lin = (int)(blockIdx.x % (unsigned)nh);
      ui = nqb - 1 - (int)(blockIdx.x / (unsigned)nh);
    }
  } else {
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    head_lin = L / nunit;
    ui = L - head_lin * nunit;
  }
  const int b = head_lin / p.Hq, h = head_lin - b * p.Hq, hk = h / p.G;

  const int kvalid = __builtin_amdgcn_readfirstlane(valid_keys(p.seqlens, b, p.N));
  const int ksb = 2 * (int)a.sk.n, vsb = 2 * (int)a.sv.n;
  const Rsrc krs = make_rsrc(static_cast<const bf16*>(a.k) + b * a.sk.b + hk * a.sk.h,
                             rows_extent(kvalid, ksb, 2 * D));
  const Rsrc vrs = make_rsrc(static_cast<const bf16*>(a.v) + b * a.sv.b + hk * a.sv.h,
                             rows_extent(kvalid, vsb, 2 * D));
  const float sl2 = p.scale_l2;
  FA_TL(fa_tl_fwd, 0, tl_now());
  FA_TL(fa_tl_fwd, 1, tl_where());

  for (int rep = 0; rep < NREP; ++rep) {
    const int qb = NREP == 2 ? (rep == 0 ? nqb - 1 - ui : ui) : ui;
    if (rep == 1) {
      if (qb == nqb - 1 - ui) break;  // the middle block of an odd count
      __syncthreads();                // the first block's last tile is no longer read
    }
    const int q0 = qb * C::BR;
    const int r0 = q0 + 32 * w;  // first row of this wave
    // Keys any row of the block may see: causal / padding / right window
    // edge bound the end, the left window edge the start.
    const int kend = min(p.causal ? min(kvalid, q0 + C::BR) : kvalid, q0 + C::BR + p.wr);
    const int ntiles = (kend + C::BC - 1) / C::BC;

    // The lane's two query rows r0 + li and r0 + 16 + li as B operands:
    // head-dim chunk dc, slots 8 lg .. 8 lg + 7.
    bf16x8 qf[2][C::NDC];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int row = r0 + 16 * rb + li;
      const bool ok = row < p.N;
      const bf16* qrow = static_cast<const bf16*>(a.q) + b * a.sq.b + h * a.sq.h +
                         (int64_t)(ok ? row : 0) * a.sq.n + 8 * lg;
#pragma unroll
      for (int dc = 0; dc < C::NDC; ++dc) qf[rb][dc] = frag_g(qrow + 32 * dc, ok);
    }
    int kvo[T::NLD], vvo[T::NLD];
    dma_offsets_t<T>(kvo, ksb, w, lane);
    dma_offsets_t<T>(vvo, vsb, w, lane);
    // K operand of key block kb, chunk dc: key row 16 kb + li, 16-byte chunk
    // 4 dc + lg; the swizzle depends on the row's low 4 bits only, so block
    // kb adds 16 kb rows as an immediate.
    int koff[C::NDC];
#pragma unroll
    for (int dc = 0; dc < C::NDC; ++dc) koff[dc] = T::off(li, 4 * dc + lg);
    // V^T operand of head-dim block db (rows 16 db + li of the result): the
    // transposing read of lane 4 e + a of group lg loads key row 4 lg + e
    // (+ 16 for the second read, + 32 c for key slice c, both immediates) at
    // head-dim 16 db + 4 a.
    int voff[C::NDB];
    {
      const int rr = 4 * lg + (li >> 2), aa = li & 3;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        const int d = 16 * db + 4 * aa;
        voff[db] = rr * T::RB + 16 * ((d >> 3) ^ T::swz(rr)) + 2 * (d & 7);
      }
    }

    f32x4 acc[C::NDB][2];
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) acc[db][0] = acc[db][1] = f32x4{};
    float m_ref[2] = {-kInf, -kInf};  // exponent references of the two rows (log2 units)
    float l_run[2] = {0.f, 0.f};      // this lane's share of each row's exp-sum
    const int64_t log_row =
        a.log ? (((int64_t)b * p.Hq + h) * p.nlb + (q0 >> 7)) * p.logw : 0;

    auto issue = [&](int kt, char* stage) {
      dma_tile<D, C::BC>(krs, kvo, (uint32_t)(kt * C::BC) * ksb, stage, w);
      dma_tile<D, C::BC>(vrs, vvo, (uint32_t)(kt * C::BC) * vsb, stage + T::BYTES, w);
    };
    FA_TL(fa_tl_fwd, 2 + 4 * rep, tl_now());
    int kt = max(0, q0 - p.wl) / C::BC;
    if (kt < ntiles) {
      issue(kt, smem[0]);
      wait_dma();
      __syncthreads();
    }
    FA_TL(fa_tl_fwd, 3 + 4 * rep, tl_now());
    auto tile = [&](const char* __restrict__ Ks, char* __restrict__ fill) {
      const char* Vs = Ks + T::BYTES;
      const int key0 = kt * C::BC;
      const int nxt = kt + 1;
      if (nxt < ntiles) {
        paranoid_before_fill();
        issue(nxt, fill);
        paranoid_after_fill();
      }
      if (a.log && tid == 0) log_tile(a.log, log_row, key0);
      // (Causal pairs never carry a window: its terms compile into the
      // one-block instances only.)
      const bool need_mask =
          (p.causal && key0 + C::BC - 1 > q0) || (key0 + C::BC > kvalid) ||
          (NREP == 1 && ((key0 < q0 + C::BR - 1 - p.wl) || (key0 + C::BC - 1 > q0 + p.wr)));
      // A wave whose rows see no key of the tile (above the causal diagonal,
      // outside the band) skips it: every score -inf, P~ = 0, and m, l and O
      // come out bit-identical.
      const bool wave_off = NREP == 2 ? key0 > r0 + 31
                                      : key0 > r0 + 31 + (p.causal ? 0 : p.wr) ||
                                            key0 + C::BC - 1 < r0 - p.wl;
      if (!wave_off) {
        f32x4 s[C::NKB][2];
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) s[kb][0] = s[kb][1] = f32x4{};
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int dc = 0; dc < C::NDC; ++dc)
#pragma unroll
          for (int kb = 0; kb < C::NKB; ++kb) {
            const bf16x8 kf = lds_row(Ks + 16 * kb * T::RB, koff[dc]);
            s[kb][0] = mfma16(kf, qf[0][dc], s[kb][0]);
            s[kb][1] = mfma16(kf, qf[1][dc], s[kb][1]);
          }
        {
          // Operand reads PF ahead of the products (two products per read).
          constexpr int NR = C::NDC * C::NKB, PF = D == 64 ? 2 : 4;
          __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);
#pragma unroll
          for (int i = 0; i < NR - PF; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, 2 * PF, 0);
        }
        __builtin_amdgcn_s_setprio(0);
        if (__builtin_expect(need_mask, false)) {
          // Register r of key block kb is key key0 + 16 kb + 4 lg + r. Row i
          // sees key j iff i - wl <= j <= i + hi (hi = 0 under the causal
          // mask, else the right window edge) and j < kvalid: one unsigned
          // compare of j - i + wl against wl + hi.
          const unsigned span = (unsigned)p.wl + (p.causal ? 0u : (unsigned)p.wr);
#pragma unroll
          for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int key = key0 + 16 * kb + 4 * lg + r;
                const int row = r0 + 16 * rb + li;
                const bool kill = key >= kvalid || (NREP == 2 ? key > row
                                                              : (unsigned)(key - row + p.wl) > span);
                s[kb][rb][r] = kill ? -kInf : s[kb][rb][r];
              }
        }
        // Row maxima: a chain of three-input maxima over the lane's 16 values
        // of each row, then one lane exchange for both rows.
        float mx[2];
        {
          float m2[2];
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            float m = fmaxf(s[0][rb][0], s[0][rb][1]);
#pragma unroll
            for (int k = 2; k < 4 * C::NKB; k += 2)
              m = fmaxf(fmaxf(m, s[k >> 2][rb][k & 3]), s[(k + 1) >> 2][rb][(k + 1) & 3]);
            m2[rb] = m;
          }
          quad_max2(m2[0], m2[1], mx[0], mx[1]);
          mx[0] *= sl2;
          mx[1] *= sl2;
        }
        if (wave_any(mx[0] > m_ref[0] + C::kLag || mx[1] > m_ref[1] + C::kLag)) {
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            const float m_new = fmaxf(m_ref[rb], mx[rb]);
            const float alpha =
                m_new == -kInf ? 1.f : __builtin_amdgcn_exp2f(m_ref[rb] - m_new);
            m_ref[rb] = m_new;
            l_run[rb] *= alpha;
#pragma unroll
            for (int db = 0; db < C::NDB; ++db)
#pragma unroll
              for (int r = 0; r < 4; ++r) acc[db][rb][r] *= alpha;
          }
        }
        const float mu0 = m_ref[0] == -kInf ? 0.f : m_ref[0];
        const float mu1 = m_ref[1] == -kInf ? 0.f : m_ref[1];
        // Per 32-key slice c: exponentials of key blocks 2 c, 2 c + 1, then
        // the PV products of the slice (the next slice's exponentials can run
        // under them).
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          bf16x8 pf[2];
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            const float mu = rb ? mu1 : mu0;
            float ps = 0.f;
#pragma unroll
            for (int hb = 0; hb < 2; ++hb)
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const float e = __builtin_amdgcn_exp2f(fmaf(s[2 * c + hb][rb][r], sl2, -mu));
                ps += e;
                pf[rb][4 * hb + r] = (bf16)e;
              }
            l_run[rb] += ps;
          }
          __builtin_amdgcn_s_setprio(1);
          const char* vp = Vs + 32 * c * T::RB;
#pragma unroll
          for (int db = 0; db < C::NDB; ++db) {
            const bf16x8 vf = lds_tr(vp, voff[db], voff[db] + 16 * T::RB);
            acc[db][0] = mfma16(vf, pf[0], acc[db][0]);
            acc[db][1] = mfma16(vf, pf[1], acc[db][1]);
          }
          {
            // PF operands (2 PF transposing reads) ahead of the products.
            constexpr int PF = D == 64 ? 2 : 4;
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * PF, 0);
#pragma unroll
            for (int i = 0; i < C::NDB - PF; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
              __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 2 * PF, 0);
          }
          __builtin_amdgcn_s_setprio(0);
        }
      }  // !wave_off
      if (nxt < ntiles) {
        wait_dma();
        __syncthreads();  // next tile landed everywhere; this tile is no longer read
      }
      kt = nxt;
    };
    while (kt < ntiles) {
      tile(smem[0], smem[1]);
      if (kt >= ntiles) break;
      tile(smem[1], smem[0]);
    }
    FA_TL(fa_tl_fwd, 4 + 4 * rep, tl_now());
    FA_TL(fa_tl_fwd, 5 + 4 * rep, ((unsigned long long)qb << 16) | (unsigned)ntiles);

#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int row = r0 + 16 * rb + li;
      const float l_tot = quad_sum(l_run[rb]);
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      if (row < p.N) {
        char* obase = static_cast<char*>(a.o);
        const int64_t orow = b * a.so.b + h * a.so.h + (int64_t)row * a.so.n;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
          const int d0 = 16 * db + 4 * lg;
          const float v0 = acc[db][rb][0] * inv, v1 = acc[db][rb][1] * inv;
          const float v2 = acc[db][rb][2] * inv, v3 = acc[db][rb][3] * inv;
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
        if (lg == 0) {
          const float lse = l_tot > 0.f ? (m_ref[rb] + __log2f(l_tot)) * kLn2 : -kInf;
          a.lse[((int64_t)b * p.Hq + h) * p.N + row] = lse;
        }
      }
    }
  }  // q-blocks of this workgroup
  FA_TL(fa_tl_fwd, 10, tl_now());
}

// fp32 inputs (reference-precision path) use the generic kernel above.
template <typename T, int D>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t s) {
  const int64_t nqb = (a.p.N + 127) / 128;
  const int64_t grid = nqb * a.p.Hq * a.p.B;
  hipLaunchKernelGGL((fwd_kernel<T, D>), dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

// Launches without a block mask or dropout at d=128 (causal, key padding
// and sliding windows allowed) take the 16x16x32 kernel; at d=64 the
// 32x32x16 kernel fits four waves per SIMD (the 16x16x32 one needs 142
// VGPRs there) and stays faster.
template <int D, bool DROP, int NREP>
static void launch_fwd_bf16_m(const FwdArgs& a, dim3 g, hipStream_t s) {
  const bool window = a.p.wl < a.p.N || a.p.wr < a.p.N;
  if (DROP || a.p.bm) {
    hipLaunchKernelGGL((fwd_kernel_bf16<D, DROP, NREP, true>), g, dim3(256), 0, s, a);
  } else if constexpr (D == 128) {
    hipLaunchKernelGGL((fwd_kernel_m16<D, NREP>), g, dim3(256), 0, s, a);
  } else if (window) {
    hipLaunchKernelGGL((fwd_kernel_bf16<D, DROP, NREP, true>), g, dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL((fwd_kernel_bf16<D, DROP, NREP, DROP>), g, dim3(256), 0, s, a);
  }
}

#ifndef FA_FWD_HEAVY_FIRST_N
#define FA_FWD_HEAVY_FIRST_N 8192
#endif

template <int D>
static hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t s) {
  const int64_t nqb = (a.p.N + FwdB<D>::BR - 1) / FwdB<D>::BR;
  const bool causal_full = a.p.causal && a.p.wl >= a.p.N;
  // Long causal rows at d = 128 (no block mask or dropout): single blocks,
  // heaviest first. A mirror pair there is two blocks of up to N / 64 tiles,
  // and the grid ends on a long tail of the last pairs; single blocks in
  // decreasing size end on the lightest ones. At N = 4096 the pairs are
  // short, and the single-block order measured no faster.
  if (D == 128 && causal_full && !a.p.drop && !a.p.bm && a.p.N >= FA_FWD_HEAVY_FIRST_N) {
    FwdArgs b = a;
    b.order = 1;
    launch_fwd_bf16_m<D, false, 1>(b, dim3((unsigned)(nqb * a.p.Hq * a.p.B)), s);
    return hipGetLastError();
  }
  // Pairs of query blocks where the work per block grows with the block
  // index (causal, no left window edge); under a sliding window every block
  // already does about the same work.
  if (causal_full) {
    const dim3 g((unsigned)(((nqb + 1) / 2) * a.p.Hq * a.p.B));
    if (a.p.drop) launch_fwd_bf16_m<D, true, 2>(a, g, s);
    else launch_fwd_bf16_m<D, false, 2>(a, g, s);
  } else {
    const dim3 g((unsigned)(nqb * a.p.Hq * a.p.B));
    if (a.p.drop) launch_fwd_bf16_m<D, true, 1>(a, g, s);
    else launch_fwd_bf16_m<D, false, 1>(a, g, s);
  }
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs& a, int dtype, int head_dim, hipStream_t s) {
  if (dtype == 0) {
    return head_dim == 64 ? launch_fwd_bf16<64>(a, s) : launch_fwd_bf16<128>(a, s);
  }
  return head_dim == 64 ? launch_fwd_t<float, 64>(a, s) : launch_fwd_t<float, 128>(a, s);
}

}  // namespace fa

#if FA_TIMELINE
// Debug build only (fa_timeline.h): copy or clear the forward's stamps.
extern "C" int fa_timeline_fwd_read(void* dst, size_t words) {
  if (words > (size_t)fa::kTlWorkgroups * fa::kTlSlots) return -1;
  return (int)hipMemcpyFromSymbol(dst, HIP_SYMBOL(fa::fa_tl_fwd), words * 8, 0,
                                  hipMemcpyDeviceToHost);
}
extern "C" int fa_timeline_fwd_clear() {
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(fa::fa_tl_fwd)) != hipSuccess) return -1;
  return (int)hipMemset(ptr, 0, (size_t)fa::kTlWorkgroups * fa::kTlSlots * 8);
}
#endif

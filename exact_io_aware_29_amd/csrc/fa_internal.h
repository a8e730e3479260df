// fa_internal.h -- argument blocks passed from the C ABI layer to the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct Strides {
  int64_t b, h, n;
};

// Shape and mask of one call, already validated on the host.
struct Problem {
  int B, Hq, Hkv, N, G;
  float scale;      // softmax scale (> 0)
  float scale_l2;   // scale * log2(e): scores enter exp2 in this unit
  int causal;
  const int32_t* seqlens;  // device [B] or null
  const uint8_t* bm;       // device block mask or null
  int bm_ld;
  int nlb;   // ceil(N / 128): 128-blocks per sequence
  int logw;  // uint32 words per tile-log row: ceil(nlb / 32)
  int wl, wr;  // sliding window: key j allowed for query i iff i - wl <= j <= i + wr
               // (both in [0, N]; N when there is no window)
  // Dropout (drop != 0): element kept iff its 16-bit Philox uniform is below
  // drop_thr (1 .. 65535); kept probabilities are scaled by drop_scale =
  // 65536 / drop_thr, and drop_q = drop_thr / 65536 is the keep probability.
  int drop;
  uint32_t drop_thr;
  float drop_scale, drop_q;
  uint32_t seed_lo, seed_hi, drop_off;
};

struct FwdArgs {
  Problem p;
  const void* q;
  const void* k;
  const void* v;
  void* o;
  Strides sq, sk, sv, so;
  float* lse;
  uint32_t* log;
  int o_fp32;
  float qk_descale;  // FP8 inputs: descale_q * descale_k (scores) ...
  float v_descale;   // ... and descale_v (output)
  // Grid order of one-block launches: 0 = head-major (XCD-remapped);
  // 1 = heaviest blocks first, workgroup i taking block nqb - 1 - i / heads
  // of head i mod heads (causal launches only).
  int order = 0;
};

struct BwdArgs {
  Problem p;
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  Strides sq, sk, sv, so, sdo, sdq, sdk, sdv;
  const float* lse;
  float* dvec;  // workspace: D = rowsum(dO * O) (q D under dropout), fp32 [B][Hq][N],
                // written by the dQ kernel and read by the dK/dV kernel
  float* lse2;  // workspace: LSE * log2(e) (+inf for empty rows), fp32 [B][Hq][N], likewise
  void* dq;
  void* dk;
  void* dv;
  uint32_t* log_kv;  // tiles visited by the dK/dV kernel (or null)
  uint32_t* log_q;   // tiles visited by the dQ kernel (or null)
  int o_fp32;
};

// Decode: one query row per head (q, o: [B][Hq][.][d], row index 0 only)
// against a cache of N keys, split into `splits` ranges of `split_len` keys.
struct DecodeArgs {
  Problem p;
  const void* q;
  const void* k;
  const void* v;
  void* o;
  Strides sq, sk, sv, so;
  float* lse;     // [B][Hq], natural log
  float* ws_o;    // workspace: per-split normalised partials [B][Hq][splits][d]
  float* ws_lse;  // workspace: per-split log2-sum-exp [B][Hq][splits]
  int splits, split_len, hblocks;
  int o_fp32;
};

// Launchers (defined next to their kernels). dtype: 0 bf16, 1 fp32.
hipError_t launch_fwd(const FwdArgs& a, int dtype, int head_dim, hipStream_t s);
hipError_t launch_fwd_fp8(const FwdArgs& a, int head_dim, hipStream_t s);
hipError_t launch_bwd_dkdv(const BwdArgs& a, int head_dim, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, int head_dim, hipStream_t s);
hipError_t launch_bwd_dq(const BwdArgs& a, int head_dim, hipStream_t s);

// Device address of the library's fixed scratch array on the current device
// (looked up once per device); it holds FA_NOALLOC_WORKSPACE_BYTES.
hipError_t scratch_address(void** out);

}  // namespace fa

// fa_api.cpp -- C ABI entry points: host-side validation, then kernel launch.
//
// Every check runs on the host before the first HIP call, so an invalid call
// returns a status code without touching the GPU (and can be tested on a
// machine without one).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/fa.h"
#include "fa_internal.h"

#define FA_CHECK(expr)            \
  do {                            \
    const int st_ = (expr);       \
    if (st_ != FA_OK) return st_; \
  } while (0)

namespace {

thread_local char g_detail[256] = "";

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_detail, sizeof(g_detail), fmt, ap);
  va_end(ap);
  return status;
}

size_t elem_size(int dtype) { return dtype == FA_BF16 ? 2 : dtype == FA_FP8_E4M3 ? 1 : 4; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Keep threshold T = round((1 - p) * 65536) (ties away from zero), in double.
int64_t keep_threshold(float p) {
  return (int64_t)std::floor((1.0 - (double)p) * 65536.0 + 0.5);
}

int check_params(const fa_params* p) {
  if (!p) return fail(FA_ERR_NULL, "params is NULL");
  if (p->dtype != FA_BF16 && p->dtype != FA_FP32 && p->dtype != FA_FP8_E4M3)
    return fail(FA_ERR_DTYPE, "dtype %d is not FA_BF16, FA_FP32 or FA_FP8_E4M3", p->dtype);
  if (p->o_dtype != FA_BF16 && p->o_dtype != FA_FP32)
    return fail(FA_ERR_DTYPE, "o_dtype %d is not FA_BF16 or FA_FP32", p->o_dtype);
  if (p->dtype == FA_FP32 && p->o_dtype != FA_FP32)
    return fail(FA_ERR_DTYPE, "fp32 inputs need an fp32 output");
  if (p->batch <= 0 || p->heads_q <= 0 || p->heads_kv <= 0 || p->seqlen <= 0)
    return fail(FA_ERR_SHAPE, "batch, heads and seqlen must be positive");
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(FA_ERR_HEADDIM, "head_dim %d is not 64 or 128", p->head_dim);
  if (p->heads_q % p->heads_kv != 0)
    return fail(FA_ERR_GQA, "heads_q %d is not a multiple of heads_kv %d", p->heads_q, p->heads_kv);
  if (!std::isfinite(p->scale) || !(p->scale > 0.f))
    return fail(FA_ERR_SCALE, "scale must be finite and positive");
  if (p->seqlen > (1 << 30)) return fail(FA_ERR_SHAPE, "seqlen above 2^30");
  const int64_t blocks = ceil_div(p->seqlen, 128);
  const int64_t grid_q = blocks * p->heads_q * p->batch;
  if (grid_q >= (int64_t(1) << 31) || (int64_t)p->batch * p->heads_q * p->seqlen >= (int64_t(1) << 40))
    return fail(FA_ERR_SHAPE, "problem too large to index");
  if (p->window && (p->window_left < 0 || p->window_right < 0))
    return fail(FA_ERR_MASK, "window widths must be >= 0 (got %d, %d)", p->window_left,
                p->window_right);
  if (!(p->dropout_p >= 0.f && p->dropout_p < 1.f))
    return fail(FA_ERR_DROPOUT, "dropout_p must lie in [0, 1) (got %g)", (double)p->dropout_p);
  if (p->dropout_p > 0.f && keep_threshold(p->dropout_p) <= 0)
    return fail(FA_ERR_DROPOUT, "dropout_p %g drops every element", (double)p->dropout_p);
  if (p->dtype == FA_FP8_E4M3) {
    const float ds[3] = {p->descale_q, p->descale_k, p->descale_v};
    for (float x : ds)
      if (!std::isfinite(x) || !(x > 0.f))
        return fail(FA_ERR_SCALE, "FP8 descale factors must be finite and positive");
    if (p->dropout_p != 0.f) return fail(FA_ERR_DROPOUT, "the FP8 forward takes no dropout");
  }
  if (p->block_mask && p->block_mask_ld < blocks)
    return fail(FA_ERR_MASK, "block_mask_ld %d < ceil(seqlen/128) = %lld", p->block_mask_ld,
                (long long)blocks);
  // The kernels read 64 consecutive blocks of a mask column at once, at
  // 32-bit byte offsets of up to 63 pitches.
  if (p->block_mask && p->block_mask_ld > (1 << 24))
    return fail(FA_ERR_MASK, "block_mask_ld %d is above 2^24", p->block_mask_ld);
  return FA_OK;
}

int check_tensor(const char* name, const void* ptr, fa_strides s, int dtype) {
  if (!ptr) return fail(FA_ERR_NULL, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(ptr) % 16 != 0)
    return fail(FA_ERR_ALIGN, "%s is not 16-byte aligned", name);
  const int64_t q = 16 / (int64_t)elem_size(dtype);
  if (s.batch < 0 || s.head < 0 || s.row < 0 || s.batch % q || s.head % q || s.row % q)
    return fail(FA_ERR_STRIDE, "%s strides must be >= 0 and multiples of 16 bytes", name);
  return FA_OK;
}

// Rows of one head must not overlap: the kernels read a tile's rows past
// the sequence (or past a batch entry's valid key count) as zeros through a
// buffer resource whose extent ends at the last valid row, which only
// excludes the rows after it if each row starts past the previous row's
// data. Outputs with overlapping rows would be written by several lanes.
int check_rows(const char* name, fa_strides s, const fa_params* p) {
  if (s.row < p->head_dim)
    return fail(FA_ERR_STRIDE, "%s: row stride %lld is below head_dim %d (rows overlap)", name,
                (long long)s.row, p->head_dim);
  return FA_OK;
}

// The kernels address a head's rows of a staged tensor (K and V; Q and dO
// in the backward) through a buffer resource with 32-bit byte offsets and a
// 32-bit extent. Tiles cover whole 128-row blocks, so the rows addressed run
// up to ceil(N / 128) * 128 - 1, past the last row when N is not a multiple
// of 128: every byte of every such row must lie below offset 2^32, or its
// offset would wrap back inside the resource and read real data where zeros
// are meant; and the extent of the N rows must itself fit 32 bits.
int check_span(const char* name, fa_strides s, const fa_params* p, int dtype) {
  FA_CHECK(check_rows(name, s, p));
  const int64_t e = (int64_t)elem_size(dtype);
  const int64_t rows = ceil_div(p->seqlen, FA_MASK_BLOCK) * FA_MASK_BLOCK;
  const int64_t span = (rows - 1) * s.row * e + (int64_t)p->head_dim * e;
  const int64_t extent = (int64_t)(p->seqlen - 1) * s.row * e + (int64_t)p->head_dim * e;
  if (span > ((int64_t)1 << 32) || extent > (int64_t)UINT32_MAX)
    return fail(FA_ERR_SHAPE,
                "%s: the %lld rows of one head's 128-row tiles span %lld bytes (row stride %lld); "
                "the limit is 4 GiB",
                name, (long long)rows, (long long)span, (long long)(s.row * e));
  return FA_OK;
}

fa::Problem make_problem(const fa_params* p) {
  fa::Problem pr;
  pr.B = p->batch;
  pr.Hq = p->heads_q;
  pr.Hkv = p->heads_kv;
  pr.N = p->seqlen;
  pr.G = p->heads_q / p->heads_kv;
  pr.scale = p->scale;
  pr.scale_l2 = p->scale * 1.4426950408889634f;
  pr.causal = p->causal != 0;
  pr.seqlens = p->seqlens_k;
  pr.bm = p->block_mask;
  pr.bm_ld = p->block_mask_ld;
  pr.nlb = (int)ceil_div(p->seqlen, 128);
  pr.logw = (int)ceil_div(pr.nlb, 32);
  // Band widths; without a window (or beyond the sequence) the band covers
  // every key, and the kernels apply it unconditionally.
  pr.wl = p->window ? (int)std::min<int64_t>(p->window_left, p->seqlen) : p->seqlen;
  pr.wr = p->window ? (int)std::min<int64_t>(p->window_right, p->seqlen) : p->seqlen;
  // T = 65536 keeps every element with scale 1: that is no dropout.
  const int64_t thr = p->dropout_p > 0.f ? keep_threshold(p->dropout_p) : 65536;
  pr.drop = thr < 65536;
  pr.drop_thr = (uint32_t)std::min<int64_t>(thr, 65535);
  pr.drop_scale = (float)(65536.0 / (double)thr);
  pr.drop_q = (float)((double)thr / 65536.0);
  pr.seed_lo = (uint32_t)(p->dropout_seed & 0xFFFFFFFFu);
  pr.seed_hi = (uint32_t)(p->dropout_seed >> 32);
  pr.drop_off = p->dropout_offset;
  return pr;
}

fa::Strides conv(fa_strides s) { return fa::Strides{s.batch, s.head, s.row}; }

int hip_fail(hipError_t e, const char* what) {
  return fail(FA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" {

size_t fa_tile_log_words(const fa_params* p) {
  if (check_params(p) != FA_OK) return 0;
  const int64_t nlb = ceil_div(p->seqlen, 128);
  return (size_t)p->batch * p->heads_q * nlb * ceil_div(nlb, 32);
}

size_t fa_bwd_workspace_size(const fa_params* p) {
  if (check_params(p) != FA_OK) return 0;
  return 2 * (size_t)p->batch * p->heads_q * p->seqlen * sizeof(float);
}

int fa_fwd(const fa_params* p, const void* q, fa_strides sq, const void* k, fa_strides sk,
           const void* v, fa_strides sv, void* o, fa_strides so, float* lse, uint32_t* tile_log,
           void* stream) {
  g_detail[0] = '\0';
  FA_CHECK(check_params(p));
  FA_CHECK(check_tensor("q", q, sq, p->dtype));
  FA_CHECK(check_tensor("k", k, sk, p->dtype));
  FA_CHECK(check_tensor("v", v, sv, p->dtype));
  FA_CHECK(check_tensor("o", o, so, p->o_dtype));
  FA_CHECK(check_span("k", sk, p, p->dtype));
  FA_CHECK(check_span("v", sv, p, p->dtype));
  FA_CHECK(check_rows("q", sq, p));
  FA_CHECK(check_rows("o", so, p));
  if (!lse) return fail(FA_ERR_NULL, "lse is NULL");
  if (reinterpret_cast<uintptr_t>(lse) % 4) return fail(FA_ERR_ALIGN, "lse is not 4-byte aligned");
  if (tile_log && reinterpret_cast<uintptr_t>(tile_log) % 4)
    return fail(FA_ERR_ALIGN, "tile_log is not 4-byte aligned");

  fa::FwdArgs a;
  a.p = make_problem(p);
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.sq = conv(sq);
  a.sk = conv(sk);
  a.sv = conv(sv);
  a.so = conv(so);
  a.lse = lse;
  a.log = tile_log;
  a.o_fp32 = p->o_dtype == FA_FP32;
  a.qk_descale = p->descale_q * p->descale_k;
  a.v_descale = p->descale_v;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e = p->dtype == FA_FP8_E4M3
                           ? fa::launch_fwd_fp8(a, p->head_dim, st)
                           : fa::launch_fwd(a, p->dtype == FA_BF16 ? 0 : 1, p->head_dim, st);
  if (e != hipSuccess) return hip_fail(e, "forward launch");
  return FA_OK;
}

}  // extern "C"

namespace {

// fa_bwd and fa_bwd_noalloc: the same checks, then the same two kernels.
// With `own_scratch` the workspace is the library's fixed device array
// (looked up only after every argument check has passed).
int bwd_call(const fa_params* p, const void* q, fa_strides sq, const void* k, fa_strides sk,
             const void* v, fa_strides sv, const void* o, fa_strides so, const void* dout,
             fa_strides sdo, const float* lse, void* dq, fa_strides sdq, void* dk,
             fa_strides sdk, void* dv, fa_strides sdv, bool own_scratch, void* workspace,
             size_t workspace_bytes, uint32_t* tile_log, void* const* stage_events,
             void* stream) {
  g_detail[0] = '\0';
  FA_CHECK(check_params(p));
  if (p->dtype != FA_BF16) return fail(FA_ERR_DTYPE, "the backward pass supports bf16 inputs only");
  FA_CHECK(check_tensor("q", q, sq, p->dtype));
  FA_CHECK(check_tensor("k", k, sk, p->dtype));
  FA_CHECK(check_tensor("v", v, sv, p->dtype));
  FA_CHECK(check_tensor("o", o, so, p->o_dtype));
  FA_CHECK(check_tensor("dout", dout, sdo, p->dtype));
  FA_CHECK(check_tensor("dq", dq, sdq, p->dtype));
  FA_CHECK(check_tensor("dk", dk, sdk, p->dtype));
  FA_CHECK(check_tensor("dv", dv, sdv, p->dtype));
  FA_CHECK(check_span("q", sq, p, p->dtype));
  FA_CHECK(check_span("k", sk, p, p->dtype));
  FA_CHECK(check_span("v", sv, p, p->dtype));
  FA_CHECK(check_span("dout", sdo, p, p->dtype));
  FA_CHECK(check_rows("o", so, p));
  FA_CHECK(check_rows("dq", sdq, p));
  FA_CHECK(check_rows("dk", sdk, p));
  FA_CHECK(check_rows("dv", sdv, p));
  if (!lse) return fail(FA_ERR_NULL, "lse is NULL");
  if (reinterpret_cast<uintptr_t>(lse) % 4) return fail(FA_ERR_ALIGN, "lse is not 4-byte aligned");
  const size_t need = fa_bwd_workspace_size(p);
  if (own_scratch) {
    if (need > FA_NOALLOC_WORKSPACE_BYTES)
      return fail(FA_ERR_WORKSPACE,
                  "the backward needs %zu bytes of workspace; the fixed array holds %zu "
                  "(batch * heads_q * seqlen above %zu)",
                  need, (size_t)FA_NOALLOC_WORKSPACE_BYTES,
                  (size_t)FA_NOALLOC_WORKSPACE_BYTES / (2 * sizeof(float)));
  } else {
    if (!workspace || workspace_bytes < need)
      return fail(FA_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need,
                  workspace ? workspace_bytes : (size_t)0);
    if (reinterpret_cast<uintptr_t>(workspace) % 16)
      return fail(FA_ERR_ALIGN, "workspace is not 16-byte aligned");
  }
  if (tile_log && reinterpret_cast<uintptr_t>(tile_log) % 4)
    return fail(FA_ERR_ALIGN, "tile_log is not 4-byte aligned");
  if (stage_events)
    for (int i = 0; i < 3; ++i)
      if (!stage_events[i]) return fail(FA_ERR_NULL, "stage_events[%d] is NULL", i);

  hipError_t e;
  if (own_scratch && (e = fa::scratch_address(&workspace)) != hipSuccess)
    return hip_fail(e, "scratch array address");

  fa::BwdArgs a;
  a.p = make_problem(p);
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.sq = conv(sq);
  a.sk = conv(sk);
  a.sv = conv(sv);
  a.so = conv(so);
  a.sdo = conv(sdo);
  a.sdq = conv(sdq);
  a.sdk = conv(sdk);
  a.sdv = conv(sdv);
  a.lse = lse;
  a.dvec = static_cast<float*>(workspace);
  a.lse2 = a.dvec + (size_t)p->batch * p->heads_q * p->seqlen;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  const size_t words = fa_tile_log_words(p);
  a.log_kv = tile_log;
  a.log_q = tile_log ? tile_log + words : nullptr;
  a.o_fp32 = p->o_dtype == FA_FP32;

  hipStream_t s = static_cast<hipStream_t>(stream);
  auto mark = [&](int i) -> hipError_t {
    return stage_events ? hipEventRecord(static_cast<hipEvent_t>(stage_events[i]), s) : hipSuccess;
  };
  // dQ first: it also writes the row statistics the dK/dV kernel reads.
  if ((e = mark(0)) != hipSuccess) return hip_fail(e, "event record");
  if ((e = fa::launch_bwd_dq(a, p->head_dim, s)) != hipSuccess) return hip_fail(e, "bwd_dq launch");
  if ((e = mark(1)) != hipSuccess) return hip_fail(e, "event record");
  if ((e = fa::launch_bwd_dkdv(a, p->head_dim, s)) != hipSuccess) return hip_fail(e, "bwd_dkdv launch");
  if ((e = mark(2)) != hipSuccess) return hip_fail(e, "event record");
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_bwd(const fa_params* p, const void* q, fa_strides sq, const void* k, fa_strides sk,
           const void* v, fa_strides sv, const void* o, fa_strides so, const void* dout,
           fa_strides sdo, const float* lse, void* dq, fa_strides sdq, void* dk, fa_strides sdk,
           void* dv, fa_strides sdv, void* workspace, size_t workspace_bytes, uint32_t* tile_log,
           void* const* stage_events, void* stream) {
  return bwd_call(p, q, sq, k, sk, v, sv, o, so, dout, sdo, lse, dq, sdq, dk, sdk, dv, sdv, false,
                  workspace, workspace_bytes, tile_log, stage_events, stream);
}

int fa_bwd_noalloc(const fa_params* p, const void* q, fa_strides sq, const void* k,
                   fa_strides sk, const void* v, fa_strides sv, const void* o, fa_strides so,
                   const void* dout, fa_strides sdo, const float* lse, void* dq, fa_strides sdq,
                   void* dk, fa_strides sdk, void* dv, fa_strides sdv, uint32_t* tile_log,
                   void* const* stage_events, void* stream) {
  return bwd_call(p, q, sq, k, sk, v, sv, o, so, dout, sdo, lse, dq, sdq, dk, sdk, dv, sdv, true,
                  nullptr, 0, tile_log, stage_events, stream);
}

namespace {

// Decode work split: enough (batch, key/value head, block of 16 query heads,
// key split) units for several workgroups per CU, every split at least four
// 64-key tiles and a multiple of 64 keys.
struct DecodePlan {
  int hblocks, splits, split_len;
};

DecodePlan decode_plan(const fa_params* p) {
  DecodePlan d;
  const int64_t G = p->heads_q / p->heads_kv;
  d.hblocks = (int)ceil_div(G, 16);
  const int64_t units = (int64_t)p->batch * p->heads_kv * d.hblocks;
  const int64_t max_splits = ceil_div(p->seqlen, 256);
  const int64_t want = std::max<int64_t>(1, ceil_div(2048, units));
  const int64_t splits = std::min<int64_t>(max_splits, want);
  const int64_t len = ceil_div(ceil_div(p->seqlen, splits), 64) * 64;
  d.split_len = (int)len;
  d.splits = (int)ceil_div(p->seqlen, len);
  return d;
}

int check_decode_params(const fa_params* p) {
  const int st = check_params(p);
  if (st != FA_OK) return st;
  if (p->dtype != FA_BF16) return fail(FA_ERR_DTYPE, "decode supports bf16 inputs only");
  if (p->block_mask) return fail(FA_ERR_MASK, "decode takes no block mask");
  if (p->window) return fail(FA_ERR_MASK, "decode takes no sliding window");
  if (p->dropout_p != 0.f) return fail(FA_ERR_DROPOUT, "decode takes no dropout");
  return FA_OK;
}

}  // namespace

size_t fa_decode_workspace_size(const fa_params* p) {
  if (check_decode_params(p) != FA_OK) return 0;
  const DecodePlan d = decode_plan(p);
  if (d.splits == 1) return 0;
  return (size_t)p->batch * p->heads_q * d.splits * (p->head_dim + 1) * sizeof(float);
}

int fa_decode(const fa_params* p, const void* q, fa_strides sq, const void* k, fa_strides sk,
              const void* v, fa_strides sv, void* o, fa_strides so, float* lse, void* workspace,
              size_t workspace_bytes, void* stream) {
  g_detail[0] = '\0';
  FA_CHECK(check_decode_params(p));
  FA_CHECK(check_tensor("q", q, sq, p->dtype));
  FA_CHECK(check_tensor("k", k, sk, p->dtype));
  FA_CHECK(check_tensor("v", v, sv, p->dtype));
  FA_CHECK(check_tensor("o", o, so, p->o_dtype));
  FA_CHECK(check_span("k", sk, p, p->dtype));
  FA_CHECK(check_span("v", sv, p, p->dtype));
  if (!lse) return fail(FA_ERR_NULL, "lse is NULL");
  if (reinterpret_cast<uintptr_t>(lse) % 4) return fail(FA_ERR_ALIGN, "lse is not 4-byte aligned");
  const size_t need = fa_decode_workspace_size(p);
  if (need && (!workspace || workspace_bytes < need))
    return fail(FA_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need,
                workspace ? workspace_bytes : (size_t)0);
  if (need && reinterpret_cast<uintptr_t>(workspace) % 16)
    return fail(FA_ERR_ALIGN, "workspace is not 16-byte aligned");

  const DecodePlan d = decode_plan(p);
  fa::DecodeArgs a;
  a.p = make_problem(p);
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.sq = conv(sq);
  a.sk = conv(sk);
  a.sv = conv(sv);
  a.so = conv(so);
  a.lse = lse;
  a.ws_o = static_cast<float*>(workspace);
  a.ws_lse = need ? a.ws_o + (size_t)p->batch * p->heads_q * d.splits * p->head_dim : nullptr;
  a.splits = d.splits;
  a.split_len = d.split_len;
  a.hblocks = d.hblocks;
  a.o_fp32 = p->o_dtype == FA_FP32;
  const hipError_t e = fa::launch_decode(a, p->head_dim, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return FA_OK;
}

const char* fa_strerror(int status) {
  switch (status) {
    case FA_OK: return "success";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "invalid or too large problem size";
    case FA_ERR_DTYPE: return "unsupported dtype combination";
    case FA_ERR_HEADDIM: return "head_dim must be 64 or 128";
    case FA_ERR_GQA: return "heads_q must be a multiple of heads_kv";
    case FA_ERR_STRIDE: return "strides must be non-negative multiples of 16 bytes";
    case FA_ERR_ALIGN: return "pointer not sufficiently aligned";
    case FA_ERR_WORKSPACE: return "workspace missing or too small";
    case FA_ERR_HIP: return "HIP runtime error";
    case FA_ERR_MASK: return "block_mask_ld smaller than the number of 128-key blocks";
    case FA_ERR_SCALE: return "scale must be finite and positive";
    case FA_ERR_DROPOUT: return "dropout_p outside [0, 1) or too close to 1";
    default: return "unknown status";
  }
}

const char* fa_last_error_detail(void) { return g_detail; }

}  // extern "C"

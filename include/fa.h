/*
 * fa.h -- C ABI of the MI355X (gfx950) exact-attention library.
 *
 * The library computes exact scaled-dot-product attention,
 *     O = softmax(Q K^T * scale + mask) V,
 * the way the FlashAttention method computes it: Q is split into row blocks,
 * K/V are streamed through on-chip memory tile by tile, and a running row
 * maximum m and scaled exponential sum l (the incremental softmax of the
 * FlashAttention deep-reading report, zako-mio, sections 2.4 and 3.2) keep
 * the result exact without the N x N score or probability matrix ever being
 * written to device memory. The backward pass is the recomputation backward
 * of the report's sections 2.5 and 3.3: the forward saves only O and one
 * statistic per row (here the natural log-sum-exp LSE = m + ln l), and the
 * backward rebuilds P tile by tile from Q, K and LSE.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Tensors are addressed as base + b*stride.batch + h*stride.head
 * + i*stride.row + t, with element (not byte) strides and unit stride along
 * the head dimension t. Q, O, dO and dQ have heads_q heads; K, V, dK and dV
 * have heads_kv heads. Query head h reads key/value head h / G with
 * G = heads_q / heads_kv (grouped-query attention, as in the bowenzhou.top
 * tutorial's remark that K/V heads may be shared).
 *
 * Masks, all combined with AND (a disallowed score counts as -infinity):
 *   causal     key j is allowed for query i iff j <= i (top-left aligned);
 *   seqlens_k  key j is allowed iff j < seqlens_k[b] (key padding); query
 *              rows past the valid length are still computed; K and V rows
 *              at or past the valid length are never read (the kernels
 *              take them as zeros), so their memory may hold anything,
 *              NaN or uninitialised values included;
 *   block_mask key j is allowed for query i iff
 *              block_mask[(i/128)*block_mask_ld + j/128] != 0; this is the
 *              block-sparse variant of the report's sections 2.6 and 3.5 at a
 *              fixed 128 x 128 granularity, shared by all batches and heads.
 * A 128 x 128 tile with no allowed entry is skipped whole: never loaded and
 * never computed. A query row with no allowed key gets O = 0 and
 * LSE = -infinity, and contributes nothing to the gradients.
 *
 * Ownership: the caller allocates and owns every buffer (inputs, outputs,
 * workspace, tile logs). The library never allocates device memory, frees
 * nothing and keeps no pointer after the call returns. Every call only
 * enqueues work on `stream` (a hipStream_t; NULL = the default stream) and
 * returns; device-side faults surface at the caller's next synchronisation.
 * Inputs are read-only; outputs are overwritten and must not alias inputs.
 *
 * Errors: every entry point validates its arguments on the host before any
 * HIP call and returns a negative fa_status on failure without touching the
 * GPU. FA_ERR_HIP means a HIP launch failed; fa_last_error_detail() then
 * holds the HIP error text. No entry point aborts or throws.
 *
 * The library keeps no global mutable state apart from the per-thread error
 * detail, so calls on different streams may run concurrently.
 */
#ifndef EXACT_IO_AWARE_FA_H
#define EXACT_IO_AWARE_FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL = -1,      /* a required pointer is NULL */
  FA_ERR_SHAPE = -2,     /* a size is <= 0, or too large to index. The
                          * kernels read K and V (and Q and dO in fa_bwd)
                          * in tiles that cover whole 128-row blocks, through
                          * 32-bit byte offsets from the head's first row:
                          * R = ceil(seqlen / 128) * 128 rows are addressed,
                          * so (R - 1) * row stride + head_dim elements must
                          * not exceed 4 GiB (and (seqlen - 1) * row stride
                          * + head_dim elements must stay below it) */
  FA_ERR_DTYPE = -3,     /* unsupported dtype combination */
  FA_ERR_HEADDIM = -4,   /* head_dim is not 64 or 128 */
  FA_ERR_GQA = -5,       /* heads_q is not a multiple of heads_kv */
  FA_ERR_STRIDE = -6,    /* a stride is negative or not a multiple of 16
                          * bytes, or the row stride of a [B][H][N][d]
                          * tensor is below head_dim (rows would overlap;
                          * fa_decode's q and o, of which only row 0 is
                          * used, are exempt) */
  FA_ERR_ALIGN = -7,     /* a base pointer is not 16-byte aligned */
  FA_ERR_WORKSPACE = -8, /* workspace missing or smaller than required */
  FA_ERR_HIP = -9,       /* a HIP call failed (see fa_last_error_detail) */
  FA_ERR_MASK = -10,     /* block_mask_ld below ceil(seqlen / 128) or above 2^24 */
  FA_ERR_SCALE = -11,    /* scale is not finite and positive */
  FA_ERR_DROPOUT = -12   /* dropout_p outside [0, 1) or too close to 1 */
};

/* Element types. */
enum fa_dtype {
  FA_BF16 = 0, /* bfloat16 storage; all arithmetic accumulates in fp32 */
  FA_FP32 = 1, /* float32 storage and fp32 matrix-core arithmetic */
  /* OCP e4m3 (E4M3FN) codes of Q, K, V, forward only: the logical inputs
   * are descale_x * decode(code); S on the FP8 matrix core (fp32
   * accumulation), softmax in fp32, P~ rounded to e4m3 for the PV product.
   * Not exact attention: FlashAttention-3's FP8 direction (cross-paper
   * synthesis page, section 2). O must be FA_BF16 or FA_FP32. */
  FA_FP8_E4M3 = 2
};

/* Granularity of block masks and of tile logs (rows and columns). */
#define FA_MASK_BLOCK 128

/* Element strides of a [batch][head][row][head_dim] tensor. */
typedef struct fa_strides {
  int64_t batch;
  int64_t head;
  int64_t row;
} fa_strides;

/* Problem description shared by the forward and backward entry points. */
typedef struct fa_params {
  int32_t dtype;    /* fa_dtype of Q, K, V (and of dO, dQ, dK, dV) */
  int32_t o_dtype;  /* fa_dtype of O: equal to dtype, or FA_FP32 with bf16 */
  int32_t batch;    /* B >= 1 */
  int32_t heads_q;  /* query heads >= 1 */
  int32_t heads_kv; /* key/value heads >= 1, divides heads_q */
  int32_t seqlen;   /* N >= 1: query and key length */
  int32_t head_dim; /* d: 64 or 128 */
  float scale;      /* softmax scale, usually 1/sqrt(d) */
  int32_t causal;   /* nonzero: causal mask */
  const int32_t* seqlens_k;  /* device [batch] valid key counts, or NULL;
                                values are clamped to [0, seqlen] */
  const uint8_t* block_mask; /* device [ceil(N/128)][block_mask_ld], or NULL */
  int32_t block_mask_ld;     /* row pitch of block_mask in bytes, at most 2^24 */
  /* Sliding-window (local) attention, ANDed with the masks above: when
   * `window` is nonzero, key j is allowed for query i only if
   * i - window_left <= j <= i + window_right (both >= 0; FA_ERR_MASK
   * otherwise). The synthesis page lists the sliding window among the
   * attention variants (section 5, item 1) and the tutorial page among the
   * block-skipping sparse patterns ("sparse attention"). A zero-initialised
   * struct has no window. */
  int32_t window;
  int32_t window_left;
  int32_t window_right;
  /* Dropout on the attention probabilities, applied on chip and regenerated
   * by every kernel that needs it, never stored (the zako-mio report,
   * section 3.2, fuses dropout into the single attention kernel). With
   * 0 < dropout_p < 1, element (b, h, i, j) draws the 16-bit uniform
   *   u = half (j mod 2) [0 = low 16 bits] of word ((j div 2) mod 4) of
   *       Philox4x32-10(counter = (j div 8, i, b * heads_q + h, dropout_offset),
   *                     key = (dropout_seed mod 2^32, dropout_seed div 2^32))
   * (Salmon et al., SC'11) and is kept iff u < T, T = round((1 - p) 65536)
   * in double precision; kept probabilities are scaled by 65536 / T.
   * O = (P o Z * 65536 / T) V with P the undropped softmax, so LSE is
   * unchanged; fa_bwd regenerates the same mask from the same fields.
   * dropout_p = 0 (a zero-initialised struct) means no dropout; p outside
   * [0, 1), or so close to 1 that T = 0, is FA_ERR_DROPOUT. fa_decode
   * accepts dropout_p = 0 only. */
  float dropout_p;
  uint32_t dropout_offset;
  uint64_t dropout_seed;
  /* FA_FP8_E4M3 inputs only: per-tensor factors that turn codes into values
   * (each finite and > 0, FA_ERR_SCALE otherwise); ignored for other
   * dtypes. The FP8 forward takes no dropout (FA_ERR_DROPOUT). */
  float descale_q;
  float descale_k;
  float descale_v;
} fa_params;

/*
 * fa_fwd -- tiled forward pass (the report's section 3.2, with the loop
 * order of FlashAttention-2 described in the zhaifeiyue.github.io
 * cross-paper synthesis, section 2: one workgroup per Q block, K/V streamed).
 *
 *   q, k, v   device inputs of dtype p->dtype with strides sq, sk, sv
 *   o         device output [B][heads_q][N][d] of dtype p->o_dtype (strides so)
 *   lse       device output, contiguous float32 [B][heads_q][N]: natural
 *             log-sum-exp of each row's scaled, masked scores (-inf if empty)
 *   tile_log  NULL, or a caller-zeroed device array of fa_tile_log_words(p)
 *             uint32 words; bit (kb % 32) of word
 *             ((b*heads_q + h)*ceil(N/128) + qb)*ceil(ceil(N/128)/32) + kb/32
 *             is set iff the kernel loaded and computed any part of the
 *             128 x 128 tile (qb, kb) of batch b, head h
 *   stream    hipStream_t to enqueue on
 * Supports dtype FA_BF16 (o_dtype FA_BF16 or FA_FP32) and FA_FP32.
 */
int fa_fwd(const fa_params* p,
           const void* q, fa_strides sq,
           const void* k, fa_strides sk,
           const void* v, fa_strides sv,
           void* o, fa_strides so,
           float* lse,
           uint32_t* tile_log,
           void* stream);

/* Number of uint32 words of one tile log (fa_fwd); fa_bwd takes twice this. */
size_t fa_tile_log_words(const fa_params* p);

/* Bytes of device workspace fa_bwd needs: two fp32 [B][Hq][N] row vectors,
 * D (q D under dropout) and the log-sum-exp in base-2 units, written by the
 * dQ kernel and read by the dK/dV kernel. */
size_t fa_bwd_workspace_size(const fa_params* p);

/*
 * fa_bwd -- recomputation backward (the report's sections 2.5 and 3.3; the
 * tutorial's backward paragraph). Two kernels run in order on `stream`:
 *   1. per block of 128 query rows: D_i = sum_t dO[i][t] * O[i][t] and
 *      LSE_i * log2(e) of its rows into the workspace (fp32; +inf for a row
 *      with no allowed key); then for every visited key tile rebuild
 *      P = exp(scale * q.k - LSE), dP = dO V^T, dS = P * (dP - D) and
 *      accumulate dQ += scale * dS K (fp32 registers);
 *   2. per block of 128 keys of one key/value head: for every query head of
 *      its group and every visited query tile, rebuild P and dS the same
 *      way and accumulate dV += P^T dO and dK += scale * dS^T Q.
 *
 *   q, k, v, o, dout  device inputs (o of dtype p->o_dtype, the others of
 *                     p->dtype) with their strides
 *   lse               the forward's log-sum-exp, float32 [B][heads_q][N]
 *   dq, dk, dv        device outputs of dtype p->dtype (overwritten)
 *   workspace         device buffer of >= fa_bwd_workspace_size(p) bytes,
 *                     16-byte aligned; its contents on entry are ignored
 *   tile_log          NULL, or caller-zeroed 2 * fa_tile_log_words(p) words:
 *                     first the tiles visited by kernel 2 (dK/dV), then by
 *                     kernel 1 (dQ) (same bit layout as fa_fwd)
 *   stage_events      NULL, or 3 hipEvent_t recorded on `stream` before
 *                     kernel 1, between the kernels and after kernel 2 (for
 *                     per-kernel timing)
 * Supports dtype FA_BF16 only (FA_ERR_DTYPE otherwise).
 */
int fa_bwd(const fa_params* p,
           const void* q, fa_strides sq,
           const void* k, fa_strides sk,
           const void* v, fa_strides sv,
           const void* o, fa_strides so,
           const void* dout, fa_strides sdo,
           const float* lse,
           void* dq, fa_strides sdq,
           void* dk, fa_strides sdk,
           void* dv, fa_strides sdv,
           void* workspace, size_t workspace_bytes,
           uint32_t* tile_log,
           void* const* stage_events,
           void* stream);

/* Size of the library's fixed device array that serves as fa_bwd_noalloc's
 * workspace: 32 MiB per GPU, enough for batch * heads_q * seqlen up to
 * 4194304 rows (fa_bwd_workspace_size(p) <= this). */
#define FA_NOALLOC_WORKSPACE_BYTES (32u << 20)

/*
 * fa_bwd_noalloc -- fa_bwd for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, and harnesses that
 * forbid hipMalloc. It takes no workspace argument and calls no allocator;
 * the two fp32 row vectors that fa_bwd keeps in the caller's workspace live
 * in a fixed device array inside the library instead, of
 * FA_NOALLOC_WORKSPACE_BYTES, which each GPU the library runs on holds
 * until the process ends. Its address is looked up once per device (with
 * that device current) on the first call there, so the stream must belong
 * to the current device.
 *
 * Arguments, outputs and errors as fa_bwd, without workspace and
 * workspace_bytes; a problem with fa_bwd_workspace_size(p) above
 * FA_NOALLOC_WORKSPACE_BYTES is FA_ERR_WORKSPACE (host check, before any
 * HIP call). Nothing in the array needs clearing: every call writes the
 * row vectors before it reads them. Every call on one GPU shares that
 * array, so calls that can overlap on one GPU (different streams without an
 * ordering between them) race and give wrong results; calls on one stream,
 * or ordered by events, are safe. Results are bit-identical to fa_bwd's.
 */
int fa_bwd_noalloc(const fa_params* p,
                   const void* q, fa_strides sq,
                   const void* k, fa_strides sk,
                   const void* v, fa_strides sv,
                   const void* o, fa_strides so,
                   const void* dout, fa_strides sdo,
                   const float* lse,
                   void* dq, fa_strides sdq,
                   void* dk, fa_strides sdk,
                   void* dv, fa_strides sdv,
                   uint32_t* tile_log,
                   void* const* stage_events,
                   void* stream);

/* Bytes of device workspace fa_decode needs for `p` (0 when the keys are
 * not split; 0 also for invalid parameters). */
size_t fa_decode_workspace_size(const fa_params* p);

/*
 * fa_decode -- attention of one new query row per head against a cache of
 * p->seqlen keys (decoding). The synthesis page (section 3, item 4) notes
 * that here the score matrix is a single row and the cost is reading the
 * K/V cache from HBM; the keys are split across workgroups and the partial
 * results merged with the tutorial page's softmax merge rule (exercise 2).
 *
 *   q, o      device [batch][heads_q][.][head_dim] (row index 0 is used;
 *             the row stride is ignored), q bf16, o of p->o_dtype
 *   k, v      device [batch][heads_kv][seqlen][head_dim] bf16, the cache
 *   lse       device float32 [batch][heads_q], natural-log log-sum-exp
 *             (-inf for an empty cache)
 *   workspace device buffer of >= fa_decode_workspace_size(p) bytes (may be
 *             NULL when that is 0), 16-byte aligned, contents ignored
 *   stream    hipStream_t to enqueue on (NULL = default stream)
 *
 * The query sees keys 0 .. L_b - 1, L_b = seqlens_k[b] (clamped to
 * [0, seqlen]) or seqlen; `causal` has no effect (the new row is the last
 * position). Requirements and errors as fa_fwd, plus: bf16 inputs only
 * (FA_ERR_DTYPE); no block mask and no window (FA_ERR_MASK).
 */
int fa_decode(const fa_params* p, const void* q, fa_strides sq, const void* k, fa_strides sk,
              const void* v, fa_strides sv, void* o, fa_strides so, float* lse, void* workspace,
              size_t workspace_bytes, void* stream);

/* Static description of a status code (never NULL). */
const char* fa_strerror(int status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* fa_last_error_detail(void);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_IO_AWARE_FA_H */

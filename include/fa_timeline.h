/* fa_timeline.h -- debug entry points of libfa_timeline.so only.
 *
 * libfa_timeline.so is libfa.so built with per-workgroup timelines: the
 * 16x16x32 forward, dQ and dK/dV kernels (d = 128 without a block mask or
 * dropout, and dQ at d = 64) have thread 0 of each workgroup store 64-bit
 * stamps into a device array per kernel, as the workgroup runs. It takes
 * the same calls as libfa.so, plus these four. The release libfa.so
 * exports none of them and its kernels carry no stamps.
 *
 * Layout: FA_TIMELINE_SLOTS words per workgroup, for the first
 * FA_TIMELINE_WORKGROUPS workgroups of the kernel's most recent launches
 * (each launch overwrites the rows of its workgroups). Word 0: the 100 MHz
 * real-time counter at entry; 1: (XCC_ID << 32) | HW_ID of the wave; 10:
 * the counter at exit. For block r = 0, 1 of the workgroup (a causal pair
 * runs two): 2 + 4r the counter at the block's start, 3 + 4r once its
 * first tile (forward, dQ) or the V block and first step (dK/dV) have
 * landed, 4 + 4r at the end of its tile or step loop, 5 + 4r the block
 * index << 16 | its tile or step count. Rows of workgroups that did not
 * run are left as they were: clear before the launch to be read.
 *
 * Return values are hipError_t codes (0 = success), or -1 for a request
 * beyond the arrays. The caller owns `dst` (host memory, `words` 64-bit
 * words). Calls must not overlap kernels that write the arrays.
 */
#ifndef FA_TIMELINE_H
#define FA_TIMELINE_H

#include <stddef.h>

#define FA_TIMELINE_WORKGROUPS 65536
#define FA_TIMELINE_SLOTS 16

#ifdef __cplusplus
extern "C" {
#endif

/* Copy the first `words` words of the forward's stamps to dst. */
int fa_timeline_fwd_read(void* dst, size_t words);
/* Zero the forward's stamps (all rows). */
int fa_timeline_fwd_clear(void);
/* Copy dQ (which = 0) or dK/dV (which = 1) stamps to dst. */
int fa_timeline_bwd_read(int which, void* dst, size_t words);
/* Zero the dQ and dK/dV stamps. */
int fa_timeline_bwd_clear(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_TIMELINE_H */

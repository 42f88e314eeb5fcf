/*
 * vlkv_attn_debug.h — entry point of the visit-counting build of the decode
 * attention library (libvlkv_attn_visits.so).
 *
 * That build is the same source as libvlkv_attn.so compiled with
 * VLKV_DEBUG_VISITS defined. It exports every entry point of vlkv_attn.h and
 * vlkv_router.h with identical behaviour and results, plus the one below; its
 * decode and combine kernels also count, with device atomics, what they
 * consume and what they write. It is a test instrument: the work-list
 * checks it enables show that the tile hand-out of the dynamic schedule, which
 * cuts each request's KV cache into uniform tiles and gives them to
 * workgroups by load, neither drops nor repeats a tile [Tencent HPC lands in
 * SGLang, challenging default inference kernels, sec. "Why Tencent HPC matters
 * for online model serving"], also as lengths change from step to step and
 * requests end [same page, sec. "What the 48.8% TPOT claim does not prove",
 * on continuous batching and cancellation]. libvlkv_attn.so does not export
 * it and carries none of the counting code.
 */
#ifndef VLKV_ATTN_DEBUG_H
#define VLKV_ATTN_DEBUG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Set the visit counters of the current device for every later decode, step
 * and combine call of this library (until the next call of this function).
 *   tok_counts  (device) int32 [B][Hkv][tok_stride], or NULL: each cached row
 *               j of request b, kv head g that the attention math consumes adds
 *               1 to tok_counts[(b * Hkv + g) * tok_stride + j] (a row at j >=
 *               tok_stride is not counted). A prefix-shared row counts once for
 *               every request it serves. Give tok_stride >= pt_stride *
 *               page_size so that every row is counted.
 *   tok_stride  > 0 with tok_counts, 0 with NULL.
 *   out_counts  (device) int32 [B][Hq], or NULL: each write of a final output
 *               row o[b][h] (with its lse) adds 1 to out_counts[b * Hq + h].
 * The caller owns and clears the counters; B, Hkv and Hq are those of the
 * calls that follow. The call waits for the device to be idle, so no kernel
 * launched before it counts into the new buffers. Returns ATTN_OK, or
 * ATTN_ERR_INVALID_ARG (pointer and stride disagree) / ATTN_ERR_HIP.
 */
int attn_debug_visits(int32_t *tok_counts, int64_t tok_stride, int32_t *out_counts);

#ifdef __cplusplus
}
#endif

#endif /* VLKV_ATTN_DEBUG_H */

/*
 * vlkv_attn.h — C ABI of the MI355X (gfx950) variable-length paged decode
 * attention library (libvlkv_attn.so).
 *
 * The operation. One decode step of attention serving many requests whose
 * context lengths differ widely: each request b has one query per query head and
 * attends to its L_b cached key/value rows. The source article motivates it with
 * a batch where one request carries 16,000 tokens of context and another has
 * just started at 1,000: under a static schedule one GPU block gets far more
 * work than the rest and the longest task decides when the launch ends. Its
 * "Dynamic Attention" cuts the KV-cache work into uniform tiles, hands them to
 * workgroups according to the current load, and rebuilds that mapping as
 * lengths change during decode; its baseline is a static split-k
 * [Tencent HPC lands in SGLang, challenging default inference kernels, sec.
 * "Why Tencent HPC matters for online model serving"]. Cache precision is one
 * of the benchmark dimensions it lists [same page, sec. "What the 48.8% TPOT
 * claim does not prove"], hence the fp8 cache option.
 *
 * Per step the caller enqueues, on one stream and with one workspace:
 *     attn_plan  -> attn_decode -> attn_combine
 * The result is, for request b and query head h (kv head g = h / (Hq/Hkv)):
 *     o[b][h] = sum_j softmax_j(sm_scale * q[b][h] . K_j) V_j,
 *     lse[b][h] = ln sum_j exp(sm_scale * q[b][h] . K_j)
 * over j = 0..L_b-1, with K_j = k_cache[page_table[b][j/P]][g][j%P][:].
 *
 * Conventions for every entry point:
 *   - Pointers marked (device) are HIP device memory on the current device;
 *     (host) pointers are ordinary host memory read before the call returns.
 *   - `stream` is a hipStream_t (NULL = the null stream). Work is enqueued and
 *     never waited for, except by attn_get_status.
 *   - The caller allocates and owns every buffer. The library allocates no
 *     memory, keeps no pointer after a call returns and has no global mutable
 *     state (apart from the per-GPU scratch of attn_step_noalloc); calls on
 *     different workspaces may run concurrently.
 *   - Return value: ATTN_OK, or an ATTN_ERR_* code. Argument and shape checks
 *     happen on the host before anything is enqueued; on error nothing is
 *     enqueued and attn_last_error() describes the problem.
 *   - Data errors that only the device can see (a length beyond the page
 *     table, a page id outside [0, num_pages)) set bits in a status word inside
 *     the workspace; the affected rows are skipped, never read out of bounds.
 */
#ifndef VLKV_ATTN_H
#define VLKV_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* return codes */
#define ATTN_OK               0
#define ATTN_ERR_INVALID_ARG  1  /* null pointer, bad shape, workspace too small */
#define ATTN_ERR_UNSUPPORTED  2  /* a shape or dtype this build does not implement */
#define ATTN_ERR_HIP          3  /* a HIP runtime call or kernel launch failed */

/* kv_dtype */
#define ATTN_KV_BF16      0      /* bfloat16 K/V rows */
#define ATTN_KV_FP8_E4M3  1      /* OCP e4m3fn codes, fp32 scale per (request, kv head) */

/* mode */
#define ATTN_DYNAMIC  0          /* balanced per-step tile plan */
#define ATTN_STATIC   1          /* static split-K: S fixed splits per (request, kv head) */
#define ATTN_SHARED   2          /* dynamic plan that reads prefix-shared pages once (see attn_plan) */

/* status word bits (attn_get_status) */
#define ATTN_STATUS_BAD_LENGTH  1u  /* some L_b < 0 or L_b > pt_stride * page_size: treated as 0 */
#define ATTN_STATUS_BAD_PAGE    2u  /* some used page id outside [0, num_pages): its rows skipped */
#define ATTN_STATUS_INTERNAL    4u  /* a library defect, never data: in attn_step a workgroup's range
                                       split more than its first and last (request, kv head) pair,
                                       which the plan rules out (the extra pair was not merged); or,
                                       in any decode, a wait of the waves of one workgroup for one
                                       another at a segment's end ran out its bound (that segment's
                                       merge was skipped). Either way some outputs are wrong. */

/*
 * Problem shape (host struct, read during the call).
 *   batch          B, number of requests (>= 1)
 *   num_q_heads    Hq;  num_kv_heads Hkv; Hq % Hkv == 0 and 1 <= Hq/Hkv <= 16
 *   head_dim       D; this build supports 128
 *   page_size      P tokens per page; a multiple of 16
 *   num_pages      physical pages in each cache
 *   pt_stride      row length of the page table (max pages per request)
 *   tile_tokens    T, the uniform tile; a multiple of 64
 *   num_wgs        W, workgroups of the decode launch (1 .. 65536), or 0 for the
 *                  library default: a launch of 2 per compute unit of the
 *                  current device, of which the dynamic plan uses all when
 *                  that leaves at least 32 units (request, kv head, tile) per
 *                  workgroup, else one per compute unit (the fixed costs of a
 *                  workgroup outweigh a second wave per SIMD on small steps).
 *                  With 0, sizes and splits below follow the current device.
 *   kv_dtype       ATTN_KV_BF16 or ATTN_KV_FP8_E4M3
 *   mode           ATTN_DYNAMIC, ATTN_STATIC or ATTN_SHARED
 *   static_splits  S for ATTN_STATIC (>= 1); 0 picks
 *                  clamp(ceil(W / (B*Hkv)), 1, ceil(pt_stride*P / T)) with
 *                  W = attn_num_wgs(shape)
 */
typedef struct attn_shape {
    int32_t batch;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t page_size;
    int32_t num_pages;
    int32_t pt_stride;
    int32_t tile_tokens;
    int32_t num_wgs;
    int32_t kv_dtype;
    int32_t mode;
    int32_t static_splits;
} attn_shape;

/*
 * Validate a shape without touching the GPU. Returns ATTN_OK,
 * ATTN_ERR_INVALID_ARG or ATTN_ERR_UNSUPPORTED (see attn_last_error()).
 */
int attn_check_shape(const attn_shape *shape);

/*
 * Bytes of workspace the three calls need for this shape, for any lengths
 * within pt_stride * page_size. Host only, pure (with num_wgs = 0 it reads the
 * current device's compute-unit count). Returns 0 for an invalid shape. The
 * workspace must be device memory aligned to 256 bytes.
 */
size_t attn_workspace_bytes(const attn_shape *shape);

/* Effective number of static splits S for this shape (ATTN_STATIC), or 0. */
int32_t attn_static_splits(const attn_shape *shape);

/*
 * Workgroups the decode launch of this shape has: num_wgs, or for num_wgs = 0
 * two per compute unit of the current device (the size of the plan's
 * per-workgroup arrays, attn_read_plan). 0 for an invalid shape or, with
 * num_wgs = 0, when no device is available.
 */
int32_t attn_num_wgs(const attn_shape *shape);

/*
 * Number of compute units of HIP device `device` in *cus (host pointer).
 * Returns ATTN_OK or ATTN_ERR_HIP.
 */
int attn_device_cu_count(int device, int32_t *cus);

/*
 * Build the tile plan for this step into the workspace (one small kernel).
 *   lengths    (device) int32 [B], current context length of each request
 *   page_table (device) int32 [B][pt_stride]; read only in ATTN_SHARED mode
 *   workspace  (device) >= attn_workspace_bytes(shape) bytes, 256-B aligned
 * Dynamic mode: the (request, kv head, tile) units are numbered request-major
 * and cut into W_eff contiguous, equal (+-1) ranges (W_eff: the workgroups the
 * plan uses, see num_wgs, and at most the number of units); each maximal run of one
 * (request, kv head) inside a range is a segment with its own partial slot.
 * Static mode: chunk = ceil(max L / S) rounded up to a multiple of
 * lcm(page_size, tile_tokens); split s of each (request, kv head) covers
 * tokens [s*chunk, min((s+1)*chunk, L_b)) and may be empty.
 * Shared mode (prefix caching, which the article lists among the situations
 * the kernels must handle [Tencent HPC lands in SGLang, challenging default
 * inference kernels, sec. "Why Tencent HPC matters for online model
 * serving"]): request b shares with b-1 the leading page slots that hold the
 * same valid page id, capped by both lengths and rounded down to whole tiles.
 * Runs of adjacent sharing requests are cut into groups of R = 32 / G for
 * G = Hq/Hkv >= 8 and R = 16 / G below (one pass holds 32 or 16 query rows);
 * a group of two or more reads its common prefix once, as one item whose query
 * rows are the members' heads, and each request keeps an item for its
 * remaining tokens. The partition above then
 * runs over (item, kv head, tile) units. Results equal the other modes' up to
 * the order of the softmax merge. The plan's arrays are over items
 * (attn_read_plan, attn_read_plan_items). Batches whose page tables alias
 * pages should use this mode: the other modes stream K/V with non-temporal
 * loads, so a page that several requests read in one step is fetched from
 * memory each time.
 * Note: "non-temporal" above is a cache policy of the loads only; it does not
 * change any result.
 * The workspace contents stay valid until the next attn_plan on it.
 */
int attn_plan(const attn_shape *shape, const int32_t *lengths, const int32_t *page_table,
              void *workspace, size_t workspace_bytes, void *stream);

/*
 * Decode attention over the plan in `workspace` (same stream): one query
 * token per request against its paged, variable-length KV history, each
 * workgroup streaming the uniform tiles the plan handed it and keeping a
 * partial softmax state per (request, kv head) it touches [Tencent HPC lands
 * in SGLang, challenging default inference kernels, sec. "Why Tencent HPC
 * matters for online model serving": work cut into uniform tiles, partial
 * results merged afterwards; KV in bf16 or fp8, sec. "What the 48.8% TPOT
 * claim does not prove": cache precision as a benchmark dimension].
 *   q          (device) bf16 [B][Hq][D]
 *   k_cache    (device) [num_pages][Hkv][P][D], bf16 or uint8 e4m3fn codes
 *   v_cache    (device) same layout and dtype as k_cache
 *   k_scale    (device) fp32 [B][Hkv] for ATTN_KV_FP8_E4M3, else NULL
 *   v_scale    (device) fp32 [B][Hkv] for ATTN_KV_FP8_E4M3, else NULL
 *   page_table (device) int32 [B][pt_stride]: page of tokens [i*P, (i+1)*P)
 * The lengths are the validated copy attn_plan stored in the workspace.
 *   sm_scale   softmax scale applied to q . k (e.g. 1/sqrt(D))
 *   out        (device) bf16 [B][Hq][D]; (request, kv head) pairs handled by
 *              a single workgroup are written here directly
 *   lse        (device) fp32 [B][Hq] natural-log log-sum-exp, or NULL
 * Rows j >= L_b of a request's last page are never used. K/V, q, scales and
 * the page table are only read.
 */
int attn_decode(const attn_shape *shape, const void *q, const void *k_cache,
                const void *v_cache, const float *k_scale, const float *v_scale,
                const int32_t *page_table, float sm_scale, void *workspace,
                size_t workspace_bytes, void *out, float *lse, void *stream);

/*
 * Merge the partial results of (request, kv head) pairs that were split over
 * several workgroups (log-sum-exp weighting), and write o = 0, lse = -inf for
 * requests with L_b = 0 [Tencent HPC lands in SGLang, challenging default
 * inference kernels, sec. "Why Tencent HPC matters for online model serving":
 * the partial results of a request's tiles are combined after the tiles are
 * processed]. Must follow attn_decode on the same stream and workspace. out,
 * lse as in attn_decode. Each pair's partials are folded in slot order, so the
 * result does not depend on timing.
 */
int attn_combine(const attn_shape *shape, const void *workspace, size_t workspace_bytes,
                 void *out, float *lse, void *stream);

/*
 * Prepare a workspace for attn_step: clears the status word and the per-(request,
 * kv head) arrival counters (one small kernel on `stream`). Call it once after
 * allocating the workspace (and after any shape change that reuses it); every
 * attn_step leaves the counters at zero again, so no per-step clearing is needed.
 */
int attn_workspace_init(const attn_shape *shape, void *workspace, size_t workspace_bytes,
                        void *stream);

/*
 * One decode step in a single kernel launch: the same plan, decode and merge as
 * attn_plan + attn_decode + attn_combine, with identical results up to the order
 * in which split partials are summed. Every workgroup derives its own unit range
 * of the current tile plan from `lengths` (the per-step rebuild of the article's
 * tile-to-CTA mapping [Tencent HPC lands in SGLang, challenging default
 * inference kernels, sec. "Why Tencent HPC matters for online model serving"]),
 * and the last workgroup to finish a (request, kv head) pair that is split over
 * several workgroups merges the pair's partials by log-sum-exp weighting.
 *   lengths    (device) int32 [B], current context length of each request
 *   other arguments as in attn_decode; shape->mode selects the dynamic plan or
 *   the static split-K. ATTN_SHARED is not fused: attn_step then enqueues
 *   attn_plan, attn_decode and attn_combine (three launches).
 * The workspace must have been prepared by attn_workspace_init. The status word
 * is sticky: bits set by any step stay set until attn_workspace_init or
 * attn_plan rewrites it. Two attn_step calls on one workspace must not overlap
 * (same stream, or ordered).
 */
int attn_step(const attn_shape *shape, const void *q, const void *k_cache, const void *v_cache,
              const float *k_scale, const float *v_scale, const int32_t *page_table,
              const int32_t *lengths, float sm_scale, void *workspace, size_t workspace_bytes,
              void *out, float *lse, void *stream);

/*
 * attn_step for callers that cannot allocate device memory: code under HIP
 * graph capture, serving loops and harnesses that forbid hipMalloc. Arguments
 * and results as in attn_step, without the workspace: the step's arrival
 * counters, partial results and a status word live in a fixed scratch array
 * inside this library's device code, one per GPU, of
 * ATTN_NOALLOC_SCRATCH_BYTES bytes (placed when the library is first used on a
 * GPU and held until the process ends). This call allocates nothing.
 *   status  (device, optional) uint32: the step ORs its ATTN_STATUS_* bits into
 *           it (the caller clears it); NULL keeps them in the scratch, unread.
 * Limits, checked on the host (ATTN_ERR_INVALID_ARG, nothing enqueued):
 * batch * num_kv_heads <= ATTN_NOALLOC_MAX_PAIRS, and the partial results must
 * fit the scratch: 2 * W slots (ATTN_DYNAMIC, W = attn_num_wgs) or batch * num_kv_heads * S
 * slots (ATTN_STATIC), each Hq/Hkv rows of head_dim + 1 floats, plus 256 bytes
 * of alignment, at most ATTN_NOALLOC_SCRATCH_BYTES - 4 * ATTN_NOALLOC_MAX_PAIRS
 * - 256 bytes. ATTN_SHARED returns ATTN_ERR_UNSUPPORTED (its plan needs a
 * workspace). Every call on a GPU shares that GPU's scratch: calls that can
 * overlap on one GPU (different streams without ordering between them) race
 * and give wrong results. The first call on a GPU also enqueues one small
 * kernel that clears the arrival counters; every step leaves them at zero.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES (16u << 20)
#define ATTN_NOALLOC_MAX_PAIRS     65536
int attn_step_noalloc(const attn_shape *shape, const void *q, const void *k_cache,
                      const void *v_cache, const float *k_scale, const float *v_scale,
                      const int32_t *page_table, const int32_t *lengths, float sm_scale,
                      void *out, float *lse, uint32_t *status, void *stream);

/*
 * Append one new token per request to the paged caches: the step that grows
 * every context by one token before decode attends to it (contexts that grow
 * at different rates under continuous batching, [Tencent HPC lands in SGLang,
 * challenging default inference kernels, sec. "Why Tencent HPC matters for
 * online model serving"]; cache precision, sec. "What the 48.8% TPOT claim does
 * not prove").
 *   k_new, v_new (device) bf16 [B][Hkv][D]: the new key and value rows
 *   positions    (device) int32 [B]: token position to write (normally the
 *                length before the append); a negative value skips the request
 *   page_table   (device) int32 [B][pt_stride]; the page of the position must
 *                already be assigned
 *   k_scale, v_scale (device) fp32 [B][Hkv] for ATTN_KV_FP8_E4M3, else NULL
 *   k_cache, v_cache (device) [num_pages][Hkv][P][D], written in place: row
 *                positions[b] % P of page page_table[b][positions[b] / P]
 *   workspace    (device, optional) a workspace of this shape whose status word
 *                receives ATTN_STATUS_BAD_LENGTH for a position at or beyond
 *                pt_stride * P and ATTN_STATUS_BAD_PAGE for a page id outside
 *                [0, num_pages); such requests are skipped. NULL: no status.
 * bf16 caches store the bits of the new rows. fp8 caches store the OCP e4m3fn
 * code of x / scale (fp32 division, nearest with ties to even, saturated at
 * +-448). Only the rows written are touched.
 */
int attn_append_kv(const attn_shape *shape, const void *k_new, const void *v_new,
                   const int32_t *positions, const int32_t *page_table, const float *k_scale,
                   const float *v_scale, void *k_cache, void *v_cache, void *workspace,
                   size_t workspace_bytes, void *stream);

/*
 * Copy the status word of the last plan/decode on this workspace into *flags
 * (host pointer). SYNCHRONISES `stream`; meant for tests and debugging, not
 * for the per-step path.
 */
int attn_get_status(const void *workspace, uint32_t *flags, void *stream);

/*
 * Copy the plan arrays out of the workspace into host memory (synchronises
 * `stream`), for checking the device planner against a CPU planner. Each host
 * pointer may be NULL to skip that array. Sizes: header[8], len_eff[B],
 * tiles_prefix[B+1], seg_prefix[B*Hkv+1], first_wg[B*Hkv], wg_begin[W+1] (W = attn_num_wgs),
 * wg_start_b[W]. header = {status, N, W_eff, max L, chunk, S, total tiles, T}.
 * ATTN_SHARED: the arrays are over items, not requests, with B replaced by 2B
 * (the first header[4] items are used): len_eff = item token counts,
 * wg_start_b = each range's first item; header = {status, N, W_eff, max L,
 * number of items, R, total tiles, T}.
 */
int attn_read_plan(const attn_shape *shape, const void *workspace, int32_t *header,
                   int32_t *len_eff, int32_t *tiles_prefix, int32_t *seg_prefix,
                   int32_t *first_wg, int32_t *wg_begin, int32_t *wg_start_b, void *stream);

/*
 * ATTN_SHARED only: copy the item description of the plan into host memory
 * (synchronises `stream`); NULL skips an array. Sizes 2B for the item arrays,
 * B for the request arrays; entries past header[4] items are unspecified.
 *   item_req[i]   first request of item i (its page table row)
 *   item_start[i] first token of item i within that request
 *   item_m[i]     requests item i serves: item_req[i] .. + item_m[i] - 1
 *   item_solo[i]  1 if item i is its request's only item
 *   req_shared[b] the shared item of request b's group, or -1
 *   req_member[b] b's position in that group (query rows member*G..)
 *   req_own[b]    the item holding b's own tokens
 */
int attn_read_plan_items(const attn_shape *shape, const void *workspace, int32_t *item_req,
                         int32_t *item_start, int32_t *item_m, int32_t *item_solo,
                         int32_t *req_shared, int32_t *req_member, int32_t *req_own,
                         void *stream);

/* Text of the last error on the calling thread ("" if none). */
const char *attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* VLKV_ATTN_H */

// C ABI of libvlkv_attn.so (declared in include/vlkv_attn.h): host-side
// argument checks, the workspace layout, the three per-step launches and the
// single-launch step.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "../../include/vlkv_attn.h"
#ifdef VLKV_DEBUG_VISITS
#include "../../include/vlkv_attn_debug.h"
#endif
#include "vlkv_internal.hpp"

namespace vlkv {

static thread_local std::string g_last_error;

int fail(int code, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int ok()
{
    g_last_error.clear();
    return ATTN_OK;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Compute units of the current device, read once per device.
static int device_cus(int *cus)
{
    constexpr int kMaxDev = 64;
    static int cache[kMaxDev];
    static std::once_flag once[kMaxDev];
    static hipError_t err[kMaxDev];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(ATTN_ERR_HIP, "num_wgs 0 needs a device: hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDev)
        return fail(ATTN_ERR_INVALID_ARG, "device %d beyond the %d this library serves", dev, kMaxDev);
    std::call_once(once[dev], [&] { err[dev] = hipDeviceGetAttribute(&cache[dev], hipDeviceAttributeMultiprocessorCount, dev); });
    if (err[dev] != hipSuccess)
        return fail(ATTN_ERR_HIP, "hipDeviceGetAttribute: %s", hipGetErrorString(err[dev]));
    *cus = cache[dev];
    return ATTN_OK;
}

// Static split count S for a launch of W workgroups.
static int32_t effective_splits(const attn_shape *s, int64_t W)
{
    if (s->static_splits > 0)
        return s->static_splits;
    const int64_t pairs = (int64_t)s->batch * s->num_kv_heads;
    int64_t S = ceil_div(W, pairs);
    const int64_t cap = ceil_div((int64_t)s->pt_stride * s->page_size, s->tile_tokens);
    if (S > cap)
        S = cap;
    if (S < 1)
        S = 1;
    return (int32_t)S;
}

// Full shape validation. Returns ATTN_OK or an error code (with message).
static int check(const attn_shape *s, Shape *out)
{
    if (!s)
        return fail(ATTN_ERR_INVALID_ARG, "shape is NULL");
    if (s->batch < 1 || s->batch > kMaxBatch)
        return fail(ATTN_ERR_INVALID_ARG, "batch %d outside [1, %d]", s->batch, kMaxBatch);
    if (s->num_q_heads < 1 || s->num_kv_heads < 1 || s->num_q_heads % s->num_kv_heads)
        return fail(ATTN_ERR_INVALID_ARG, "num_q_heads %d must be a positive multiple of num_kv_heads %d",
                    s->num_q_heads, s->num_kv_heads);
    const int G = s->num_q_heads / s->num_kv_heads;
    if (G > kMaxGroup)
        return fail(ATTN_ERR_UNSUPPORTED, "query heads per kv head %d > %d", G, kMaxGroup);
    if (s->head_dim != kHeadDim)
        return fail(ATTN_ERR_UNSUPPORTED, "head_dim %d (only %d is built)", s->head_dim, kHeadDim);
    if (s->page_size < 16 || s->page_size % 16)
        return fail(ATTN_ERR_INVALID_ARG, "page_size %d must be a positive multiple of 16", s->page_size);
    if (s->num_pages < 1)
        return fail(ATTN_ERR_INVALID_ARG, "num_pages %d < 1", s->num_pages);
    if (s->pt_stride < 1)
        return fail(ATTN_ERR_INVALID_ARG, "pt_stride %d < 1", s->pt_stride);
    if (s->tile_tokens < kBlockTokens || s->tile_tokens % kBlockTokens)
        return fail(ATTN_ERR_UNSUPPORTED, "tile_tokens %d must be a positive multiple of %d",
                    s->tile_tokens, kBlockTokens);
    if (s->num_wgs < 0 || s->num_wgs > (1 << 16))
        return fail(ATTN_ERR_INVALID_ARG, "num_wgs %d outside [0, 2^16]", s->num_wgs);
    if (s->kv_dtype != ATTN_KV_BF16 && s->kv_dtype != ATTN_KV_FP8_E4M3)
        return fail(ATTN_ERR_UNSUPPORTED, "kv_dtype %d", s->kv_dtype);
    if (s->mode != ATTN_DYNAMIC && s->mode != ATTN_STATIC && s->mode != ATTN_SHARED)
        return fail(ATTN_ERR_INVALID_ARG, "mode %d", s->mode);
    if (s->static_splits < 0)
        return fail(ATTN_ERR_INVALID_ARG, "static_splits %d < 0", s->static_splits);
    // every index the kernels form must fit its type
    const int64_t max_tokens = (int64_t)s->pt_stride * s->page_size;
    if (max_tokens > INT32_MAX / 2)
        return fail(ATTN_ERR_INVALID_ARG, "pt_stride * page_size too large");
    // (mode 2 splits a request into at most two items: one more tile each)
    const int64_t max_units = (int64_t)s->batch * s->num_kv_heads * (ceil_div(max_tokens, s->tile_tokens) + 1);
    if (max_units > INT32_MAX / 2)
        return fail(ATTN_ERR_INVALID_ARG, "batch * kv heads * tiles per request too large");
    // num_wgs 0: the library default, two workgroups per compute unit of the
    // current device (read only when the shape is resolved for a call)
    int W = s->num_wgs, W_auto = 0;
    if (W == 0) {
        if (!out)
            W = 2;   // any device has a compute unit: check the rest with the smallest count
        else {
            int cus = 0;
            const int rc = device_cus(&cus);
            if (rc != ATTN_OK)
                return rc;
            W = 2 * cus;
            W_auto = cus;
        }
    }
    const int32_t S = s->mode == ATTN_STATIC ? effective_splits(s, W) : 0;
    if (s->mode == ATTN_STATIC && (int64_t)s->batch * s->num_kv_heads * S > INT32_MAX / 2)
        return fail(ATTN_ERR_INVALID_ARG, "batch * kv heads * splits too large");
    if (s->mode == ATTN_STATIC && (int64_t)S * max_tokens > ((int64_t)INT32_MAX) * 4)
        return fail(ATTN_ERR_INVALID_ARG, "static splits too large");
    if (out) {
        *out = Shape{s->batch, s->num_q_heads, s->num_kv_heads, G, s->head_dim, s->page_size,
                     s->num_pages, s->pt_stride, s->tile_tokens, W,
                     s->kv_dtype == ATTN_KV_FP8_E4M3, s->mode, S, W_auto};
    }
    return ATTN_OK;
}

WsLayout ws_layout(const Shape &s)
{
    WsLayout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align256(off + bytes);
        return at;
    };
    const int64_t nbg = (int64_t)s.B * s.Hkv;
    const bool shared = s.mode == ATTN_SHARED;
    // the plan's "items": requests, or in mode 2 up to two per request
    L.max_items = shared ? 2 * (int64_t)s.B : s.B;
    const int64_t nig = L.max_items * s.Hkv;
    // dynamic: at most W_eff + (item, kv head) pairs segments with attn_plan's
    // slots, and two slots per workgroup (its first and last segment) in the
    // single launch
    L.max_slots = s.mode == ATTN_STATIC ? nbg * s.S : nig + 2 * (int64_t)s.W;
    L.slot_rows = shared ? shared_group(s.G) * s.G : s.G;
    L.header = take(sizeof(int32_t) * kHeaderInts);
    L.len_eff = take(sizeof(int32_t) * L.max_items);
    L.tiles_prefix = take(sizeof(int32_t) * (L.max_items + 1));
    L.seg_prefix = take(sizeof(int32_t) * (nig + 1));
    L.first_wg = take(sizeof(int32_t) * nig);
    L.wg_begin = take(sizeof(int32_t) * (s.W + 1));
    L.wg_start_b = take(sizeof(int32_t) * s.W);
    const int64_t ni = shared ? L.max_items : 0, nr = shared ? s.B : 0;
    L.item_req = take(sizeof(int32_t) * ni);
    L.item_start = take(sizeof(int32_t) * ni);
    L.item_m = take(sizeof(int32_t) * ni);
    L.item_solo = take(sizeof(int32_t) * ni);
    L.req_shared = take(sizeof(int32_t) * nr);
    L.req_member = take(sizeof(int32_t) * nr);
    L.req_own = take(sizeof(int32_t) * nr);
    L.counters = take(sizeof(int32_t) * nbg);
    L.part_lse = take(sizeof(float) * L.max_slots * L.slot_rows);
    L.part_o = take(sizeof(float) * L.max_slots * L.slot_rows * s.D);
    L.total = off;
    return L;
}

template <typename T>
static T *at(void *ws, size_t off)
{
    return reinterpret_cast<T *>(static_cast<char *>(ws) + off);
}
template <typename T>
static const T *at(const void *ws, size_t off)
{
    return reinterpret_cast<const T *>(static_cast<const char *>(ws) + off);
}

static int check_ws(const Shape &s, const void *ws, size_t bytes, WsLayout *L)
{
    *L = ws_layout(s);
    if (!ws)
        return fail(ATTN_ERR_INVALID_ARG, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(ws) % 256)
        return fail(ATTN_ERR_INVALID_ARG, "workspace not 256-byte aligned");
    if (bytes < L->total)
        return fail(ATTN_ERR_INVALID_ARG, "workspace %zu bytes < %zu needed", bytes, L->total);
    return ATTN_OK;
}

static int hip_fail(hipError_t e, const char *what)
{
    return fail(ATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace vlkv

using namespace vlkv;

extern "C" {

int attn_check_shape(const attn_shape *shape)
{
    const int rc = check(shape, nullptr);
    return rc == ATTN_OK ? ok() : rc;
}

size_t attn_workspace_bytes(const attn_shape *shape)
{
    Shape s;
    if (check(shape, &s) != ATTN_OK)
        return 0;
    return ws_layout(s).total;
}

int32_t attn_static_splits(const attn_shape *shape)
{
    Shape s;
    if (check(shape, &s) != ATTN_OK)
        return 0;
    return effective_splits(shape, s.W);
}

int32_t attn_num_wgs(const attn_shape *shape)
{
    Shape s;
    if (check(shape, &s) != ATTN_OK)
        return 0;
    return s.W;
}

int attn_device_cu_count(int device, int32_t *cus)
{
    if (!cus)
        return fail(ATTN_ERR_INVALID_ARG, "cus is NULL");
    int n = 0;
    const hipError_t e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, device);
    if (e != hipSuccess)
        return hip_fail(e, "hipDeviceGetAttribute");
    *cus = n;
    return ok();
}

static int enqueue_plan(const Shape &s, const WsLayout &L, const int32_t *lengths, const int32_t *page_table,
                        void *workspace, hipStream_t st);
static int enqueue_decode(const Shape &s, const WsLayout &L, const void *q, const void *k_cache,
                          const void *v_cache, const float *k_scale, const float *v_scale,
                          const int32_t *page_table, float sm_scale, void *workspace, void *out, float *lse,
                          hipStream_t st);
static int enqueue_combine(const Shape &s, const WsLayout &L, const void *workspace, void *out, float *lse,
                           hipStream_t st);

int attn_plan(const attn_shape *shape, const int32_t *lengths, const int32_t *page_table,
              void *workspace, size_t workspace_bytes, void *stream)
{
    Shape s;
    WsLayout L;
    int rc = check(shape, &s);
    if (rc != ATTN_OK)
        return rc;
    if (!lengths)
        return fail(ATTN_ERR_INVALID_ARG, "lengths is NULL");
    if (s.mode == ATTN_SHARED && !page_table)
        return fail(ATTN_ERR_INVALID_ARG, "mode ATTN_SHARED needs the page table");
    if ((rc = check_ws(s, workspace, workspace_bytes, &L)) != ATTN_OK)
        return rc;
    return enqueue_plan(s, L, lengths, page_table, workspace, static_cast<hipStream_t>(stream));
}

static int enqueue_plan(const Shape &s, const WsLayout &L, const int32_t *lengths, const int32_t *page_table,
                        void *workspace, hipStream_t st)
{
    PlanArgs a{};
    a.lengths = lengths;
    a.page_table = page_table;
    a.header = at<int32_t>(workspace, L.header);
    a.len_eff = at<int32_t>(workspace, L.len_eff);
    a.tiles_prefix = at<int32_t>(workspace, L.tiles_prefix);
    a.seg_prefix = at<int32_t>(workspace, L.seg_prefix);
    a.first_wg = at<int32_t>(workspace, L.first_wg);
    a.wg_begin = at<int32_t>(workspace, L.wg_begin);
    a.wg_start_b = at<int32_t>(workspace, L.wg_start_b);
    a.item_req = at<int32_t>(workspace, L.item_req);
    a.item_start = at<int32_t>(workspace, L.item_start);
    a.item_m = at<int32_t>(workspace, L.item_m);
    a.item_solo = at<int32_t>(workspace, L.item_solo);
    a.req_shared = at<int32_t>(workspace, L.req_shared);
    a.req_member = at<int32_t>(workspace, L.req_member);
    a.req_own = at<int32_t>(workspace, L.req_own);
    a.B = s.B;
    a.Hkv = s.Hkv;
    a.G = s.G;
    a.P = s.P;
    a.pt_stride = s.pt_stride;
    a.num_pages = s.num_pages;
    a.T = s.T;
    a.W = s.W;
    a.W_auto = s.W_auto;
    a.W_auto = s.W_auto;
    a.mode = s.mode;
    a.S = s.S;
    const hipError_t e = launch_plan(a, st);
    if (e != hipSuccess)
        return hip_fail(e, "plan launch");
    return ok();
}

int attn_decode(const attn_shape *shape, const void *q, const void *k_cache, const void *v_cache,
                const float *k_scale, const float *v_scale, const int32_t *page_table,
                float sm_scale, void *workspace, size_t workspace_bytes, void *out, float *lse,
                void *stream)
{
    Shape s;
    WsLayout L;
    int rc = check(shape, &s);
    if (rc != ATTN_OK)
        return rc;
    if (!q || !k_cache || !v_cache || !page_table || !out)
        return fail(ATTN_ERR_INVALID_ARG, "q, k_cache, v_cache, page_table and out must be non-NULL");
    if (s.kv_fp8 && (!k_scale || !v_scale))
        return fail(ATTN_ERR_INVALID_ARG, "fp8 cache needs k_scale and v_scale");
    if (!(sm_scale == sm_scale) || sm_scale == INFINITY || sm_scale == -INFINITY)
        return fail(ATTN_ERR_INVALID_ARG, "sm_scale is not finite");
    if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_cache) |
         reinterpret_cast<uintptr_t>(v_cache) | reinterpret_cast<uintptr_t>(out)) % 16)
        return fail(ATTN_ERR_INVALID_ARG, "q, caches and out must be 16-byte aligned");
    if ((rc = check_ws(s, workspace, workspace_bytes, &L)) != ATTN_OK)
        return rc;
    return enqueue_decode(s, L, q, k_cache, v_cache, k_scale, v_scale, page_table, sm_scale, workspace, out, lse,
                          static_cast<hipStream_t>(stream));
}

static int enqueue_decode(const Shape &s, const WsLayout &L, const void *q, const void *k_cache,
                          const void *v_cache, const float *k_scale, const float *v_scale,
                          const int32_t *page_table, float sm_scale, void *workspace, void *out, float *lse,
                          hipStream_t st)
{
    DecodeArgs a{};
    a.lengths = nullptr;
    a.counters = nullptr;
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint8_t *>(k_cache);
    a.v = static_cast<const uint8_t *>(v_cache);
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.page_table = page_table;
    a.header = at<int32_t>(workspace, L.header);
    a.len_eff = at<int32_t>(workspace, L.len_eff);
    a.tiles_prefix = at<int32_t>(workspace, L.tiles_prefix);
    a.seg_prefix = at<int32_t>(workspace, L.seg_prefix);
    a.first_wg = at<int32_t>(workspace, L.first_wg);
    a.wg_begin = at<int32_t>(workspace, L.wg_begin);
    a.wg_start_b = at<int32_t>(workspace, L.wg_start_b);
    a.item_req = at<int32_t>(workspace, L.item_req);
    a.item_start = at<int32_t>(workspace, L.item_start);
    a.item_m = at<int32_t>(workspace, L.item_m);
    a.item_solo = at<int32_t>(workspace, L.item_solo);
    a.part_o = at<float>(workspace, L.part_o);
    a.part_lse = at<float>(workspace, L.part_lse);
    a.out = static_cast<uint16_t *>(out);
    a.lse = lse;
    a.B = s.B;
    a.Hq = s.Hq;
    a.Hkv = s.Hkv;
    a.G = s.G;
    a.P = s.P;
    a.num_pages = s.num_pages;
    a.pt_stride = s.pt_stride;
    a.S = s.S;
    a.T = s.T;
    a.W = s.W;
    a.slot_rows = L.slot_rows;
    a.scale_log2 = sm_scale * 1.4426950408889634f;
    const int grid = s.mode == ATTN_STATIC ? s.B * s.Hkv * s.S : s.W;
    const int src = s.mode == ATTN_STATIC   ? SRC_STATIC
                    : s.mode == ATTN_SHARED ? (shared_blocks(s.G) == 2 ? SRC_SHARED_WIDE : SRC_SHARED)
                                            : SRC_DYNAMIC;
    const hipError_t e = launch_decode(a, src, s.kv_fp8, grid, st);
    if (e != hipSuccess)
        return hip_fail(e, "decode launch");
    return ok();
}

int attn_combine(const attn_shape *shape, const void *workspace, size_t workspace_bytes, void *out,
                 float *lse, void *stream)
{
    Shape s;
    WsLayout L;
    int rc = check(shape, &s);
    if (rc != ATTN_OK)
        return rc;
    if (!out)
        return fail(ATTN_ERR_INVALID_ARG, "out is NULL");
    if (reinterpret_cast<uintptr_t>(out) % 16)
        return fail(ATTN_ERR_INVALID_ARG, "out must be 16-byte aligned");
    if ((rc = check_ws(s, workspace, workspace_bytes, &L)) != ATTN_OK)
        return rc;
    return enqueue_combine(s, L, workspace, out, lse, static_cast<hipStream_t>(stream));
}

static int enqueue_combine(const Shape &s, const WsLayout &L, const void *workspace, void *out, float *lse,
                           hipStream_t st)
{
    CombineArgs a{};
    a.header = at<int32_t>(workspace, L.header);
    a.req_shared = at<int32_t>(workspace, L.req_shared);
    a.req_member = at<int32_t>(workspace, L.req_member);
    a.req_own = at<int32_t>(workspace, L.req_own);
    a.item_solo = at<int32_t>(workspace, L.item_solo);
    a.seg_prefix = at<int32_t>(workspace, L.seg_prefix);
    a.part_o = at<float>(workspace, L.part_o);
    a.part_lse = at<float>(workspace, L.part_lse);
    a.out = static_cast<uint16_t *>(out);
    a.lse = lse;
    a.B = s.B;
    a.Hq = s.Hq;
    a.Hkv = s.Hkv;
    a.G = s.G;
    a.mode = s.mode;
    a.S = s.S;
    a.slot_rows = L.slot_rows;
    const hipError_t e = launch_combine(a, st);
    if (e != hipSuccess)
        return hip_fail(e, "combine launch");
    return ok();
}

int attn_workspace_init(const attn_shape *shape, void *workspace, size_t workspace_bytes, void *stream)
{
    Shape s;
    WsLayout L;
    int rc = check(shape, &s);
    if (rc != ATTN_OK)
        return rc;
    if ((rc = check_ws(s, workspace, workspace_bytes, &L)) != ATTN_OK)
        return rc;
    const hipError_t e = launch_ws_init(at<int32_t>(workspace, L.header), at<int32_t>(workspace, L.counters),
                                        s.B * s.Hkv, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "workspace init launch");
    return ok();
}

// Checks shared by attn_step and attn_step_noalloc (everything but the
// workspace).
static int check_step_args(const attn_shape *shape, Shape *s, const void *q, const void *k_cache,
                           const void *v_cache, const float *k_scale, const float *v_scale,
                           const int32_t *page_table, const int32_t *lengths, float sm_scale, const void *out)
{
    int rc = check(shape, s);
    if (rc != ATTN_OK)
        return rc;
    if (!q || !k_cache || !v_cache || !page_table || !lengths || !out)
        return fail(ATTN_ERR_INVALID_ARG, "q, k_cache, v_cache, page_table, lengths and out must be non-NULL");
    if (s->kv_fp8 && (!k_scale || !v_scale))
        return fail(ATTN_ERR_INVALID_ARG, "fp8 cache needs k_scale and v_scale");
    if (!(sm_scale == sm_scale) || sm_scale == INFINITY || sm_scale == -INFINITY)
        return fail(ATTN_ERR_INVALID_ARG, "sm_scale is not finite");
    if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_cache) |
         reinterpret_cast<uintptr_t>(v_cache) | reinterpret_cast<uintptr_t>(out)) % 16)
        return fail(ATTN_ERR_INVALID_ARG, "q, caches and out must be 16-byte aligned");
    return ATTN_OK;
}

// The single-launch step (dynamic or static) on the given arrival counters,
// status word and partial-result arrays.
static int enqueue_step(const Shape &s, const void *q, const void *k_cache, const void *v_cache,
                        const float *k_scale, const float *v_scale, const int32_t *page_table,
                        const int32_t *lengths, float sm_scale, int32_t *counters, int32_t *status,
                        float *part_o, float *part_lse, int slot_rows, void *out, float *lse, hipStream_t st)
{
    DecodeArgs a{};
    a.lengths = lengths;
    a.counters = counters;
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint8_t *>(k_cache);
    a.v = static_cast<const uint8_t *>(v_cache);
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.page_table = page_table;
    a.header = status;   // the single launch uses only the status word (H_STATUS = 0)
    a.part_o = part_o;
    a.part_lse = part_lse;
    a.out = static_cast<uint16_t *>(out);
    a.lse = lse;
    a.B = s.B;
    a.Hq = s.Hq;
    a.Hkv = s.Hkv;
    a.G = s.G;
    a.P = s.P;
    a.num_pages = s.num_pages;
    a.pt_stride = s.pt_stride;
    a.S = s.S;
    a.T = s.T;
    a.W = s.W;
    a.W_auto = s.W_auto;
    a.slot_rows = slot_rows;
    a.scale_log2 = sm_scale * 1.4426950408889634f;
    const int grid = s.mode == ATTN_STATIC ? s.B * s.Hkv * s.S : s.W;
    const hipError_t e = launch_decode(a, s.mode == ATTN_STATIC ? SRC_FUSED_STATIC : SRC_FUSED_DYNAMIC,
                                       s.kv_fp8, grid, st);
    if (e != hipSuccess)
        return hip_fail(e, "step launch");
    return ok();
}

int attn_step(const attn_shape *shape, const void *q, const void *k_cache, const void *v_cache,
              const float *k_scale, const float *v_scale, const int32_t *page_table,
              const int32_t *lengths, float sm_scale, void *workspace, size_t workspace_bytes,
              void *out, float *lse, void *stream)
{
    Shape s;
    WsLayout L;
    int rc = check_step_args(shape, &s, q, k_cache, v_cache, k_scale, v_scale, page_table, lengths, sm_scale, out);
    if (rc != ATTN_OK)
        return rc;
    if ((rc = check_ws(s, workspace, workspace_bytes, &L)) != ATTN_OK)
        return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (s.mode == ATTN_SHARED) {
        // the prefix-shared plan groups requests by comparing page tables; it
        // runs as its own launch, followed by the decode and the combine
        if ((rc = enqueue_plan(s, L, lengths, page_table, workspace, st)) != ATTN_OK)
            return rc;
        if ((rc = enqueue_decode(s, L, q, k_cache, v_cache, k_scale, v_scale, page_table, sm_scale, workspace, out,
                                 lse, st)) != ATTN_OK)
            return rc;
        return enqueue_combine(s, L, workspace, out, lse, st);
    }
    return enqueue_step(s, q, k_cache, v_cache, k_scale, v_scale, page_table, lengths, sm_scale,
                        at<int32_t>(workspace, L.counters), at<int32_t>(workspace, L.header),
                        at<float>(workspace, L.part_o), at<float>(workspace, L.part_lse), L.slot_rows, out, lse, st);
}

}  // extern "C"

// ---- attn_step_noalloc: the step without a caller workspace -----------------
// Its scratch (arrival counters, a status word, partial results) is this
// file-scope device array: one copy per GPU, placed when the library's code
// object is loaded on that GPU and held until the process ends. Host code never
// passes `scratch` itself to a kernel (on the host the name is only a stand-in);
// it uses the device address that hipGetSymbolAddress returns for the current
// GPU, taken once per GPU at its first call.
namespace vlkv {
namespace {

constexpr size_t kScratchBytes = ATTN_NOALLOC_SCRATCH_BYTES;
constexpr int64_t kScratchPairs = ATTN_NOALLOC_MAX_PAIRS;
constexpr size_t kScratchCounters = 0;                                     // int32 [kScratchPairs]
constexpr size_t kScratchStatus = kScratchPairs * sizeof(int32_t);         // int32 [kHeaderInts]
constexpr size_t kScratchParts = kScratchStatus + 256;                     // part_lse, then part_o
static_assert(kScratchStatus % 256 == 0, "scratch regions must stay 256-byte aligned");

__device__ __align__(256) static uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
uint8_t *g_scratch_ptr[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Partial-result bytes the single launch needs for this shape: two slots per
// workgroup (its first and last segment) in dynamic mode, S per (request, kv
// head) in static mode; each slot holds G rows of (D + 1) floats.
size_t noalloc_parts_bytes(const Shape &s, int64_t *slots)
{
    *slots = s.mode == ATTN_STATIC ? (int64_t)s.B * s.Hkv * s.S : 2 * (int64_t)s.W;
    return align256((size_t)*slots * s.G * sizeof(float)) + (size_t)*slots * s.G * s.D * sizeof(float);
}

}  // namespace
}  // namespace vlkv

extern "C" {

int attn_step_noalloc(const attn_shape *shape, const void *q, const void *k_cache, const void *v_cache,
                      const float *k_scale, const float *v_scale, const int32_t *page_table,
                      const int32_t *lengths, float sm_scale, void *out, float *lse, uint32_t *status,
                      void *stream)
{
    Shape s;
    int rc = check_step_args(shape, &s, q, k_cache, v_cache, k_scale, v_scale, page_table, lengths, sm_scale, out);
    if (rc != ATTN_OK)
        return rc;
    if (s.mode == ATTN_SHARED)
        return fail(ATTN_ERR_UNSUPPORTED, "attn_step_noalloc: mode ATTN_SHARED needs a workspace (attn_step)");
    if ((int64_t)s.B * s.Hkv > kScratchPairs)
        return fail(ATTN_ERR_INVALID_ARG, "attn_step_noalloc: batch * num_kv_heads = %lld exceeds the scratch limit %lld",
                    (long long)s.B * s.Hkv, (long long)kScratchPairs);
    int64_t slots;
    const size_t parts = noalloc_parts_bytes(s, &slots);
    if (parts > kScratchBytes - kScratchParts)
        return fail(ATTN_ERR_INVALID_ARG,
                    "attn_step_noalloc: %lld partial slots need %zu bytes, more than the %zu-byte scratch holds",
                    (long long)slots, parts, kScratchBytes - kScratchParts);
    if (reinterpret_cast<uintptr_t>(status) % 4)
        return fail(ATTN_ERR_INVALID_ARG, "status must be 4-byte aligned");
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(ATTN_ERR_INVALID_ARG, "attn_step_noalloc: device %d beyond the %d it serves", dev, kMaxDevices);
    hipStream_t st = static_cast<hipStream_t>(stream);
    bool first = false;
    std::call_once(g_scratch_once[dev], [&] {
        void *p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = static_cast<uint8_t *>(p);
        first = true;
    });
    if (g_scratch_err[dev] != hipSuccess)
        return hip_fail(g_scratch_err[dev], "hipGetSymbolAddress(scratch)");
    uint8_t *base = g_scratch_ptr[dev];
    int32_t *counters = reinterpret_cast<int32_t *>(base + kScratchCounters);
    int32_t *own_status = reinterpret_cast<int32_t *>(base + kScratchStatus);
    if (first) {
        // the counters must start at zero (every completed step leaves them
        // there); cleared by a fill kernel on the caller's stream, not a memset
        if ((e = launch_ws_init(own_status, counters, (int)kScratchPairs, st)) != hipSuccess)
            return hip_fail(e, "scratch init launch");
    }
    float *part_lse = reinterpret_cast<float *>(base + kScratchParts);
    float *part_o = reinterpret_cast<float *>(base + kScratchParts + align256((size_t)slots * s.G * sizeof(float)));
    return enqueue_step(s, q, k_cache, v_cache, k_scale, v_scale, page_table, lengths, sm_scale, counters,
                        status ? reinterpret_cast<int32_t *>(status) : own_status, part_o, part_lse, s.G, out, lse,
                        st);
}

int attn_append_kv(const attn_shape *shape, const void *k_new, const void *v_new, const int32_t *positions,
                   const int32_t *page_table, const float *k_scale, const float *v_scale, void *k_cache,
                   void *v_cache, void *workspace, size_t workspace_bytes, void *stream)
{
    Shape s;
    WsLayout L;
    int rc = check(shape, &s);
    if (rc != ATTN_OK)
        return rc;
    if (!k_new || !v_new || !positions || !page_table || !k_cache || !v_cache)
        return fail(ATTN_ERR_INVALID_ARG,
                    "k_new, v_new, positions, page_table, k_cache and v_cache must be non-NULL");
    if (s.kv_fp8 && (!k_scale || !v_scale))
        return fail(ATTN_ERR_INVALID_ARG, "fp8 cache needs k_scale and v_scale");
    if ((reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new) |
         reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache)) % 16)
        return fail(ATTN_ERR_INVALID_ARG, "new rows and caches must be 16-byte aligned");
    int32_t *header = nullptr;
    if (workspace) {
        if ((rc = check_ws(s, workspace, workspace_bytes, &L)) != ATTN_OK)
            return rc;
        header = at<int32_t>(workspace, L.header);
    }
    AppendArgs a;
    a.k_new = static_cast<const uint16_t *>(k_new);
    a.v_new = static_cast<const uint16_t *>(v_new);
    a.positions = positions;
    a.page_table = page_table;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.k_cache = static_cast<uint8_t *>(k_cache);
    a.v_cache = static_cast<uint8_t *>(v_cache);
    a.header = header;
    a.B = s.B;
    a.Hkv = s.Hkv;
    a.P = s.P;
    a.num_pages = s.num_pages;
    a.pt_stride = s.pt_stride;
    const hipError_t e = launch_append(a, s.kv_fp8, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "append launch");
    return ok();
}

#ifdef VLKV_DEBUG_VISITS
int attn_debug_visits(int32_t *tok_counts, int64_t tok_stride, int32_t *out_counts)
{
    if ((tok_counts != nullptr) != (tok_stride > 0))
        return fail(ATTN_ERR_INVALID_ARG, "tok_counts needs tok_stride > 0 (and null needs 0)");
    hipError_t e = hipDeviceSynchronize();   // no kernel of an earlier step still counts
    if (e == hipSuccess)
        e = set_debug_visits(tok_counts, tok_stride, out_counts);
    if (e != hipSuccess)
        return hip_fail(e, "visit counters");
    return ok();
}
#endif

int attn_get_status(const void *workspace, uint32_t *flags, void *stream)
{
    if (!workspace || !flags)
        return fail(ATTN_ERR_INVALID_ARG, "workspace and flags must be non-NULL");
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(flags, workspace, sizeof(uint32_t), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess)
        e = hipStreamSynchronize(st);
    if (e != hipSuccess)
        return hip_fail(e, "status copy");
    return ok();
}

int attn_read_plan(const attn_shape *shape, const void *workspace, int32_t *header, int32_t *len_eff,
                   int32_t *tiles_prefix, int32_t *seg_prefix, int32_t *first_wg, int32_t *wg_begin,
                   int32_t *wg_start_b, void *stream)
{
    Shape s;
    int rc = check(shape, &s);
    if (rc != ATTN_OK)
        return rc;
    if (!workspace)
        return fail(ATTN_ERR_INVALID_ARG, "workspace is NULL");
    const WsLayout L = ws_layout(s);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t ni = L.max_items, nig = L.max_items * s.Hkv;
    struct Item {
        int32_t *dst;
        size_t off;
        int64_t n;
    } items[] = {
        {header, L.header, kHeaderInts},      {len_eff, L.len_eff, ni},
        {tiles_prefix, L.tiles_prefix, ni + 1}, {seg_prefix, L.seg_prefix, nig + 1},
        {first_wg, L.first_wg, nig},           {wg_begin, L.wg_begin, s.W + 1},
        {wg_start_b, L.wg_start_b, s.W},
    };
    for (const Item &it : items) {
        if (!it.dst)
            continue;
        const hipError_t e = hipMemcpyAsync(it.dst, at<int32_t>(workspace, it.off),
                                            sizeof(int32_t) * it.n, hipMemcpyDeviceToHost, st);
        if (e != hipSuccess)
            return hip_fail(e, "plan copy");
    }
    const hipError_t e = hipStreamSynchronize(st);
    if (e != hipSuccess)
        return hip_fail(e, "plan copy sync");
    return ok();
}

int attn_read_plan_items(const attn_shape *shape, const void *workspace, int32_t *item_req, int32_t *item_start,
                         int32_t *item_m, int32_t *item_solo, int32_t *req_shared, int32_t *req_member,
                         int32_t *req_own, void *stream)
{
    Shape s;
    int rc = check(shape, &s);
    if (rc != ATTN_OK)
        return rc;
    if (s.mode != ATTN_SHARED)
        return fail(ATTN_ERR_INVALID_ARG, "attn_read_plan_items needs mode ATTN_SHARED");
    if (!workspace)
        return fail(ATTN_ERR_INVALID_ARG, "workspace is NULL");
    const WsLayout L = ws_layout(s);
    hipStream_t st = static_cast<hipStream_t>(stream);
    struct Item {
        int32_t *dst;
        size_t off;
        int64_t n;
    } items[] = {
        {item_req, L.item_req, L.max_items},     {item_start, L.item_start, L.max_items},
        {item_m, L.item_m, L.max_items},         {item_solo, L.item_solo, L.max_items},
        {req_shared, L.req_shared, s.B},         {req_member, L.req_member, s.B},
        {req_own, L.req_own, s.B},
    };
    for (const Item &it : items) {
        if (!it.dst)
            continue;
        const hipError_t e = hipMemcpyAsync(it.dst, at<int32_t>(workspace, it.off),
                                            sizeof(int32_t) * it.n, hipMemcpyDeviceToHost, st);
        if (e != hipSuccess)
            return hip_fail(e, "plan copy");
    }
    const hipError_t e = hipStreamSynchronize(st);
    if (e != hipSuccess)
        return hip_fail(e, "plan copy sync");
    return ok();
}

const char *attn_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"

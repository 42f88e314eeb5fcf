// Internal declarations shared by the planner, decode/combine kernels and the
// C ABI of libvlkv_attn.so. Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace vlkv {

constexpr int kHeadDim = 128;      // D supported by the decode kernel
constexpr int kWaves = 4;          // wavefronts per decode workgroup
constexpr int kBlockTokens = 64;   // tile granularity: 4 waves x 16 bf16 rows
constexpr int kDecodeThreads = 256;
constexpr int kMaxGroup = 16;      // query heads per kv head (one MFMA column block)
constexpr int kMaxBatch = 8192;    // planner keeps the tile prefix in LDS
constexpr int kHeaderInts = 8;
// status word bit for a broken plan invariant (ATTN_STATUS_INTERNAL)
constexpr unsigned kStatusInternal = 4u;

// header fields (mode 2: H_CHUNK holds the number of items, H_SPLITS the
// requests per shared pass R)
enum : int { H_STATUS = 0, H_UNITS = 1, H_WEFF = 2, H_MAXLEN = 3, H_CHUNK = 4, H_SPLITS = 5,
             H_TILES = 6, H_TILE = 7 };
enum : int { H_ITEMS = 4, H_GROUP = 5 };

// plan modes (the public ATTN_DYNAMIC / ATTN_STATIC / ATTN_SHARED)
enum : int { MODE_DYNAMIC = 0, MODE_STATIC = 1, MODE_SHARED = 2 };

// Requests per shared pass: the shared decode stacks them in MFMA column
// blocks of kMaxGroup query rows, two blocks when one holds two requests or
// fewer (G >= 8), else one (G <= kMaxGroup).
__host__ __device__ constexpr int shared_blocks(int G) { return G >= 8 ? 2 : 1; }
__host__ __device__ constexpr int shared_group(int G) { return shared_blocks(G) * kMaxGroup / G; }

// Byte offsets of the workspace regions (all 256-B aligned). In mode 2 the
// plan is over items (at most 2B): len_eff, tiles_prefix, seg_prefix, first_wg
// and wg_start_b are indexed by item, and the item_* / req_* regions exist.
struct WsLayout {
    size_t header, len_eff, tiles_prefix, seg_prefix, first_wg, wg_begin, wg_start_b;
    size_t item_req, item_start, item_m, item_solo, req_shared, req_member, req_own;
    size_t counters, part_lse, part_o, total;
    int64_t max_slots, max_items;
    int slot_rows;   // query rows per partial slot
};

// Where a decode workgroup's sequence of segments comes from.
enum PlanSrc : int {
    SRC_DYNAMIC = 0,        // plan arrays written by attn_plan (dynamic mode)
    SRC_STATIC = 1,         // plan arrays written by attn_plan (static mode)
    SRC_FUSED_DYNAMIC = 2,  // single launch: each workgroup derives its range from the lengths
    SRC_FUSED_STATIC = 3,   // single launch, static split-K
    SRC_SHARED = 4,         // plan arrays written by attn_plan (mode 2: items, prefix-shared pages)
    SRC_SHARED_WIDE = 5,    // the same with two MFMA column blocks of query rows (G >= 8)
};

__host__ __device__ constexpr bool is_shared(int src) { return src == SRC_SHARED || src == SRC_SHARED_WIDE; }

// Workgroups a dynamic plan of N units uses. W is the launch's workgroup
// count; with the library default (W_auto = the device's compute units,
// W = 2 * W_auto) two per compute unit when that leaves at least 32 units per
// workgroup, else one per compute unit. Never more than N.
__host__ __device__ inline int64_t plan_wgs(int64_t N, int W, int W_auto)
{
    const int64_t Wu = (W_auto > 0 && N < 32 * (int64_t)W) ? W_auto : W;
    return N < Wu ? N : Wu;
}

struct Shape {
    int B, Hq, Hkv, G, D, P, num_pages, pt_stride, T, W, kv_fp8, mode, S;
    int W_auto;   // compute units when num_wgs = 0 chose W = 2 * W_auto, else 0
};

WsLayout ws_layout(const Shape &s);

struct PlanArgs {
    const int32_t *lengths;
    const int32_t *page_table;   // mode 2 only
    int32_t *header, *len_eff, *tiles_prefix, *seg_prefix, *first_wg, *wg_begin, *wg_start_b;
    // mode 2 only
    int32_t *item_req, *item_start, *item_m, *item_solo, *req_shared, *req_member, *req_own;
    int B, Hkv, G, P, pt_stride, num_pages, T, W, mode, S;
    int W_auto;   // see plan_wgs
};

struct DecodeArgs {
    const int32_t *lengths;    // raw per-request lengths (single-launch sources only)
    int32_t *counters;         // [B*Hkv] arrival counters (single-launch sources only)
    const uint16_t *q;         // [B][Hq][D] bf16 bits
    const uint8_t *k;          // cache base (bytes)
    const uint8_t *v;
    const float *k_scale, *v_scale;
    const int32_t *page_table;
    int32_t *header;
    const int32_t *len_eff, *tiles_prefix, *seg_prefix, *first_wg, *wg_begin, *wg_start_b;
    const int32_t *item_req, *item_start, *item_m, *item_solo;   // SRC_SHARED only
    float *part_o, *part_lse;
    uint16_t *out;             // [B][Hq][D] bf16 bits
    float *lse;                // [B][Hq] or null
    int B, Hq, Hkv, G, P, num_pages, pt_stride, S, T, W;
    int W_auto;                // see plan_wgs (single launch, dynamic)
    int slot_rows;             // query rows per partial slot
    float scale_log2;          // sm_scale * log2(e)
};

struct CombineArgs {
    const int32_t *header, *seg_prefix;
    const int32_t *req_shared, *req_member, *req_own, *item_solo;   // mode 2 only
    const float *part_o, *part_lse;
    uint16_t *out;
    float *lse;
    int B, Hq, Hkv, G, mode, S, slot_rows;
};

struct AppendArgs {
    const uint16_t *k_new, *v_new;   // [B][Hkv][D] bf16 bits
    const int32_t *positions;        // [B]
    const int32_t *page_table;       // [B][pt_stride]
    const float *k_scale, *v_scale;  // [B][Hkv] (fp8 only)
    uint8_t *k_cache, *v_cache;      // [num_pages][Hkv][P][D]
    int32_t *header;                 // status word, or null
    int B, Hkv, P, num_pages, pt_stride;
};

// Error reporting of the C ABI (attn_last_error): set the message, return code.
int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int ok();

hipError_t launch_plan(const PlanArgs &a, hipStream_t st);
hipError_t launch_append(const AppendArgs &a, int kv_fp8, hipStream_t st);
hipError_t launch_decode(const DecodeArgs &a, int src, int kv_fp8, int grid, hipStream_t st);
hipError_t launch_combine(const CombineArgs &a, hipStream_t st);
hipError_t launch_ws_init(int32_t *header, int32_t *counters, int n_counters, hipStream_t st);

#ifdef VLKV_DEBUG_VISITS
// Visit-counting build only: every decode and combine kernel adds 1 to
// tok[(b * Hkv + g) * tok_stride + j] for each cached row j of request b, kv
// head g that its attention math consumes, and 1 to out[b * Hq + h] for each
// write of a final output row (null pointers: nothing is counted).
hipError_t set_debug_visits(int32_t *tok, int64_t tok_stride, int32_t *out);
#endif

}  // namespace vlkv

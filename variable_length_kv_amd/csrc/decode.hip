// Split-KV paged decode attention and its log-sum-exp combine, for gfx950.
//
// The source article's Dynamic Attention spreads uneven decode work over GPU
// execution units: KV-cache work is cut into uniform tiles handed to CTAs by
// current load, and split results are merged ("split-k"); the static split-k is
// the comparison point [Tencent HPC lands in SGLang, challenging default
// inference kernels, sec. "Why Tencent HPC matters for online model serving"].
// All variants here share one per-block body and differ only in where a
// workgroup's sequence of (request, kv head, block range) segments comes from:
// the plan arrays attn_plan wrote, or (single launch) the lengths themselves,
// from which every workgroup derives its own unit range; then the last
// workgroup to finish a split (request, kv head) pair merges its partials,
// after its own blocks.
//
// Workgroup = 4 wave64s. A block of one (request b, kv head g), 64 tokens for a
// bf16 cache and 128 for fp8, is split into four slices, one per wave: 16 bf16
// or 32 fp8 cache rows, 4 KB of K and 4 KB of V either way. Every wave walks the
// same sequence of blocks and keeps its own online-softmax state for the G query
// heads of g; the four states are merged through LDS at the end of each segment.
//
// Per wave and slice:
//   * The slice's K and V rows (contiguous in the page) are read by raw buffer
//     loads through descriptors whose range is exactly the slice's valid rows,
//     lane l taking bytes 16 l + 1024 i of load i: each instruction reads 1 KB
//     of whole 128-byte lines, non-temporally (every K/V byte is read once per
//     step). Two slices per wave are in flight in registers, on top of two
//     resident waves per SIMD.
//   * At the slice's compute the wave writes its registers to its own LDS
//     staging rows and reads back the K operand layout (lane l: token row l%16,
//     a run of dims selected by l/16). Loading that layout straight from memory
//     reads 64 bytes of each of 16 rows per instruction, half lines that a
//     non-temporal load would fetch twice; through LDS the loads stream at the
//     rate of contiguous reads.
//   * S^T = K Q^T with bf16 MFMAs 16x16x32 (16 tokens x 16 query rows; rows >= G
//     are zero): one 16-token sub-tile for bf16, two for fp8, whose codes are
//     widened to bf16 exactly first. The result's lane layout (lane l: tokens
//     4*(l/16)+i, query row l%16) is the B operand of the P.V MFMA, so P^T needs
//     no data movement.
//   * Online softmax in base 2 (sm_scale*log2 e, times the fp8 k scale, folded
//     into one multiply); per-row maxima across the 4 lane groups by permlane
//     swaps; the reference maximum moves only when it is exceeded by more than
//     kLazy.
//   * V^T, the A operand of P.V, is read from the staged V rows by LDS transpose
//     loads (16-bit or 8-bit elements), fp8 codes widened to bf16 after them.
//   * O^T (128 dims x 16 query rows) += V^T P^T with 8 MFMAs into 32 fp32
//     registers.
#include "vlkv_device.hpp"
#include "vlkv_internal.hpp"

namespace vlkv {
namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef uint32_t u32x2 __attribute__((__vector_size__(2 * sizeof(uint32_t))));
typedef float f32x2 __attribute__((__vector_size__(2 * sizeof(float))));
typedef short s16x4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef int i32x2 __attribute__((ext_vector_type(2)));      // LDS transpose loads' types
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.6931471805599453f;
constexpr int kLdsRow = kHeadDim + 4;  // padded fp32 row of the segment-end mailbox
// A staged K or V row: 256 bytes of data (one bf16 cache row, or two fp8 cache
// rows with a 16-byte gap between them) padded to 288 bytes, which keeps the
// row-strided operand reads and the transpose loads on distinct LDS banks.
constexpr int kStgRow = kHeadDim * 2 + 32;
constexpr int kFp8HalfGap = 16;   // offset of an fp8 staged row's second cache row: 128 + 16
constexpr float kLazy = 8.f;           // lazy-rescale threshold (log2 units)
constexpr int kMergeBatch = 4;         // partials folded together by the LSE merge
constexpr int kMailboxSpin = 1 << 22;  // bound of a mailbox wait (s_sleep 1 each, ~0.1 s)
// Word 3 of a raw buffer descriptor (gfx9 family): 32-bit data format, no
// swizzle, no index. A data format of 0 would make every access read zero.
constexpr int kRsrcWord3 = 0x00020000;
// Cache policy of the K/V loads: non-temporal (every K/V byte is read once per step).
constexpr int kLoadNT = 2;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

#ifdef VLKV_DEBUG_VISITS
// Counters of the visit-counting build (see set_debug_visits).
struct DebugVisits {
    int32_t *tok, *out;
    int64_t tok_stride;
};
__device__ DebugVisits g_visits;

__device__ __forceinline__ void debug_count_out(size_t hq, int d4)
{
    if (g_visits.out && d4 == 0)
        atomicAdd(g_visits.out + hq, 1);
}
#define VLKV_COUNT_OUT(hq, d4) debug_count_out(hq, d4)
#else
#define VLKV_COUNT_OUT(hq, d4) ((void)0)
#endif

// Wave priority from a workgroup's progress through its blocks: 3 for the
// first half, 2 up to 80%, 1 up to 95%, 0 for the rest. Two workgroups share a
// CU, and among ready waves of equal priority the SIMD issues the older one
// first, so the workgroup dispatched second falls behind and finishes last,
// alone on its CU. With priorities that fall as the work progresses, the
// workgroup that is behind issues first whenever both are ready.
__device__ __forceinline__ void set_progress_priority(int done, int total)
{
    // wave-uniform 32-bit compares (block counts stay far below 2^26): scalar
    // instructions only, no division in the loop
    const int d = __builtin_amdgcn_readfirstlane(done), t = __builtin_amdgcn_readfirstlane(total);
    if (2 * d < t)
        __builtin_amdgcn_s_setprio(3);
    else if (5 * d < 4 * t)
        __builtin_amdgcn_s_setprio(2);
    else if (20 * d < 19 * t)
        __builtin_amdgcn_s_setprio(1);
    else
        __builtin_amdgcn_s_setprio(0);
}

// Read-only data of the step (plan arrays, lengths, page table, scales) is read
// through the constant address space: wave-uniform addresses then become scalar
// loads, which are counted apart from the K/V vector loads, so waiting for a
// page id never waits for K/V data still in flight.
template <typename T>
__device__ __forceinline__ T ldc(const T *p, size_t i)
{
    return ((const __attribute__((address_space(4))) T *)(p))[i];
}

// Four fp32 values rounded to bf16 (nearest even) and packed as an MFMA
// operand. Converting in pairs keeps one v_cvt_pk_bf16_f32 per two values;
// converting the whole vector into an MFMA operand lowers to one convert per
// value plus byte permutes.
__device__ __forceinline__ s16x4 pack_bf16x4(f32x4 x)
{
    const bf16x2 lo = __builtin_convertvector((f32x2){x[0], x[1]}, bf16x2);
    const bf16x2 hi = __builtin_convertvector((f32x2){x[2], x[3]}, bf16x2);
    return __builtin_bit_cast(s16x4, (u32x2){__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)});
}

// Two packed 4-value operands side by side: an 8-value MFMA operand.
__device__ __forceinline__ bf16x8 cat_bf16x8(s16x4 a, s16x4 b)
{
    const u32x2 x = __builtin_bit_cast(u32x2, a), y = __builtin_bit_cast(u32x2, b);
    return __builtin_bit_cast(bf16x8, (u32x4){x[0], x[1], y[0], y[1]});
}

// The bf16 values of a packed operand, widened back to fp32 (exact).
__device__ __forceinline__ f32x4 unpack_bf16x4(s16x4 v)
{
    const u32x2 w = __builtin_bit_cast(u32x2, v);
    return f32x4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u), __uint_as_float(w[1] << 16),
                 __uint_as_float(w[1] & 0xffff0000u)};
}

// max / sum over lanes l, l^16, l^32, l^48 (the 4 row groups of an MFMA tile)
__device__ __forceinline__ float xmax4(float x)
{
    auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xsum4(float x)
{
    auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Validated length of request b as the planner defines it: L_b if
// 0 <= L_b <= pt_stride * P, else 0.
__device__ __forceinline__ int len_valid(const DecodeArgs *a, int b)
{
    const int L = ldc(a->lengths, b);
    return (L < 0 || (int64_t)L > (int64_t)a->pt_stride * a->P) ? 0 : L;
}

// Registers of one in-flight slice (fp8 uses k[0..1], v[0..1]) and q of the
// first column block of 16 query rows (a second block's q is loaded when its
// segment starts: carrying it in every slot would not fit the registers).
struct Slot {
    u32x4 k[4];
    u32x4 v[4];
    u32x4 q[4];
};

// Scalar description of one block as seen by one wave.
struct Meta {
    int valid;   // a block exists
    int b, g;    // request, kv head
    int tok0;    // first token of this wave's slice
    int nv;      // valid tokens of this wave's slice (0..16)
    int first;   // first block of its segment
    int last;    // last block of its segment
    int slot;    // partial slot
    int direct;  // write the final output directly
    int nseg;    // single launch: segments of the pair (arrivals before its merge)
    int wfirst;  // single launch, dynamic: workgroup of the pair's first segment
    int first_off;  // single launch, dynamic: slot offset of that first segment
    int m;       // query requests b, b+1, .., b+m-1 (more than one: a shared prefix)
    int tbase;   // first token of the item (0 unless a request's own rest)
    float ksc, vsc;   // fp8 scales of the first column block (per row in SRC_SHARED)
};

// Walks a workgroup's blocks in order. SRC_DYNAMIC / SRC_FUSED_DYNAMIC /
// SRC_SHARED: the contiguous unit range of the plan (SRC_SHARED: over items,
// b is then the item index); SRC_STATIC / SRC_FUSED_STATIC: the one
// (b, g, split) of this workgroup. A block is KBT tokens counted from its
// segment's first token (a segment starts at a tile boundary), one slice of
// KBT / kWaves tokens per wave; a segment's last block may be short.
template <int SRC, int KBT>
struct Walker {
    static constexpr int kSliceT = KBT / kWaves;   // tokens per wave per block
    static constexpr bool kFused = SRC == SRC_FUSED_DYNAMIC || SRC == SRC_FUSED_STATIC;
    static constexpr bool kShared = is_shared(SRC);
    static constexpr bool kPlanned = SRC == SRC_DYNAMIC || kShared;   // ranges from attn_plan's arrays
    static constexpr bool kDyn = kPlanned || SRC == SRC_FUSED_DYNAMIC;

    const DecodeArgs *a;
    int w, wave;
    int b, g, L, nt, units_left, done;
    int tok, tok_seg, tok_end;   // current block's first token, the segment's first and end tokens
    int slot, direct, nseg, wfirst, first_off;
    // SRC_SHARED: the item's first request, first token, request count and
    // whether it is its request's only item
    int req = 0, ist = 0, mm = 1, solo = 1;
    __device__ void load_item()
    {
        if (kShared) {
            req = ldc(a->item_req, b);
            ist = ldc(a->item_start, b);
            mm = ldc(a->item_m, b);
            solo = ldc(a->item_solo, b);
        }
    }
    // single launch, dynamic
    int tpb;                 // tiles before request b
    int first_seg;           // the next segment entered is the workgroup's first
    int64_t N, We, u_beg, u_end;
    UniformSplit split;   // the plan's cuts: begin(w) = floor(w N / We)

    __device__ int64_t owner(int64_t u) const { return split.owner((uint32_t)u); }
    __device__ int64_t begin_of(int64_t ww) const { return split.begin((uint32_t)ww); }

    // single launch, dynamic: the prologue's LDS copies of the tiles prefix and
    // the validated lengths, used until the block loop starts (then nullptr)
    const int32_t *ltp = nullptr, *llen = nullptr;

    __device__ int tiles_of(int bb) const
    {
        if (kFused && ltp)
            return __builtin_amdgcn_readfirstlane(ltp[bb + 1]) - __builtin_amdgcn_readfirstlane(ltp[bb]);
        return kFused ? (len_valid(a, bb) + a->T - 1) / a->T
                      : ldc(a->tiles_prefix, bb + 1) - ldc(a->tiles_prefix, bb);
    }
    __device__ int length_of(int bb) const
    {
        if (kFused && llen)
            return __builtin_amdgcn_readfirstlane(llen[bb]);
        return kFused ? len_valid(a, bb) : ldc(a->len_eff, bb);
    }

    __device__ void enter_segment(int ta, int tb)
    {
        tok = tok_seg = ta * a->T;
        tok_end = (int)min((int64_t)tb * a->T, (int64_t)L);
        const int bg = b * a->Hkv + g;
        if (kPlanned) {
            const int s0 = ldc(a->seg_prefix, bg);
            const int s1 = ldc(a->seg_prefix, bg + 1);
            slot = s0 + (w - ldc(a->first_wg, bg));
            // an item that is not its request's only item always leaves a partial
            direct = (s1 - s0) == 1 && solo;
        } else {
            // slot 2w for the workgroup's first segment, 2w+1 for its last; a
            // segment that is neither covers its whole pair and is direct
            const int64_t pu0 = (int64_t)tpb * a->Hkv + (int64_t)g * nt;
            direct = pu0 >= u_beg && pu0 + nt <= u_end;
            slot = 2 * w + (first_seg ? 0 : 1);
            first_seg = 0;
            if (!direct) {
                const int64_t wf = owner(pu0);
                wfirst = (int)wf;
                nseg = (int)(owner(pu0 + nt - 1) - wf + 1);
                first_off = begin_of(wf) < pu0 ? 1 : 0;
            }
        }
    }

    // lds_tp, lds_len: tiles prefix and validated lengths (single launch, dynamic only)
    __device__ void init(const DecodeArgs *args, int wg, int wv, const int32_t *lds_tp, const int32_t *lds_len,
                         int64_t N_, int64_t We_, int chunk)
    {
        a = args;
        if (SRC == SRC_FUSED_DYNAMIC) {
            ltp = lds_tp;
            llen = lds_len;
        }
        w = wg;
        wave = wv;
        done = 0;
        nseg = 1;
        wfirst = 0;
        first_off = 0;
        if (kDyn) {
            int u0, u1;
            if (kPlanned) {
                u0 = ldc(a->wg_begin, w);
                u1 = ldc(a->wg_begin, w + 1);
                b = ldc(a->wg_start_b, w);
                tpb = ldc(a->tiles_prefix, b);
                nt = ldc(a->tiles_prefix, b + 1) - tpb;
                load_item();
            } else {
                N = N_;
                We = We_;
                split.init((uint32_t)N, (uint32_t)We);
                u_beg = begin_of(w);
                u_end = begin_of(w + 1);
                u0 = (int)u_beg;
                u1 = (int)u_end;
                // largest b in [0, B) with Hkv * tp[b] <= u0: the request of unit u0
                // (tp is non-decreasing and tp[0] = 0). Each round, the wave's
                // lanes test 64 evenly spaced candidates of the remaining range
                // at once; the count of passing ones locates the answer within
                // one stride (one round for B <= 64, two for B <= 4096).
                int lo = 0, n = a->B;
                const int lane = threadIdx.x & 63;
                while (n > 1) {
                    const int st = (n + 63) >> 6;
                    const bool ok = lane * st < n && (int64_t)lds_tp[lo + lane * st] * a->Hkv <= u0;
                    const int c = __builtin_popcountll(__builtin_amdgcn_ballot_w64(ok));   // >= 1 (lane 0)
                    lo += (c - 1) * st;
                    n = min(st, n - (c - 1) * st);
                }
                b = lo;
                tpb = __builtin_amdgcn_readfirstlane(lds_tp[b]);
                nt = __builtin_amdgcn_readfirstlane(lds_tp[b + 1]) - tpb;
                first_seg = 1;
            }
            L = length_of(b);
            const int rem = u0 - tpb * a->Hkv;
            g = rem / nt;
            const int t = rem - g * nt;
            const int take = min(nt - t, u1 - u0);
            units_left = u1 - u0 - take;
            enter_segment(t, t + take);
        } else {
            const int S = a->S;
            const int bg = w / S, s = w - bg * S;
            b = bg / a->Hkv;
            g = bg - b * a->Hkv;
            L = length_of(b);
            const int C = SRC == SRC_STATIC ? ldc(a->header, H_CHUNK) : chunk;
            const int lo = s * C, hi = min(lo + C, L);
            units_left = 0;
            slot = w;
            direct = S == 1;
            nseg = S;
            tok = tok_seg = lo;
            if (hi > lo) {
                tok_end = hi;
            } else {
                // empty split: one pseudo-block without valid tokens, so the
                // workgroup still writes its (empty) result
                tok_end = lo + 1;
                L = 0;
            }
        }
    }

    // Step to the next request that has tiles.
    __device__ void next_request()
    {
        do {
            tpb += nt;
            ++b;
            nt = tiles_of(b);
        } while (nt == 0);
        L = length_of(b);
        load_item();
    }

    // Number of blocks this workgroup will process (a scalar walk over its
    // segments; the walker itself is not advanced).
    __device__ int count_blocks() const
    {
        const int n0 = tok < tok_end ? (tok_end - tok + KBT - 1) / KBT : 0;
        if (!kDyn)
            return n0;
        int n = n0;
        int bb = b, gg = g, ntt = nt, LL = L, left = units_left;
        while (left > 0) {
            if (++gg == a->Hkv) {
                gg = 0;
                do {
                    ++bb;
                    ntt = tiles_of(bb);
                } while (ntt == 0);
                LL = length_of(bb);
            }
            const int take = min(ntt, left);
            left -= take;
            n += (int)((min((int64_t)take * a->T, (int64_t)LL) + KBT - 1) / KBT);
        }
        return n;
    }

    // Describe the current block and step to the next one. Past the end the
    // description is invalid: no valid tokens, no segment start or end.
    __device__ Meta next()
    {
        Meta m;
        m.valid = !done;
        m.b = b;
        m.g = g;
        m.tok0 = tok + wave * kSliceT;
        m.nv = done ? 0 : max(0, min(kSliceT, min(tok_end, L) - m.tok0));
        m.first = !done && tok == tok_seg;
        m.last = !done && tok + KBT >= tok_end;
        m.slot = slot;
        m.direct = direct;
        m.nseg = nseg;
        m.wfirst = wfirst;
        m.first_off = first_off;
        m.m = kShared ? mm : 1;
        m.tbase = kShared ? ist : 0;
        if (kShared)
            m.b = req;
        m.ksc = 1.f;
        m.vsc = 1.f;
        if (done)
            return m;
        tok += KBT;
        if (tok >= tok_end) {
            if (kDyn && units_left > 0) {
                ++g;
                if (g == a->Hkv) {
                    g = 0;
                    next_request();
                }
                const int take = min(nt, units_left);
                units_left -= take;
                enter_segment(0, take);
            } else {
                done = 1;
            }
        }
        return m;
    }
};

// Stores of the partials exchanged between workgroups inside one launch:
// relaxed atomic stores at agent scope, which the chip makes coherent across
// its XCDs' L2 caches by writing them through to the device's coherence
// point (the readers' side is the acquire fence before the merge).
__device__ __forceinline__ void store_coherent(float *p, float x)
{
    __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Four consecutive floats base[i .. i+3] with the same cache policy as
// store_coherent (sc1: written through to the device's coherence point), as
// one 16-byte store: the per-float stores would each be a separate partial
// write of a memory line. `base` is wave-uniform (a buffer descriptor) and
// 0 <= i < 2^29.
constexpr int kStoreSc1 = 16;   // cache-policy bit sc1 of a buffer store (gfx950)
__device__ __forceinline__ void store_coherent4(float *base, int i, f32x4 x)
{
    const auto r = __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7fffffff, kRsrcWord3);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, i * (int)sizeof(float), 0, kStoreSc1);
}

// The LSE merge of partial results (o normalised, lse in base 2) of one
// (request, kv head) pair, for one (head, 4 dims) of the output. The running
// state is M (largest lse so far), den = sum 2^(lse_s - M) and
// o = sum 2^(lse_s - M) o_s; partials are folded in slot order, kMergeBatch at a
// time. Both merges (the combine kernel and the single launch's last arriver)
// go through these two functions, with contraction off, so they round
// identically wherever they are inlined.
__device__ __forceinline__ void merge_fold(float &M, float &den, f32x4 &o, const float (&ls)[kMergeBatch],
                                           const f32x4 (&xs)[kMergeBatch], int nb)
{
#pragma clang fp contract(off)
    float Mb = M;
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j)
        if (j < nb)
            Mb = fmaxf(Mb, ls[j]);
    if (Mb == -INFINITY)
        return;   // every partial so far is empty
    const float r = fast_exp2(M - Mb);   // 0 when M is -inf
    den *= r;
    o *= r;
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
        if (j < nb) {
            const float e = fast_exp2(ls[j] - Mb);
            den += e;
            o += e * xs[j];
        }
    }
    M = Mb;
}

// Final step of the merge: o / den as bf16 and the natural-log lse.
__device__ __forceinline__ void merge_write(float M, float den, f32x4 o, uint16_t *out, float *lse, size_t hq, int d4)
{
#pragma clang fp contract(off)
    float lse2 = -INFINITY;
    if (M != -INFINITY) {
        o *= 1.f / den;
        lse2 = M + log2f(den);
    } else {
        o = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    *reinterpret_cast<bf16x4 *>(out + hq * kHeadDim + d4) = __builtin_convertvector(o, bf16x4);
    if (lse && d4 == 0)
        lse[hq] = lse2 * kLn2;
    VLKV_COUNT_OUT(hq, d4);
}

// Merge n partials of one (request, kv head) pair into the bf16 output and the
// natural-log lse. base_of(s) is the partial row of head 0 of the s-th partial
// (its heads are the G rows from there). Run by all threads of a workgroup.
template <typename BaseOf>
__device__ __forceinline__ void merge_partials(const float *part_o, const float *part_lse, int n, BaseOf base_of,
                                               int G, int Hq, int b, int g, uint16_t *out, float *lse)
{
    constexpr int D = kHeadDim;
    for (int idx = threadIdx.x; idx < G * 32; idx += kDecodeThreads) {
        const int h = idx >> 5, d4 = (idx & 31) * 4;
        float M = -INFINITY, den = 0.f;
        f32x4 o = {0.f, 0.f, 0.f, 0.f};
        for (int s0 = 0; s0 < n; s0 += kMergeBatch) {
            float ls[kMergeBatch];
            f32x4 xs[kMergeBatch];
#pragma unroll
            for (int j = 0; j < kMergeBatch; ++j) {
                const size_t sl = (size_t)base_of(s0 + j < n ? s0 + j : s0) + h;
                ls[j] = part_lse[sl];
                xs[j] = *reinterpret_cast<const f32x4 *>(part_o + sl * D + d4);
            }
            merge_fold(M, den, o, ls, xs, n - s0);
        }
        merge_write(M, den, o, out, lse, (size_t)b * Hq + (size_t)g * G + h, d4);
    }
}

// The single launch's end-of-kernel merge of the (up to two) pairs this
// workgroup arrived at last. Every partial of an item (up to kEndPre per pair)
// is loaded before any is folded, for both pairs at once, so the merge costs
// one memory round trip; the folds then run in the same batches and order as
// merge_partials, so the results are bitwise those of the combine kernel.
// base_of(k, s): partial row of head 0 of the s-th partial of pair k.
constexpr int kEndPre = 8;
template <typename BaseOf>
__device__ __forceinline__ void merge_pairs_at_end(const float *part_o, const float *part_lse, int npairs,
                                                   const int (&n)[2], const int (&b)[2], const int (&g)[2],
                                                   BaseOf base_of, int G, int Hq, uint16_t *out, float *lse)
{
    constexpr int D = kHeadDim;
    for (int idx = threadIdx.x; idx < G * 32; idx += kDecodeThreads) {
        const int h = idx >> 5, d4 = (idx & 31) * 4;
        float ls[2][kEndPre];
        f32x4 xs[2][kEndPre];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
#pragma unroll
            for (int j = 0; j < kEndPre; ++j) {
                if (k < npairs && j < n[k]) {
                    const size_t sl = (size_t)base_of(k, j) + h;
                    ls[k][j] = part_lse[sl];
                    xs[k][j] = *reinterpret_cast<const f32x4 *>(part_o + sl * D + d4);
                }
            }
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            if (k >= npairs)
                continue;
            float M = -INFINITY, den = 0.f;
            f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s0 = 0; s0 < kEndPre; s0 += kMergeBatch) {
                if (s0 >= n[k])
                    break;
                float lb[kMergeBatch];
                f32x4 xb[kMergeBatch];
#pragma unroll
                for (int j = 0; j < kMergeBatch; ++j) {
                    lb[j] = ls[k][s0 + j];
                    xb[j] = xs[k][s0 + j];
                }
                merge_fold(M, den, o, lb, xb, n[k] - s0);
            }
            for (int s0 = kEndPre; s0 < n[k]; s0 += kMergeBatch) {   // pairs of more pieces
                float lb[kMergeBatch];
                f32x4 xb[kMergeBatch];
#pragma unroll
                for (int j = 0; j < kMergeBatch; ++j) {
                    const size_t sl = (size_t)base_of(k, s0 + j < n[k] ? s0 + j : s0) + h;
                    lb[j] = part_lse[sl];
                    xb[j] = *reinterpret_cast<const f32x4 *>(part_o + sl * D + d4);
                }
                merge_fold(M, den, o, lb, xb, n[k] - s0);
            }
            merge_write(M, den, o, out, lse, (size_t)b[k] * Hq + (size_t)g[k] * G + h, d4);
        }
    }
}

// LDS of a decode workgroup. With one column block, the per-wave states of a
// segment's end go to a mailbox of their own beside the staging rows, so a
// wave posts its state without waiting for the others to finish staging; with
// two column blocks (32 query rows) the mailbox would not fit beside the
// staging rows at two workgroups per CU, so it aliases them.
template <int NCB>
struct DecodeLdsRegion {   // NCB == 1
    uint8_t stg[kWaves][2][16 * kStgRow];          // per-wave K and V slice staging (during blocks)
    float acc[kWaves][kMaxGroup * NCB][kLdsRow];   // per-wave states at a segment's end
};
template <>
struct DecodeLdsRegion<2> {
    union {
        uint8_t stg[kWaves][2][16 * kStgRow];
        float acc[kWaves][kMaxGroup * 2][kLdsRow];
    };
};

template <int NCB>
struct DecodeLds {
    union {
        DecodeLdsRegion<NCB> r;
        struct {
            int32_t tp[kMaxBatch + 1];          // single launch: tiles prefix (prologue only)
            int32_t len[kMaxBatch];             // and validated lengths
        };
    };
    // per mailbox buffer (two only with one column block and G <= 8)
    float m[2][kWaves][kMaxGroup * NCB];
    float l[2][kWaves][kMaxGroup * NCB];
    float e[2][kWaves][kMaxGroup * NCB];
    int red[3 * kWaves];
    // one column block: the latest segment end reached by any wave, and per
    // buffer, counted from the block loop's start, the states posted (kWaves
    // per segment) and the segments merged; the held segments' descriptions
    int mb_first, mb_posted[2], mb_merged[2];
    int mb_desc[2][8];   // b, g, slot, direct, nseg, wfirst, first_off, m
    float mb_vsc[2];
    // single launch: the split pairs this workgroup arrived at last, merged
    // after its block loop (at most two: only a first and a last segment split)
    int npend;
    int pend[2][5];   // b, g, nseg, wfirst, first_off
    int pend_last[2];   // this workgroup brought the pair's counter to nseg
    float vs[kMaxGroup * NCB];   // SRC_SHARED: V scale of each query row
};

template <int SRC, int KVFP8>
__global__ __launch_bounds__(kDecodeThreads, 2) void decode_kernel(DecodeArgs a)
{
    constexpr bool kFused = SRC == SRC_FUSED_DYNAMIC || SRC == SRC_FUSED_STATIC;
    const int w = blockIdx.x;
    if ((SRC == SRC_DYNAMIC || is_shared(SRC)) && w >= ldc(a.header, H_WEFF))
        return;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int row = lane & 15;   // MFMA row / column within a 16x16 tile
    const int grp = lane >> 4;   // MFMA row group

    // Column blocks of 16 query rows: a shared prefix item stacks up to
    // 32 / G requests' heads in two blocks that read each K/V slice once.
    constexpr int NCB = SRC == SRC_SHARED_WIDE ? 2 : 1;
    __shared__ __attribute__((aligned(16))) DecodeLds<NCB> lds;

    const int G = a.G;
    constexpr int D = kHeadDim;
    constexpr int EB = KVFP8 ? 1 : 2;             // bytes per cached element
    constexpr int kSlots = 2;                      // slices in flight per wave
    // block tokens: a wave's slice is 16 bf16 or 32 fp8 cache rows (4 KB of K
    // and 4 KB of V either way)
    constexpr int kBT = KVFP8 ? 128 : 64;
    constexpr int kSliceT = kBT / kWaves;
    constexpr bool kEarlyRefill = NCB == 1;        // refill a slot before its block's math
    const size_t page_head_bytes = (size_t)a.P * D * EB;

    // ---- single launch: this workgroup's share of the plan ---------------
    int64_t N = 0, We = 0;
    int chunk = 0;
    if (kFused) {
        const int tid = threadIdx.x;
        const int cA = (a.B + kDecodeThreads - 1) / kDecodeThreads;
        const int b0 = min(a.B, tid * cA), b1 = min(a.B, b0 + cA);
        int sum = 0, mx = 0, bad = 0;
        const int64_t limit = (int64_t)a.pt_stride * a.P;
        for (int bb = b0; bb < b1; ++bb) {
            const int raw = a.lengths[bb];
            const int Lb = (raw < 0 || (int64_t)raw > limit) ? 0 : raw;
            bad |= Lb != raw;
            mx = max(mx, Lb);
            const int n = (Lb + a.T - 1) / a.T;
            if (SRC == SRC_FUSED_DYNAMIC) {
                lds.tp[bb + 1] = n;
                lds.len[bb] = Lb;
            }
            sum += n;
        }
        int maxle, bits, total;
        int run = block_scan_max_or<kDecodeThreads>(sum, mx, bad, lds.red, &total, &maxle, &bits);
        maxle = __builtin_amdgcn_readfirstlane(maxle);
        bits = __builtin_amdgcn_readfirstlane(bits);
        total = __builtin_amdgcn_readfirstlane(total);
        if (bits && w == 0 && tid == 0)
            atomicOr(reinterpret_cast<unsigned *>(a.header + H_STATUS), 1u);
        if (SRC == SRC_FUSED_DYNAMIC) {
            for (int bb = b0; bb < b1; ++bb) {
                run += lds.tp[bb + 1];
                lds.tp[bb + 1] = run;
            }
            if (tid == 0)
                lds.tp[0] = 0;
            N = (int64_t)total * a.Hkv;
            We = plan_wgs(N, a.W, a.W_auto);
            __syncthreads();   // the tiles prefix and the lengths are complete
            // requests without tiles: o = 0, lse = -inf (spread over the grid)
            for (int bb = w; bb < a.B; bb += gridDim.x) {
                if (lds.len[bb] != 0)
                    continue;
                for (int idx = tid; idx < a.Hq * 32; idx += kDecodeThreads) {
                    const int h = idx >> 5, d4 = (idx & 31) * 4;
                    const size_t hq = (size_t)bb * a.Hq + h;
                    *reinterpret_cast<bf16x4 *>(a.out + hq * D + d4) = bf16x4{0, 0, 0, 0};
                    if (a.lse && d4 == 0)
                        a.lse[hq] = -INFINITY;
                    VLKV_COUNT_OUT(hq, d4);
                }
            }
            if (w >= We)
                return;
        } else {
            const int64_t S = a.S;
            const int64_t gran = (int64_t)a.P / gcd64(a.P, a.T) * a.T;
            if (maxle > 0) {
                int64_t C = (maxle + S - 1) / S;
                chunk = (int)((C + gran - 1) / gran * gran);
            }
        }
    }

    Walker<SRC, kBT> wk;
    wk.init(&a, w, wave, lds.tp, lds.len, N, We, chunk);

    // per-wave softmax state, head = row. m_run is uniform over the 4 row
    // groups; l_run is this lane's partial sum, reduced at segment end.
    // l_run sums the bf16-rounded weights that multiply V (normalises o exactly
    // like P.V); e_run sums the unrounded fp32 weights (gives an accurate lse).
    // One set per column block.
    float m_run[NCB], l_run[NCB], e_run[NCB], sc[NCB], vsc_run[NCB];
    f32x4 acc[NCB][8];
    u32x4 qreg[NCB][4];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        m_run[cb] = -INFINITY;
        l_run[cb] = e_run[cb] = 0.f;
        sc[cb] = a.scale_log2;
        vsc_run[cb] = 1.f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            acc[cb][i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i)
            qreg[cb][i] = u32x4{0u, 0u, 0u, 0u};
    }

    int bad_page = 0;
    if (threadIdx.x == 0) {
        lds.npend = 0;   // these are read after the barrier before the block loop
        lds.mb_first = -1;
        lds.mb_posted[0] = lds.mb_posted[1] = lds.mb_merged[0] = lds.mb_merged[1] = 0;
    }

    // ---- loads of one block into a slot ---------------------------------
    // K/V loads are issued for every slot, also past the end of the work or
    // for an empty or invalid slice (then with an empty range: no memory
    // access), so the number of vector loads between any two points of the
    // pipeline is fixed and the wait before each compute covers its own slot only.
    // q of query rows 16 cb .. 16 cb + 15 of a segment: row r is head r % G of
    // request b + r / G (a shared prefix stacks m requests; rows past m G
    // read head 0 and are zeroed at use); fp8: the scales of each row's request
    auto load_q = [&](u32x4 (&q)[4], const Meta &mt, int cb, float &ksc, float &vsc) {
        const int rr = 16 * cb + row;
        const int hrow = rr < mt.m * G ? rr : 0;
        int qb = mt.b, qh = hrow;
        if (is_shared(SRC)) {
            const int mem = hrow / G;
            qb += mem;
            qh = hrow - mem * G;
        }
        const uint16_t *qp = a.q + ((size_t)qb * a.Hq + (size_t)mt.g * G + qh) * D;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int d0 = KVFP8 ? 16 * grp + 64 * (kk >> 1) + 8 * (kk & 1) : 32 * kk + 8 * grp;
            q[kk] = *reinterpret_cast<const u32x4 *>(qp + d0);
        }
        if (KVFP8) {
            if (is_shared(SRC)) {   // per row
                ksc = a.k_scale[(size_t)qb * a.Hkv + mt.g];
                vsc = a.v_scale[(size_t)qb * a.Hkv + mt.g];
            } else {
                ksc = ldc(a.k_scale, (size_t)mt.b * a.Hkv + mt.g);
                vsc = ldc(a.v_scale, (size_t)mt.b * a.Hkv + mt.g);
            }
        }
    };

    // Describe the slot's next block; a segment's first block also brings q
    // (query rows as the B operand: head = row). Branch-free: rows >= G read
    // head 0 and are zeroed when copied at the segment's first block, so
    // nothing here waits for the load and no divergent control flow separates
    // the scalar bookkeeping of the pipeline.
    auto next_block = [&](Slot &s, Meta &m) {
        m = wk.next();
        if (m.valid && m.first)
            load_q(s.q, m, 0, m.ksc, m.vsc);
    };
    // page ids of a block's slice (scalar loads), -1 when it has no rows. An
    // fp8 slice (32 rows) starts on a 32-token boundary; its second half is on
    // another page only when the page size is an odd multiple of 16.
    struct Pages {
        int p0, p1;   // pages of the slice's rows 0-15 and (fp8) 16-31
        int r0;       // row of the slice's first token in page p0
    };
    auto slice_pages = [&](const Meta &m) -> Pages {
        if (!m.valid || m.nv <= 0)
            return {-1, -1, 0};
        const int tok = m.tbase + m.tok0;   // token index in the request
        const int pi = tok / a.P, r0 = tok - pi * a.P;
        const size_t base = (size_t)m.b * a.pt_stride;
        const int p0 = ldc(a.page_table, base + pi);
        int p1 = p0;
        if (KVFP8 && m.nv > 16 && r0 + 16 >= a.P)
            p1 = ldc(a.page_table, base + pi + 1);
        return {p0, p1, r0};
    };
    // The slice's K and V rows are read through buffer descriptors whose base
    // is the slice's first row (wave-uniform, scalar registers) and whose
    // range is exactly its valid rows: a row past the request's length, or a
    // whole slice past the end of the work or on an invalid page (range 0),
    // reads as zeros without touching memory. Each lane adds its fixed 32-bit
    // offset (16 bytes per lane, 1 KB per load): four loads of K and four of
    // V, 16 bf16 rows or 32 fp8 rows (the second 16 through a second
    // descriptor, their page being possibly another).
    auto load_slice = [&](Slot &s, Meta &m, Pages pg) {
        constexpr int RB = D * EB;   // bytes per cache row
        size_t slab0 = 0, slab1 = 0;
        int n0 = 0, n1 = 0;
        if (m.valid && m.nv > 0) {
            const bool bad1 = KVFP8 && m.nv > 16 && (pg.p1 < 0 || pg.p1 >= a.num_pages);
            if (pg.p0 < 0 || pg.p0 >= a.num_pages || bad1) {
                bad_page = 1;   // reported once at the end of the kernel
                m.nv = 0;
            } else {
                slab0 = ((size_t)pg.p0 * a.Hkv + m.g) * page_head_bytes + (size_t)pg.r0 * RB;
                // (wave-uniform; kept in scalar registers so that the
                // descriptors are, and the loads need no per-lane loop)
                n0 = __builtin_amdgcn_readfirstlane(min(m.nv, 16) * RB);
                if (KVFP8) {
                    const int r1 = pg.r0 + 16 >= a.P ? pg.r0 + 16 - a.P : pg.r0 + 16;
                    slab1 = ((size_t)pg.p1 * a.Hkv + m.g) * page_head_bytes + (size_t)r1 * RB;
                    n1 = __builtin_amdgcn_readfirstlane(max(m.nv - 16, 0) * RB);
                }
            }
        }
        const auto rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(a.k + slab0), 0, n0, kRsrcWord3);
        const auto rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(a.v + slab0), 0, n0, kRsrcWord3);
        if (KVFP8) {
            const auto rk1 = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(a.k + slab1), 0, n1, kRsrcWord3);
            const auto rv1 = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(a.v + slab1), 0, n1, kRsrcWord3);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                s.k[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, 16 * lane + 1024 * i, 0, kLoadNT));
                s.k[2 + i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk1, 16 * lane + 1024 * i, 0, kLoadNT));
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                s.v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, 16 * lane + 1024 * i, 0, kLoadNT));
                s.v[2 + i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv1, 16 * lane + 1024 * i, 0, kLoadNT));
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                s.k[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, 16 * lane + 1024 * i, 0, kLoadNT));
#pragma unroll
            for (int i = 0; i < 4; ++i)
                s.v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, 16 * lane + 1024 * i, 0, kLoadNT));
        }
    };
    auto issue = [&](Slot &s, Meta &m) {
        next_block(s, m);
        load_slice(s, m, slice_pages(m));
    };

    // ---- end of a segment: merge the 4 waves and write ------------------
    // The mailbox: per wave, the segment's running max and sums per query row
    // and its o rows. One column block with G <= 8 (and not a shared prefix,
    // whose items stack up to 16 rows): two buffers of 8 rows in the same
    // LDS, used by alternate segments; otherwise one buffer.
    const int nbuf = NCB == 1 && !is_shared(SRC) && G <= kMaxGroup / 2 ? 2 : 1;
    const int rows_buf = kMaxGroup * NCB / nbuf;
    auto acc_row = [&](int buf, int v, int r) -> float * {
        return &lds.r.acc[0][0][0] + ((buf * kWaves + v) * rows_buf + r) * kLdsRow;
    };
    // Post this wave's state of the segment (running max, sums and o) to a buffer.
    auto post_state = [&](int rows, int buf) {
        // (the lane's LDS addresses are recomputed here from an opaque copy of
        // the thread index rather than kept in registers across the block loop)
        int t = threadIdx.x;
        asm volatile("" : "+v"(t));
        const int prow = t & 15, pgrp = (t & 63) >> 4;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const float l_tot = xsum4(l_run[cb]);
            const float e_tot = xsum4(e_run[cb]);
            const int rr = 16 * cb + prow;
            if (rr < rows) {
                if (pgrp == 0) {
                    lds.m[buf][wave][rr] = m_run[cb];
                    lds.l[buf][wave][rr] = l_tot;
                    lds.e[buf][wave][rr] = e_tot;
                    if (is_shared(SRC) && wave == 0)
                        lds.vs[rr] = vsc_run[cb];   // per row: its request's V scale
                }
                float *ar = acc_row(buf, wave, rr);
#pragma unroll
                for (int mb = 0; mb < 8; ++mb)
                    *reinterpret_cast<f32x4 *>(ar + 16 * mb + 4 * pgrp) = acc[cb][mb];
            }
        }
    };
    // Merge the four states of a buffer and write the segment's output (a
    // direct result or a partial), items t0, t0 + step, ...; thread t0 == 0
    // also records a split pair for the end of the launch.
    auto merge_out = [&](const Meta &mt, int rows, float vsc, int buf, int t0, int step) {
        asm volatile("" : "+v"(t0));   // (addresses from t0 are not hoisted into the block loop)
#pragma unroll 1
        for (int idx = t0; idx < rows * 32; idx += step) {
            const int h = idx >> 5, d4 = (idx & 31) * 4;
            // every wave's state is read before any is used (one LDS round trip)
            float mv[kWaves], lv[kWaves], ev[kWaves];
            f32x4 xv[kWaves];
#pragma unroll
            for (int v = 0; v < kWaves; ++v) {
                mv[v] = lds.m[buf][v][h];
                lv[v] = lds.l[buf][v][h];
                ev[v] = lds.e[buf][v][h];
                xv[v] = *reinterpret_cast<const f32x4 *>(acc_row(buf, v, h) + d4);
            }
            float M = -INFINITY;
#pragma unroll
            for (int v = 0; v < kWaves; ++v)
                M = fmaxf(M, mv[v]);
            f32x4 o = {0.f, 0.f, 0.f, 0.f};
            float lse2 = -INFINITY;
            if (M != -INFINITY) {
                float den = 0.f, ex = 0.f;
#pragma unroll
                for (int v = 0; v < kWaves; ++v) {
                    const float e = fast_exp2(mv[v] - M);
                    den += e * lv[v];
                    ex += e * ev[v];
                    o += e * xv[v];
                }
                const float r = (is_shared(SRC) ? lds.vs[h] : vsc) / den;
                o *= r;
                lse2 = M + log2f(ex);
            }
            const int mem = is_shared(SRC) ? h / G : 0;   // row h: head h % G of request b + h / G
            const size_t hq = (size_t)(mt.b + mem) * a.Hq + (size_t)mt.g * G + (h - mem * G);
            const size_t prow = (size_t)mt.slot * a.slot_rows + h;   // partial row
            if (mt.direct) {
                const bf16x4 ob = __builtin_convertvector(o, bf16x4);
                *reinterpret_cast<bf16x4 *>(a.out + hq * D + d4) = ob;
                if (a.lse && d4 == 0)
                    a.lse[hq] = lse2 * kLn2;
                VLKV_COUNT_OUT(hq, d4);
            } else if (kFused) {
                // (the slot's rows start at a wave-uniform address)
                store_coherent4(a.part_o + (size_t)mt.slot * a.slot_rows * D, h * D + d4, o);
                if (d4 == 0)
                    store_coherent(a.part_lse + prow, lse2);
            } else {
                *reinterpret_cast<f32x4 *>(a.part_o + prow * D + d4) = o;
                if (d4 == 0)
                    a.part_lse[prow] = lse2;
            }
        }
        if (kFused && !mt.direct && t0 == 0) {
            // The pair's arrival is deferred to the end of this workgroup's
            // blocks (no wait for the stores here, so the loads in flight keep
            // streaming). A contiguous unit range splits at most its first and
            // last pair; a third would break the plan's invariant and is
            // reported instead of merged. (Two merges may run at once, in two
            // waves: the list's slot is taken atomically.)
            const int k = __hip_atomic_fetch_add(&lds.npend, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            if (k < 2) {
                lds.pend[k][0] = mt.b;
                lds.pend[k][1] = mt.g;
                lds.pend[k][2] = mt.nseg;
                lds.pend[k][3] = mt.wfirst;
                lds.pend[k][4] = mt.first_off;
            } else {
                atomicOr(reinterpret_cast<unsigned *>(a.header + H_STATUS), kStatusInternal);
            }
        }
    };
    // One column block: a segment's end does not stop the waves. Each wave
    // posts its state to the segment's mailbox buffer and goes on with its
    // next block. The first wave to reach the next segment's end (the wave
    // with the most slack) merges the segment as soon as all four have posted
    // it, which frees its buffer; the last segment is merged by every thread
    // after the block loop. A wave waits only to post into a buffer whose
    // previous segment is not merged yet. The first wave at segment end j is
    // the one whose atomic max of j into mb_first returns less than j (the
    // waves may reach different segment ends in any interleaving; mb_first
    // only grows). Ordering: each post ends with a release increment of its
    // buffer's mb_posted (workgroup scope, LDS), which the merging wave
    // acquires before reading; the merge ends with a release of the buffer's
    // mb_merged, which a wave acquires before writing the buffer again. Waits
    // cannot last (every wave reaches each segment end after finitely many
    // blocks, and each merge waits only for posts that wait only for earlier
    // merges); they are still bounded, and a wait that ran out is reported in
    // the status word (its merge is then skipped).
    // Two column blocks: the mailbox aliases the staging rows, so all waves
    // meet at barriers: post, merge (one item per thread), and go on.
    int seg_idx = 0;   // segment ends this wave has passed (the same in every wave)
    auto wait_at_least = [&](int *ctr, int v) -> bool {
        for (int spin = 0; __hip_atomic_load(ctr, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < v; ++spin) {
            if (spin >= kMailboxSpin) {
                if (lane == 0)
                    atomicOr(reinterpret_cast<unsigned *>(a.header + H_STATUS), kStatusInternal);
                return false;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        return true;
    };
    // merge the segment held in a buffer (items t0, t0 + step, ...)
    auto merge_held = [&](int buf, int t0, int step) {
        Meta hm;
        hm.b = __builtin_amdgcn_readfirstlane(lds.mb_desc[buf][0]);
        hm.g = __builtin_amdgcn_readfirstlane(lds.mb_desc[buf][1]);
        hm.slot = __builtin_amdgcn_readfirstlane(lds.mb_desc[buf][2]);
        hm.direct = __builtin_amdgcn_readfirstlane(lds.mb_desc[buf][3]);
        hm.nseg = __builtin_amdgcn_readfirstlane(lds.mb_desc[buf][4]);
        hm.wfirst = __builtin_amdgcn_readfirstlane(lds.mb_desc[buf][5]);
        hm.first_off = __builtin_amdgcn_readfirstlane(lds.mb_desc[buf][6]);
        hm.m = __builtin_amdgcn_readfirstlane(lds.mb_desc[buf][7]);
        merge_out(hm, hm.m * G, lds.mb_vsc[buf], buf, t0, step);
    };
    auto finish = [&](const Meta &mt) {
        const int rows = mt.m * G;   // query rows of this segment
        if (NCB == 1) {
            const int j = seg_idx++;
            const int buf = j & (nbuf - 1), use = nbuf == 2 ? j >> 1 : j;   // this segment's buffer and its use
            int old = 0;
            if (lane == 0)
                old = __hip_atomic_fetch_max(&lds.mb_first, j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            old = __builtin_amdgcn_readfirstlane(old);
            if (j > 0 && old < j) {
                // first at this segment end: merge segment j - 1 once all four posted it
                const int bp = (j - 1) & (nbuf - 1), up = nbuf == 2 ? (j - 1) >> 1 : j - 1;
                if (wait_at_least(&lds.mb_posted[bp], kWaves * (up + 1)))
                    merge_held(bp, lane, 64);
                if (lane == 0)
                    __hip_atomic_store(&lds.mb_merged[bp], up + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
            }
            wait_at_least(&lds.mb_merged[buf], use);   // the buffer's previous segment is merged
            post_state(rows, buf);
            if (lane == 0) {
                lds.mb_desc[buf][0] = mt.b;
                lds.mb_desc[buf][1] = mt.g;
                lds.mb_desc[buf][2] = mt.slot;
                lds.mb_desc[buf][3] = mt.direct;
                lds.mb_desc[buf][4] = mt.nseg;
                lds.mb_desc[buf][5] = mt.wfirst;
                lds.mb_desc[buf][6] = mt.first_off;
                lds.mb_desc[buf][7] = mt.m;
                lds.mb_vsc[buf] = vsc_run[0];
                __hip_atomic_fetch_add(&lds.mb_posted[buf], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
            }
        } else {
            __syncthreads();   // every wave is done with its staging rows, which the mailbox aliases
            post_state(rows, 0);
            __syncthreads();
            merge_out(mt, rows, vsc_run[0], 0, threadIdx.x, kDecodeThreads);
            __syncthreads();
        }
    };

    // a segment whose end is still to be posted (one column block)
    Meta fin_mt;
    bool pend_fin = false;

    // ---- math of one block ----------------------------------------------
    // The slot's K/V registers are staged into LDS first; the slot is then
    // refilled with the loads of its next block, so those are in flight during
    // this block's math and every wave keeps kSlots slices in flight.
    auto compute = [&](Slot &s, Meta &mslot) {
        const Meta mcopy = mslot;   // the slot's description is replaced by the refill
        const Meta &mt = kEarlyRefill ? mcopy : mslot;
#ifdef VLKV_DEBUG_VISITS
        // lane j: the slice's row j, for each request the block serves
        if (g_visits.tok && lane < mt.nv) {
            const int64_t j = (int64_t)mt.tbase + mt.tok0 + lane;
            for (int r = 0; r < mt.m; ++r)
                if (j < g_visits.tok_stride)
                    atomicAdd(g_visits.tok + ((int64_t)(mt.b + r) * a.Hkv + mt.g) * g_visits.tok_stride + j, 1);
        }
#endif
        constexpr int NL = 4;
        // K operand registers: the slot's own once it is not refilled before the math
        u32x4 kbuf[4];
        u32x4(&kop)[4] = kEarlyRefill ? kbuf : s.k;
        // Load i of lane l brought slice bytes [1024 i + 16 l, +16): staged row
        // (1024 i + 16 l) / 256, column byte (1024 i + 16 l) % 256 (a staged row
        // is one bf16 cache row, or two fp8 cache rows, the second kFp8HalfGap
        // bytes after the first's end). Write them to this wave's staging rows,
        // then read back the operand layout (row = lane % 16, bytes 64 i + 16 *
        // (lane / 16)). LDS operations of one wave complete in order, so no
        // barrier is needed.
        constexpr int RB = 256;
        uint8_t *sk = lds.r.stg[wave][0];
        uint8_t *sv = lds.r.stg[wave][1];
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int byte = 1024 * i + 16 * lane;
            const int o = (byte / RB) * kStgRow + byte % RB + (KVFP8 && byte % RB >= RB / 2 ? kFp8HalfGap : 0);
            *reinterpret_cast<u32x4 *>(sk + o) = s.k[i];
            *reinterpret_cast<u32x4 *>(sv + o) = s.v[i];
        }
        // the second column block only when the segment's rows reach it
        // (wave-uniform: a shared item of more than 16 query rows)
        const bool two = NCB == 2 && mt.m * G > 16;
        float ksc1 = 1.f, vsc1 = 1.f;
        if (mt.first) {
            // q arrived with this slot (only a segment's first block loads it);
            // copied before the refill reuses the slot's registers
            if (NCB == 2 && two)   // loaded here, once per segment (a memory round trip)
                load_q(qreg[NCB - 1], mt, 1, ksc1, vsc1);
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const u32x4 q = cb == 0 ? s.q[kk] : qreg[cb][kk];
                    qreg[cb][kk] = (cb == 0 || two) && 16 * cb + row < mt.m * G ? q : u32x4{0u, 0u, 0u, 0u};
                }
            }
        }
        // (the two-column-block kernel refills after its math: its second
        // block's state leaves no registers for a slice in flight beside the
        // operands)
        if (kEarlyRefill)
            issue(s, mslot);
        if (mt.first) {
            // the previous segment's end, deferred to here so that both slots'
            // loads are in flight while it runs
            if (kEarlyRefill && pend_fin) {
                finish(fin_mt);
                pend_fin = false;
            }
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                m_run[cb] = -INFINITY;
                l_run[cb] = 0.f;
                e_run[cb] = 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    acc[cb][i] = f32x4{0.f, 0.f, 0.f, 0.f};
                sc[cb] = a.scale_log2 * (cb == 0 ? mt.ksc : ksc1);
                vsc_run[cb] = cb == 0 ? mt.vsc : vsc1;
            }
        }
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int o = row * kStgRow + 64 * i + 16 * grp + (KVFP8 && i >= NL / 2 ? kFp8HalfGap : 0);
            kop[i] = *reinterpret_cast<const u32x4 *>(sk + o);
        }
        {
            // Scores S^T[sub-tile row 4*grp+i][head row], per column block and
            // 16-token sub-tile: sub-tile s, row m is token m (bf16) or 2m + s
            // (fp8: a staged row holds two cache rows), so each fp8 sub-tile
            // reads its own half of the staged row pairs.
            constexpr int NST = KVFP8 ? 2 : 1;   // 16-token sub-tiles per slice
            f32x4 st[NCB][NST];
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                for (int sub = 0; sub < NST; ++sub)
                    st[cb][sub] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int sub = 0; sub < NST; ++sub) {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    bf16x8 kv;
                    if (KVFP8) {
                        const uint32_t w0 = kop[2 * sub + (kk >> 1)][2 * (kk & 1)];
                        const uint32_t w1 = kop[2 * sub + (kk >> 1)][2 * (kk & 1) + 1];
                        const bf16x2 c0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
                        const bf16x2 c1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
                        const bf16x2 c2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
                        const bf16x2 c3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
                        kv = bf16x8{c0[0], c0[1], c1[0], c1[1], c2[0], c2[1], c3[0], c3[1]};
                    } else {
                        kv = __builtin_bit_cast(bf16x8, kop[kk]);
                    }
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb)
                        if (cb == 0 || two)
                            st[cb][sub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                kv, __builtin_bit_cast(bf16x8, qreg[cb][kk]), st[cb][sub], 0, 0, 0);
                }
            }
            s16x4 pb[NCB][NST];
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                if (!(cb == 0 || two))
                    continue;
#pragma unroll
                for (int sub = 0; sub < NST; ++sub)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        st[cb][sub][i] *= sc[cb];
                if (mt.nv < kSliceT) {
#pragma unroll
                    for (int sub = 0; sub < NST; ++sub)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int t = KVFP8 ? 2 * (4 * grp + i) + sub : 4 * grp + i;
                            st[cb][sub][i] = t >= mt.nv ? -INFINITY : st[cb][sub][i];
                        }
                }
                float mx = -INFINITY;
#pragma unroll
                for (int sub = 0; sub < NST; ++sub)
                    mx = fmaxf(mx, fmaxf(fmaxf(st[cb][sub][0], st[cb][sub][1]), fmaxf(st[cb][sub][2], st[cb][sub][3])));
                mx = xmax4(mx);
                // Lazy rescaling: the reference maximum m_run only moves (and the
                // running sums are rescaled) when a head's scores exceed it by more
                // than kLazy (log2 units). Weights 2^(s - m_run) then stay <= 2^kLazy,
                // exact in fp32 and bf16 alike, and every later step uses the same
                // reference, so the result is unchanged while most slices skip the
                // 34 multiplies of a rescale.
                if (__builtin_amdgcn_ballot_w64(mx > m_run[cb] + kLazy) != 0) {
                    const float m_new = fmaxf(m_run[cb], mx);
                    const float alpha = fast_exp2(m_run[cb] - m_new);
                    l_run[cb] *= alpha;
                    e_run[cb] *= alpha;
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        acc[cb][i] *= alpha;
                    m_run[cb] = m_new;
                }
                const float m_use = m_run[cb] == -INFINITY ? 0.f : m_run[cb];
#pragma unroll
                for (int sub = 0; sub < NST; ++sub) {
                    f32x4 p;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        p[i] = fast_exp2(st[cb][sub][i] - m_use);
                    pb[cb][sub] = pack_bf16x4(p);
                    const f32x4 pr = unpack_bf16x4(pb[cb][sub]);
                    l_run[cb] += (pr[0] + pr[1]) + (pr[2] + pr[3]);
                    e_run[cb] += (p[0] + p[1]) + (p[2] + p[3]);
                }
            }
            // rows past the length were read as zeros (the loads' range ends at
            // the last valid row), so they add nothing to P.V.
            // V^T, the A operand of P.V, is read from the staged V rows by
            // LDS transpose loads: in each 16-lane row group, lane 8h + c (tr_b8)
            // or 4h + c (tr_b16) receives element c of the 8-byte chunks that
            // lanes 2j + h (j = 0..7) or 4j + h (j = 0..3) address. Lane (16 g +
            // i) addresses the chunk of V[token of its group's reduction index
            // j][dims 16 mb + 8h .. or 4h ..], so that lane (16 g + d) receives
            // V[token(g, j)][16 mb + d], j = 0.. in the reduction order of P^T:
            // bf16, token 4g + j; fp8, the token of sub-tile j / 4, row
            // 4g + j % 4 (token 2 (4g + j % 4) + j / 4 of the staged row pairs).
            {
                const int gi = lane & 15;
                int vrow;
                if (KVFP8) {
                    const int j = gi >> 1, h = gi & 1;
                    vrow = (4 * grp + (j & 3)) * kStgRow + (j >> 2) * (128 + kFp8HalfGap) + 8 * h;
                } else {
                    const int j = gi >> 2, h = gi & 3;
                    vrow = (4 * grp + j) * kStgRow + 8 * h;
                }
#pragma unroll
                for (int mb = 0; mb < 8; ++mb) {
                    if (KVFP8) {
                        const i32x2 raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                            (__attribute__((address_space(3))) i32x2 *)(sv + vrow + 16 * mb));
                        const bf16x2 c0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[0], 1.0f, false);
                        const bf16x2 c1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[0], 1.0f, true);
                        const bf16x2 c2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[1], 1.0f, false);
                        const bf16x2 c3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[1], 1.0f, true);
                        const bf16x8 va = bf16x8{c0[0], c0[1], c1[0], c1[1], c2[0], c2[1], c3[0], c3[1]};
#pragma unroll
                        for (int cb = 0; cb < NCB; ++cb)
                            if (cb == 0 || two)
                                acc[cb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    va, cat_bf16x8(pb[cb][0], pb[cb][NST - 1]), acc[cb][mb], 0, 0, 0);
                    } else {
                        const s16x4 vt = __builtin_bit_cast(s16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) i16x4 *)(sv + vrow + 32 * mb)));
#pragma unroll
                        for (int cb = 0; cb < NCB; ++cb)
                            if (cb == 0 || two)
                                acc[cb][mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, pb[cb][0], acc[cb][mb], 0, 0,
                                                                                          0);
                    }
                }
            }
        }
        if (mt.last) {
            if (kEarlyRefill) {   // ended at the next segment's first block, or after the loop
                fin_mt = mt;
                pend_fin = true;
            } else {
                finish(mt);
            }
        }
        if (!kEarlyRefill)
            issue(s, mslot);
    };

    // ---- software pipeline: kSlots slices in flight per wave --------------
    // A counted loop (the block count is known from the plan) with every slot
    // handled in each iteration; trailing invalid blocks do nothing. (Three or
    // four slots measured slower on gfx950 for both cache types: more registers,
    // no more useful bytes in flight.)
    Slot sl[kSlots];
    Meta mt[kSlots];
    {
        // the first blocks' page ids are fetched together (one round trip)
        Pages pg[kSlots];
#pragma unroll
        for (int i = 0; i < kSlots; ++i)
            next_block(sl[i], mt[i]);
#pragma unroll
        for (int i = 0; i < kSlots; ++i)
            pg[i] = slice_pages(mt[i]);
#pragma unroll
        for (int i = 0; i < kSlots; ++i)
            load_slice(sl[i], mt[i], pg[i]);
    }
    // the block count is walked while the first slices are in flight: the
    // blocks still ahead of the walker plus those already issued
    int nblk = wk.count_blocks();
#pragma unroll
    for (int i = 0; i < kSlots; ++i)
        nblk += mt[i].valid;
    nblk = __builtin_amdgcn_readfirstlane(nblk);   // wave-uniform: a scalar loop bound
    if (SRC == SRC_FUSED_DYNAMIC)
        wk.ltp = wk.llen = nullptr;   // from here on the walker reads lengths from memory
    // every wave is done with the LDS prefix (which the staging rows alias) and
    // sees the cleared counters
    __syncthreads();
    for (int it = 0; it < nblk; it += kSlots) {
        set_progress_priority(it, nblk);
#pragma unroll
        for (int i = 0; i < kSlots; ++i)
            compute(sl[i], mt[i]);
    }
    if (kEarlyRefill && pend_fin)
        finish(fin_mt);
    if (NCB == 1) {
        __syncthreads();   // every wave has posted its last segment
        if (seg_idx > 0)
            merge_held((seg_idx - 1) & (nbuf - 1), threadIdx.x, kDecodeThreads);
    }

    // single launch: arrive at the split pairs and merge those this workgroup
    // completes. Ordering across workgroups:
    //  * every partial was stored with agent-scope (device-coherent) stores,
    //    which write through this XCD's L2; each wave waits for its stores to
    //    complete (s_waitcnt 0, the stores' acknowledgement from the device's
    //    coherence point) before the barrier, and only then does thread 0 add
    //    this workgroup's arrival (an agent-scope atomic, performed at that
    //    same coherence point);
    //  * the workgroup whose addition brings a pair's counter to its number of
    //    pieces has seen every other piece's arrival, hence the completion of
    //    their stores; it then runs an agent-scope acquire fence (invalidating
    //    this XCD's caches) before its merge reads the partials, so those reads
    //    cannot return data cached before the stores.
    // A release ordering on the arrival would write back this XCD's whole L2
    // at every workgroup's end (measured 7-12% slower); the device-coherent
    // stores plus the completion wait give the same order for the partials,
    // the only data the counter publishes. The merging workgroup leaves the
    // counter at 0 for the next step.
    if (kFused) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (threadIdx.x == 0) {
            const int np = lds.npend;
            int old[2] = {0, 0};
#pragma unroll
            for (int k = 0; k < 2; ++k)
                if (k < np)
                    old[k] = __hip_atomic_fetch_add(a.counters + lds.pend[k][0] * a.Hkv + lds.pend[k][1], 1,
                                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            int any = 0;
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                if (k < np) {
                    const int last = old[k] == lds.pend[k][2] - 1;
                    if (last)
                        __hip_atomic_store(a.counters + lds.pend[k][0] * a.Hkv + lds.pend[k][1], 0,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    lds.pend_last[k] = last;
                    any |= last;
                }
            }
            if (any)
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        }
        __syncthreads();
        // the pairs to merge here: those whose counter this workgroup completed
        const int np = __builtin_amdgcn_readfirstlane(lds.npend);
        const int l0 = np > 0 && __builtin_amdgcn_readfirstlane(lds.pend_last[0]);
        const int l1 = np > 1 && __builtin_amdgcn_readfirstlane(lds.pend_last[1]);
        const int nm = l0 + l1;
        // merge slot 0 is the first pending pair this workgroup completed, slot 1 the second
        const int e0 = l0 ? 0 : 1;
        int mn[2], mb[2], mg[2], mw[2], mo[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int e = k == 0 ? e0 : 1;
            mb[k] = __builtin_amdgcn_readfirstlane(lds.pend[e][0]);
            mg[k] = __builtin_amdgcn_readfirstlane(lds.pend[e][1]);
            mn[k] = __builtin_amdgcn_readfirstlane(lds.pend[e][2]);
            mw[k] = __builtin_amdgcn_readfirstlane(lds.pend[e][3]);
            mo[k] = __builtin_amdgcn_readfirstlane(lds.pend[e][4]);
        }
        if (nm > 0) {
            const int sr = a.slot_rows;
            if (SRC == SRC_FUSED_DYNAMIC) {
                merge_pairs_at_end(a.part_o, a.part_lse, nm, mn, mb, mg,
                                   [&](int k, int s) { return (2 * (mw[k] + s) + (s == 0 ? mo[k] : 0)) * sr; }, G,
                                   a.Hq, a.out, a.lse);
            } else {
                merge_pairs_at_end(a.part_o, a.part_lse, nm, mn, mb, mg,
                                   [&](int k, int s) { return ((mb[k] * a.Hkv + mg[k]) * a.S + s) * sr; }, G, a.Hq,
                                   a.out, a.lse);
            }
        }
    }

    if (bad_page && lane == 0)
        atomicOr(reinterpret_cast<unsigned *>(a.header + H_STATUS), 2u);
}

// One workgroup per (request, kv head): merge its partial slots, or write the
// empty result; pairs written directly by the decode are left alone.
__global__ __launch_bounds__(kDecodeThreads) void combine_kernel(CombineArgs a)
{
    const int bg = blockIdx.x;
    const int b = bg / a.Hkv, g = bg - b * a.Hkv;
    int s0, n;
    if (a.mode == 0) {
        s0 = a.seg_prefix[bg];
        n = a.seg_prefix[bg + 1] - s0;
    } else {
        s0 = bg * a.S;
        n = a.S;
    }
    if (n == 1)
        return;
    const int sr = a.slot_rows;
    merge_partials(a.part_o, a.part_lse, n, [=](int s) { return (s0 + s) * sr; }, a.G, a.Hq, b, g, a.out,
                          a.lse);
}

// Mode 2: one workgroup per (request, kv head). The request's partials are
// those of its group's shared item (rows member*G..) followed by those of its
// own item; a solo item with one segment was written directly by the decode.
__global__ __launch_bounds__(kDecodeThreads) void combine_shared_kernel(CombineArgs a)
{
    const int bg = blockIdx.x;
    const int b = bg / a.Hkv, g = bg - b * a.Hkv;
    const int io = a.req_own[b], is = a.req_shared[b];
    const int o0 = a.seg_prefix[io * a.Hkv + g], no = a.seg_prefix[io * a.Hkv + g + 1] - o0;
    if (a.item_solo[io] && no == 1)
        return;
    int s0 = 0, ns = 0;
    if (is >= 0) {
        s0 = a.seg_prefix[is * a.Hkv + g];
        ns = a.seg_prefix[is * a.Hkv + g + 1] - s0;
    }
    const int sr = a.slot_rows, off = a.req_member[b] * a.G;
    merge_partials(a.part_o, a.part_lse, ns + no,
                          [=](int s) { return s < ns ? (s0 + s) * sr + off : (o0 + s - ns) * sr; }, a.G, a.Hq, b,
                          g, a.out, a.lse);
}

// Clears the status word and the arrival counters of a workspace.
__global__ __launch_bounds__(256) void ws_init_kernel(int32_t *header, int32_t *counters, int n)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < kHeaderInts)
        header[i] = 0;
    if (i < n)
        counters[i] = 0;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, int src, int kv_fp8, int grid, hipStream_t st)
{
    if (grid <= 0)
        return hipSuccess;
#define VLKV_LAUNCH(S, F) hipLaunchKernelGGL((decode_kernel<S, F>), dim3(grid), dim3(kDecodeThreads), 0, st, a)
    switch (src * 2 + (kv_fp8 ? 1 : 0)) {
    case 0: VLKV_LAUNCH(SRC_DYNAMIC, 0); break;
    case 1: VLKV_LAUNCH(SRC_DYNAMIC, 1); break;
    case 2: VLKV_LAUNCH(SRC_STATIC, 0); break;
    case 3: VLKV_LAUNCH(SRC_STATIC, 1); break;
    case 4: VLKV_LAUNCH(SRC_FUSED_DYNAMIC, 0); break;
    case 5: VLKV_LAUNCH(SRC_FUSED_DYNAMIC, 1); break;
    case 6: VLKV_LAUNCH(SRC_FUSED_STATIC, 0); break;
    case 7: VLKV_LAUNCH(SRC_FUSED_STATIC, 1); break;
    case 8: VLKV_LAUNCH(SRC_SHARED, 0); break;
    case 9: VLKV_LAUNCH(SRC_SHARED, 1); break;
    case 10: VLKV_LAUNCH(SRC_SHARED_WIDE, 0); break;
    case 11: VLKV_LAUNCH(SRC_SHARED_WIDE, 1); break;
    default: return hipErrorInvalidValue;
    }
#undef VLKV_LAUNCH
    return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs &a, hipStream_t st)
{
    const int grid = a.B * a.Hkv;
    if (grid <= 0)
        return hipSuccess;
    if (a.mode == MODE_SHARED)
        hipLaunchKernelGGL(combine_shared_kernel, dim3(grid), dim3(kDecodeThreads), 0, st, a);
    else
        hipLaunchKernelGGL(combine_kernel, dim3(grid), dim3(kDecodeThreads), 0, st, a);
    return hipGetLastError();
}

#ifdef VLKV_DEBUG_VISITS
hipError_t set_debug_visits(int32_t *tok, int64_t tok_stride, int32_t *out)
{
    const DebugVisits v{tok, out, tok_stride};
    return hipMemcpyToSymbol(HIP_SYMBOL(g_visits), &v, sizeof(v));
}
#endif

hipError_t launch_ws_init(int32_t *header, int32_t *counters, int n_counters, hipStream_t st)
{
    const int n = n_counters > kHeaderInts ? n_counters : kHeaderInts;
    hipLaunchKernelGGL(ws_init_kernel, dim3((n + 255) / 256), dim3(256), 0, st, header, counters, n_counters);
    return hipGetLastError();
}

}  // namespace vlkv

// Router GEMM with split bf16 weights (declared in include/vlkv_router.h).
//
// The source article's Router GEMM keeps fp32-level precision for the matmul
// that scores MoE experts by splitting each fp32 weight into a bf16 high part
// and a bf16 residual scaled by 1/256, and running two bf16 tensor-core
// products in one kernel whose accumulators stay in registers until a single
// write [Tencent HPC lands in SGLang, challenging default inference kernels,
// sec. "Dynamic Attention and Fused MoE target different bottlenecks"].
//
// Here the residual is stored as w_lo = bf16(256 (w - w_hi)) and the kernel
// computes y = X w_hi^T + 2^-8 X w_lo^T with v_mfma_f32_16x16x32_bf16:
//   - a workgroup (8 wave64s) owns a 128-token x 64-expert tile of y and a
//     range of K; each wave owns 64 tokens x 32 experts (4 x 2 blocks of
//     16 x 16) and one 32-wide half of every 64-wide k step, with separate
//     accumulators for the two products (16 MFMAs per step from 8 LDS
//     reads); the two k halves are added in a fixed order at the end;
//   - each k step's token and weight tiles are staged through LDS (four
//     16-byte global loads per thread, double-buffered in LDS, the loads
//     issued two steps ahead into registers, and the next step's operands
//     read from LDS while the current step's MFMAs run, the memory
//     instructions interleaved with the MFMAs); rows are padded to 144 bytes
//     so that the 16-byte operand reads do not conflict;
//   - lane (r = lane % 16, g = lane / 16) reads the 16 bytes of k = 8g..8g+7
//     of row r of its block, the operand layout of both A (tokens x k) and
//     B (k x experts, i.e. a row of w);
//   - bf16 x bf16 products are exact in fp32, so only the accumulation and
//     the final acc_hi + 2^-8 acc_lo round;
//   - few-token shapes split K over workgroups (the weights then stream from
//     many CUs); the fp32 partials are summed in split order by a second
//     kernel, so the result does not depend on timing.
#include "../../include/vlkv_attn.h"
#include "../../include/vlkv_router.h"
#include "vlkv_internal.hpp"

namespace vlkv {
namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));

constexpr int kRT = 512;          // threads per workgroup: 2 k groups x 2 x 2 waves
constexpr int kTM = 128;          // tokens per tile (64 per wave)
constexpr int kTE = 64;           // experts per tile (32 per wave)
constexpr int kKS = 64;           // k per step (two 16x16x32 MFMAs deep)
constexpr int kMinSteps = 2;      // k steps per split at least
constexpr int kXcds = 8;          // XCDs of the part; workgroups go to them round-robin
constexpr int kRow = kKS + 8;     // LDS row: 64 bf16 + 16 bytes of padding (144 B) against bank conflicts

struct RouterArgs {
    const uint16_t *x, *whi, *wlo;
    float *y, *part;
    int M, K, E, S, kchunk;
    int mt, et;   // token tiles, expert tiles
    int upx;      // units per XCD
};

union RouterLds {
    struct {
        uint16_t a[2][kTM][kRow];    // tokens x k, double-buffered
        uint16_t h[2][kTE][kRow];    // experts x k (high parts)
        uint16_t l[2][kTE][kRow];    // experts x k (scaled residuals)
    };
    f32x4 half[4][64][8];            // the second k group's sums, per wave of it: [wave][lane][block]
};

__global__ __launch_bounds__(256) void split_kernel(const float *w, uint16_t *hi, uint16_t *lo, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n)
        return;
    const float x = w[i];
    const __bf16 h = (__bf16)x;                      // nearest even (v_cvt_pk_bf16_f32)
    const float r = (x - (float)h) * 256.f;          // exact for finite x below bf16 overflow
    const __bf16 l = (__bf16)r;
    hi[i] = __builtin_bit_cast(uint16_t, h);
    lo[i] = __builtin_bit_cast(uint16_t, l);
}

typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));

// One k step's share of the global -> LDS copy for one thread: 16-byte chunk
// c = t % 8 of token rows t / 8 and t / 8 + 64 and of expert row t / 8 of
// both weight tiles.
struct Stage {
    u32x4 a[2], h, l;
};

__global__ __launch_bounds__(kRT) void router_gemm_kernel(RouterArgs a)
{
    __shared__ __attribute__((aligned(16))) RouterLds lds;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, g = lane >> 4;
    // this wave: k half kg of every step, tokens 64 wm.., experts 32 we..
    const int kg = wave >> 2, wm = (wave >> 1) & 1, we = wave & 1;
    // Workgroup i runs on XCD i % 8. Units (token tile, k range) are numbered
    // token tile first and dealt to the XCDs in contiguous runs of a.upx, and
    // consecutive workgroups of one XCD take the E tiles of one unit in turn:
    // a unit's token rows, and the weight rows of a k range that several
    // token tiles share, are then fetched into one XCD's L2 once.
    const int xcd = blockIdx.x % kXcds, q = blockIdx.x / kXcds;
    const int unit = xcd * a.upx + q / a.et;
    if (q / a.et >= a.upx || unit >= a.mt * a.S)
        return;
    const int mt0 = (unit % a.mt) * kTM, et0 = (q % a.et) * kTE;
    const int s = unit / a.mt;
    const int k0 = s * a.kchunk, k1 = min(a.K, k0 + a.kchunk);
    const int nsteps = k1 > k0 ? (k1 - k0) / kKS : 0;

    // Rows past M or E read the last valid row (their results are not
    // stored). Loads are unconditional (a step index past the end is clamped
    // to the last step), so that they stay in flight across the math instead
    // of waiting at a branch join.
    const int cr = tid >> 3, cc = (tid & 7) * 8;
    const uint16_t *ga0 = a.x + (size_t)min(mt0 + cr, a.M - 1) * a.K + cc;
    const uint16_t *ga1 = a.x + (size_t)min(mt0 + cr + 64, a.M - 1) * a.K + cc;
    const size_t wrow = (size_t)min(et0 + cr, a.E - 1) * a.K + cc;
    const uint16_t *gh = a.whi + wrow, *gl = a.wlo + wrow;
    auto fetch = [&](Stage &st, int t) {
        const int k = k0 + min(t, nsteps - 1) * kKS;
        st.a[0] = *reinterpret_cast<const u32x4 *>(ga0 + k);
        st.a[1] = *reinterpret_cast<const u32x4 *>(ga1 + k);
        st.h = *reinterpret_cast<const u32x4 *>(gh + k);
        st.l = *reinterpret_cast<const u32x4 *>(gl + k);
    };
    auto stash = [&](const Stage &st, int b) {
        *reinterpret_cast<u32x4 *>(&lds.a[b][cr][cc]) = st.a[0];
        *reinterpret_cast<u32x4 *>(&lds.a[b][cr + 64][cc]) = st.a[1];
        *reinterpret_cast<u32x4 *>(&lds.h[b][cr][cc]) = st.h;
        *reinterpret_cast<u32x4 *>(&lds.l[b][cr][cc]) = st.l;
    };

    f32x4 ch[4][2], cl[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            ch[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
            cl[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

    // operands: lane (r, g) reads k = 32 kg + 8g .. + 7 of row r of each block
    struct Ops {
        bf16x8 A[4], H[2], L[2];
    };
    const int kc = 32 * kg + 8 * g;
    auto read_ops = [&](Ops &o, int b) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            o.A[i] = *reinterpret_cast<const bf16x8 *>(&lds.a[b][64 * wm + 16 * i + r][kc]);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            o.H[j] = *reinterpret_cast<const bf16x8 *>(&lds.h[b][32 * we + 16 * j + r][kc]);
            o.L[j] = *reinterpret_cast<const bf16x8 *>(&lds.l[b][32 * we + 16 * j + r][kc]);
        }
    };
    auto math = [&](const Ops &o) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                ch[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.A[i], o.H[j], ch[i][j], 0, 0, 0);
                cl[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.A[i], o.L[j], cl[i][j], 0, 0, 0);
            }
    };

    // The order asked of the scheduler inside a step: the step's 16 MFMAs
    // with its memory instructions spread between them (the next step's 8
    // LDS operand reads, then the 4 LDS stores and the 4 global loads), so
    // that the matrix cores, LDS and the memory pipeline work at the same
    // time instead of in turn (measured 13% faster than issuing them in
    // groups at 8192 x 7168 x 256).
    auto interleave = [] {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);   // LDS write
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // global load
        }
    };

    // Pipeline, at the start of step t: step t's operands are in registers,
    // step t + 1's tiles in LDS buffer (t + 1) % 2, steps t + 2 and t + 3 in
    // flight from global memory. Step t reads step t + 1's operands while its
    // MFMAs run, then stores step t + 2 into buffer t % 2 (read into
    // registers during step t - 1, before the last barrier) and issues the
    // loads of step t + 4.
    if (nsteps > 0) {
        Stage s0, s1;
        Ops o0, o1;
        fetch(s0, 0);
        fetch(s1, 1);
        stash(s0, 0);
        fetch(s0, 2);
        __syncthreads();
        read_ops(o0, 0);
        stash(s1, 1);
        fetch(s1, 3);
        __syncthreads();
        int t = 0;
        for (; t + 1 < nsteps; t += 2) {
            read_ops(o1, 1);   // step t + 1
            math(o0);          // step t
            stash(s0, 0);      // step t + 2
            fetch(s0, t + 4);
            interleave();
            __syncthreads();
            read_ops(o0, 0);   // step t + 2 (unused past the end)
            math(o1);          // step t + 1
            stash(s1, 1);      // step t + 3
            fetch(s1, t + 5);
            interleave();
            __syncthreads();
        }
        if (t < nsteps)
            math(o0);          // odd step count: the last step
        __syncthreads();       // LDS is reused below
    }

    // Each k group combines its two products (the 2^-8 scale is exact); the
    // second group hands its sums to the first through LDS, which adds them
    // in that fixed order. Lane (r, g) holds rows 4g..4g+3 of column r of
    // each 16x16 block.
    f32x4 v[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            v[i][j] = ch[i][j] + cl[i][j] * 0.00390625f;
    if (kg == 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                lds.half[wave - 4][lane][2 * i + j] = v[i][j];
    }
    __syncthreads();
    if (kg == 1)
        return;
    float *dst = a.S == 1 ? a.y : a.part + (size_t)s * a.M * a.E;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int e = et0 + 32 * we + 16 * j + r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f32x4 o = v[i][j] + lds.half[wave][lane][2 * i + j];
            if (e >= a.E)
                continue;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int m = mt0 + 64 * wm + 16 * i + 4 * g + u;
                if (m < a.M)
                    dst[(size_t)m * a.E + e] = o[u];
            }
        }
    }
}

// y = sum over the S splits of the partials, in a fixed order: a workgroup
// owns 256 consecutive outputs (a float4 per lane); wave w sums splits
// w, w + 4, w + 8, ... in increasing order, then wave 0 adds the four wave
// sums in wave order. Loads of one wave are independent, so they are all in
// flight together.
constexpr int kRedWaves = 4;

__global__ __launch_bounds__(256) void router_reduce_kernel(const float *part, float *y, int64_t n, int S)
{
    __shared__ f32x4 sums[kRedWaves - 1][64];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t i = ((int64_t)blockIdx.x * 64 + lane) * 4;   // n is a multiple of 16
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (i < n) {
        int s = w;
        if (s < S)
            acc = *reinterpret_cast<const f32x4 *>(part + (size_t)s * n + i);
#pragma unroll 8
        for (s += kRedWaves; s < S; s += kRedWaves)
            acc += *reinterpret_cast<const f32x4 *>(part + (size_t)s * n + i);
    }
    if (w > 0)
        sums[w - 1][lane] = acc;
    __syncthreads();
    if (w == 0 && i < n) {
#pragma unroll
        for (int v = 0; v < kRedWaves - 1; ++v)
            acc += sums[v][lane];
        *reinterpret_cast<f32x4 *>(y + i) = acc;
    }
}

// Splits of K for a shape: about one workgroup per CU of a 256-CU part, at
// least kMinSteps k steps per split.
int router_splits(int M, int K, int E)
{
    const int64_t tiles = (int64_t)((M + kTM - 1) / kTM) * ((E + kTE - 1) / kTE);
    const int64_t steps = K / kKS;
    const int64_t max_s = steps / kMinSteps > 1 ? steps / kMinSteps : 1;
    const int64_t want = (256 + tiles - 1) / tiles;
    return (int)(want < max_s ? want : max_s);
}

int router_check(int M, int K, int E)
{
    if (M < 1 || K < kKS || K % kKS || E < 16 || E % 16)
        return fail(ATTN_ERR_INVALID_ARG, "router shape M=%d K=%d E=%d: need M >= 1, K a positive multiple of %d, "
                    "E a positive multiple of 16", M, K, E, kKS);
    if (M > (1 << 24) || K > (1 << 20) || E > (1 << 16))
        return fail(ATTN_ERR_INVALID_ARG, "router shape too large (M <= 2^24, K <= 2^20, E <= 2^16)");
    return ATTN_OK;
}

}  // namespace
}  // namespace vlkv

using namespace vlkv;

extern "C" {

int router_split_weights(const float *w, void *w_hi, void *w_lo, int64_t n, void *stream)
{
    if (n < 0)
        return fail(ATTN_ERR_INVALID_ARG, "n %lld < 0", (long long)n);
    if (n == 0)
        return ok();
    if (!w || !w_hi || !w_lo)
        return fail(ATTN_ERR_INVALID_ARG, "w, w_hi and w_lo must be non-NULL");
    if ((reinterpret_cast<uintptr_t>(w) % 4) || (reinterpret_cast<uintptr_t>(w_hi) % 2) ||
        (reinterpret_cast<uintptr_t>(w_lo) % 2))
        return fail(ATTN_ERR_INVALID_ARG, "w must be 4-byte and w_hi, w_lo 2-byte aligned");
    const int64_t blocks = (n + 255) / 256;
    if (blocks > INT32_MAX)
        return fail(ATTN_ERR_INVALID_ARG, "n too large");
    hipLaunchKernelGGL(split_kernel, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream), w,
                       static_cast<uint16_t *>(w_hi), static_cast<uint16_t *>(w_lo), n);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(ATTN_ERR_HIP, "split launch: %s", hipGetErrorString(e));
    return ok();
}

size_t router_workspace_bytes(int32_t M, int32_t K, int32_t E)
{
    if (router_check(M, K, E) != ATTN_OK)
        return 0;
    const int S = router_splits(M, K, E);
    return S == 1 ? 0 : sizeof(float) * (size_t)S * M * E;
}

int router_gemm(int32_t M, int32_t K, int32_t E, const void *x, const void *w_hi, const void *w_lo, float *y,
                void *workspace, size_t workspace_bytes, void *stream)
{
    int rc = router_check(M, K, E);
    if (rc != ATTN_OK)
        return rc;
    if (!x || !w_hi || !w_lo || !y)
        return fail(ATTN_ERR_INVALID_ARG, "x, w_hi, w_lo and y must be non-NULL");
    if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(w_hi) | reinterpret_cast<uintptr_t>(w_lo)) %
        16)
        return fail(ATTN_ERR_INVALID_ARG, "x, w_hi and w_lo must be 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(y) % 16)
        return fail(ATTN_ERR_INVALID_ARG, "y must be 16-byte aligned");
    const int S = router_splits(M, K, E);
    const size_t need = S == 1 ? 0 : sizeof(float) * (size_t)S * M * E;
    if (need && (!workspace || workspace_bytes < need || reinterpret_cast<uintptr_t>(workspace) % 256))
        return fail(ATTN_ERR_INVALID_ARG, "workspace of %zu bytes (256-byte aligned) needed, got %zu", need,
                    workspace ? workspace_bytes : (size_t)0);
    RouterArgs a;
    a.x = static_cast<const uint16_t *>(x);
    a.whi = static_cast<const uint16_t *>(w_hi);
    a.wlo = static_cast<const uint16_t *>(w_lo);
    a.y = y;
    a.part = static_cast<float *>(workspace);
    a.M = M;
    a.K = K;
    a.E = E;
    a.S = S;
    a.kchunk = ((K / kKS + S - 1) / S) * kKS;
    hipStream_t st = static_cast<hipStream_t>(stream);
    a.mt = (M + kTM - 1) / kTM;
    a.et = (E + kTE - 1) / kTE;
    const int64_t units = (int64_t)a.mt * S;
    a.upx = (int)((units + kXcds - 1) / kXcds);
    const dim3 grid((unsigned)((int64_t)a.upx * kXcds * a.et));
    hipLaunchKernelGGL(router_gemm_kernel, grid, dim3(kRT), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && S > 1) {
        const int64_t n = (int64_t)M * E;
        hipLaunchKernelGGL(router_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a.part, y, n,
                           S);
        e = hipGetLastError();
    }
    if (e != hipSuccess)
        return fail(ATTN_ERR_HIP, "router launch: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"

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
//   - a workgroup (4 wave64s) owns a 128-token x 64-expert tile of y and a
//     range of K; wave v owns tokens 32v..32v+31 of it (2 row blocks) against
//     all 4 expert blocks, with separate accumulators for the two products
//     (16 MFMAs per 32-wide k step);
//   - operands go from global memory straight into MFMA registers: lane
//     (r = lane % 16, g = lane / 16) loads the 16 bytes of k = 8g..8g+7 of row
//     r of its block, which is the operand layout of both A (tokens x k) and
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

constexpr int kRT = 256;          // threads per workgroup
constexpr int kTM = 128;          // tokens per tile (32 per wave)
constexpr int kTE = 64;           // experts per tile
constexpr int kKS = 32;           // k per MFMA step
constexpr int kMinSteps = 8;      // k steps per split at least

struct RouterArgs {
    const uint16_t *x, *whi, *wlo;
    float *y, *part;
    int M, K, E, S, kchunk;
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

__global__ __launch_bounds__(kRT) void router_gemm_kernel(RouterArgs a)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, g = lane >> 4;
    const int m0 = blockIdx.x * kTM + 32 * wave;     // this wave's first token
    const int e0 = blockIdx.y * kTE;
    const int s = blockIdx.z;
    const int nb = min(4, (a.E - e0) >> 4);          // expert blocks in this tile (E % 16 == 0)
    const int k0 = s * a.kchunk, k1 = min(a.K, k0 + a.kchunk);

    // operand rows: tokens past M read row M-1 (their results are not stored),
    // expert blocks past E read the tile's first block (not computed)
    const uint16_t *xa[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
        xa[i] = a.x + (size_t)min(m0 + 16 * i + r, a.M - 1) * a.K + 8 * g;
    const uint16_t *bh[4], *bl[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const size_t row = (size_t)(e0 + 16 * (j < nb ? j : 0) + r) * a.K + 8 * g;
        bh[j] = a.whi + row;
        bl[j] = a.wlo + row;
    }

    f32x4 ch[2][4], cl[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            ch[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
            cl[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

#pragma unroll 2
    for (int k = k0; k < k1; k += kKS) {
        bf16x8 A[2], H[4], L[4];
#pragma unroll
        for (int i = 0; i < 2; ++i)
            A[i] = *reinterpret_cast<const bf16x8 *>(xa[i] + k);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            H[j] = *reinterpret_cast<const bf16x8 *>(bh[j] + k);
            L[j] = *reinterpret_cast<const bf16x8 *>(bl[j] + k);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j < nb) {
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    ch[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[i], H[j], ch[i][j], 0, 0, 0);
                    cl[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[i], L[j], cl[i][j], 0, 0, 0);
                }
            }
        }
    }

    // lane (r, g) holds rows 4g..4g+3 of column r of each 16x16 block
    float *dst = a.S == 1 ? a.y : a.part + (size_t)s * a.M * a.E;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j >= nb)
                continue;
            const int e = e0 + 16 * j + r;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int m = m0 + 16 * i + 4 * g + t;
                if (m < a.M)
                    dst[(size_t)m * a.E + e] = ch[i][j][t] + cl[i][j][t] * 0.00390625f;   // 2^-8, exact
            }
        }
    }
}

// y = sum over the S splits of the partials, in split order.
__global__ __launch_bounds__(256) void router_reduce_kernel(const float *part, float *y, int64_t n, int S)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n)
        return;
    float acc = part[i];
    for (int s = 1; s < S; ++s)
        acc += part[(size_t)s * n + i];
    y[i] = acc;
}

// Splits of K for a shape: about one workgroup per CU of a 256-CU part, at
// least kMinSteps k steps per split.
int router_splits(int M, int K, int E)
{
    const int64_t tiles = (int64_t)((M + kTM - 1) / kTM) * ((E + kTE - 1) / kTE);
    const int64_t max_s = K / kKS / kMinSteps > 1 ? K / kKS / kMinSteps : 1;
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
    if (reinterpret_cast<uintptr_t>(y) % 4)
        return fail(ATTN_ERR_INVALID_ARG, "y must be 4-byte aligned");
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
    const dim3 grid((M + kTM - 1) / kTM, (E + kTE - 1) / kTE, S);
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

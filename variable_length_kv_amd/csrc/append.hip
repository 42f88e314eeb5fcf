// Per-step KV append: one new key/value row per request written into its page.
//
// Decode grows every request's context by one token per step; the source
// article names continuous batching with contexts that grow at different rates
// as the traffic its scheduler serves, and cache precision as a benchmark
// dimension [Tencent HPC lands in SGLang, challenging default inference
// kernels, secs. "Why Tencent HPC matters for online model serving" and "What
// the 48.8% TPOT claim does not prove"]. This kernel is the write half of that
// step: request b's rows k_new[b][g][:], v_new[b][g][:] go to token position
// positions[b], row positions[b] % P of page page_table[b][positions[b] / P].
// A bf16 cache stores the bf16 bits; an fp8 cache stores the e4m3fn code of
// x / scale (fp32 division, nearest with ties to even, saturated at +-448).
//
// 16 lanes per (request, kv head), 16 bytes of new bf16 data per lane: the
// loads and the bf16 stores are whole 16-byte transactions, the fp8 stores 8.
#include "vlkv_internal.hpp"

namespace vlkv {
namespace {

typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef uint32_t u32x2 __attribute__((__vector_size__(2 * sizeof(uint32_t))));

constexpr int kLanesPerRow = kHeadDim / 8;   // 8 bf16 values per lane

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// x / s saturated to the e4m3fn range; NaN stays NaN (and becomes the NaN code).
__device__ __forceinline__ float scaled_sat(float x, float s)
{
    const float y = x / s;
    return y != y ? y : fminf(fmaxf(y, -448.f), 448.f);
}

// Four fp32 values (already in range) to four e4m3fn codes, nearest-even.
__device__ __forceinline__ uint32_t to_e4m3fn4(float a, float b, float c, float d)
{
    uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0u, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

template <int KVFP8>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a)
{
    const int t = blockIdx.x * 256 + threadIdx.x;
    const int bg = t / kLanesPerRow, c = t - bg * kLanesPerRow;
    if (bg >= a.B * a.Hkv)
        return;
    const int b = bg / a.Hkv, g = bg - b * a.Hkv;
    const int pos = a.positions[b];
    if (pos < 0)
        return;
    if ((int64_t)pos >= (int64_t)a.pt_stride * a.P) {
        if (a.header && g == 0 && c == 0)
            atomicOr(reinterpret_cast<unsigned *>(a.header + H_STATUS), 1u);
        return;
    }
    const int page = a.page_table[(size_t)b * a.pt_stride + pos / a.P];
    if (page < 0 || page >= a.num_pages) {
        if (a.header && g == 0 && c == 0)
            atomicOr(reinterpret_cast<unsigned *>(a.header + H_STATUS), 2u);
        return;
    }
    const size_t src = (size_t)bg * kHeadDim + 8 * c;                       // elements
    const size_t dst = (((size_t)page * a.Hkv + g) * a.P + pos % a.P) * kHeadDim + 8 * c;
    const u32x4 kx = *reinterpret_cast<const u32x4 *>(a.k_new + src);
    const u32x4 vx = *reinterpret_cast<const u32x4 *>(a.v_new + src);
    if (KVFP8) {
        const float ks = a.k_scale[bg], vs = a.v_scale[bg];
        u32x2 kc, vc;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            kc[h] = to_e4m3fn4(scaled_sat(bf16_lo(kx[2 * h]), ks), scaled_sat(bf16_hi(kx[2 * h]), ks),
                               scaled_sat(bf16_lo(kx[2 * h + 1]), ks), scaled_sat(bf16_hi(kx[2 * h + 1]), ks));
            vc[h] = to_e4m3fn4(scaled_sat(bf16_lo(vx[2 * h]), vs), scaled_sat(bf16_hi(vx[2 * h]), vs),
                               scaled_sat(bf16_lo(vx[2 * h + 1]), vs), scaled_sat(bf16_hi(vx[2 * h + 1]), vs));
        }
        *reinterpret_cast<u32x2 *>(a.k_cache + dst) = kc;
        *reinterpret_cast<u32x2 *>(a.v_cache + dst) = vc;
    } else {
        *reinterpret_cast<u32x4 *>(a.k_cache + 2 * dst) = kx;
        *reinterpret_cast<u32x4 *>(a.v_cache + 2 * dst) = vx;
    }
}

}  // namespace

hipError_t launch_append(const AppendArgs &a, int kv_fp8, hipStream_t st)
{
    const int64_t threads = (int64_t)a.B * a.Hkv * kLanesPerRow;
    const int grid = (int)((threads + 255) / 256);
    if (grid <= 0)
        return hipSuccess;
    if (kv_fp8)
        hipLaunchKernelGGL((append_kernel<1>), dim3(grid), dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((append_kernel<0>), dim3(grid), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace vlkv

// Per-step tile planner (one workgroup).
//
// The source article's Dynamic Attention cuts each request's KV-cache work into
// uniform tiles, hands them to CTAs according to the current load, and rebuilds
// that mapping as request lengths change during decode; a static split-k is its
// comparison point [Tencent HPC lands in SGLang, challenging default inference
// kernels, sec. "Why Tencent HPC matters for online model serving"]. Here the
// plan is rebuilt on the device every step from the lengths alone, so the host
// never waits for the GPU:
//
//   units   (b, g, t), t < ceil(Le_b / T), numbered b-major, then g, then t;
//           Le_b = L_b if 0 <= L_b <= pt_stride*P, else 0 (status bit 1)
//   dynamic workgroup w owns units [floor(w*N/We), floor((w+1)*N/We)),
//           We = min(W, N); unit u's owner is floor(((u+1)*We - 1) / N);
//           pair bg = b*Hkv+g has owner(last) - owner(first) + 1 segments,
//           each with a partial slot seg_prefix[bg] + (w - first_wg[bg])
//   static  chunk C = ceil(max Le / S) rounded up to lcm(P, T); split s of a
//           pair covers tokens [s*C, min((s+1)*C, Le_b)); slot = bg*S + s
//
// The work is O(B*Hkv + W) and latency-bound: each thread owns a contiguous
// chunk of every array, so a prefix sum is one serial pass per thread, one
// wave scan and one exchange of 4 wave totals through LDS.
#include "vlkv_device.hpp"
#include "vlkv_internal.hpp"

namespace vlkv {
namespace {

constexpr int kPT = 256;  // planner threads
constexpr int kPW = kPT / 64;

__global__ __launch_bounds__(kPT) void plan_kernel(PlanArgs a)
{
    __shared__ int32_t tp[kMaxBatch + 1];   // tiles prefix
    __shared__ int scan_lds[kPW];
    __shared__ int red_lds[2 * kPW];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

    // 1) validated lengths and the tiles prefix
    const int64_t limit = (int64_t)a.pt_stride * a.P;
    const int cA = (a.B + kPT - 1) / kPT;
    const int b0 = min(a.B, tid * cA), b1 = min(a.B, b0 + cA);
    int sum = 0, mx = 0, st = 0;
    for (int b = b0; b < b1; ++b) {
        int L = a.lengths[b];
        if (L < 0 || (int64_t)L > limit) {
            st = 1;
            L = 0;
        }
        a.len_eff[b] = L;
        mx = max(mx, L);
        const int n = (L + a.T - 1) / a.T;
        tp[b + 1] = n;   // tile count for now; turned into the prefix below
        sum += n;
    }
    int total;
    int run = block_excl_scan<kPT>(sum, scan_lds, &total);
    for (int b = b0; b < b1; ++b) {
        run += tp[b + 1];
        tp[b + 1] = run;
        a.tiles_prefix[b + 1] = run;
    }
    mx = wave_max(mx);
    st = wave_or(st);
    if (lane == 0) {
        red_lds[wave] = mx;
        red_lds[kPW + wave] = st;
    }
    if (tid == 0) {
        tp[0] = 0;
        a.tiles_prefix[0] = 0;
    }
    __syncthreads();
    int maxle = 0, status = 0;
#pragma unroll
    for (int i = 0; i < kPW; ++i) {
        maxle = max(maxle, red_lds[i]);
        status |= red_lds[kPW + i];
    }
    const int nbg = a.B * a.Hkv;

    if (a.mode == 1) {
        // 2s) static split-K
        const int64_t S = a.S;
        const int64_t gran = (int64_t)a.P / gcd64(a.P, a.T) * a.T;
        int64_t C = 0;
        if (maxle > 0) {
            C = (maxle + S - 1) / S;
            C = (C + gran - 1) / gran * gran;
        }
        for (int bg = tid; bg <= nbg; bg += kPT) {
            a.seg_prefix[bg] = (int32_t)(bg * S);
            if (bg < nbg)
                a.first_wg[bg] = (int32_t)(bg * S);
        }
        if (tid == 0) {
            const int32_t NB = (int32_t)(nbg * S);
            const int32_t h[kHeaderInts] = {status, NB, NB, maxle, (int32_t)C, (int32_t)S, total, a.T};
            for (int i = 0; i < kHeaderInts; ++i)
                a.header[i] = h[i];
        }
        return;
    }

    // 2d) dynamic: segments per (b, g) and their prefix
    const int64_t N = (int64_t)total * a.Hkv;
    const int64_t We = N < a.W ? N : a.W;
    const int cB = (nbg + kPT - 1) / kPT;
    const int g0 = min(nbg, tid * cB), g1 = min(nbg, g0 + cB);
    int segs = 0;
    for (int bg = g0; bg < g1; ++bg) {
        const int b = bg / a.Hkv, g = bg - b * a.Hkv;
        const int64_t nb = tp[b + 1] - tp[b];
        if (nb == 0) {
            a.first_wg[bg] = -1;
        } else {
            const int64_t u0 = (int64_t)tp[b] * a.Hkv + g * nb;
            const int64_t w0 = div_floor((u0 + 1) * We - 1, N);
            const int64_t w1 = div_floor((u0 + nb) * We - 1, N);
            a.first_wg[bg] = (int32_t)w0;
            segs += (int)(w1 - w0 + 1);
        }
    }
    int nseg;
    run = block_excl_scan<kPT>(segs, scan_lds, &nseg);
    for (int bg = g0; bg < g1; ++bg) {
        const int b = bg / a.Hkv, g = bg - b * a.Hkv;
        const int64_t nb = tp[b + 1] - tp[b];
        if (nb) {
            const int64_t u0 = (int64_t)tp[b] * a.Hkv + g * nb;
            run += (int)(div_floor((u0 + nb) * We - 1, N) - div_floor((u0 + 1) * We - 1, N) + 1);
        }
        a.seg_prefix[bg + 1] = run;
    }
    if (tid == 0)
        a.seg_prefix[0] = 0;

    // 3) workgroup ranges and the request of each range's first unit
    const int cC = (a.W + 1 + kPT - 1) / kPT;
    const int w0 = min(a.W + 1, tid * cC), w1 = min(a.W + 1, w0 + cC);
    int sb = 0;
    if (w0 < w1 && We > 0) {
        // largest b in [0, B) with Hkv * tp[b] <= begin(w0)
        const int64_t begin = w0 <= We ? div_floor((int64_t)w0 * N, We) : N;
        int lo = 0, hi = a.B - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if ((int64_t)tp[mid] * a.Hkv <= begin)
                lo = mid;
            else
                hi = mid - 1;
        }
        sb = lo;
    }
    for (int w = w0; w < w1; ++w) {
        const int64_t begin = (w <= We && We > 0) ? div_floor((int64_t)w * N, We) : N;
        a.wg_begin[w] = (int32_t)begin;
        if (w < a.W) {
            if (w < We) {
                while (sb + 1 < a.B && (int64_t)tp[sb + 1] * a.Hkv <= begin)
                    ++sb;
                a.wg_start_b[w] = sb;
            } else {
                a.wg_start_b[w] = a.B;
            }
        }
    }
    if (tid == 0) {
        const int32_t h[kHeaderInts] = {status, (int32_t)N, (int32_t)We, maxle, 0, 0, total, a.T};
        for (int i = 0; i < kHeaderInts; ++i)
            a.header[i] = h[i];
    }
}

}  // namespace

hipError_t launch_plan(const PlanArgs &a, hipStream_t st)
{
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPT), 0, st, a);
    return hipGetLastError();
}

}  // namespace vlkv

// Per-step tile planner (one workgroup of 1024 threads).
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
// Work is O(B*Hkv + W) with one block-wide scan per array.
#include "vlkv_internal.hpp"

namespace vlkv {
namespace {

// Inclusive scan of one int per thread across the workgroup; returns this
// thread's inclusive prefix and the workgroup total in *total.
__device__ int64_t block_inclusive_scan(int64_t v, int64_t *lds_waves, int64_t *total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nwaves = blockDim.x >> 6;
    int64_t x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int64_t y = __shfl_up(x, off, 64);
        if (lane >= off)
            x += y;
    }
    if (lane == 63)
        lds_waves[wave] = x;
    __syncthreads();
    if (wave == 0) {
        int64_t w = lane < nwaves ? lds_waves[lane] : 0;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            int64_t y = __shfl_up(w, off, 64);
            if (lane >= off)
                w += y;
        }
        if (lane < nwaves)
            lds_waves[lane] = w;  // inclusive totals of waves
    }
    __syncthreads();
    const int64_t before = wave ? lds_waves[wave - 1] : 0;
    *total = lds_waves[nwaves - 1];
    __syncthreads();  // lds_waves is reused by the next call
    return x + before;
}

__device__ int64_t gcd64(int64_t a, int64_t b)
{
    while (b) {
        int64_t t = a % b;
        a = b;
        b = t;
    }
    return a;
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a)
{
    __shared__ int32_t tp[kMaxBatch + 1];   // tiles prefix
    __shared__ int64_t scan_tmp[kPlanThreads / 64];
    __shared__ int32_t red_max, red_status;
    const int tid = threadIdx.x;
    if (tid == 0) {
        red_max = 0;
        red_status = 0;
        tp[0] = 0;
    }
    __syncthreads();

    // 1) validated lengths and tile prefix
    const int64_t limit = (int64_t)a.pt_stride * a.P;
    int64_t carry = 0;
    int local_max = 0, local_status = 0;
    for (int base = 0; base < a.B; base += kPlanThreads) {
        const int b = base + tid;
        int64_t n = 0;
        if (b < a.B) {
            int64_t L = a.lengths[b];
            if (L < 0 || L > limit) {
                local_status |= 1;
                L = 0;
            }
            a.len_eff[b] = (int32_t)L;
            local_max = L > local_max ? (int)L : local_max;
            n = (L + a.T - 1) / a.T;
        }
        int64_t tot;
        const int64_t incl = block_inclusive_scan(n, scan_tmp, &tot);
        if (b < a.B) {
            tp[b + 1] = (int32_t)(carry + incl);
            a.tiles_prefix[b + 1] = (int32_t)(carry + incl);
        }
        carry += tot;
    }
    if (tid == 0)
        a.tiles_prefix[0] = 0;
    atomicMax(&red_max, local_max);
    atomicOr(&red_status, local_status);
    __syncthreads();
    const int64_t total = carry;   // sum of tiles (same in every thread)
    const int32_t maxle = red_max;
    const int32_t status = red_status;
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
        for (int bg = tid; bg <= nbg; bg += kPlanThreads) {
            a.seg_prefix[bg] = (int32_t)(bg * S);
            if (bg < nbg)
                a.first_wg[bg] = (int32_t)(bg * S);
        }
        if (tid == 0) {
            const int32_t NB = (int32_t)(nbg * S);
            const int32_t h[kHeaderInts] = {status, NB, NB, maxle, (int32_t)C, (int32_t)S,
                                            (int32_t)total, a.T};
            for (int i = 0; i < kHeaderInts; ++i)
                a.header[i] = h[i];
        }
        return;
    }

    // 2d) dynamic: segments per (b, g) and their prefix
    const int64_t N = total * a.Hkv;
    const int64_t We = N < a.W ? N : a.W;
    carry = 0;
    for (int base = 0; base < nbg; base += kPlanThreads) {
        const int bg = base + tid;
        int64_t segs = 0;
        if (bg < nbg) {
            const int b = bg / a.Hkv, g = bg % a.Hkv;
            const int64_t nb = tp[b + 1] - tp[b];
            if (nb == 0) {
                a.first_wg[bg] = -1;
            } else {
                const int64_t u0 = (int64_t)tp[b] * a.Hkv + g * nb;
                const int64_t u1 = u0 + nb - 1;
                const int64_t w0 = ((u0 + 1) * We - 1) / N;
                const int64_t w1 = ((u1 + 1) * We - 1) / N;
                a.first_wg[bg] = (int32_t)w0;
                segs = w1 - w0 + 1;
            }
        }
        int64_t tot;
        const int64_t incl = block_inclusive_scan(segs, scan_tmp, &tot);
        if (bg < nbg)
            a.seg_prefix[bg + 1] = (int32_t)(carry + incl);
        carry += tot;
    }
    if (tid == 0)
        a.seg_prefix[0] = 0;

    // 3) workgroup ranges and the request of each range's first unit
    for (int w = tid; w <= a.W; w += kPlanThreads) {
        const int64_t begin = (w <= We && We > 0) ? (int64_t)w * N / We : N;
        a.wg_begin[w] = (int32_t)begin;
        if (w < a.W) {
            int32_t sb = a.B;
            if (w < We) {
                // largest b in [0, B) with Hkv * tp[b] <= begin
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
            a.wg_start_b[w] = sb;
        }
    }
    if (tid == 0) {
        const int32_t h[kHeaderInts] = {status, (int32_t)N, (int32_t)We, maxle, 0, 0,
                                        (int32_t)total, a.T};
        for (int i = 0; i < kHeaderInts; ++i)
            a.header[i] = h[i];
    }
}

}  // namespace

hipError_t launch_plan(const PlanArgs &a, hipStream_t st)
{
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace vlkv

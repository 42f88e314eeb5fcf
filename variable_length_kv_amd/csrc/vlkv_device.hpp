// Device helpers shared by the planner and the decode kernels: wave and
// workgroup scans/reductions over wave64, and exact integer division used by
// the tile partition. Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>

namespace vlkv {

// Wave64 scans and reductions. Within each row of 16 lanes the running value
// moves by DPP row shifts (1, 2, 4, 8: a lane whose source falls outside its
// row keeps the identity); the rows are then joined through the row totals
// (lanes 15, 31, 47, 63), read into scalar registers. No LDS traffic, so
// each step costs a few cycles instead of a cross-lane permute's round trip.
template <typename Op>
__device__ __forceinline__ int row_incl_scan(int x, int id, Op op)
{
    x = op(x, __builtin_amdgcn_update_dpp(id, x, 0x111, 0xf, 0xf, false));   // row_shr:1
    x = op(x, __builtin_amdgcn_update_dpp(id, x, 0x112, 0xf, 0xf, false));   // row_shr:2
    x = op(x, __builtin_amdgcn_update_dpp(id, x, 0x114, 0xf, 0xf, false));   // row_shr:4
    x = op(x, __builtin_amdgcn_update_dpp(id, x, 0x118, 0xf, 0xf, false));   // row_shr:8
    return x;
}

template <typename Op>
__device__ __forceinline__ int wave_incl_scan_op(int x, int id, Op op)
{
    x = row_incl_scan(x, id, op);
    const int r0 = __builtin_amdgcn_readlane(x, 15);
    const int r1 = __builtin_amdgcn_readlane(x, 31);
    const int r2 = __builtin_amdgcn_readlane(x, 47);
    const int row = (threadIdx.x & 63) >> 4;
    const int c1 = r0, c2 = op(r0, r1), c3 = op(c2, r2);   // carries into rows 1, 2, 3
    const int carry = row == 0 ? id : row == 1 ? c1 : row == 2 ? c2 : c3;
    return op(carry, x);
}

// Reduction over the wave; the result is wave-uniform.
template <typename Op>
__device__ __forceinline__ int wave_reduce_op(int x, int id, Op op)
{
    x = row_incl_scan(x, id, op);
    const int r0 = __builtin_amdgcn_readlane(x, 15);
    const int r1 = __builtin_amdgcn_readlane(x, 31);
    const int r2 = __builtin_amdgcn_readlane(x, 47);
    const int r3 = __builtin_amdgcn_readlane(x, 63);
    return op(op(r0, r1), op(r2, r3));
}

struct OpAdd {
    __device__ int operator()(int a, int b) const { return a + b; }
};
struct OpMax {
    __device__ int operator()(int a, int b) const { return max(a, b); }
};
struct OpOr {
    __device__ int operator()(int a, int b) const { return a | b; }
};

__device__ __forceinline__ int wave_incl_scan(int x) { return wave_incl_scan_op(x, 0, OpAdd{}); }
__device__ __forceinline__ int wave_max(int x) { return wave_reduce_op(x, INT_MIN, OpMax{}); }
__device__ __forceinline__ int wave_or(int x) { return wave_reduce_op(x, 0, OpOr{}); }

// Exclusive prefix of one int per thread over a workgroup of NT threads (in
// thread order); *total receives the sum over all threads. `lds` holds NT/64
// ints. Every thread of the workgroup must call it.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int *lds, int *total)
{
    constexpr int NW = NT / 64;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int incl = wave_incl_scan(v);
    if (lane == 63)
        lds[wave] = incl;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const int t = lds[i];
        before += i < wave ? t : 0;
        all += t;
    }
    __syncthreads();  // lds is reused by the next call
    *total = all;
    return before + incl - v;
}

// Exclusive prefix sum of one int per thread over a workgroup of NT threads
// (in thread order), with the workgroup's maximum of a second int and OR of a
// third, through a single barrier. *total receives the sum over all threads.
// `lds` holds 3*NT/64 ints and must not be written again before the caller's
// next barrier. Every thread of the workgroup must call it.
template <int NT>
__device__ __forceinline__ int block_scan_max_or(int v, int mx, int bits, int *lds, int *total, int *mx_out,
                                                 int *bits_out)
{
    constexpr int NW = NT / 64;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int incl = wave_incl_scan(v);
    mx = wave_max(mx);
    bits = wave_or(bits);
    if (lane == 63)
        lds[wave] = incl;
    if (lane == 0) {
        lds[NW + wave] = mx;
        lds[2 * NW + wave] = bits;
    }
    __syncthreads();
    int before = 0, all = 0, m = 0, o = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const int t = lds[i];
        before += i < wave ? t : 0;
        all += t;
        m = max(m, lds[NW + i]);
        o |= lds[2 * NW + i];
    }
    *total = all;
    *mx_out = m;
    *bits_out = o;
    return before + incl - v;
}

// Exclusive running maximum of one int per thread over a workgroup of NT
// threads (in thread order; `lo` is the identity, returned to thread 0), with
// the workgroup's maximum of a second int and OR of a third, through a single
// barrier. `lds` holds 3*NT/64 ints and must not be written again
// before the caller's next barrier. Every thread of the workgroup must call it.
template <int NT>
__device__ __forceinline__ int block_excl_max_scan_max_or(int v, int lo, int mx, int bits, int *lds, int *mx_out,
                                                          int *bits_out)
{
    constexpr int NW = NT / 64;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int incl = wave_incl_scan_op(v, INT_MIN, OpMax{});
    int excl = __shfl_up(incl, 1, 64);
    if (lane == 0)
        excl = lo;
    mx = wave_max(mx);
    bits = wave_or(bits);
    if (lane == 63)
        lds[wave] = incl;
    if (lane == 0) {
        lds[NW + wave] = mx;
        lds[2 * NW + wave] = bits;
    }
    __syncthreads();
    int m = INT_MIN, o = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        if (i < wave)
            excl = max(excl, lds[i]);
        m = max(m, lds[NW + i]);
        o |= lds[2 * NW + i];
    }
    *mx_out = m;
    *bits_out = o;
    return excl;
}

// Exclusive prefix sums of two ints per thread over a workgroup of NT threads
// (in thread order), through a single barrier; *total1 / *total2 receive the
// sums. `lds` holds 2*NT/64 ints and must not be written again before the
// caller's next barrier. Every thread of the workgroup must call it.
template <int NT>
__device__ __forceinline__ void block_excl_scan2(int v1, int v2, int *lds, int *excl1, int *excl2, int *total1,
                                                 int *total2)
{
    constexpr int NW = NT / 64;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int i1 = wave_incl_scan(v1), i2 = wave_incl_scan(v2);
    if (lane == 63) {
        lds[wave] = i1;
        lds[NW + wave] = i2;
    }
    __syncthreads();
    int b1 = 0, b2 = 0, a1 = 0, a2 = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const int t1 = lds[i], t2 = lds[NW + i];
        b1 += i < wave ? t1 : 0;
        b2 += i < wave ? t2 : 0;
        a1 += t1;
        a2 += t2;
    }
    *excl1 = b1 + i1 - v1;
    *excl2 = b2 + i2 - v2;
    *total1 = a1;
    *total2 = a2;
}

// The uniform partition of N units into We contiguous ranges, range w being
// [begin(w), begin(w + 1)) with begin(w) = floor(w N / We), for N < 2^31 and
// 1 <= We <= 2^16, in 32-bit integer arithmetic: with N = qN We + rN,
// begin(w) = w qN + floor(w rN / We), where w rN < 2^32.
struct UniformSplit {
    uint32_t N, We, qN, rN;
    __device__ void init(uint32_t n, uint32_t we)
    {
        N = n;
        We = we;
        qN = n / we;
        rN = n - qN * we;
    }
    __device__ uint32_t begin(uint32_t w) const { return w * qN + (w * rN) / We; }
    // The range holding unit u < N: the largest w with begin(w) <= u. A
    // single-precision estimate of u We / N (below 2^16, so off by less than
    // one) is stepped to the answer.
    __device__ uint32_t owner(uint32_t u) const
    {
        int w = (int)((float)u * ((float)We / (float)N));
        w = w < 0 ? 0 : (w >= (int)We ? (int)We - 1 : w);
        while (w + 1 < (int)We && begin(w + 1) <= u)
            ++w;
        while (w > 0 && begin(w) > u)
            --w;
        return (uint32_t)w;
    }
};

// floor(x / d) for 0 <= x < 2^53, d > 0: double estimate, exact correction.
__device__ __forceinline__ int64_t div_floor(int64_t x, int64_t d)
{
    int64_t q = (int64_t)((double)x / (double)d);
    if (q * d > x)
        --q;
    else if ((q + 1) * d <= x)
        ++q;
    return q;
}

__device__ __forceinline__ int64_t gcd64(int64_t a, int64_t b)
{
    while (b) {
        const int64_t t = a % b;
        a = b;
        b = t;
    }
    return a;
}

}  // namespace vlkv

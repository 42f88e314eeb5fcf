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
//           We = min(W, N) (W: the launch's count, or by default two per
//           compute unit when that leaves 32 units each, else one);
//           unit u's owner is floor(((u+1)*We - 1) / N);
//           pair bg = b*Hkv+g has owner(last) - owner(first) + 1 segments,
//           each with a partial slot seg_prefix[bg] + (w - first_wg[bg])
//   static  chunk C = ceil(max Le / S) rounded up to lcm(P, T); split s of a
//           pair covers tokens [s*C, min((s+1)*C, Le_b)); slot = bg*S + s
//
//   shared  (mode 2) requests whose page tables begin with the same valid
//           pages are grouped (runs of adjacent sharers cut into groups of
//           R = 32 / G for G >= 8, 16 / G below); a group reads its common
//           prefix once as one "item" whose query rows are the members'
//           heads, and each request keeps an item for the rest of its tokens. The partition above then runs
//           over (item, g, t) units. Prefix caching is on the article's list
//           of situations the kernels must handle [same page, same section,
//           production-reliability paragraph].
//
// The work is O(B*Hkv + W) and latency-bound: each thread owns a contiguous
// chunk of every array, so a prefix sum is one serial pass per thread, one
// wave scan and one exchange of 4 wave totals through LDS. Mode 2 adds the
// page-table comparison of adjacent requests: 256 slots per coalesced wave
// step, 8 requests in flight in each of 16 waves.
#include "vlkv_device.hpp"
#include "vlkv_internal.hpp"

namespace vlkv {
namespace {

constexpr int kPT = 256;  // planner threads
constexpr int kPW = kPT / 64;
constexpr int kST = 1024; // threads of the prefix-shared planner: more waves keep more
constexpr int kSW = kST / 64;   // page-table loads in flight (each wave holds at most 63)

// The dynamic partition over n "items" (requests in modes 0, items in mode
// 2) whose tiles prefix is tp[0..n]: segments of each (item, kv head) pair and
// their prefix, each workgroup's range and first item, and the header.
template <int NT>
__device__ void plan_partition(const PlanArgs &a, const int32_t *tp, int n, int total, int status, int maxle,
                               int h4, int h5, int *scan_lds)
{
    const int tid = threadIdx.x;
    int run;
    // segments per (item, g) and their prefix
    const int nbg = n * a.Hkv;
    const int64_t N = (int64_t)total * a.Hkv;
    const int64_t We = plan_wgs(N, a.W, a.W_auto);
    const int cB = (nbg + NT - 1) / NT;
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
    run = block_excl_scan<NT>(segs, scan_lds, &nseg);
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
    const int cC = (a.W + 1 + NT - 1) / NT;
    const int w0 = min(a.W + 1, tid * cC), w1 = min(a.W + 1, w0 + cC);
    int sb = 0;
    if (w0 < w1 && We > 0) {
        // largest item i in [0, n) with Hkv * tp[i] <= begin(w0)
        const int64_t begin = w0 <= We ? div_floor((int64_t)w0 * N, We) : N;
        int lo = 0, hi = n - 1;
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
                while (sb + 1 < n && (int64_t)tp[sb + 1] * a.Hkv <= begin)
                    ++sb;
                a.wg_start_b[w] = sb;
            } else {
                a.wg_start_b[w] = n;
            }
        }
    }
    if (tid == 0) {
        const int32_t h[kHeaderInts] = {status, (int32_t)N, (int32_t)We, maxle, h4, h5, total, a.T};
        for (int i = 0; i < kHeaderInts; ++i)
            a.header[i] = h[i];
    }
}

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

    plan_partition<kPT>(a, tp, a.B, total, status, maxle, 0, 0, scan_lds);
}


// Group of request b (mode 2): its leader, member count m and the group's
// shared tokens Ls (0 when m < 2). rs is the start of b's run; share[] holds
// each request's tokens shared with the previous one.
__device__ __forceinline__ void group_of(const int32_t *share, int B, int R, int b, int rs, int &leader, int &m,
                                         int &Ls)
{
    leader = rs + (b - rs) / R * R;
    m = 1;
    Ls = INT32_MAX;
    while (m < R && leader + m < B) {
        const int sh = share[leader + m];
        if (sh == 0)
            break;
        Ls = min(Ls, sh);
        ++m;
    }
    if (m < 2)
        Ls = 0;
}

// Mode 2: prefix-shared pages. All threads are in one workgroup; the
// per-request intermediates (shared tokens, validated lengths) stay in LDS,
// so the phases that read other threads' entries cost no memory round trips.
__global__ __launch_bounds__(kST) void plan_shared_kernel(PlanArgs a)
{
    __shared__ int32_t tp_lds[kMaxBatch + 1];   // item tiles prefix, when at most kMaxBatch items
    __shared__ int32_t share_lds[kMaxBatch];    // tokens shared with the previous request
    __shared__ int32_t len_lds[kMaxBatch];      // validated lengths
    __shared__ int scan_lds[kSW];
    __shared__ int red_lds[2 * kSW];
    const int tid = threadIdx.x;
    const int R = shared_group(a.G);
    const int64_t limit = (int64_t)a.pt_stride * a.P;
    const int cA = (a.B + kST - 1) / kST;
    const int b0 = min(a.B, tid * cA), b1 = min(a.B, b0 + cA);

    // 1) tokens shared with the previous request: leading page slots with the
    //    same valid id, capped by both lengths, whole tiles; and the validated
    //    lengths (out-of-range lengths count as 0 and set the status bit). It
    //    reads only the inputs, so it goes first. Lane l of a wave
    //    compares slots 4l..4l+3 (256 consecutive slots per step, coalesced);
    //    a ballot over the lanes whose 4 slots all agree finds the first
    //    mismatch. Each of the 16 waves takes kNB requests at a time
    //    (b = wave + 16 k), so all their loads share one round trip per step,
    //    and the first step's loads go out together with the lengths';
    //    the round trips, not the bytes, are what this phase costs (a wave
    //    holds at most 63 loads in flight, hence the 16 waves).
    int mx = 0, st = 0;
    {
        constexpr int kNB = 8, kSub = 4, kSpan = 64 * kSub;
        const int wave = tid >> 6, lane = tid & 63;
        for (int base = wave; base < a.B; base += kSW * kNB) {
            int c[kNB], n[kNB], lmin[kNB];
            bool done[kNB];
            int x[kNB][kSub], y[kNB][kSub];
            // the first step's slots of rows b and b - 1 do not depend on the
            // lengths: their loads go out with the lengths' (one round trip)
#pragma unroll
            for (int k = 0; k < kNB; ++k) {
                const int b = base + kSW * k;
                const int32_t *ra = a.page_table + (size_t)b * a.pt_stride;
#pragma unroll
                for (int i = 0; i < kSub; ++i) {
                    const int j = kSub * lane + i;
                    x[k][i] = -1;
                    y[k][i] = -2;
                    if (b > 0 && b < a.B && j < a.pt_stride) {
                        x[k][i] = ra[j];
                        y[k][i] = ra[j - a.pt_stride];
                    }
                }
            }
#pragma unroll
            for (int k = 0; k < kNB; ++k) {
                // branch-free, in-bounds loads
                const int b = base + kSW * k;
                const int ia = max(min(b, a.B - 1), 0), ip = max(ia - 1, 0);
                int la = a.lengths[ia], lp = a.lengths[ip];
                if (b < a.B && (la < 0 || (int64_t)la > limit))
                    st = 1;
                la = (la < 0 || (int64_t)la > limit) ? 0 : la;
                lp = (lp < 0 || (int64_t)lp > limit) ? 0 : lp;
                if (b < a.B) {
                    mx = max(mx, la);
                    if (lane == 0)
                        len_lds[b] = la;
                }
                lmin[k] = min(la, lp);
                c[k] = 0;
                n[k] = (b > 0 && b < a.B) ? (lmin[k] + a.P - 1) / a.P : 0;
                done[k] = n[k] == 0;
            }
            for (bool first = true;; first = false) {
                if (!first) {
#pragma unroll
                    for (int k = 0; k < kNB; ++k) {
                        const int32_t *ra = a.page_table + (size_t)(base + kSW * k) * a.pt_stride;
#pragma unroll
                        for (int i = 0; i < kSub; ++i) {
                            x[k][i] = -1;
                            y[k][i] = -2;
                            const int j = c[k] + kSub * lane + i;
                            if (!done[k] && j < n[k]) {
                                x[k][i] = ra[j];
                                y[k][i] = ra[j - a.pt_stride];
                            }
                        }
                    }
                }
                bool any = false;
#pragma unroll
                for (int k = 0; k < kNB; ++k) {
                    if (done[k])
                        continue;
                    int m = 0;   // this lane's slots that agree (slots past n do not)
#pragma unroll
                    for (int i = 0; i < kSub; ++i)
                        m |= (c[k] + kSub * lane + i < n[k] && x[k][i] == y[k][i] && x[k][i] >= 0 &&
                              x[k][i] < a.num_pages)
                             << i;
                    const uint64_t full = __builtin_amdgcn_ballot_w64(m == (1 << kSub) - 1);
                    int run = kSpan;
                    if (full != ~0ull) {
                        const int fl = __builtin_ctzll(~full);   // first lane with a mismatch
                        const int mf = __builtin_amdgcn_readlane(m, fl);
                        run = kSub * fl + __builtin_ctz(~mf);
                    }
                    c[k] += run;
                    done[k] = run < kSpan || c[k] >= n[k];
                    any |= !done[k];
                }
                if (!any)
                    break;
            }
            if (lane == 0) {
#pragma unroll
                for (int k = 0; k < kNB; ++k) {
                    const int b = base + kSW * k;
                    if (b < a.B) {
                        const int64_t t = b > 0 ? min((int64_t)c[k] * a.P, (int64_t)lmin[k]) : 0;
                        share_lds[b] = (int)(t / a.T * a.T);
                    }
                }
            }
        }
    }

    // 2) the largest length and the status bit (the barriers of the reduction
    //    also publish share_lds and len_lds)
    int maxle, status;
    block_max_or<kST>(mx, st, red_lds, &maxle, &status);

    // 3) runs (start at b = 0 and wherever share = 0), groups of R, and the
    //    item and tile counts of each thread's requests
    int last_start = -1;
    for (int b = b0; b < b1; ++b)
        if (b == 0 || share_lds[b] == 0)
            last_start = b;
    const int carry = block_excl_max_scan<kST>(last_start, -1, scan_lds);
    int nitems = 0, ntiles = 0;
    {
        int rs = carry;
        for (int b = b0; b < b1; ++b) {
            if (b == 0 || share_lds[b] == 0)
                rs = b;
            int leader, m, Ls;
            group_of(share_lds, a.B, R, b, rs, leader, m, Ls);
            if (b == leader && m >= 2) {
                ++nitems;
                ntiles += (Ls + a.T - 1) / a.T;
            }
            ++nitems;
            ntiles += (len_lds[b] - Ls + a.T - 1) / a.T;
        }
    }
    int n_items, total;
    const int ibase = block_excl_scan<kST>(nitems, scan_lds, &n_items);
    const int tbase = block_excl_scan<kST>(ntiles, scan_lds, &total);

    // 4) items, in request order
    {
        int i = ibase, t = tbase, rs = carry;
        for (int b = b0; b < b1; ++b) {
            if (b == 0 || share_lds[b] == 0)
                rs = b;
            int leader, m, Ls;
            group_of(share_lds, a.B, R, b, rs, leader, m, Ls);
            if (b == leader && m >= 2) {
                a.item_req[i] = b;
                a.item_start[i] = 0;
                a.len_eff[i] = Ls;
                a.item_m[i] = m;
                a.item_solo[i] = 0;
                t += (Ls + a.T - 1) / a.T;
                a.tiles_prefix[i + 1] = t;
                if (i + 1 <= kMaxBatch)
                    tp_lds[i + 1] = t;
                ++i;
            }
            const int Lb = len_lds[b];
            a.item_req[i] = b;
            a.item_start[i] = Ls;
            a.len_eff[i] = Lb - Ls;
            a.item_m[i] = 1;
            a.item_solo[i] = m >= 2 ? 0 : 1;
            t += (Lb - Ls + a.T - 1) / a.T;
            a.tiles_prefix[i + 1] = t;
            if (i + 1 <= kMaxBatch)
                tp_lds[i + 1] = t;
            a.req_own[b] = i;
            a.req_member[b] = m >= 2 ? b - leader : 0;
            // the group's shared item precedes the own items of leader..b
            a.req_shared[b] = m >= 2 ? i - 1 - (b - leader) : -1;
            ++i;
        }
        if (tid == 0) {
            a.tiles_prefix[0] = 0;
            tp_lds[0] = 0;
        }
    }
    __syncthreads();

    // 5) the dynamic partition over items (tiles prefix from LDS when it fits)
    plan_partition<kST>(a, n_items <= kMaxBatch ? tp_lds : a.tiles_prefix, n_items, total, status, maxle, n_items, R,
                   scan_lds);
}

}  // namespace

hipError_t launch_plan(const PlanArgs &a, hipStream_t st)
{
    if (a.mode == MODE_SHARED)
        hipLaunchKernelGGL(plan_shared_kernel, dim3(1), dim3(kST), 0, st, a);
    else
        hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPT), 0, st, a);
    return hipGetLastError();
}

}  // namespace vlkv

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
// page-table comparison of adjacent requests: 4 consecutive requests per wave
// (16 waves) at a time, their 5 rows loaded once, 256 slots per row and step.
#include "vlkv_device.hpp"
#include "vlkv_internal.hpp"

namespace vlkv {
namespace {

constexpr int kPT = 256;  // planner threads
constexpr int kPW = kPT / 64;
constexpr int kST = 1024; // threads of the prefix-shared planner
constexpr int kSW = kST / 64;

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
    __shared__ int run_lds[3 * kSW];   // (each block pass has its own LDS, so one barrier each)
    __shared__ int cnt_lds[2 * kSW];
    const int tid = threadIdx.x;
    const int R = shared_group(a.G);
    const int64_t limit = (int64_t)a.pt_stride * a.P;
    const int cA = (a.B + kST - 1) / kST;
    const int b0 = min(a.B, tid * cA), b1 = min(a.B, b0 + cA);

    // 1) tokens shared with the previous request: leading page slots with the
    //    same valid id, capped by both lengths, whole tiles; and the validated
    //    lengths (out-of-range lengths count as 0 and set the status bit). It
    //    reads only the inputs, so it goes first. Each wave takes kNB
    //    consecutive requests at a time and loads the kNB + 1 page-table rows
    //    they span once (row b is request b's row and request b + 1's
    //    previous one), 256 slots each: lane l holds slots l + 64 i, so every
    //    load instruction reads contiguous bytes. The lengths come in one load
    //    issued first, and one wait covers the step. The per-request
    //    arithmetic runs across lanes (lane k: request base + k); only the
    //    search for the first slot that differs, one ballot per 64 slots, runs
    //    per request. A run that goes on past 256 slots continues in further
    //    steps for its request alone.
    int mx = 0, st = 0;
    {
        constexpr int kNB = 64 / kSW, kSub = 4, kSpan = 64 * kSub;
        // (wave-uniform in scalar registers: rows and their addresses are scalar)
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
        // first slot in [c0, c0 + kSpan) where xs and ys differ (or either is
        // not a valid page id, or the slot is at or past nk); kSpan if none
        auto first_mismatch = [&](const int (&xs)[kSub], const int (&ys)[kSub], int c0, int nk) {
            int run = kSpan;
#pragma unroll
            for (int i = kSub - 1; i >= 0; --i) {
                const bool ok = c0 + lane + 64 * i < nk && xs[i] == ys[i] && xs[i] >= 0 && xs[i] < a.num_pages;
                const uint64_t full = __builtin_amdgcn_ballot_w64(ok);
                if (full != ~0ull)
                    run = 64 * i + __builtin_ctzll(~full);
            }
            return run;
        };
        auto load_row = [&](int (&xs)[kSub], int row, int c0, int nk) {
            const int32_t *ra = a.page_table + (size_t)row * a.pt_stride;
#pragma unroll
            for (int i = 0; i < kSub; ++i) {
                const int j = c0 + lane + 64 * i;
                xs[i] = j < nk ? ra[j] : -1;
            }
        };
        for (int base = wave * kNB; base < a.B; base += kSW * kNB) {
            // lane r <= kNB: the length of row base - 1 + r
            const int lv = a.lengths[max(min(base - 1 + lane, a.B - 1), 0)];
            // rows base - 1 .. base + kNB - 1, slots lane + 64 i (-1 past the
            // row's end or for a row outside [0, B))
            int rw[kNB + 1][kSub];
#pragma unroll
            for (int i = 0; i < kSub; ++i) {
#pragma unroll
                for (int r = 0; r <= kNB; ++r)
                    rw[r][i] = -1;
                if (lane + 64 * i < a.pt_stride) {
#pragma unroll
                    for (int r = 0; r <= kNB; ++r) {
                        const int row = base - 1 + r;
                        if (row >= 0 && row < a.B)
                            rw[r][i] = a.page_table[(size_t)row * a.pt_stride + lane + 64 * i];
                    }
                }
            }
            // lane k < kNB: request b = base + k, its length and the previous request's
            const int b = base + lane;
            const bool mine = lane < kNB && b < a.B;
            int la = __shfl_down(lv, 1), lp = lv;
            if (mine && (la < 0 || (int64_t)la > limit))
                st = 1;
            la = (la < 0 || (int64_t)la > limit) ? 0 : la;
            lp = (lp < 0 || (int64_t)lp > limit) ? 0 : lp;
            if (mine) {
                mx = max(mx, la);
                len_lds[b] = la;
            }
            const int lmin = min(la, lp);
            const int nv = mine && b > 0 ? (lmin + a.P - 1) / a.P : 0;   // slots to compare
            int cv = 0;   // lane k: the common run of request k, in slots
#pragma unroll
            for (int k = 0; k < kNB; ++k) {
                const int nk = __builtin_amdgcn_readlane(nv, k);
                if (nk == 0)
                    continue;
                int c = first_mismatch(rw[k + 1], rw[k], 0, nk);
                // further steps while a whole 256-slot window agreed (each
                // adds 256 to c < nk, so the loop ends)
                bool more = c == kSpan && c < nk;
                while (more) {
                    int x[kSub], y[kSub];
                    load_row(x, base + k, c, nk);
                    load_row(y, base + k - 1, c, nk);
                    const int run = first_mismatch(x, y, c, nk);
                    c += run;
                    more = run == kSpan && c < nk;
                }
                cv = lane == k ? c : cv;
            }
            if (mine) {
                const int64_t t = b > 0 ? min((int64_t)cv * a.P, (int64_t)lmin) : 0;
                share_lds[b] = (int)(t / a.T * a.T);
            }
        }
    }

    __syncthreads();   // share_lds and len_lds are complete

    // 2) runs (start at b = 0 and wherever share = 0), groups of R, and the
    //    item and tile counts of each thread's requests; the largest length
    //    and the status bit reduce in the same pass as the runs' starts
    int last_start = -1;
    for (int b = b0; b < b1; ++b)
        if (b == 0 || share_lds[b] == 0)
            last_start = b;
    int maxle, status;
    const int carry = block_excl_max_scan_max_or<kST>(last_start, -1, mx, st, run_lds, &maxle, &status);
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
    int n_items, total, ibase, tbase;
    block_excl_scan2<kST>(nitems, ntiles, cnt_lds, &ibase, &tbase, &n_items, &total);

    // 3) items, in request order
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

    // 4) the dynamic partition over items (tiles prefix from LDS when it fits;
    //    two calls, so that each reads its array with its own instructions
    //    rather than generic ones)
    if (n_items <= kMaxBatch)
        plan_partition<kST>(a, tp_lds, n_items, total, status, maxle, n_items, R, scan_lds);
    else
        plan_partition<kST>(a, a.tiles_prefix, n_items, total, status, maxle, n_items, R, scan_lds);
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

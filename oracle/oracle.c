/*
 * CPU reference ("oracle") for variable-length paged decode attention.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library. The product path never calls it,
 * and it shares no code, header, table or helper with the HIP path.
 *
 * What it computes. One decode step: each request b has one query per query
 * head and attends to all L_b cached key/value rows of its kv head. The KV cache
 * is split into pages; the source article only says the cache holds earlier
 * attention state and that longer histories mean more cached data to read
 * [Tencent HPC lands in SGLang, challenging default inference kernels, sec.
 * "Why Tencent HPC matters for online model serving"]. Splitting the KV work
 * into tiles and merging partial softmax states (the "split-k" the same section
 * names) is an exact re-association of softmax, so the oracle is the plain
 * definition written out in fp64, for request b, query head h, kv head
 * g = h / (Hq/Hkv), L = L_b:
 *
 *   K_j = K[page_table[b][j / P]][g][j % P][:],  V_j likewise,  j = 0..L-1
 *   s_j = sm_scale * sum_d q[b][h][d] * K_j[d]
 *   m   = max_j s_j,   l = sum_j exp(s_j - m)
 *   o[b][h][:] = sum_j exp(s_j - m) * V_j / l,   lse[b][h] = m + ln l
 *
 * An empty request (L = 0) gives o = 0 and lse = -inf. bf16 values widen
 * exactly to fp64. fp8 caches hold OCP e4m3fn codes; a code is decoded exactly
 * and multiplied, in fp64, by the fp32 scale of its (request, kv head).
 *
 * The planner below is the integer specification of the per-step tile plan:
 * uniform tiles handed to workgroups, rebuilt from the current lengths
 * [same page and section: the scheduler that splits requests into uniform
 * tiles and hands them to CTAs, remapped as lengths change], and the static
 * split-k comparison point [same section]. The GPU planner must reproduce its
 * arrays byte for byte.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- values -- */

/* bfloat16 bit pattern -> double (exact: bf16 is the top half of a float). */
double oracle_bf16_to_f64(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP 8-bit floating point, E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits with
 * bias 7, 3 mantissa bits; no infinities; S.1111.111 is NaN; exponent field 0
 * encodes subnormals m/8 * 2^-6. */
double oracle_e4m3fn_to_f64(uint8_t c)
{
    int sign = c >> 7, e = (c >> 3) & 0xF, m = c & 0x7;
    double v;
    if (e == 0xF && m == 0x7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);          /* (m/8) * 2^(1-7) */
    else
        v = ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
    return sign ? -v : v;
}

/* ---------------------------------------------------------------- decode -- */

/* Error codes (negative): */
#define ORACLE_EINVAL (-1)  /* bad shape or argument */
#define ORACLE_ELEN   (-2)  /* a length outside [0, pt_stride * P] */
#define ORACLE_EPAGE  (-3)  /* a used page id outside [0, num_pages) */

/*
 * Decode attention for the requests listed in req_ids (n_req entries; NULL
 * means all B requests in order). Host pointers:
 *   q          [B][Hq][D] bf16 bits
 *   k_cache    [num_pages][Hkv][P][D] bf16 bits (kv_fp8 = 0) or e4m3fn codes
 *   v_cache    same layout as k_cache
 *   k_scale, v_scale [B][Hkv] fp32 (fp8 only; ignored for bf16)
 *   page_table [B][pt_stride] int32, lengths [B] int32
 *   out        [n_req][Hq][D] fp64, lse [n_req][Hq] fp64
 * threads <= 0 uses the OpenMP default.
 */
int oracle_decode(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t P,
                  int32_t num_pages, int32_t pt_stride, int32_t kv_fp8,
                  const uint16_t *q, const void *k_cache, const void *v_cache,
                  const float *k_scale, const float *v_scale,
                  const int32_t *page_table, const int32_t *lengths, double sm_scale,
                  const int32_t *req_ids, int32_t n_req, double *out, double *lse,
                  int32_t threads)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || D <= 0 || P <= 0 || pt_stride < 0 ||
        num_pages < 0 || !out || !lse || (kv_fp8 && (!k_scale || !v_scale)))
        return ORACLE_EINVAL;
    if (!req_ids)
        n_req = B;
    const int32_t G = Hq / Hkv;

    /* validate everything first, so no worker thread ever reads out of bounds */
    for (int32_t i = 0; i < n_req; ++i) {
        int32_t b = req_ids ? req_ids[i] : i;
        if (b < 0 || b >= B)
            return ORACLE_EINVAL;
        int64_t L = lengths[b];
        if (L < 0 || L > (int64_t)pt_stride * P)
            return ORACLE_ELEN;
        for (int64_t pg = 0; pg < (L + P - 1) / P; ++pg) {
            int32_t id = page_table[(int64_t)b * pt_stride + pg];
            if (id < 0 || id >= num_pages)
                return ORACLE_EPAGE;
        }
    }

    const int64_t n_items = (int64_t)n_req * Hkv;
    int failed = 0;
#ifdef _OPENMP
    if (threads <= 0)
        threads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(threads)
#endif
    for (int64_t item = 0; item < n_items; ++item) {
        const int32_t i = (int32_t)(item / Hkv), g = (int32_t)(item % Hkv);
        const int32_t b = req_ids ? req_ids[i] : i;
        const int64_t L = lengths[b];
        double *o = out + ((int64_t)i * Hq + (int64_t)g * G) * D;
        double *ls = lse + (int64_t)i * Hq + (int64_t)g * G;
        if (L == 0) {
            memset(o, 0, sizeof(double) * (size_t)G * D);
            for (int32_t hh = 0; hh < G; ++hh)
                ls[hh] = -INFINITY;
            continue;
        }
        double *qd = malloc(sizeof(double) * (size_t)G * D);
        double *row = malloc(sizeof(double) * (size_t)D);
        double *s = malloc(sizeof(double) * (size_t)L * G);
        double *mx = malloc(sizeof(double) * (size_t)G);
        double *sum = malloc(sizeof(double) * (size_t)G);
        if (!qd || !row || !s || !mx || !sum) {
            free(qd); free(row); free(s); free(mx); free(sum);
#ifdef _OPENMP
#pragma omp atomic write
#endif
            failed = 1;
            continue;
        }
        for (int32_t hh = 0; hh < G; ++hh)
            for (int32_t d = 0; d < D; ++d)
                qd[(int64_t)hh * D + d] =
                    oracle_bf16_to_f64(q[((int64_t)b * Hq + (int64_t)g * G + hh) * D + d]);
        const double ksc = kv_fp8 ? (double)k_scale[(int64_t)b * Hkv + g] : 1.0;
        const double vsc = kv_fp8 ? (double)v_scale[(int64_t)b * Hkv + g] : 1.0;

        /* pass 1: scores */
        for (int64_t j = 0; j < L; ++j) {
            const int64_t page = page_table[(int64_t)b * pt_stride + j / P];
            const int64_t off = ((page * Hkv + g) * P + j % P) * D;
            for (int32_t d = 0; d < D; ++d)
                row[d] = kv_fp8 ? oracle_e4m3fn_to_f64(((const uint8_t *)k_cache)[off + d]) * ksc
                                : oracle_bf16_to_f64(((const uint16_t *)k_cache)[off + d]);
            for (int32_t hh = 0; hh < G; ++hh) {
                double acc = 0.0;
                for (int32_t d = 0; d < D; ++d)
                    acc += qd[(int64_t)hh * D + d] * row[d];
                s[j * G + hh] = sm_scale * acc;
            }
        }
        /* pass 2: max, then weights exp(s - m) and their sum */
        for (int32_t hh = 0; hh < G; ++hh) {
            double m = -INFINITY;
            for (int64_t j = 0; j < L; ++j)
                if (s[j * G + hh] > m)
                    m = s[j * G + hh];
            mx[hh] = m;
            sum[hh] = 0.0;
        }
        for (int64_t j = 0; j < L; ++j)
            for (int32_t hh = 0; hh < G; ++hh) {
                s[j * G + hh] = exp(s[j * G + hh] - mx[hh]);
                sum[hh] += s[j * G + hh];
            }
        /* pass 3: weighted sum of value rows */
        memset(o, 0, sizeof(double) * (size_t)G * D);
        for (int64_t j = 0; j < L; ++j) {
            const int64_t page = page_table[(int64_t)b * pt_stride + j / P];
            const int64_t off = ((page * Hkv + g) * P + j % P) * D;
            for (int32_t d = 0; d < D; ++d)
                row[d] = kv_fp8 ? oracle_e4m3fn_to_f64(((const uint8_t *)v_cache)[off + d]) * vsc
                                : oracle_bf16_to_f64(((const uint16_t *)v_cache)[off + d]);
            for (int32_t hh = 0; hh < G; ++hh) {
                const double w = s[j * G + hh];
                for (int32_t d = 0; d < D; ++d)
                    o[(int64_t)hh * D + d] += w * row[d];
            }
        }
        for (int32_t hh = 0; hh < G; ++hh) {
            for (int32_t d = 0; d < D; ++d)
                o[(int64_t)hh * D + d] /= sum[hh];
            ls[hh] = mx[hh] + log(sum[hh]);
        }
        free(qd); free(row); free(s); free(mx); free(sum);
    }
    return failed ? ORACLE_EINVAL : 0;
}

/* ------------------------------------------------------------------ plan -- */

/*
 * Tile plan of one decode step (integer only, int64 internally).
 *
 * Units. Request b has n_b = ceil(Le_b / T) uniform tiles of T tokens (the last
 * may be short), where Le_b = L_b if 0 <= L_b <= pt_stride*P, else 0 and status
 * bit 1 is set. A unit is (b, g, t) with g < Hkv, t < n_b, numbered in the order
 * b, then g, then t; N = Hkv * sum_b n_b units in all.
 *
 * Workgroup count. W is given, or chosen by the library default: with cus > 0
 * (the device's compute units; then W must be 2*cus) the plan uses W_use = W
 * when that leaves at least 32 units per workgroup (N >= 32*W) and W_use = cus
 * otherwise; with cus = 0, W_use = W. The arrays below still span W.
 *
 * Dynamic mode (mode 0). With W_use workgroups, W_eff = min(W_use, N). Workgroup w owns
 * the contiguous unit range [floor(w*N/W_eff), floor((w+1)*N/W_eff)), so no two
 * workgroups differ by more than one unit. Unit u's owner is
 * floor(((u+1)*W_eff - 1) / N). A segment is a maximal run of one (b, g) inside
 * one workgroup; pair bg = b*Hkv + g has segs(bg) = owner(last) - owner(first) + 1
 * segments (0 if n_b = 0), and its segments take partial-result slots
 * seg_prefix[bg] .. seg_prefix[bg+1]-1 in workgroup order; first_wg[bg] is the
 * owner of its first unit (-1 if it has none). A pair with one segment is
 * written directly; pairs with two or more are merged afterwards.
 *
 * Static mode (mode 1). S splits per pair (S > 0, given). Chunk C =
 * ceil(maxLe / S) rounded up to a multiple of lcm(P, T) (0 if maxLe = 0);
 * split s of pair bg covers tokens [s*C, min((s+1)*C, Le_b)) and may be empty.
 * One workgroup per (b, g, s): N = W_eff = B*Hkv*S, seg_prefix[bg] = bg*S,
 * first_wg[bg] = bg*S. wg_begin and wg_start_b are not written.
 *
 * Outputs (caller-allocated):
 *   header[8]      = {status, N, W_eff, maxLe, C (static) or 0, S (static) or 0,
 *                     sum_b n_b, T}
 *   len_eff[B], tiles_prefix[B+1], seg_prefix[B*Hkv+1], first_wg[B*Hkv],
 *   wg_begin[W+1]  (dynamic: floor(w*N/W_eff) for w <= W_eff, N beyond),
 *   wg_start_b[W]  (dynamic: request of workgroup w's first unit; B if none).
 * Returns 0, or ORACLE_EINVAL for bad arguments, or -4 if N exceeds INT32_MAX.
 */
static int64_t gcd64(int64_t a, int64_t b)
{
    while (b) {
        int64_t t = a % b;
        a = b;
        b = t;
    }
    return a;
}

/* The workgroups a dynamic plan of N units uses (see "Workgroup count"). */
static int64_t wgs_used(int64_t N, int32_t W, int32_t cus)
{
    if (cus > 0 && N < (int64_t)32 * W)
        return cus;
    return W;
}

int oracle_plan(int32_t mode, int32_t B, int32_t Hkv, int32_t P, int32_t pt_stride,
                int32_t T, int32_t W, int32_t S, int32_t cus, const int32_t *lengths,
                int32_t *header, int32_t *len_eff, int32_t *tiles_prefix,
                int32_t *seg_prefix, int32_t *first_wg, int32_t *wg_begin,
                int32_t *wg_start_b)
{
    if (B < 0 || Hkv <= 0 || P <= 0 || pt_stride < 0 || T <= 0 || W <= 0 ||
        (mode != 0 && mode != 1) || (mode == 1 && S <= 0) || cus < 0 ||
        (cus > 0 && W != 2 * cus))
        return ORACLE_EINVAL;
    int32_t status = 0;
    int64_t total = 0, maxle = 0;
    tiles_prefix[0] = 0;
    for (int32_t b = 0; b < B; ++b) {
        int64_t L = lengths[b];
        if (L < 0 || L > (int64_t)pt_stride * P) {
            status |= 1;
            L = 0;
        }
        len_eff[b] = (int32_t)L;
        if (L > maxle)
            maxle = L;
        total += (L + T - 1) / T;
        if (total > INT32_MAX)
            return -4;
        tiles_prefix[b + 1] = (int32_t)total;
    }
    if (mode == 1) {
        const int64_t NB = (int64_t)B * Hkv * S;
        if (NB > INT32_MAX)
            return -4;
        const int64_t gran = (int64_t)P / gcd64(P, T) * T;
        int64_t C = 0;
        if (maxle > 0) {
            C = (maxle + S - 1) / S;
            C = (C + gran - 1) / gran * gran;
        }
        for (int64_t bg = 0; bg < (int64_t)B * Hkv; ++bg) {
            seg_prefix[bg] = (int32_t)(bg * S);
            first_wg[bg] = (int32_t)(bg * S);
        }
        seg_prefix[(int64_t)B * Hkv] = (int32_t)NB;
        const int32_t h[8] = {status, (int32_t)NB, (int32_t)NB, (int32_t)maxle,
                              (int32_t)C, S, (int32_t)total, T};
        memcpy(header, h, sizeof h);
        return 0;
    }
    const int64_t N = total * Hkv;
    if (N > INT32_MAX)
        return -4;
    const int64_t Wu = wgs_used(N, W, cus);
    const int64_t We = N < Wu ? N : Wu;
    int64_t nseg = 0;
    seg_prefix[0] = 0;
    for (int32_t b = 0; b < B; ++b) {
        const int64_t nb = tiles_prefix[b + 1] - tiles_prefix[b];
        for (int32_t g = 0; g < Hkv; ++g) {
            const int64_t bg = (int64_t)b * Hkv + g;
            if (nb == 0) {
                first_wg[bg] = -1;
            } else {
                const int64_t u0 = (int64_t)tiles_prefix[b] * Hkv + g * nb;
                const int64_t u1 = u0 + nb - 1;
                const int64_t w0 = ((u0 + 1) * We - 1) / N;
                const int64_t w1 = ((u1 + 1) * We - 1) / N;
                first_wg[bg] = (int32_t)w0;
                nseg += w1 - w0 + 1;
            }
            seg_prefix[bg + 1] = (int32_t)nseg;
        }
    }
    for (int64_t w = 0; w <= W; ++w)
        wg_begin[w] = (int32_t)(w <= We && We > 0 ? w * N / We : N);
    /* request of each workgroup's first unit: the b with
       Hkv*tiles_prefix[b] <= u < Hkv*tiles_prefix[b+1] */
    int32_t b = 0;
    for (int64_t w = 0; w < W; ++w) {
        if (w >= We) {
            wg_start_b[w] = B;
            continue;
        }
        const int64_t u = wg_begin[w];
        while (b < B && (int64_t)tiles_prefix[b + 1] * Hkv <= u)
            ++b;
        wg_start_b[w] = b;
    }
    const int32_t h[8] = {status, (int32_t)N, (int32_t)We, (int32_t)maxle, 0, 0,
                          (int32_t)total, T};
    memcpy(header, h, sizeof h);
    return 0;
}

/* ------------------------------------------------------- KV append -- */

/* ---------------------------------------------------- prefix-shared plan -- */
/*
 * Integer specification of the plan with prefix-shared pages (mode 2). The
 * source article lists prefix caching among the situations the kernels must
 * handle [Tencent HPC lands in SGLang, challenging default inference kernels,
 * sec. "Why Tencent HPC matters for online model serving", the production-
 * reliability paragraph]; requests whose page tables begin with the same
 * physical pages hold the same cached rows there. This plan reads such a
 * shared prefix once for several requests. The result is the same attention
 * (the oracle decode above, per request); only the work decomposition changes:
 *
 * 1. Le_b = L_b if 0 <= L_b <= pt_stride * P, else 0 (status bit 1).
 * 2. share_b (b >= 1): c = number of leading page slots j < min(ceil(Le_b / P),
 *    ceil(Le_{b-1} / P)) with page_table[b][j] == page_table[b-1][j] and that
 *    id valid (0 <= id < num_pages); share_b = min(c P, Le_b, Le_{b-1}) rounded
 *    down to a multiple of T. share_0 = 0.
 * 3. Runs: a run starts at b = 0 and at every b with share_b = 0. A run is cut,
 *    from its start, into groups of R consecutive requests: R = 32 / G for
 *    G >= 8 (two MFMA column blocks of 16 query rows per pass), R = 16 / G
 *    below (one block); R requests times G query heads of one kv head.
 *    A group with m >= 2 members shares Ls = min of share over its members
 *    other than the first (its pages agree with the first member's there).
 * 4. Items, in request order: a group leader with m >= 2 first emits the
 *    shared item (req = leader, start 0, len Ls, m members, solo 0); every
 *    request then emits its own item: (b, Ls, Le_b - Ls, 1, 0) inside a group
 *    of m >= 2, else (b, 0, Le_b, 1, 1). req_shared[b] / req_member[b] /
 *    req_own[b] map requests to items (-1 / 0 without a shared item).
 * 5. From here on mode 0 with items in place of requests: tiles ceil(len/T),
 *    units (item, kv head, tile) in order, W_eff contiguous ranges, segments
 *    and their prefix over (item, kv head) pairs, each workgroup's first item.
 *
 * header = {status, N, W_eff, max Le, number of items, R, total tiles, T}.
 * Item arrays hold up to 2B entries; tiles_prefix 2B+1; seg_prefix
 * 2B*Hkv+1; first_wg 2B*Hkv; wg_begin W+1; wg_start W.
 */
int oracle_plan_shared(int32_t B, int32_t Hkv, int32_t G, int32_t P, int32_t pt_stride, int32_t num_pages,
                       int32_t T, int32_t W, int32_t cus, const int32_t *lengths, const int32_t *page_table,
                       int32_t *header,
                       int32_t *item_req, int32_t *item_start, int32_t *item_len, int32_t *item_m,
                       int32_t *item_solo, int32_t *req_shared, int32_t *req_member, int32_t *req_own,
                       int32_t *tiles_prefix, int32_t *seg_prefix, int32_t *first_wg, int32_t *wg_begin,
                       int32_t *wg_start)
{
    if (B < 0 || Hkv <= 0 || G <= 0 || P <= 0 || pt_stride < 0 || num_pages <= 0 || T <= 0 || W <= 0 ||
        cus < 0 || (cus > 0 && W != 2 * cus))
        return ORACLE_EINVAL;
    const int32_t R = G >= 32 ? 1 : G >= 8 ? 32 / G : 16 / G;
    int32_t status = 0;
    int64_t maxle = 0;
    int32_t *Le = calloc((size_t)(B > 0 ? B : 1), sizeof *Le);
    int32_t *share = calloc((size_t)(B > 0 ? B : 1), sizeof *share);
    if (!Le || !share) {
        free(Le);
        free(share);
        return -5;
    }
    /* 1. validated lengths */
    for (int32_t b = 0; b < B; ++b) {
        int64_t L = lengths[b];
        if (L < 0 || L > (int64_t)pt_stride * P) {
            status |= 1;
            L = 0;
        }
        Le[b] = (int32_t)L;
        if (L > maxle)
            maxle = L;
    }
    /* 2. tokens shared with the previous request */
    for (int32_t b = 1; b < B; ++b) {
        const int64_t na = ((int64_t)Le[b] + P - 1) / P, nb = ((int64_t)Le[b - 1] + P - 1) / P;
        const int64_t n = na < nb ? na : nb;
        int64_t c = 0;
        while (c < n) {
            const int32_t x = page_table[(int64_t)b * pt_stride + c];
            const int32_t y = page_table[(int64_t)(b - 1) * pt_stride + c];
            if (x != y || x < 0 || x >= num_pages)
                break;
            ++c;
        }
        int64_t t = c * P;
        if (t > Le[b])
            t = Le[b];
        if (t > Le[b - 1])
            t = Le[b - 1];
        share[b] = (int32_t)(t / T * T);
    }
    /* 3 + 4. groups and items */
    int64_t I = 0, total = 0;
    int32_t run0 = 0;
    tiles_prefix[0] = 0;
    for (int32_t b = 0; b < B; ++b) {
        if (b == 0 || share[b] == 0)
            run0 = b;
        const int32_t leader = run0 + (b - run0) / R * R;
        /* members of the group led by `leader`: it and the next requests of
           the same run (share != 0), at most R */
        int32_t m = 1, Ls = 0;
        while (m < R && leader + m < B && share[leader + m] != 0)
            ++m;
        if (m >= 2) {
            Ls = share[leader + 1];
            for (int32_t k = 2; k < m; ++k)
                if (share[leader + k] < Ls)
                    Ls = share[leader + k];
        }
        if (b == leader && m >= 2) {
            item_req[I] = b;
            item_start[I] = 0;
            item_len[I] = Ls;
            item_m[I] = m;
            item_solo[I] = 0;
            total += (Ls + T - 1) / T;
            tiles_prefix[I + 1] = (int32_t)total;
            ++I;
        }
        req_shared[b] = m >= 2 ? (int32_t)(I - 1 - (b - leader)) : -1;
        req_member[b] = m >= 2 ? b - leader : 0;
        /* the shared item of b's group was emitted at the leader, b - leader own
           items ago: I - 1 - (b - leader) when b's own item is not yet counted */
        item_req[I] = b;
        item_start[I] = m >= 2 ? Ls : 0;
        item_len[I] = Le[b] - (m >= 2 ? Ls : 0);
        item_m[I] = 1;
        item_solo[I] = m >= 2 ? 0 : 1;
        req_own[b] = (int32_t)I;
        total += ((int64_t)item_len[I] + T - 1) / T;
        if (total > INT32_MAX) {
            free(Le);
            free(share);
            return -4;
        }
        tiles_prefix[I + 1] = (int32_t)total;
        ++I;
    }
    free(Le);
    free(share);
    /* 5. mode 0 over items */
    const int64_t N = total * Hkv;
    if (N > INT32_MAX)
        return -4;
    const int64_t Wu = wgs_used(N, W, cus);
    const int64_t We = N < Wu ? N : Wu;
    int64_t nseg = 0;
    seg_prefix[0] = 0;
    for (int64_t i = 0; i < I; ++i) {
        const int64_t ni = tiles_prefix[i + 1] - tiles_prefix[i];
        for (int32_t g = 0; g < Hkv; ++g) {
            const int64_t ig = i * Hkv + g;
            if (ni == 0) {
                first_wg[ig] = -1;
            } else {
                const int64_t u0 = (int64_t)tiles_prefix[i] * Hkv + g * ni;
                const int64_t u1 = u0 + ni - 1;
                const int64_t w0 = ((u0 + 1) * We - 1) / N;
                const int64_t w1 = ((u1 + 1) * We - 1) / N;
                first_wg[ig] = (int32_t)w0;
                nseg += w1 - w0 + 1;
            }
            seg_prefix[ig + 1] = (int32_t)nseg;
        }
    }
    for (int64_t w = 0; w <= W; ++w)
        wg_begin[w] = (int32_t)(w <= We && We > 0 ? w * N / We : N);
    int64_t i = 0;
    for (int64_t w = 0; w < W; ++w) {
        if (w >= We) {
            wg_start[w] = (int32_t)I;
            continue;
        }
        const int64_t u = wg_begin[w];
        while (i < I && (int64_t)tiles_prefix[i + 1] * Hkv <= u)
            ++i;
        wg_start[w] = (int32_t)i;
    }
    const int32_t h[8] = {status, (int32_t)N, (int32_t)We, (int32_t)maxle, (int32_t)I, R, (int32_t)total, T};
    memcpy(header, h, sizeof h);
    return 0;
}

/*
 * The e4m3fn code nearest to the fp32 value y: ties to even, magnitudes at or
 * above 448 (the largest finite e4m3fn value) saturate to +-448, NaN gives the
 * NaN code 0x7F. Written from the format's definition (see
 * oracle_e4m3fn_to_f64): normal numbers are (8 + m) * 2^(E-3) with E in
 * [-6, 8] and exponent field E + 7; below 2^-6 the values are the multiples
 * of 2^-9 with exponent field 0.
 */
uint8_t oracle_e4m3fn_encode(float y)
{
    if (y != y)
        return 0x7F;
    const uint8_t sign = signbit(y) ? 0x80 : 0x00;
    const double a = fabs((double)y);
    if (a >= 448.0)
        return sign | 0x7E;
    if (a < ldexp(1.0, -6)) {
        const double m = nearbyint(a * 512.0);   /* exact scaling; 8 is the smallest normal */
        return sign | (uint8_t)m;
    }
    int e;
    frexp(a, &e);                                /* a = f * 2^e, f in [0.5, 1) */
    int E = e - 1;
    double m = nearbyint(ldexp(a, 3 - E));       /* in [8, 16] */
    if (m == 16.0) {
        m = 8.0;
        ++E;
    }
    if (E > 8)
        return sign | 0x7E;
    return sign | (uint8_t)(((E + 7) << 3) | ((int)m - 8));
}

void oracle_e4m3fn_encode_array(const float *y, uint8_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_e4m3fn_encode(y[i]);
}

/*
 * Append one token per request to a paged cache: request b's new key and value
 * rows k_new[b][g][:], v_new[b][g][:] (bf16 bits, [B][Hkv][D]) go to token
 * position positions[b], i.e. row positions[b] % P of page
 * page_table[b][positions[b] / P]. A bf16 cache stores the bits unchanged; an
 * fp8 cache stores oracle_e4m3fn_encode(x / scale) with x the bf16 value and
 * scale = k_scale[b][g] (v_scale for values), the division done in fp32.
 * A negative position means "no append". A position at or beyond
 * pt_stride * P sets status bit 1 and a page id outside [0, num_pages) sets
 * bit 2; such requests are skipped. Returns the status bits.
 */
int oracle_append(int32_t B, int32_t Hkv, int32_t D, int32_t P, int32_t num_pages, int32_t pt_stride,
                  int32_t kv_fp8, const uint16_t *k_new, const uint16_t *v_new, const int32_t *positions,
                  const int32_t *page_table, const float *k_scale, const float *v_scale, void *k_cache,
                  void *v_cache)
{
    int status = 0;
    for (int32_t b = 0; b < B; ++b) {
        const int64_t pos = positions[b];
        if (pos < 0)
            continue;
        if (pos >= (int64_t)pt_stride * P) {
            status |= 1;
            continue;
        }
        const int64_t page = page_table[(int64_t)b * pt_stride + pos / P];
        if (page < 0 || page >= num_pages) {
            status |= 2;
            continue;
        }
        for (int32_t g = 0; g < Hkv; ++g) {
            const int64_t src = ((int64_t)b * Hkv + g) * D;
            const int64_t dst = ((page * Hkv + g) * P + pos % P) * D;
            for (int32_t d = 0; d < D; ++d) {
                if (kv_fp8) {
                    const float ks = k_scale[(int64_t)b * Hkv + g], vs = v_scale[(int64_t)b * Hkv + g];
                    const float kx = (float)oracle_bf16_to_f64(k_new[src + d]);
                    const float vx = (float)oracle_bf16_to_f64(v_new[src + d]);
                    ((uint8_t *)k_cache)[dst + d] = oracle_e4m3fn_encode(kx / ks);
                    ((uint8_t *)v_cache)[dst + d] = oracle_e4m3fn_encode(vx / vs);
                } else {
                    ((uint16_t *)k_cache)[dst + d] = k_new[src + d];
                    ((uint16_t *)v_cache)[dst + d] = v_new[src + d];
                }
            }
        }
    }
    return status;
}

/* ------------------------------------------------------------ router GEMM -- */
/*
 * Router GEMM with split weights. The source article describes the router
 * matmul that picks MoE experts as precision-sensitive: each fp32 weight is
 * split into two bf16 parts, one holding the high part of the weight and one
 * holding a scaled residual, with a documented scale of 1/256; the kernel runs
 * two bf16 tensor-core products and combines them [Tencent HPC lands in SGLang,
 * challenging default inference kernels, sec. "Dynamic Attention and Fused MoE
 * target different bottlenecks"]. The reading used here:
 *
 *   hi = bf16(w),  lo = bf16(256 (w - hi)),  w ~ hi + lo / 256
 *
 * with bf16() round-to-nearest-even of the fp32 value (w - hi is exact in fp32:
 * hi keeps w's 8 leading significant bits). The product of bf16 activations
 * x[M][K] with the weights w[E][K] (one row per expert) is
 *
 *   y[m][e] = sum_k x[m][k] w[e][k]
 *
 * oracle_router_gemm returns it twice in fp64: with the exact fp32 weights (the
 * accuracy target) and with hi + lo/256 (what the split computes before any
 * accumulation rounding).
 */

/* fp32 -> bf16 bits, round to nearest, ties to even; NaN stays a quiet NaN. */
uint16_t oracle_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu))
        return (uint16_t)((u >> 16) | 0x0040u);
    /* add half an ulp of the kept part (minus one when the kept lsb is 0, so
       an exact tie stays even), then truncate */
    const uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

void oracle_router_split(const float *w, uint16_t *hi, uint16_t *lo, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) {
        const uint16_t h = oracle_bf16_rne(w[i]);
        const float hf = (float)oracle_bf16_to_f64(h);
        const float r = (w[i] - hf) * 256.0f;   /* both steps exact for finite w below bf16 overflow */
        hi[i] = h;
        lo[i] = oracle_bf16_rne(r);
    }
}

int oracle_router_gemm(int32_t M, int32_t K, int32_t E, const uint16_t *x, const float *w, const uint16_t *hi,
                       const uint16_t *lo, double *y_exact, double *y_split, int32_t threads)
{
    if (M < 0 || K < 0 || E < 0 || !x || !w || !hi || !lo || !y_exact || !y_split)
        return ORACLE_EINVAL;
#ifdef _OPENMP
    if (threads <= 0)
        threads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(threads)
#endif
    for (int64_t me = 0; me < (int64_t)M * E; ++me) {
        const int64_t m = me / E, e = me % E;
        double a = 0.0, s = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double xv = oracle_bf16_to_f64(x[m * K + k]);
            a += xv * (double)w[e * K + k];
            s += xv * (oracle_bf16_to_f64(hi[e * K + k]) + oracle_bf16_to_f64(lo[e * K + k]) / 256.0);
        }
        y_exact[me] = a;
        y_split[me] = s;
    }
    (void)threads;
    return 0;
}

// Split-KV paged decode attention and its log-sum-exp combine, for gfx950.
//
// The source article's Dynamic Attention spreads uneven decode work over GPU
// execution units: KV-cache work is cut into uniform tiles handed to CTAs by
// current load, and split results are merged ("split-k"); the static split-k is
// the comparison point [Tencent HPC lands in SGLang, challenging default
// inference kernels, sec. "Why Tencent HPC matters for online model serving"].
// Both variants here share one per-block body and differ only in where a
// workgroup's sequence of (request, kv head, block range) segments comes from.
//
// Workgroup = 4 wave64s. A 64-token block of one (request b, kv head g) is split
// into four 16-token slices, one per wave; every wave walks the same sequence of
// blocks, keeps its own online-softmax state for the G query heads of g, and the
// four states are merged through LDS at the end of each segment.
//
// Per wave and slice (16 tokens x 128 dims of K and of V):
//   * K and V rows are loaded with 16-byte loads straight into MFMA operand
//     registers: lane l holds token row l%16 and a run of dims selected by
//     l/16. For bf16 each load instruction reads 64 contiguous bytes of 16 rows
//     and four instructions read the slice once; for fp8 two instructions do.
//     Two slices per wave are in flight (register double buffering) on top of
//     several resident waves per SIMD; no LDS staging is needed for K or V.
//   * S^T = K Q^T with 4 bf16 MFMAs 16x16x32 (16 tokens x 16 heads; heads >= G
//     are zero). fp8 K codes are widened to bf16 exactly first. The result's
//     lane layout (lane l: tokens 4*(l/16)+i, head l%16) is exactly the B
//     operand of the 16x16x16 bf16 MFMA, so P^T needs no data movement.
//   * Online softmax in base 2 (sm_scale*log2 e, times the fp8 k scale, folded
//     into one multiply); per-head maxima across the 4 lane groups by permlane
//     swaps.
//   * V is transposed in registers by an MFMA against a 0/1 selection matrix:
//     D = V_rows x Sel gives, in lane l, V[token 4*(l/16)+i][one dim per l%16],
//     which is the A operand (V^T) of the 16x16x16 bf16 MFMA. The product is
//     exact (one nonzero term), so it also widens fp8 codes to bf16 for free.
//   * O^T (128 dims x 16 heads) += V^T P^T with 8 MFMAs into 32 fp32 registers.
#include "vlkv_internal.hpp"

namespace vlkv {
namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef uint32_t u32x2 __attribute__((__vector_size__(2 * sizeof(uint32_t))));

constexpr float kLn2 = 0.6931471805599453f;
constexpr int kLdsRow = kHeadDim + 4;  // padded fp32 row of the merge buffer

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Read-only data of the step (plan arrays, page table, scales) is read through
// the constant address space: wave-uniform addresses then become scalar loads,
// which are counted apart from the K/V vector loads, so waiting for a page id
// never waits for K/V data still in flight.
template <typename T>
__device__ __forceinline__ T ldc(const T *p, size_t i)
{
    return ((const __attribute__((address_space(4))) T *)(p))[i];
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

// Head dim held by output register i of accumulator block mb in row group grp.
// bf16: block mb = 2*kk + s covers dims 32*kk + 16*s + [0,16) in order.
// fp8 : lane (row, grp) loads dims 16*(grp + 4p) + [0,16) for p = 0,1; the
//       selection MFMA (p, h, s) with columns n then yields
//       dim 64p + 32s + 16*(n/8) + 8h + n%8 for block mb = 4p + 2h + s.
template <int KVFP8>
__device__ __forceinline__ int out_dim(int mb, int c)
{
    if (KVFP8) {
        const int p = mb >> 2, h = (mb >> 1) & 1, s = mb & 1;
        return 64 * p + 32 * s + 16 * (c >> 3) + 8 * h + (c & 7);
    }
    return 16 * mb + c;
}

// Registers of one in-flight slice (fp8 uses k[0..1], v[0..1]).
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
    float ksc, vsc;
};

// Walks a workgroup's blocks in order. Dynamic: the contiguous unit range of
// the plan; static: the one (b, g, split) of this workgroup.
template <int MODE>
struct Walker {
    const DecodeArgs *a;
    int w, wave;
    int b, g, blk, blk0, blk_end, L, nt, units_left, done;
    int slot, direct;

    __device__ void enter_segment(int ta, int tb)
    {
        const int R = a->blocks_per_tile;
        blk = blk0 = ta * R;
        const int nblk = (L + kBlockTokens - 1) / kBlockTokens;
        blk_end = min(tb * R, nblk);
        const int bg = b * a->Hkv + g;
        const int s0 = ldc(a->seg_prefix, bg);
        const int s1 = ldc(a->seg_prefix, bg + 1);
        slot = s0 + (w - ldc(a->first_wg, bg));
        direct = (s1 - s0) == 1;
    }

    __device__ void init(const DecodeArgs *args, int wg, int wv)
    {
        a = args;
        w = wg;
        wave = wv;
        done = 0;
        if (MODE == 0) {
            const int u0 = ldc(a->wg_begin, w);
            const int u1 = ldc(a->wg_begin, w + 1);
            b = ldc(a->wg_start_b, w);
            const int tp0 = ldc(a->tiles_prefix, b);
            nt = ldc(a->tiles_prefix, b + 1) - tp0;
            L = ldc(a->len_eff, b);
            const int rem = u0 - tp0 * a->Hkv;
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
            L = ldc(a->len_eff, b);
            const int C = ldc(a->header, H_CHUNK);
            const int lo = s * C, hi = min(lo + C, L);
            units_left = 0;
            slot = w;
            direct = S == 1;
            blk = blk0 = lo / kBlockTokens;
            if (hi > lo) {
                blk_end = (hi + kBlockTokens - 1) / kBlockTokens;
            } else {
                // empty split: one pseudo-block without valid tokens, so the
                // workgroup still writes its (empty) result
                blk_end = blk + 1;
                L = 0;
            }
        }
    }

    // Number of blocks this workgroup will process (a scalar walk over its
    // segments; the walker itself is not advanced).
    __device__ int count_blocks() const
    {
        if (MODE != 0)
            return blk_end - blk;
        int n = blk_end - blk;
        int bb = b, gg = g, ntt = nt, LL = L, left = units_left;
        const int R = a->blocks_per_tile;
        while (left > 0) {
            if (++gg == a->Hkv) {
                gg = 0;
                do {
                    ++bb;
                    ntt = ldc(a->tiles_prefix, bb + 1) - ldc(a->tiles_prefix, bb);
                } while (ntt == 0);
                LL = ldc(a->len_eff, bb);
            }
            const int take = min(ntt, left);
            left -= take;
            n += min(take * R, (LL + kBlockTokens - 1) / kBlockTokens);
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
        m.tok0 = blk * kBlockTokens + wave * kSlice;
        m.nv = done ? 0 : max(0, min(kSlice, L - m.tok0));
        m.first = !done && blk == blk0;
        m.last = !done && blk + 1 == blk_end;
        m.slot = slot;
        m.direct = direct;
        m.ksc = 1.f;
        m.vsc = 1.f;
        if (done)
            return m;
        ++blk;
        if (blk == blk_end) {
            if (MODE == 0 && units_left > 0) {
                ++g;
                if (g == a->Hkv) {
                    g = 0;
                    do {
                        ++b;
                        nt = ldc(a->tiles_prefix, b + 1) - ldc(a->tiles_prefix, b);
                    } while (nt == 0);
                    L = ldc(a->len_eff, b);
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

template <int MODE, int KVFP8>
__global__ __launch_bounds__(kDecodeThreads, 2) void decode_kernel(DecodeArgs a)
{
    const int w = blockIdx.x;
    if (MODE == 0 && w >= ldc(a.header, H_WEFF))
        return;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int row = lane & 15;   // MFMA row / column within a 16x16 tile
    const int grp = lane >> 4;   // MFMA row group

    __shared__ __attribute__((aligned(16))) float lds_acc[kWaves][kMaxGroup][kLdsRow];
    __shared__ float lds_m[kWaves][kMaxGroup];
    __shared__ float lds_l[kWaves][kMaxGroup];
    __shared__ float lds_e[kWaves][kMaxGroup];

    const int G = a.G;
    constexpr int D = kHeadDim;
    constexpr int EB = KVFP8 ? 1 : 2;             // bytes per cached element
    const size_t page_head_bytes = (size_t)a.P * D * EB;

    // 0/1 selection matrices for the in-register V transpose: B operand, lane
    // (n = row, grp) element j stands for k = 8*grp + j; Sel_s[k][n] = (k == n + 16 s)
    bf16x8 sel16[2];
    uint64_t sel8[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        uint64_t bits = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const bool one = 8 * grp + j == row + 16 * s;
            sel16[s][j] = one ? (__bf16)1.0f : (__bf16)0.0f;
            bits |= (uint64_t)(one ? 0x38u : 0u) << (8 * j);  // e4m3fn 1.0 = 0x38
        }
        sel8[s] = bits;
    }

    Walker<MODE> wk;
    wk.init(&a, w, wave);

    // per-wave softmax state, head = row. m_run is uniform over the 4 row
    // groups; l_run is this lane's partial sum, reduced at segment end.
    // l_run sums the bf16-rounded weights that multiply V (normalises o exactly
    // like P.V); e_run sums the unrounded fp32 weights (gives an accurate lse).
    float m_run = -INFINITY, l_run = 0.f, e_run = 0.f, sc = a.scale_log2, vsc_run = 1.f;
    f32x4 acc[8];
    u32x4 qreg[4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i)
        qreg[i] = u32x4{0u, 0u, 0u, 0u};

    int bad_page = 0;

    // ---- loads of one block into a slot ---------------------------------
    // K/V loads are issued for every slot, also past the end of the work or
    // for an empty or invalid slice (then from page 0, which always exists, and
    // never used), so the number of vector loads between any two points of the
    // pipeline is fixed and the wait before each compute covers its own slot only.
    auto issue = [&](Slot &s, Meta &mt) {
        mt = wk.next();
        if (mt.valid && mt.first) {
            // q of (b, g) as the B operand: head = row. Branch-free: rows >= G
            // read head 0 and are zeroed when copied at the segment's first block,
            // so nothing here waits for the load and no divergent control flow
            // separates the scalar bookkeeping of the pipeline.
            const int hrow = row < G ? row : 0;
            const uint16_t *qp = a.q + ((size_t)mt.b * a.Hq + (size_t)mt.g * G + hrow) * D;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int d0 = KVFP8 ? 16 * grp + 64 * (kk >> 1) + 8 * (kk & 1) : 32 * kk + 8 * grp;
                s.q[kk] = *reinterpret_cast<const u32x4 *>(qp + d0);  // zeroed at use
            }
            if (KVFP8) {
                mt.ksc = ldc(a.k_scale, (size_t)mt.b * a.Hkv + mt.g);
                mt.vsc = ldc(a.v_scale, (size_t)mt.b * a.Hkv + mt.g);
            }
        }
        size_t off = (size_t)mt.g * page_head_bytes + (size_t)row * (D * EB);  // page 0
        if (mt.valid && mt.nv > 0) {
            const int page = ldc(a.page_table, (size_t)mt.b * a.pt_stride + mt.tok0 / a.P);
            if (page < 0 || page >= a.num_pages) {
                bad_page = 1;   // reported once at the end of the kernel
                mt.nv = 0;
            } else {
                off = ((size_t)page * a.Hkv + mt.g) * page_head_bytes +
                      (size_t)(mt.tok0 % a.P + row) * (D * EB);
            }
        }
        if (!mt.valid)
            off = (size_t)row * (D * EB);
        const uint8_t *kp = a.k + off;
        const uint8_t *vp = a.v + off;
        if (KVFP8) {
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                s.k[p] = *reinterpret_cast<const u32x4 *>(kp + 16 * grp + 64 * p);
                s.v[p] = *reinterpret_cast<const u32x4 *>(vp + 16 * grp + 64 * p);
            }
        } else {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                s.k[kk] = *reinterpret_cast<const u32x4 *>(kp + 64 * kk + 16 * grp);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                s.v[kk] = *reinterpret_cast<const u32x4 *>(vp + 64 * kk + 16 * grp);
        }
    };

    // ---- end of a segment: merge the 4 waves and write ------------------
    auto finish = [&](const Meta &mt) {
        const float l_tot = xsum4(l_run);
        const float e_tot = xsum4(e_run);
        if (row < G) {
            if (grp == 0) {
                lds_m[wave][row] = m_run;
                lds_l[wave][row] = l_tot;
                lds_e[wave][row] = e_tot;
            }
#pragma unroll
            for (int mb = 0; mb < 8; ++mb) {
                if (KVFP8) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        lds_acc[wave][row][out_dim<1>(mb, 4 * grp + i)] = acc[mb][i];
                } else {
                    *reinterpret_cast<f32x4 *>(&lds_acc[wave][row][16 * mb + 4 * grp]) = acc[mb];
                }
            }
        }
        __syncthreads();
        const int tid = threadIdx.x;
        for (int idx = tid; idx < G * 32; idx += kDecodeThreads) {
            const int h = idx >> 5, d4 = (idx & 31) * 4;
            float M = -INFINITY;
#pragma unroll
            for (int v = 0; v < kWaves; ++v)
                M = fmaxf(M, lds_m[v][h]);
            f32x4 o = {0.f, 0.f, 0.f, 0.f};
            float lse2 = -INFINITY;
            if (M != -INFINITY) {
                float den = 0.f, ex = 0.f;
#pragma unroll
                for (int v = 0; v < kWaves; ++v) {
                    const float e = fast_exp2(lds_m[v][h] - M);
                    den += e * lds_l[v][h];
                    ex += e * lds_e[v][h];
                    const f32x4 x = *reinterpret_cast<const f32x4 *>(&lds_acc[v][h][d4]);
                    o += e * x;
                }
                const float r = vsc_run / den;
                o *= r;
                lse2 = M + log2f(ex);
            }
            const size_t hq = (size_t)mt.b * a.Hq + (size_t)mt.g * G + h;
            if (mt.direct) {
                const bf16x4 ob = __builtin_convertvector(o, bf16x4);
                *reinterpret_cast<bf16x4 *>(a.out + hq * D + d4) = ob;
                if (a.lse && d4 == 0)
                    a.lse[hq] = lse2 * kLn2;
            } else {
                *reinterpret_cast<f32x4 *>(a.part_o + ((size_t)mt.slot * G + h) * D + d4) = o;
                if (d4 == 0)
                    a.part_lse[(size_t)mt.slot * G + h] = lse2;
            }
        }
        __syncthreads();
    };

    // ---- math of one block ----------------------------------------------
    auto compute = [&](Slot &s, const Meta &mt) {
        // Every register of the slot is consumed on every path (q through a
        // select, K/V by the math, which runs even for an empty slice and then
        // contributes nothing), so the compiler's load-wait bookkeeping never
        // sees a load whose registers are reloaded without being waited for.
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            qreg[kk] = mt.first ? (row < G ? s.q[kk] : u32x4{0u, 0u, 0u, 0u}) : qreg[kk];
        if (mt.first) {
            m_run = -INFINITY;
            l_run = 0.f;
            e_run = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            sc = a.scale_log2 * mt.ksc;
            vsc_run = mt.vsc;
        }
        {
            // scores: S^T[token 4*grp+i][head row]
            f32x4 st = {0.f, 0.f, 0.f, 0.f};
            if (KVFP8) {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const uint32_t w0 = s.k[kk >> 1][2 * (kk & 1)];
                    const uint32_t w1 = s.k[kk >> 1][2 * (kk & 1) + 1];
                    const bf16x2 c0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
                    const bf16x2 c1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
                    const bf16x2 c2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
                    const bf16x2 c3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
                    const bf16x8 kv = {c0[0], c0[1], c1[0], c1[1], c2[0], c2[1], c3[0], c3[1]};
                    st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, __builtin_bit_cast(bf16x8, qreg[kk]), st, 0, 0, 0);
                }
            } else {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, s.k[kk]),
                                                                 __builtin_bit_cast(bf16x8, qreg[kk]), st, 0, 0, 0);
            }
            float mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float x = st[i] * sc;
                if (4 * grp + i >= mt.nv)
                    x = -INFINITY;
                st[i] = x;
                mx = fmaxf(mx, x);
            }
            mx = xmax4(mx);
            const float m_new = fmaxf(m_run, mx);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            const float alpha = fast_exp2(m_run - m_use);
            f32x4 p;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                p[i] = fast_exp2(st[i] - m_use);
            const bf16x4 pb = __builtin_convertvector(p, bf16x4);
            const f32x4 pr = __builtin_convertvector(pb, f32x4);
            l_run = l_run * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
            e_run = e_run * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
            m_run = m_new;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                acc[i] *= alpha;
            // rows past the length may hold anything (NaN): zero them
            if (mt.nv < kSlice && row >= mt.nv) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    s.v[i] = u32x4{0u, 0u, 0u, 0u};
            }
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
                for (int ss = 0; ss < 2; ++ss) {
                    f32x4 t;
                    if (KVFP8) {
                        const u32x2 src = {s.v[kk >> 1][2 * (kk & 1)], s.v[kk >> 1][2 * (kk & 1) + 1]};
                        t = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(__builtin_bit_cast(long, src),
                                                                       (long)sel8[ss], zero, 0, 0, 0);
                    } else {
                        t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, s.v[kk]),
                                                                    sel16[ss], zero, 0, 0, 0);
                    }
                    const bf16x4 vt = __builtin_convertvector(t, bf16x4);
                    acc[2 * kk + ss] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, pb, acc[2 * kk + ss], 0, 0, 0);
                }
            }
        }
        if (mt.last)
            finish(mt);
    };

    // ---- software pipeline: two slices in flight per wave ---------------
    // A counted loop (the block count is known from the plan) with both slots
    // handled in every iteration; a trailing invalid block does nothing.
    const int nblk = wk.count_blocks();
    Slot s0, s1;
    Meta m0, m1;
    issue(s0, m0);
    issue(s1, m1);
    for (int it = 0; it < nblk; it += 2) {
        compute(s0, m0);
        issue(s0, m0);
        compute(s1, m1);
        issue(s1, m1);
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
    const int G = a.G;
    constexpr int D = kHeadDim;
    for (int idx = threadIdx.x; idx < G * 32; idx += kDecodeThreads) {
        const int h = idx >> 5, d4 = (idx & 31) * 4;
        float M = -INFINITY;
        for (int s = 0; s < n; ++s)
            M = fmaxf(M, a.part_lse[(size_t)(s0 + s) * G + h]);
        f32x4 o = {0.f, 0.f, 0.f, 0.f};
        float lse2 = -INFINITY;
        if (M != -INFINITY) {
            float den = 0.f;
            for (int s = 0; s < n; ++s) {
                const size_t sl = (size_t)(s0 + s) * G + h;
                const float e = fast_exp2(a.part_lse[sl] - M);
                den += e;
                o += e * *reinterpret_cast<const f32x4 *>(a.part_o + sl * D + d4);
            }
            o *= 1.f / den;
            lse2 = M + log2f(den);
        }
        const size_t hq = (size_t)b * a.Hq + (size_t)g * G + h;
        *reinterpret_cast<bf16x4 *>(a.out + hq * D + d4) = __builtin_convertvector(o, bf16x4);
        if (a.lse && d4 == 0)
            a.lse[hq] = lse2 * kLn2;
    }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, int mode, int kv_fp8, int grid, hipStream_t st)
{
    if (grid <= 0)
        return hipSuccess;
    if (mode == 0 && !kv_fp8)
        hipLaunchKernelGGL((decode_kernel<0, 0>), dim3(grid), dim3(kDecodeThreads), 0, st, a);
    else if (mode == 0)
        hipLaunchKernelGGL((decode_kernel<0, 1>), dim3(grid), dim3(kDecodeThreads), 0, st, a);
    else if (!kv_fp8)
        hipLaunchKernelGGL((decode_kernel<1, 0>), dim3(grid), dim3(kDecodeThreads), 0, st, a);
    else
        hipLaunchKernelGGL((decode_kernel<1, 1>), dim3(grid), dim3(kDecodeThreads), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs &a, hipStream_t st)
{
    const int grid = a.B * a.Hkv;
    if (grid <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(combine_kernel, dim3(grid), dim3(kDecodeThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace vlkv

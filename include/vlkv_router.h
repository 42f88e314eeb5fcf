/*
 * vlkv_router.h — C ABI of the router GEMM with split bf16 weights
 * (libvlkv_attn.so, MI355X / gfx950).
 *
 * The operation. The router of an MoE layer multiplies the layer's activations
 * by a small weight matrix (one row per expert) to score the experts; the
 * source article calls this product precision-sensitive, since small weight
 * errors can change which experts are chosen. Its Router GEMM splits each fp32
 * weight into two bf16 parts, the high part and a residual scaled by 1/256,
 * runs two bf16 tensor-core products in one kernel and combines them, keeping
 * the accumulators in registers and writing the result once [Tencent HPC lands
 * in SGLang, challenging default inference kernels, sec. "Dynamic Attention and
 * Fused MoE target different bottlenecks"]. Here:
 *
 *     w_hi = bf16(w),  w_lo = bf16(256 (w - w_hi))       (round to nearest even)
 *     y[m][e] = sum_k x[m][k] w_hi[e][k] + 2^-8 sum_k x[m][k] w_lo[e][k]
 *
 * with each sum accumulated in fp32 by the matrix cores (bf16 x bf16 products
 * are exact in fp32). |w - (w_hi + w_lo/256)| <= 2^-16 |w|, and a product term
 * goes through at most K + K/256 + 4 fp32 additions (the accumulation in any
 * order, the combine and the sums of a split K), so y differs from the exact
 * fp32-weight product by at most (2^-16 + (K + K/256 + 4) 2^-24) times
 * sum_k |x[m][k] w[e][k]|.
 *
 * Conventions: as in vlkv_attn.h. (device) pointers are HIP device memory,
 * `stream` is a hipStream_t (NULL = null stream), work is only enqueued, the
 * library allocates nothing, and errors return ATTN_ERR_* codes (vlkv_attn.h)
 * with attn_last_error() describing them; nothing is enqueued on error.
 */
#ifndef VLKV_ROUTER_H
#define VLKV_ROUTER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Split n fp32 weights into their bf16 high parts and 256x residuals, a
 * one-time step per weight matrix.
 *   w     (device) fp32 [n]
 *   w_hi  (device) bf16 [n]: bf16(w)
 *   w_lo  (device) bf16 [n]: bf16(256 (w - w_hi))
 * n >= 0; pointers 4-byte aligned. Weights of magnitude near the bf16 overflow
 * threshold are outside the method's range (w_hi rounds to infinity).
 */
int router_split_weights(const float *w, void *w_hi, void *w_lo, int64_t n, void *stream);

/*
 * Workspace bytes router_gemm needs for this shape (0 if none), or 0 for an
 * invalid shape. Host only, pure. The split over K that the library picks for
 * few-token shapes keeps fp32 partials there.
 */
size_t router_workspace_bytes(int32_t M, int32_t K, int32_t E);

/*
 * y = x w^T with the split weights.
 *   M, K, E   tokens (>= 1), hidden size (a positive multiple of 64), experts
 *             (a positive multiple of 16)
 *   x         (device) bf16 [M][K], row-major
 *   w_hi,w_lo (device) bf16 [E][K], row-major (one row per expert), from
 *             router_split_weights
 *   y         (device) fp32 [M][E]
 *   workspace (device) >= router_workspace_bytes(M, K, E) bytes, 256-byte
 *             aligned; may be NULL when that size is 0
 * x, w_hi, w_lo and y 16-byte aligned. The result does not depend on the run:
 * the partial sums of a split K are added in a fixed order.
 */
int router_gemm(int32_t M, int32_t K, int32_t E, const void *x, const void *w_hi, const void *w_lo, float *y,
                void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* VLKV_ROUTER_H */

/*
 * attention_f16.h -- C ABI of the attention forward pass (FlashAttention) in
 * the MI355X (gfx950) library libgemm_f16.so (status codes: gemm_status_t in
 * gemm_f16.h).
 *
 * The operation is the tutorial's fused attention kernel (TileLang news
 * article, paragraph on FlashAttention: query/key/value tiles, no attention
 * matrix in global memory, an online softmax with running maxima, normalising
 * sums and rescale factors, causal and non-causal, checked against PyTorch's
 * scaled dot-product attention; TileLang blog post, "three-piece set" section,
 * item 3):
 *
 *     O[b][h][i][:] = sum_j p_j V[b][h][j][:],
 *     p_j = softmax over the allowed j of  scale * sum_d Q[b][h][i][d] K[b][h][j][d]
 *
 * with the allowed keys j < Nkv, and with causal != 0 also j <= i (the
 * top-left-aligned mask of PyTorch's is_causal).  Products run on fp16 inputs
 * with fp32 accumulation, the softmax state is fp32, and O is rounded to fp16
 * once.
 *
 * Layout: Q and O are [B][H][Nq][D], K and V are [B][H][Nkv][D], all dense
 * row-major fp16 DEVICE pointers, 16-byte aligned.  D must be 64 or 128.  O
 * must not overlap Q, K or V.
 *
 * Ownership and streams: the caller owns every buffer; the call allocates
 * nothing, is asynchronous on `stream` (a hipStream_t, NULL = default stream)
 * and does not synchronise.
 *
 * Errors (nothing is launched on any of them):
 *   GEMM_ERR_INVALID_DIM    a negative size, Nkv == 0 with Nq > 0, a
 *                           non-finite scale, or a (batch, head) K/V slab of
 *                           2 GiB or more
 *   GEMM_ERR_UNSUPPORTED    D other than 64 or 128
 *   GEMM_ERR_NULL_POINTER   a NULL pointer with B * H * Nq > 0
 *   GEMM_ERR_MISALIGNED     a pointer not 16-byte aligned
 *   GEMM_ERR_LAUNCH         the launch failed
 * B, H or Nq == 0 is a successful no-op.
 */
#ifndef ATTENTION_F16_H
#define ATTENTION_F16_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* O = attention(Q, K, V) as above on `stream`; scale is usually 1/sqrt(D).
 * Returns a gemm_status_t.  Same as flash_attn_fwd_f16_kernel with
 * FLASH_ATTN_KERNEL_AUTO. */
int flash_attn_fwd_f16(int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t D,
                       const void* Q, const void* K, const void* V, void* O,
                       int causal, float scale, void* stream);

/* Kernels of the forward pass.  Both form the same fp16 probabilities (the
 * same lazily raised reference maximum, the same fp32 exponent arithmetic);
 * the pipelined kernel adds a block's row sums in another order, so the two
 * agree to fp32 rounding of the normaliser, not bit for bit.  They differ in
 * instruction order:
 *   BLOCK_SERIAL  per 64-key block: scores, softmax, PV product, in turn
 *                 (D = 64 or 128)
 *   PIPELINED     the scores of block j+1 and the PV product of block j run on
 *                 the matrix cores while the same wave computes the softmax of
 *                 its neighbouring blocks (D = 64 or 128)
 *   AUTO          PIPELINED */
enum {
    FLASH_ATTN_KERNEL_AUTO = 0,
    FLASH_ATTN_KERNEL_BLOCK_SERIAL = 1,
    FLASH_ATTN_KERNEL_PIPELINED = 2
};

/* flash_attn_fwd_f16 with the kernel chosen by the caller (for comparisons and
 * tests).  Additional status: GEMM_ERR_NO_CONFIG for an unknown `kernel`. */
int flash_attn_fwd_f16_kernel(int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t D,
                              const void* Q, const void* K, const void* V, void* O,
                              int causal, float scale, int kernel, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTENTION_F16_H */

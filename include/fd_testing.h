/*
 * fd_testing.h - test hooks of the MI355X decode-attention library.  Not
 * for production callers: the entry points of fd.h choose their kernels
 * from the shapes alone, and nothing here changes that.
 */
#ifndef FD_TESTING_H
#define FD_TESTING_H

#include "fd.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Partial kernel of fd_testing_decode_attn. */
#define FD_TESTING_KERNEL_AUTO 0   /* the one fd_decode_attn picks              */
#define FD_TESTING_KERNEL_VALU 1   /* vector-ALU kernel (every supported shape)  */
#define FD_TESTING_KERNEL_MFMA 2   /* matrix-core kernel: bf16 or E4M3, D 128    */

/*
 * fd_testing_decode_attn - fd_decode_attn (and, for dtype FD_FP8_E4M3,
 * fd_decode_attn_fp8 with its k_scale / v_scale) run on the partial kernel
 * named by partial_kernel, so that a test can hold both kernels to the
 * oracle on the shapes both support ([FD] "¿Qué es Flash-Decoding y cuándo
 * acelera los LLMs?", section "Por qué la decodificación necesita otra
 * planificación": any cut of the history into pieces gives the same
 * attention; which kernel computes a piece does not change it either).
 * Arguments, workspace and errors are those of fd_decode_attn; k_scale and
 * v_scale are ignored for other dtypes.  A kernel that does not support the
 * shape returns FD_ERR_UNSUPPORTED; an unknown partial_kernel
 * FD_ERR_INVALID_ARG.
 */
fd_status fd_testing_decode_attn(const void* q, const void* k, const void* v, const float* k_scale,
                                 const float* v_scale, const int32_t* lens, int32_t batch,
                                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int64_t max_len, int32_t dtype, int32_t n_splits, void* out,
                                 int32_t out_dtype, float* lse_out, float scale, void* workspace,
                                 size_t workspace_bytes, void* stream, int32_t partial_kernel);

#ifdef __cplusplus
}
#endif

#endif /* FD_TESTING_H */

/* validate.h -- argument checks of the C ABI; pure host code, no HIP calls. */
#ifndef NG_VALIDATE_H
#define NG_VALIDATE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Returns NG_OK or the first failing ng_status_t, checked in this order:
 * NULL pointers, enums, shapes, eps, 2-byte alignment, output aliasing. */
int ng_validate_gemm(const void *x, const void *gamma, const void *beta, const void *W,
                     const void *bias, const void *y, int64_t M, int64_t N, int64_t K,
                     float eps, int norm, int act, int dtype);

/* As above for the FFN; adds the workspace (size and aliasing) last. */
int ng_validate_ffn(const void *x, const void *gamma, const void *beta, const void *W1,
                    const void *b1, const void *W2, const void *b2, const void *y,
                    int64_t M, int64_t K, int64_t F, int64_t N, float eps, int norm, int act,
                    int dtype, const void *workspace, size_t workspace_bytes);

/* As ng_validate_ffn with W1 [2F, K], b1 [2F] and a 3 M F workspace. */
int ng_validate_gated_ffn(const void *x, const void *gamma, const void *beta, const void *W1,
                          const void *b1, const void *W2, const void *b2, const void *y,
                          int64_t M, int64_t K, int64_t F, int64_t N, float eps, int norm,
                          int act, int dtype, const void *workspace, size_t workspace_bytes);

/* Inference-mode folding: W, W' (Wf) [N,K] of dtype, gamma/beta [K], bias [N]
 * (each optional), c1/c2 [N] fp32; outputs may overlap nothing. */
int ng_validate_fold(const void *W, const void *gamma, const void *beta, const void *bias,
                     const void *Wf, const void *c1, const void *c2, int64_t N, int64_t K,
                     int dtype);

/* The GEMM on folded weights: norm is LayerNorm or RMSNorm (c1 required for
 * LayerNorm, ignored for RMSNorm), c2 required. */
int ng_validate_folded(const void *x, const void *Wf, const void *c1, const void *c2,
                       const void *y, int64_t M, int64_t N, int64_t K, float eps, int norm,
                       int act, int dtype);

/* Post-GEMM normalization: norm is LayerNorm or RMSNorm; bias, gamma, beta
 * [N] optional; the workspace (16-byte aligned) holds at least one fp32 plane
 * of the M x N sums (ng_gemm_norm_workspace_size). */
int ng_validate_gemm_norm(const void *x, const void *W, const void *bias, const void *gamma,
                          const void *beta, const void *y, int64_t M, int64_t N, int64_t K,
                          float eps, int norm, int dtype, const void *workspace,
                          size_t workspace_bytes);
size_t ng_gemm_norm_workspace_size(int64_t M, int64_t N);

/* 1 when every given pointer is 16-byte aligned and K % 8 == 0. */
int ng_vector_ok(int64_t K, const void *a, const void *b, const void *c, const void *d);

size_t ng_ffn_workspace_size(int64_t M, int64_t F, int dtype);
size_t ng_gated_ffn_workspace_size(int64_t M, int64_t F, int dtype);

#ifdef __cplusplus
}
#endif

#endif

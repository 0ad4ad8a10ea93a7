/*
 * norm_gemm.h -- C ABI of the MI355X (gfx950) normalization-prologue GEMM.
 *
 * Operation (page "LayerNorm 融合算子如何让大模型推理再快 15%？深度拆解 ATB 的实现",
 * sections 1.1 and 2.1; page "昇腾CANN的MatMul融合玩法，让大模型推理快3倍",
 * section 二, strategies 1-3):
 *
 *     a[m,:] = norm_affine(x[m,:])          LayerNorm, RMSNorm or none
 *     y[m,n] = act( sum_k a[m,k] * W[n,k] + bias[n] )
 *
 * LayerNorm: a = (x - mean) / sqrt(var + eps) * gamma + beta with the biased
 * variance; RMSNorm: a = x / sqrt(mean(x^2) + eps) * gamma (+ beta if given).
 * Row statistics are reduced in fp32 in one pass (sum and sum of squares of
 * the row shifted by its first element); the normalize + affine runs in fp32
 * and is rounded once (round-to-nearest-even) to the operand type. The
 * normalized activation exists only in on-chip memory and registers: it is
 * never written to device memory. Products accumulate in fp32; the epilogue
 * adds bias, applies the activation in fp32 and rounds once to the output
 * type. The activations are those page "昇腾CANN的MatMul融合玩法…" names for
 * MatMul + activation fusion (section 二 strategy 1: ReLU, GELU, SiLU); the
 * pages define none of them, so the textbook forms are used:
 *     SiLU  z / (1 + exp(-z))
 *     ReLU  max(z, 0)
 *     GELU  z * Phi(z) = z / 2 * (1 + erf(z / sqrt 2))   (exact, not tanh)
 *
 * Conventions for every entry point:
 *  - All tensor pointers are caller-owned DEVICE memory on the current HIP
 *    device, contiguous row-major, one dtype (fp16 or bf16) for x, gamma,
 *    beta, W, bias and y. x is [M,K], W is [N,K] (K contiguous, the "w.T"
 *    convention of the pages), gamma/beta are [K], bias is [N], y is [M,N].
 *  - Pointers must be at least 2-byte aligned; 16-byte aligned pointers with
 *    K % 8 == 0 take 128-bit loads, anything else uses element loads. Any
 *    M, N, K (and F) in [1, 2^31 - 1] is supported. The tiled MFMA kernel
 *    addresses the rows of a tile with 32-bit byte offsets, so it serves
 *    aligned calls with M > 32 only up to K = 8,388,600 (256 rows of K
 *    elements below 2^32 bytes); larger K takes the generic tiled kernel,
 *    which forms 64-bit row addresses. The same bound, on F + 256 rows,
 *    selects the gated FFN's one-kernel phase 1.
 *  - gamma == NULL means gamma = 1; beta == NULL means beta = 0; bias == NULL
 *    means no bias. With norm == NG_NORM_NONE, gamma, beta and eps are ignored.
 *  - y is overwritten, never accumulated into. y must not overlap any input.
 *  - stream is a hipStream_t (NULL = the null stream). Work is enqueued on it
 *    and the call returns without synchronizing. Nothing is allocated. The
 *    only process-wide state is a cache of each device's compute-unit count,
 *    filled on a device's first call and read-only after; calls are
 *    re-entrant and thread-safe.
 *  - On any validation error no kernel is launched and y is untouched. A
 *    launch failure reports NG_ERR_HIP. Faults inside a kernel surface, as in
 *    HIP, at the caller's next synchronization.
 *  - There is no silent fallback to unfused operators: unsupported requests
 *    return an error code.
 */
#ifndef NORM_GEMM_H
#define NORM_GEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NORM_GEMM_ABI_VERSION 5   /* 2: NG_ACT_RELU, NG_ACT_GELU; 3: fused_gated_ffn;
                                     4: fused_ffn_noalloc, NG_ERR_SCRATCH;
                                     5: norm_gemm_fold_weights, fused_norm_gemm_folded,
                                        fused_gemm_norm */

typedef enum { NG_NORM_NONE = 0, NG_NORM_LAYERNORM = 1, NG_NORM_RMSNORM = 2 } ng_norm_t;
typedef enum { NG_ACT_NONE = 0, NG_ACT_SILU = 1, NG_ACT_RELU = 2, NG_ACT_GELU = 3 } ng_act_t;
typedef enum { NG_DTYPE_F16 = 0, NG_DTYPE_BF16 = 1 } ng_dtype_t;

typedef enum {
    NG_OK = 0,
    NG_ERR_NULL = -1,         /* a required pointer is NULL                      */
    NG_ERR_SHAPE = -2,        /* M, N, K or F < 1, or a size overflows int64      */
    NG_ERR_ENUM = -3,         /* norm, act or dtype out of range                  */
    NG_ERR_EPS = -4,          /* eps is NaN, infinite or negative                 */
    NG_ERR_ALIAS = -5,        /* the output overlaps an input (or the workspace) */
    NG_ERR_WORKSPACE = -6,    /* workspace missing or smaller than required       */
    NG_ERR_UNSUPPORTED = -7,  /* no kernel for this request                       */
    NG_ERR_ALIGN = -8,        /* a pointer is not 2-byte aligned                  */
    NG_ERR_HIP = -9,          /* the HIP runtime reported an error                */
    NG_ERR_SCRATCH = -10      /* fused_ffn_noalloc: workspace beyond its scratch   */
} ng_status_t;

/*
 * fused_norm_gemm: y[M,N] = act( norm_affine(x)[M,K] . W[N,K]^T + bias[N] ).
 * M <= 32 runs the skinny (decode) kernel that streams W once, one launch;
 * larger M runs the tiled MFMA kernel, preceded for LayerNorm / RMSNorm by a
 * row-statistics launch on the same stream. Returns an ng_status_t.
 */
int fused_norm_gemm(const void *x, const void *gamma, const void *beta,
                    const void *W, const void *bias, void *y,
                    int64_t M, int64_t N, int64_t K,
                    float eps, int norm, int act, int dtype, void *stream);

/*
 * Fused FFN (page "昇腾CANN的MatMul融合玩法，让大模型推理快3倍", section 二,
 * strategy 2: FFN(x) = MatMul2(SiLU(MatMul1(x)))), with an optional
 * normalization prologue, optional biases and any activation: with LayerNorm,
 * biases and ReLU it is the chain LayerNorm -> MatMul -> BiasAdd -> ReLU ->
 * MatMul -> BiasAdd of page "LayerNorm 融合算子如何让大模型推理再快 15%？深度拆解
 * ATB 的实现", section 3.3:
 *
 *     h[M,F] = act( norm_affine(x)[M,K] . W1[F,K]^T + b1[F] )   (stored as dtype)
 *     y[M,N] = h . W2[N,F]^T + b2[N]
 *
 * h lives in the caller-provided workspace (device memory of at least
 * fused_ffn_workspace_size(M, F, dtype) bytes, 256-byte aligned recommended).
 * A workspace of at least fused_ffn_workspace_size(M, F, dtype) + 8 M N bytes
 * also holds two fp32 partial sums of y: when the second GEMM's 128 x 256
 * tiles (M > 32, aligned) leave compute units idle, its K is then split over
 * two workgroups per tile and the partials are added in a fixed order
 * (deterministic) by a second kernel. Tiles on at most half of the CUs take
 * two equal K ranges; tiles on more than half but not all of them (their
 * column blocks a multiple of 8, as many on each XCD) keep one workgroup per
 * tile that skips one slice of K steps, which the spare CUs compute. Every workspace byte the
 * call may touch is checked against the inputs and y (NG_ERR_ALIAS).
 * All kernels (the statistics pass when normalizing with M > 32, the two
 * GEMMs, the partial sum when K is split) run on `stream`, in order, without
 * synchronizing. The workspace must not overlap
 * any input or y; it may be reused once the call's work has completed on the
 * stream. Returns an ng_status_t.
 */
size_t fused_ffn_workspace_size(int64_t M, int64_t F, int dtype);

int fused_ffn(const void *x, const void *gamma, const void *beta,
              const void *W1, const void *b1, const void *W2, const void *b2,
              void *y, int64_t M, int64_t K, int64_t F, int64_t N,
              float eps, int norm, int act, int dtype,
              void *workspace, size_t workspace_bytes, void *stream);

/*
 * Gated FFN (page "CANN推理加速库ascend-transformer-boost ATB算子融合实战…", Llama2
 * section: the FFN's SwiGLU, a SiLU-gated linear unit, fused with its
 * MatMuls), with the same optional normalization prologue and biases:
 *
 *     a       = norm_affine(x)[M,K]
 *     h[M,F]  = act( a . W_gate^T + b_gate ) * ( a . W_up^T + b_up )   (stored as dtype)
 *     y[M,N]  = h . W2[N,F]^T + b2[N]
 *
 * W1 is [2F, K]: the F gate rows first, then the F up rows (one concatenated
 * projection); b1, when given, is [2F] in the same order. act = SiLU gives
 * SwiGLU. For M > 32 with 16-byte aligned operands and K % 8 == 0, phase 1
 * is one tiled kernel whose tiles hold the gate and up rows of the same
 * output columns, so g and u meet in registers and only h is written; when
 * those 128 x 128-column tiles take more than one round of the compute units
 * and the last round holds at most half of them, each tile of that round is
 * computed as two halves of its K steps whose fp32 sums go to the workspace
 * past h (262144 bytes per tile, within the size below) and a small kernel
 * forms h for those tiles (fixed order, deterministic). Else the [gate | up]
 * projections of every row go to the workspace and a second kernel forms h. The workspace must hold fused_gated_ffn_workspace_size(M,
 * F, dtype) bytes (3 M F elements: h, then the [M, 2F] projections); other
 * conventions as fused_ffn, including the split K of the second GEMM, whose
 * partials (8 M N bytes after the 256-byte-rounded h) fit in this size when
 * 2 N <= F, up to that rounding. Returns an ng_status_t.
 */
size_t fused_gated_ffn_workspace_size(int64_t M, int64_t F, int dtype);

int fused_gated_ffn(const void *x, const void *gamma, const void *beta,
                    const void *W1, const void *b1, const void *W2, const void *b2,
                    void *y, int64_t M, int64_t K, int64_t F, int64_t N,
                    float eps, int norm, int act, int dtype,
                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * Inference-mode folding (page "LayerNorm 融合算子如何让大模型推理再快 15%？深度拆解
 * ATB 的实现", section 6.2, tip 2: at inference gamma and beta are fixed, so
 * gamma is folded once, ahead of time, into the weights of the MatMul that
 * follows). With xhat = (x - mu) rs the row normalized without its affine
 * terms (RMSNorm: mu = 0),
 *     y[m,n] = act( sum_k (xhat_k gamma_k + beta_k) W[n,k] + bias[n] )
 *            = act( rs_m (sum_k x[m,k] W'[n,k] - mu_m c1[n]) + c2[n] )
 *     W'[n,k] = W[n,k] gamma[k],  c1[n] = sum_k W'[n,k],
 *     c2[n]   = sum_k W[n,k] beta[k] + bias[n].
 *
 * norm_gemm_fold_weights: prepares W_folded ([N,K], dtype, each element
 * W[n,k] gamma[k] rounded once), c1 and c2 ([N] fp32; c1 sums the rounded
 * W_folded so that the GEMM's sums centre exactly). gamma == NULL means 1;
 * beta or bias == NULL means 0. All pointers are caller-owned device memory;
 * W_folded, c1 and c2 must not overlap each other or an input (NG_ERR_ALIAS);
 * c1 and c2 4-byte aligned. Reads W once, writes W_folded once, on `stream`.
 *
 * fused_norm_gemm_folded: y = act(rs (x . W_folded^T - mu c1) + c2) for
 * norm = LayerNorm or RMSNorm (NG_ERR_ENUM otherwise) with the row statistics
 * of fused_norm_gemm; x goes to the matrix cores unnormalized, and the
 * statistics and c1, c2 are applied in the epilogue in fp32. c1 is required
 * for LayerNorm and not read for RMSNorm; c2 is required. The GEMM runs on
 * the tiled kernel for any M: x and W_folded must be 16-byte aligned with
 * K % 8 == 0 and K <= 8,388,600, else NG_ERR_UNSUPPORTED. With |mean| >>
 * sigma the difference x . W'^T - mu c1 cancels in fp32; fused_norm_gemm
 * (which centres the row before the product) is the accurate choice there.
 * Other conventions as fused_norm_gemm. Return an ng_status_t.
 */
int norm_gemm_fold_weights(const void *W, const void *gamma, const void *beta,
                           const void *bias, void *W_folded, float *c1, float *c2,
                           int64_t N, int64_t K, int dtype, void *stream);

int fused_norm_gemm_folded(const void *x, const void *W_folded, const float *c1,
                           const float *c2, void *y, int64_t M, int64_t N, int64_t K,
                           float eps, int norm, int act, int dtype, void *stream);

/*
 * Post-GEMM normalization (page "昇腾CANN的MatMul融合玩法，让大模型推理快3倍",
 * section 五, optimization 3: the fused "MatMul(Output)_RMSNorm" of the LLaMA
 * layer, the attention output projection followed by its RMSNorm):
 *
 *     z[m,n] = sum_k x[m,k] W[n,k] + bias[n]
 *     y[m,n] = (z[m,n] - mu_m) / sqrt(var_m + eps) * gamma[n] + beta[n]
 *
 * with the statistics over the N outputs of row m: RMSNorm mu = 0 and var =
 * mean of z^2; LayerNorm the mean and the biased variance (norm = NONE is
 * NG_ERR_ENUM). bias, gamma, beta are [N]; NULL means 0 / 1 / 0. The sums z
 * are kept in fp32 in the workspace (a 16-byte aligned device buffer of at
 * least fused_gemm_norm_workspace_size(M, N) = 4 M N bytes rounded up to 256;
 * twice that lets the GEMM split K over two workgroups per tile when its
 * tiles leave CUs idle, as in fused_ffn); a second kernel adds the bias, takes
 * the row statistics in two passes and writes y rounded once. Two kernels
 * on `stream`, no synchronization. x and W must be 16-byte aligned with K % 8
 * == 0 and K <= 8,388,600 (the tiled kernel, any M), else NG_ERR_UNSUPPORTED.
 * Other conventions as fused_ffn (workspace checked for size and overlaps).
 */
size_t fused_gemm_norm_workspace_size(int64_t M, int64_t N);

int fused_gemm_norm(const void *x, const void *W, const void *bias, const void *gamma,
                    const void *beta, void *y, int64_t M, int64_t N, int64_t K,
                    float eps, int norm, int dtype, void *workspace,
                    size_t workspace_bytes, void *stream);

/*
 * fused_ffn_noalloc: fused_ffn for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation). Same arguments, results and kernels as fused_ffn, without the
 * workspace: h (and, when they fit, the split-K partial sums of y) live in a
 * static device array of NG_FFN_NOALLOC_SCRATCH_BYTES bytes that the library
 * holds on each device it runs on until the process ends. The call allocates
 * nothing and calls no allocating routine; its output equals fused_ffn's
 * with a 256-byte aligned workspace of NG_FFN_NOALLOC_SCRATCH_BYTES bytes.
 * Requests whose h exceeds the array (M * F * 2 bytes, rounded up to 256, >
 * NG_FFN_NOALLOC_SCRATCH_BYTES) return NG_ERR_SCRATCH, checked before any
 * HIP call. All calls on one device share its array: calls that overlap in
 * time on one device (different streams, or threads with no ordering
 * between them) race and give wrong results; calls ordered on one stream are
 * safe. Nothing in the array needs to start at zero (every byte a call
 * reads, it wrote first). Returns an ng_status_t.
 */
#define NG_FFN_NOALLOC_SCRATCH_BYTES (64u << 20) /* 64 MiB per device */

int fused_ffn_noalloc(const void *x, const void *gamma, const void *beta,
                      const void *W1, const void *b1, const void *W2, const void *b2,
                      void *y, int64_t M, int64_t K, int64_t F, int64_t N,
                      float eps, int norm, int act, int dtype, void *stream);

/* Human-readable text of a status code (static storage, never NULL). */
const char *norm_gemm_status_string(int status);

/* NORM_GEMM_ABI_VERSION of the loaded library. */
int norm_gemm_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NORM_GEMM_H */

/*
 * oracle.c -- plain, slow, fp64 CPU reference of the normalization-prologue
 * GEMM and the fused FFN.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this file's library. The GPU path shares
 * no code, header, table or helper with it, and no product code calls it.
 *
 * What it computes is the *unfused* composition the pages define; fusion only
 * changes where intermediates live, so the plain definition is the oracle:
 *
 *   LayerNorm  (page "LayerNorm 融合算子如何让大模型推理再快 15%？深度拆解 ATB
 *              的实现", section 1.1 "LayerNorm的计算流程"): mean and variance
 *              of the row, x_norm = (x - mean) / sqrt(var + eps), then
 *              gamma * x_norm + beta.  Read as the biased (1/K) variance with
 *              eps inside the root, the textbook LayerNorm that the same page
 *              calls through F.layer_norm in section 2.1.
 *   RMSNorm    (page "昇腾CANN的MatMul融合玩法，让大模型推理快3倍", section 二,
 *              strategy 3 "MatMul + 归一化融合"): the pages never write the
 *              formula; read as x / sqrt(mean(x^2) + eps) * gamma (+ beta when
 *              supplied), no mean subtraction.
 *   GEMM       (same page, strategies 1-3): y = a . W^T with W stored [N,K]
 *              and passed as w.T.
 *   bias / act (page 3 above, section 3.3 chain "MatMul -> BiasAdd -> ReLU"):
 *              act(z + bias). The activations are those page 1 names for
 *              MatMul + activation fusion (section 二 strategy 1, and its
 *              table of fused GEMM+ReLU / GELU / SiLU instructions); the pages
 *              define none of them, so the textbook forms are used:
 *              SiLU z * sigmoid(z) = z / (1 + exp(-z)); ReLU max(z, 0);
 *              GELU the exact form z * Phi(z) = z / 2 * (1 + erf(z / sqrt 2)),
 *              Phi the standard normal distribution function.
 *   FFN        (page 1 above, section 二 strategy 2): FFN(x) =
 *              MatMul2(SiLU(MatMul1(x))); page 3's section 3.3 chain
 *              LayerNorm -> MatMul -> BiasAdd -> ReLU -> MatMul -> BiasAdd is
 *              the same composition with a norm prologue, biases and another
 *              activation. The intermediate h is kept in fp64.
 *
 * Every input is the raw 16-bit pattern (IEEE binary16 or bfloat16) that the
 * GPU receives; this file decodes it exactly to double with its own decoder.
 * All arithmetic is double precision, in the order the definition states:
 * two-pass mean/variance, plain left-to-right dot products, no blocking.
 * eps arrives as the float the GPU receives and is widened exactly.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F16 = 0, OR_BF16 = 1 };
enum { OR_NORM_NONE = 0, OR_NORM_LAYERNORM = 1, OR_NORM_RMSNORM = 2 };
enum { OR_ACT_NONE = 0, OR_ACT_SILU = 1, OR_ACT_RELU = 2, OR_ACT_GELU = 3 };
enum { OR_OK = 0, OR_ERR_ARG = -1, OR_ERR_NOMEM = -2 };

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                  /* zero / subnormal: f * 2^-24 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp(1.0 + (double)f / 1024.0, e - 15);
    return sign ? -v : v;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits. */
double oracle_bf16_to_f64(uint16_t b)
{
    int sign = (b >> 15) & 1;
    int e = (b >> 7) & 0xff;
    int f = b & 0x7f;
    double v;
    if (e == 0)
        v = ldexp((double)f, -133);                 /* zero / subnormal: f * 2^-133 */
    else if (e == 255)
        v = f ? NAN : INFINITY;
    else
        v = ldexp(1.0 + (double)f / 128.0, e - 127);
    return sign ? -v : v;
}

static double dec(uint16_t v, int dtype)
{
    return dtype == OR_BF16 ? oracle_bf16_to_f64(v) : oracle_f16_to_f64(v);
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* One row of the normalization prologue, in fp64:
 *   LayerNorm: mu = (1/K) sum x, var = (1/K) sum (x - mu)^2 (two passes),
 *              a = (x - mu) / sqrt(var + eps) * gamma + beta
 *   RMSNorm:   ms = (1/K) sum x^2, a = x / sqrt(ms + eps) * gamma + beta
 *   none:      a = x
 * gamma == NULL means 1, beta == NULL means 0. */
static void normalize_row(const uint16_t *xrow, int64_t K, const uint16_t *gamma,
                          const uint16_t *beta, double eps, int norm, int dtype,
                          double *a)
{
    for (int64_t k = 0; k < K; ++k)
        a[k] = dec(xrow[k], dtype);
    if (norm == OR_NORM_NONE)
        return;
    double r;
    if (norm == OR_NORM_LAYERNORM) {
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k)
            s += a[k];
        double mu = s / (double)K;
        double q = 0.0;
        for (int64_t k = 0; k < K; ++k)
            q += (a[k] - mu) * (a[k] - mu);
        double var = q / (double)K;
        r = 1.0 / sqrt(var + eps);
        for (int64_t k = 0; k < K; ++k)
            a[k] = (a[k] - mu) * r;
    } else {
        double q = 0.0;
        for (int64_t k = 0; k < K; ++k)
            q += a[k] * a[k];
        double ms = q / (double)K;
        r = 1.0 / sqrt(ms + eps);
        for (int64_t k = 0; k < K; ++k)
            a[k] = a[k] * r;
    }
    for (int64_t k = 0; k < K; ++k) {
        double g = gamma ? dec(gamma[k], dtype) : 1.0;
        double b = beta ? dec(beta[k], dtype) : 0.0;
        a[k] = a[k] * g + b;
    }
}

static double apply_act(double z, int act)
{
    if (act == OR_ACT_SILU)
        return z / (1.0 + exp(-z));
    if (act == OR_ACT_RELU)
        return z < 0.0 ? 0.0 : z;
    if (act == OR_ACT_GELU)
        return 0.5 * z * (1.0 + erf(z / sqrt(2.0)));
    return z;
}

static int check_common(int64_t M, int64_t K, int norm, int act, int dtype)
{
    if (M < 1 || K < 1)
        return OR_ERR_ARG;
    if (norm < OR_NORM_NONE || norm > OR_NORM_RMSNORM)
        return OR_ERR_ARG;
    if (act < OR_ACT_NONE || act > OR_ACT_GELU)
        return OR_ERR_ARG;
    if (dtype != OR_F16 && dtype != OR_BF16)
        return OR_ERR_ARG;
    return OR_OK;
}

/* a_out[i, :] = normalized row rows[i] of x (fp64, [n_rows, K]). */
int oracle_normalize(const uint16_t *x, const uint16_t *gamma, const uint16_t *beta,
                     int64_t M, int64_t K, float eps, int norm, int dtype,
                     const int64_t *rows, int64_t n_rows, double *a_out)
{
    if (check_common(M, K, norm, OR_ACT_NONE, dtype) || !x || !rows || !a_out)
        return OR_ERR_ARG;
    for (int64_t i = 0; i < n_rows; ++i)
        if (rows[i] < 0 || rows[i] >= M)
            return OR_ERR_ARG;
    double e = (double)eps;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_rows; ++i)
        normalize_row(x + rows[i] * K, K, gamma, beta, e, norm, dtype, a_out + i * K);
    return OR_OK;
}

/* y_out[i, j] = act( sum_k a[rows[i], k] * W[cols[j], k] + bias[cols[j]] )
 * for a = the normalized x; y_out is fp64 [n_rows, n_cols]. */
int oracle_norm_gemm(const uint16_t *x, const uint16_t *gamma, const uint16_t *beta,
                     const uint16_t *W, const uint16_t *bias, int64_t M, int64_t N,
                     int64_t K, float eps, int norm, int act, int dtype,
                     const int64_t *rows, int64_t n_rows, const int64_t *cols,
                     int64_t n_cols, double *y_out)
{
    if (check_common(M, K, norm, act, dtype) || N < 1 || !x || !W || !rows ||
        !cols || !y_out)
        return OR_ERR_ARG;
    for (int64_t i = 0; i < n_rows; ++i)
        if (rows[i] < 0 || rows[i] >= M)
            return OR_ERR_ARG;
    for (int64_t j = 0; j < n_cols; ++j)
        if (cols[j] < 0 || cols[j] >= N)
            return OR_ERR_ARG;
    if (n_rows == 0 || n_cols == 0)
        return OR_OK;
    double *a = (double *)malloc(sizeof(double) * (size_t)n_rows * (size_t)K);
    if (!a)
        return OR_ERR_NOMEM;
    double e = (double)eps;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_rows; ++i)
        normalize_row(x + rows[i] * K, K, gamma, beta, e, norm, dtype, a + i * K);

    int64_t total = n_rows * n_cols;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t t = 0; t < total; ++t) {
        int64_t i = t / n_cols, j = t % n_cols;
        const double *ar = a + i * K;
        const uint16_t *wr = W + cols[j] * K;
        double z = 0.0;
        for (int64_t k = 0; k < K; ++k)
            z += ar[k] * dec(wr[k], dtype);
        if (bias)
            z += dec(bias[cols[j]], dtype);
        y_out[t] = apply_act(z, act);
    }
    free(a);
    return OR_OK;
}

/* Fused FFN, unfused definition:
 *   h[f]  = act( sum_k a[k] * W1[f, k] + b1[f] )   for every f < F (fp64, not rounded)
 *   y[n]  = sum_f h[f] * W2[n, f] + b2[n]
 * with a = the (optionally) normalized row of x; y_out is fp64 [n_rows, n_cols].
 * Gated (gated != 0; page "CANN推理加速库ascend-transformer-boost ATB算子融合实战…",
 * Llama2 section: the SwiGLU FFN, a SiLU-gated linear unit): W1 is [2F, K],
 * the gate rows first, then the up rows (b1 likewise [2F]), and
 *   h[f]  = act( sum_k a[k] W1[f, k] + b1[f] ) * ( sum_k a[k] W1[F + f, k] + b1[F + f] ) */
static int ffn_impl(const uint16_t *x, const uint16_t *gamma, const uint16_t *beta,
                    const uint16_t *W1, const uint16_t *b1, const uint16_t *W2,
                    const uint16_t *b2, int64_t M, int64_t K, int64_t F, int64_t N,
                    float eps, int norm, int act, int dtype, int gated, const int64_t *rows,
                    int64_t n_rows, const int64_t *cols, int64_t n_cols, double *y_out)
{
    if (check_common(M, K, norm, act, dtype) || F < 1 || N < 1 || !x || !W1 ||
        !W2 || !rows || !cols || !y_out)
        return OR_ERR_ARG;
    for (int64_t i = 0; i < n_rows; ++i)
        if (rows[i] < 0 || rows[i] >= M)
            return OR_ERR_ARG;
    for (int64_t j = 0; j < n_cols; ++j)
        if (cols[j] < 0 || cols[j] >= N)
            return OR_ERR_ARG;
    if (n_rows == 0 || n_cols == 0)
        return OR_OK;
    double *a = (double *)malloc(sizeof(double) * (size_t)K);
    double *h = (double *)malloc(sizeof(double) * (size_t)F);
    if (!a || !h) {
        free(a);
        free(h);
        return OR_ERR_NOMEM;
    }
    double e = (double)eps;
    for (int64_t i = 0; i < n_rows; ++i) {
        normalize_row(x + rows[i] * K, K, gamma, beta, e, norm, dtype, a);
#pragma omp parallel for schedule(dynamic, 16)
        for (int64_t f = 0; f < F; ++f) {
            const uint16_t *wr = W1 + f * K;
            double z = 0.0;
            for (int64_t k = 0; k < K; ++k)
                z += a[k] * dec(wr[k], dtype);
            if (b1)
                z += dec(b1[f], dtype);
            h[f] = apply_act(z, act);
            if (gated) {
                const uint16_t *ur = W1 + (F + f) * K;
                double u = 0.0;
                for (int64_t k = 0; k < K; ++k)
                    u += a[k] * dec(ur[k], dtype);
                if (b1)
                    u += dec(b1[F + f], dtype);
                h[f] *= u;
            }
        }
#pragma omp parallel for schedule(dynamic, 16)
        for (int64_t j = 0; j < n_cols; ++j) {
            const uint16_t *wr = W2 + cols[j] * F;
            double z = 0.0;
            for (int64_t f = 0; f < F; ++f)
                z += h[f] * dec(wr[f], dtype);
            if (b2)
                z += dec(b2[cols[j]], dtype);
            y_out[i * n_cols + j] = z;
        }
    }
    free(a);
    free(h);
    return OR_OK;
}

int oracle_ffn(const uint16_t *x, const uint16_t *gamma, const uint16_t *beta,
               const uint16_t *W1, const uint16_t *b1, const uint16_t *W2,
               const uint16_t *b2, int64_t M, int64_t K, int64_t F, int64_t N,
               float eps, int norm, int act, int dtype, const int64_t *rows,
               int64_t n_rows, const int64_t *cols, int64_t n_cols, double *y_out)
{
    return ffn_impl(x, gamma, beta, W1, b1, W2, b2, M, K, F, N, eps, norm, act, dtype, 0, rows,
                    n_rows, cols, n_cols, y_out);
}

int oracle_gated_ffn(const uint16_t *x, const uint16_t *gamma, const uint16_t *beta,
                     const uint16_t *W1, const uint16_t *b1, const uint16_t *W2,
                     const uint16_t *b2, int64_t M, int64_t K, int64_t F, int64_t N,
                     float eps, int norm, int act, int dtype, const int64_t *rows,
                     int64_t n_rows, const int64_t *cols, int64_t n_cols, double *y_out)
{
    return ffn_impl(x, gamma, beta, W1, b1, W2, b2, M, K, F, N, eps, norm, act, dtype, 1, rows,
                    n_rows, cols, n_cols, y_out);
}

/* Inference-mode folding (page "LayerNorm 融合算子如何让大模型推理再快 15%？深度拆解
 * ATB 的实现", section 6.2, tip 2: in inference gamma and beta are fixed, so
 * gamma is folded once, ahead of time, into the weights of the MatMul that
 * follows, which saves the multiplication after the normalization). The
 * algebra of the unfused definition, with xhat = (x - mu) r (RMSNorm: mu = 0):
 *   z_n = sum_k (xhat_k gamma_k + beta_k) W[n,k] + bias_n
 *       = r (sum_k x_k W'[n,k] - mu c1_n) + c2_n
 *   W'[n,k] = W[n,k] gamma_k,  c1_n = sum_k W'[n,k],
 *   c2_n = sum_k W[n,k] beta_k + bias_n.
 * oracle_fold_weights computes W' (fp64, exact: a product of two 16-bit
 * values), c1 and c2; gamma == NULL means 1, beta or bias == NULL means 0.
 * Wf may be NULL (only c1, c2). */
int oracle_fold_weights(const uint16_t *W, const uint16_t *gamma, const uint16_t *beta,
                        const uint16_t *bias, int64_t N, int64_t K, int dtype, double *Wf,
                        double *c1, double *c2)
{
    if (N < 1 || K < 1 || !W || !c1 || !c2 || (dtype != OR_F16 && dtype != OR_BF16))
        return OR_ERR_ARG;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t n = 0; n < N; ++n) {
        double s1 = 0.0, s2 = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double w = dec(W[n * K + k], dtype);
            double gk = gamma ? dec(gamma[k], dtype) : 1.0;
            double bk = beta ? dec(beta[k], dtype) : 0.0;
            double wf = w * gk;
            if (Wf)
                Wf[n * K + k] = wf;
            s1 += wf;
            s2 += w * bk;
        }
        c1[n] = s1;
        c2[n] = s2 + (bias ? dec(bias[n], dtype) : 0.0);
    }
    return OR_OK;
}

/* y[i, j] = act( r (sum_k x[rows[i], k] Wf[cols[j], k] - mu c1[cols[j]]) + c2[cols[j]] )
 * with the row statistics of the definition (LayerNorm: mean and biased
 * variance, two passes; RMSNorm: mu = 0, r = 1/sqrt(mean(x^2) + eps)), for
 * given folded weights Wf [N,K] and vectors c1, c2 (fp64). With the outputs of
 * oracle_fold_weights it equals oracle_norm_gemm up to fp64 rounding. */
int oracle_norm_gemm_folded(const uint16_t *x, const double *Wf, const double *c1,
                            const double *c2, int64_t M, int64_t N, int64_t K, float eps,
                            int norm, int act, int dtype, const int64_t *rows, int64_t n_rows,
                            const int64_t *cols, int64_t n_cols, double *y_out)
{
    if (check_common(M, K, norm, act, dtype) || N < 1 || norm == OR_NORM_NONE || !x || !Wf ||
        !c1 || !c2 || !rows || !cols || !y_out)
        return OR_ERR_ARG;
    for (int64_t i = 0; i < n_rows; ++i)
        if (rows[i] < 0 || rows[i] >= M)
            return OR_ERR_ARG;
    for (int64_t j = 0; j < n_cols; ++j)
        if (cols[j] < 0 || cols[j] >= N)
            return OR_ERR_ARG;
    const double e = (double)eps;
    int64_t total = n_rows * n_cols;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t t = 0; t < total; ++t) {
        int64_t i = t / n_cols, j = t % n_cols;
        const uint16_t *xr = x + rows[i] * K;
        double mu = 0.0, r;
        if (norm == OR_NORM_LAYERNORM) {
            double s = 0.0, q = 0.0;
            for (int64_t k = 0; k < K; ++k)
                s += dec(xr[k], dtype);
            mu = s / (double)K;
            for (int64_t k = 0; k < K; ++k) {
                double d = dec(xr[k], dtype) - mu;
                q += d * d;
            }
            r = 1.0 / sqrt(q / (double)K + e);
        } else {
            double q = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double v = dec(xr[k], dtype);
                q += v * v;
            }
            r = 1.0 / sqrt(q / (double)K + e);
        }
        const double *wr = Wf + cols[j] * K;
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k)
            acc += dec(xr[k], dtype) * wr[k];
        y_out[t] = apply_act(r * (acc - mu * c1[cols[j]]) + c2[cols[j]], act);
    }
    return OR_OK;
}

/* Post-GEMM normalization (page "昇腾CANN的MatMul融合玩法，让大模型推理快3倍",
 * section 五, optimization 3: the fused "MatMul(Output)_RMSNorm" of the LLaMA
 * layer, the attention output projection followed by the RMSNorm). The pages
 * give no formula; read as the normalization of each output row of the GEMM:
 *   z[m,n] = sum_k x[m,k] W[n,k] + bias[n]
 *   RMSNorm:   y[m,n] = z[m,n] / sqrt(mean_n z[m,n]^2 + eps) * gamma[n] + beta[n]
 *   LayerNorm: y[m,n] = (z[m,n] - mu_m) / sqrt(var_m + eps) * gamma[n] + beta[n]
 *              (mean and biased variance over the N outputs of the row)
 * gamma/beta/bias are [N]; NULL means 1 / 0 / 0. The statistics need every
 * output of a row, so each requested row is computed in full (fp64). */
int oracle_gemm_norm(const uint16_t *x, const uint16_t *W, const uint16_t *bias,
                     const uint16_t *gamma, const uint16_t *beta, int64_t M, int64_t N,
                     int64_t K, float eps, int norm, int dtype, const int64_t *rows,
                     int64_t n_rows, const int64_t *cols, int64_t n_cols, double *y_out)
{
    if (check_common(M, K, norm, OR_ACT_NONE, dtype) || N < 1 || norm == OR_NORM_NONE || !x ||
        !W || !rows || !cols || !y_out)
        return OR_ERR_ARG;
    for (int64_t i = 0; i < n_rows; ++i)
        if (rows[i] < 0 || rows[i] >= M)
            return OR_ERR_ARG;
    for (int64_t j = 0; j < n_cols; ++j)
        if (cols[j] < 0 || cols[j] >= N)
            return OR_ERR_ARG;
    double *z = (double *)malloc(sizeof(double) * (size_t)N);
    if (!z)
        return OR_ERR_NOMEM;
    const double e = (double)eps;
    for (int64_t i = 0; i < n_rows; ++i) {
        const uint16_t *xr = x + rows[i] * K;
#pragma omp parallel for schedule(dynamic, 16)
        for (int64_t n = 0; n < N; ++n) {
            const uint16_t *wr = W + n * K;
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += dec(xr[k], dtype) * dec(wr[k], dtype);
            z[n] = acc + (bias ? dec(bias[n], dtype) : 0.0);
        }
        double mu = 0.0, r;
        if (norm == OR_NORM_LAYERNORM) {
            double sz = 0.0, q = 0.0;
            for (int64_t n = 0; n < N; ++n)
                sz += z[n];
            mu = sz / (double)N;
            for (int64_t n = 0; n < N; ++n)
                q += (z[n] - mu) * (z[n] - mu);
            r = 1.0 / sqrt(q / (double)N + e);
        } else {
            double q = 0.0;
            for (int64_t n = 0; n < N; ++n)
                q += z[n] * z[n];
            r = 1.0 / sqrt(q / (double)N + e);
        }
        for (int64_t j = 0; j < n_cols; ++j) {
            const int64_t n = cols[j];
            double g = gamma ? dec(gamma[n], dtype) : 1.0;
            double b = beta ? dec(beta[n], dtype) : 0.0;
            y_out[i * n_cols + j] = (z[n] - mu) * r * g + b;
        }
    }
    free(z);
    return OR_OK;
}


/* validate.c -- argument checks of the C ABI (pure host code, no HIP). */
#include "validate.h"

#include <math.h>

#include "norm_gemm.h"

/* Kernels index rows and columns with 32-bit ints and offsets with 64 bits. */
#define NG_MAX_DIM ((int64_t)0x7fffffff)

typedef struct {
    uintptr_t lo, hi; /* [lo, hi) */
} range_t;

static range_t rng(const void *p, int64_t elems)
{
    range_t r;
    r.lo = (uintptr_t)p;
    r.hi = p ? r.lo + (uintptr_t)elems * 2u : r.lo;
    return r;
}

static int overlap(range_t a, range_t b)
{
    if (a.lo == a.hi || b.lo == b.hi)
        return 0;
    return a.lo < b.hi && b.lo < a.hi;
}

static int mul_ok(int64_t a, int64_t b)
{
    return a <= (INT64_MAX / 4) / b; /* keeps byte counts of a*b elements in range */
}

static int enums_ok(int norm, int act, int dtype)
{
    return norm >= NG_NORM_NONE && norm <= NG_NORM_RMSNORM && act >= NG_ACT_NONE &&
           act <= NG_ACT_GELU && (dtype == NG_DTYPE_F16 || dtype == NG_DTYPE_BF16);
}

static int dim_ok(int64_t d)
{
    return d >= 1 && d <= NG_MAX_DIM;
}

static int eps_ok(float eps, int norm)
{
    if (norm == NG_NORM_NONE)
        return 1;
    return isfinite(eps) && eps >= 0.0f;
}

static int align2(const void *p)
{
    return ((uintptr_t)p & 1u) == 0;
}

int ng_validate_gemm(const void *x, const void *gamma, const void *beta, const void *W,
                     const void *bias, const void *y, int64_t M, int64_t N, int64_t K,
                     float eps, int norm, int act, int dtype)
{
    if (!x || !W || !y)
        return NG_ERR_NULL;
    if (!enums_ok(norm, act, dtype))
        return NG_ERR_ENUM;
    if (!dim_ok(M) || !dim_ok(N) || !dim_ok(K) || !mul_ok(M, K) || !mul_ok(N, K) ||
        !mul_ok(M, N))
        return NG_ERR_SHAPE;
    if (!eps_ok(eps, norm))
        return NG_ERR_EPS;
    if (!align2(x) || !align2(gamma) || !align2(beta) || !align2(W) || !align2(bias) ||
        !align2(y))
        return NG_ERR_ALIGN;
    range_t ry = rng(y, M * N);
    if (overlap(ry, rng(x, M * K)) || overlap(ry, rng(W, N * K)) ||
        overlap(ry, rng(gamma, K)) || overlap(ry, rng(beta, K)) || overlap(ry, rng(bias, N)))
        return NG_ERR_ALIAS;
    return NG_OK;
}

/* Workspace elements per M * F: h, plus [gate | up] of every row when gated. */
static size_t ffn_workspace(int64_t M, int64_t F, int dtype, int per)
{
    if (M < 1 || F < 1 || (dtype != NG_DTYPE_F16 && dtype != NG_DTYPE_BF16) ||
        !mul_ok(M, F * per))
        return 0;
    size_t bytes = (size_t)M * (size_t)F * (size_t)per * 2u;
    return (bytes + 255u) & ~(size_t)255u;
}

size_t ng_ffn_workspace_size(int64_t M, int64_t F, int dtype)
{
    return ffn_workspace(M, F, dtype, 1);
}

size_t ng_gated_ffn_workspace_size(int64_t M, int64_t F, int dtype)
{
    return F <= NG_MAX_DIM / 2 ? ffn_workspace(M, F, dtype, 3) : 0;
}

/* gated: W1 is [2F, K] and b1 [2F]; the workspace holds 3 M F elements. */
static int validate_ffn(const void *x, const void *gamma, const void *beta, const void *W1,
                        const void *b1, const void *W2, const void *b2, const void *y,
                        int64_t M, int64_t K, int64_t F, int64_t N, float eps, int norm,
                        int act, int dtype, const void *workspace, size_t workspace_bytes,
                        int gated)
{
    const int64_t F1 = gated ? 2 * F : F;     /* rows of W1 */
    if (!x || !W1 || !W2 || !y)
        return NG_ERR_NULL;
    if (!enums_ok(norm, act, dtype))
        return NG_ERR_ENUM;
    if (!dim_ok(M) || !dim_ok(K) || !dim_ok(F) || !dim_ok(N) || (gated && F > NG_MAX_DIM / 2) ||
        !mul_ok(M, K) || !mul_ok(F1, K) || !mul_ok(N, F) || !mul_ok(M, F1 + F) || !mul_ok(M, N))
        return NG_ERR_SHAPE;
    if (!eps_ok(eps, norm))
        return NG_ERR_EPS;
    if (!align2(x) || !align2(gamma) || !align2(beta) || !align2(W1) || !align2(b1) ||
        !align2(W2) || !align2(b2) || !align2(y) || !align2(workspace))
        return NG_ERR_ALIGN;
    range_t in[7] = {rng(x, M * K), rng(gamma, K), rng(beta, K), rng(W1, F1 * K),
                     rng(b1, F1),   rng(W2, N * F), rng(b2, N)};
    range_t ry = rng(y, M * N);
    for (int i = 0; i < 7; ++i)
        if (overlap(ry, in[i]))
            return NG_ERR_ALIAS;
    const size_t need = ffn_workspace(M, F, dtype, gated ? 3 : 1);
    if (!workspace || workspace_bytes < need)
        return NG_ERR_WORKSPACE;
    /* bytes the library may touch: the required size, or h (rounded to 256
     * bytes) followed by two fp32 partial sums of y when the caller's
     * workspace is that large (split K of the second GEMM) */
    size_t touch = need;
    if ((size_t)M * (size_t)N <= (SIZE_MAX / 16u) - ((size_t)M * (size_t)F)) {
        const size_t split = ffn_workspace(M, F, dtype, 1) + 8u * (size_t)M * (size_t)N;
        if (split > touch)
            touch = split <= workspace_bytes ? split : need;
    }
    range_t rw;
    rw.lo = (uintptr_t)workspace;
    rw.hi = rw.lo + touch;
    if (overlap(rw, ry))
        return NG_ERR_ALIAS;
    for (int i = 0; i < 7; ++i)
        if (overlap(rw, in[i]))
            return NG_ERR_ALIAS;
    return NG_OK;
}

int ng_validate_ffn(const void *x, const void *gamma, const void *beta, const void *W1,
                    const void *b1, const void *W2, const void *b2, const void *y,
                    int64_t M, int64_t K, int64_t F, int64_t N, float eps, int norm, int act,
                    int dtype, const void *workspace, size_t workspace_bytes)
{
    return validate_ffn(x, gamma, beta, W1, b1, W2, b2, y, M, K, F, N, eps, norm, act, dtype,
                        workspace, workspace_bytes, 0);
}

int ng_validate_gated_ffn(const void *x, const void *gamma, const void *beta, const void *W1,
                          const void *b1, const void *W2, const void *b2, const void *y,
                          int64_t M, int64_t K, int64_t F, int64_t N, float eps, int norm,
                          int act, int dtype, const void *workspace, size_t workspace_bytes)
{
    return validate_ffn(x, gamma, beta, W1, b1, W2, b2, y, M, K, F, N, eps, norm, act, dtype,
                        workspace, workspace_bytes, 1);
}

int ng_vector_ok(int64_t K, const void *a, const void *b, const void *c, const void *d)
{
    const void *p[4] = {a, b, c, d};
    if (K % 8 != 0)
        return 0;
    for (int i = 0; i < 4; ++i)
        if (p[i] && ((uintptr_t)p[i] & 15u) != 0)
            return 0;
    return 1;
}

static int align4(const void *p)
{
    return ((uintptr_t)p & 3u) == 0;
}

static range_t rng_bytes(const void *p, int64_t bytes)
{
    range_t r;
    r.lo = (uintptr_t)p;
    r.hi = p ? r.lo + (uintptr_t)bytes : r.lo;
    return r;
}

int ng_validate_fold(const void *W, const void *gamma, const void *beta, const void *bias,
                     const void *Wf, const void *c1, const void *c2, int64_t N, int64_t K,
                     int dtype)
{
    if (!W || !Wf || !c1 || !c2)
        return NG_ERR_NULL;
    if (dtype != NG_DTYPE_F16 && dtype != NG_DTYPE_BF16)
        return NG_ERR_ENUM;
    if (!dim_ok(N) || !dim_ok(K) || !mul_ok(N, K))
        return NG_ERR_SHAPE;
    if (!align2(W) || !align2(gamma) || !align2(beta) || !align2(bias) || !align2(Wf) ||
        !align4(c1) || !align4(c2))
        return NG_ERR_ALIGN;
    /* outputs: W', c1, c2; none may overlap an input or another output */
    range_t in[4] = {rng(W, N * K), rng(gamma, K), rng(beta, K), rng(bias, N)};
    range_t out[3] = {rng(Wf, N * K), rng_bytes(c1, N * 4), rng_bytes(c2, N * 4)};
    for (int o = 0; o < 3; ++o) {
        for (int i = 0; i < 4; ++i)
            if (overlap(out[o], in[i]))
                return NG_ERR_ALIAS;
        for (int p = o + 1; p < 3; ++p)
            if (overlap(out[o], out[p]))
                return NG_ERR_ALIAS;
    }
    return NG_OK;
}

int ng_validate_folded(const void *x, const void *Wf, const void *c1, const void *c2,
                       const void *y, int64_t M, int64_t N, int64_t K, float eps, int norm,
                       int act, int dtype)
{
    if (!x || !Wf || !c2 || !y || (norm == NG_NORM_LAYERNORM && !c1))
        return NG_ERR_NULL;
    /* folding is a normalization strategy: LayerNorm or RMSNorm only */
    if (!enums_ok(norm, act, dtype) || norm == NG_NORM_NONE)
        return NG_ERR_ENUM;
    if (!dim_ok(M) || !dim_ok(N) || !dim_ok(K) || !mul_ok(M, K) || !mul_ok(N, K) ||
        !mul_ok(M, N))
        return NG_ERR_SHAPE;
    if (!eps_ok(eps, norm))
        return NG_ERR_EPS;
    if (!align2(x) || !align2(Wf) || !align2(y) || !align4(c1) || !align4(c2))
        return NG_ERR_ALIGN;
    range_t ry = rng(y, M * N);
    if (overlap(ry, rng(x, M * K)) || overlap(ry, rng(Wf, N * K)) ||
        overlap(ry, rng_bytes(norm == NG_NORM_LAYERNORM ? c1 : 0, N * 4)) ||
        overlap(ry, rng_bytes(c2, N * 4)))
        return NG_ERR_ALIAS;
    return NG_OK;
}

size_t ng_gemm_norm_workspace_size(int64_t M, int64_t N)
{
    if (!dim_ok(M) || !dim_ok(N) || !mul_ok(M, N) || (size_t)M * (size_t)N > SIZE_MAX / 8u)
        return 0;
    return (((size_t)M * (size_t)N * 4u) + 255u) & ~(size_t)255u;
}

int ng_validate_gemm_norm(const void *x, const void *W, const void *bias, const void *gamma,
                          const void *beta, const void *y, int64_t M, int64_t N, int64_t K,
                          float eps, int norm, int dtype, const void *workspace,
                          size_t workspace_bytes)
{
    if (!x || !W || !y)
        return NG_ERR_NULL;
    if (!enums_ok(norm, NG_ACT_NONE, dtype) || norm == NG_NORM_NONE)
        return NG_ERR_ENUM;
    if (!dim_ok(M) || !dim_ok(N) || !dim_ok(K) || !mul_ok(M, K) || !mul_ok(N, K) ||
        !mul_ok(M, N))
        return NG_ERR_SHAPE;
    if (!eps_ok(eps, norm))
        return NG_ERR_EPS;
    if (!align2(x) || !align2(W) || !align2(bias) || !align2(gamma) || !align2(beta) ||
        !align2(y) || ((uintptr_t)workspace & 15u) != 0)
        return NG_ERR_ALIGN;
    range_t in[5] = {rng(x, M * K), rng(W, N * K), rng(bias, N), rng(gamma, N), rng(beta, N)};
    range_t ry = rng(y, M * N);
    for (int i = 0; i < 5; ++i)
        if (overlap(ry, in[i]))
            return NG_ERR_ALIAS;
    const size_t need = ng_gemm_norm_workspace_size(M, N);
    if (!workspace || need == 0 || workspace_bytes < need)
        return NG_ERR_WORKSPACE;
    /* bytes the library may touch: one fp32 plane of the sums, or two when
     * the workspace holds them (split K) */
    const size_t touch = workspace_bytes >= 2u * need ? 2u * need : need;
    range_t rw = rng_bytes(workspace, (int64_t)touch);
    if (overlap(rw, ry))
        return NG_ERR_ALIAS;
    for (int i = 0; i < 5; ++i)
        if (overlap(rw, in[i]))
            return NG_ERR_ALIAS;
    return NG_OK;
}

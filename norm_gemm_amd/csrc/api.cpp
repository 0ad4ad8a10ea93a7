// api.cpp -- the extern "C" entry points declared in include/norm_gemm.h:
// validate (pure host code), pick the kernel, launch on the caller's stream.
#include <hip/hip_runtime.h>

#include <atomic>

#include "launch.h"
#include "norm_gemm.h"
#include "route.h"
#include "validate.h"

namespace ng {

// Workspace of fused_ffn_noalloc: one array per device, held until the
// process ends. Host code never uses this name as an address (in host code it
// is a stand-in symbol); it uses the device address that scratch_ptr() takes
// once per device with hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[NG_FFN_NOALLOC_SCRATCH_BYTES];

// Device address of this device's scratch array, taken on the device's first
// call with that device current, or nullptr when the query fails.
void *scratch_ptr()
{
    constexpr int kMaxDev = 64;
    static std::atomic<void *> ptrs[kMaxDev];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev)
        return nullptr;
    void *p = ptrs[dev].load(std::memory_order_acquire);
    if (p)
        return p;
    void *q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q)
        return nullptr;
    ptrs[dev].store(q, std::memory_order_release);
    return q;
}

int cu_count()
{
    // one entry per device ordinal; filled on first use, read-only after
    constexpr int kMaxDev = 64;
    static std::atomic<int> cache[kMaxDev];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return 256;
    int c = (dev >= 0 && dev < kMaxDev) ? cache[dev].load(std::memory_order_relaxed) : 0;
    if (c > 0)
        return c;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c < 1)
        c = 256;
    if (dev >= 0 && dev < kMaxDev)
        cache[dev].store(c, std::memory_order_relaxed);
    return c;
}

}  // namespace ng

namespace {

ng::GemmArgs make_args(const void *x, const void *gamma, const void *beta, const void *W,
                       const void *bias, void *y, int64_t M, int64_t N, int64_t K, float eps,
                       int norm, int act, int dtype)
{
    ng::GemmArgs a;
    a.x = x;
    a.gamma = norm == NG_NORM_NONE ? nullptr : gamma;
    a.beta = norm == NG_NORM_NONE ? nullptr : beta;
    a.W = W;
    a.bias = bias;
    a.y = y;
    a.M = M;
    a.N = N;
    a.K = K;
    a.eps = eps;
    a.norm = norm;
    a.act = act;
    a.dtype = dtype;
    a.vec = ng_vector_ok(K, x, W, a.gamma, a.beta) != 0;
    return a;
}

// 256 x 192 tiles for normalizing calls when they fit the request and move
// fewer bytes per CU than 128 x 256 tiles, and y can hold the statistics
// records (N % 8 == 0, 16-byte aligned rows)
bool wide_tiles(const ng::GemmArgs &a)
{
    return a.norm != NG_NORM_NONE && !a.c2 && a.N % 8 == 0 && ((uintptr_t)a.y & 15u) == 0 &&
           ng_wide_tiles_fit(a.M, a.N, a.K, a.vec ? 1 : 0) &&
           ng_wide_tiles_pay(a.M, a.N, ng::cu_count());
}

int run(const ng::GemmArgs &a, hipStream_t s)
{
    hipError_t e;
    switch (ng_route_gemm(a.M, a.N, a.K, a.vec ? 1 : 0, ng::cu_count())) {
    case NG_ROUTE_DECODE_ELEM: e = ng::launch_decode(a, s); break;
    case NG_ROUTE_DECODE_WIDE: e = ng::launch_decode_wide(a, s); break;
    case NG_ROUTE_DECODE_LDS: e = ng::launch_decode_lds(a, s); break;
    case NG_ROUTE_PREFILL_LDS:
        e = wide_tiles(a) ? ng::launch_prefill_wide(a, s) : ng::launch_prefill_lds(a, s);
        break;
    default: e = ng::launch_prefill(a, s); break;
    }
    return e == hipSuccess ? NG_OK : NG_ERR_HIP;
}

// Second GEMM of an FFN: y = h . W2^T + b2. When the workspace past h holds
// two fp32 partial sums of y and the tiles leave CUs idle, K is split over
// two workgroups per tile (tiles on at most half of the CUs: two equal
// ranges; on more than half: the skipped-slice schedule of
// ng_skip_slice_plan), and the two partials are added in a fixed order by a
// second kernel.
int ffn_down(const void *h, const void *W2, const void *b2, void *y, int64_t M, int64_t F,
             int64_t N, int dtype, void *workspace, size_t workspace_bytes, hipStream_t s)
{
    const ng::GemmArgs a = make_args(h, nullptr, nullptr, W2, b2, y, M, N, F, 0.0f,
                                     NG_NORM_NONE, NG_ACT_NONE, dtype);
    const int cus = ng::cu_count();
    const size_t hbytes = (((size_t)M * (size_t)F * 2u) + 255u) & ~(size_t)255u;
    const size_t pbytes = 2u * (size_t)M * (size_t)N * 4u;
    char *part = (char *)workspace + hbytes;
    if (ng_route_gemm(M, N, F, a.vec ? 1 : 0, cus) == NG_ROUTE_PREFILL_LDS &&
        workspace_bytes >= hbytes + pbytes && ((uintptr_t)part & 15u) == 0) {
        hipError_t e = hipErrorInvalidValue;
        if (2 * ng::prefill_tiles(M, N) <= cus && ng::prefill_k_steps(F) >= 4)
            e = ng::launch_prefill_lds_splitk(a, (float *)part, 2, s);
        else if (ng_skip_slice_plan(M, N, F, cus, nullptr, nullptr))
            e = ng::launch_prefill_lds_skip_slice(a, (float *)part, s);
        else
            return run(a, s);
        if (e != hipSuccess ||
            ng::launch_splitk_sum((const float *)part, b2, y, M, N, 2, NG_ACT_NONE, dtype, s) !=
                hipSuccess)
            return NG_ERR_HIP;
        return NG_OK;
    }
    return run(a, s);
}

}  // namespace

extern "C" {

int fused_norm_gemm(const void *x, const void *gamma, const void *beta, const void *W,
                    const void *bias, void *y, int64_t M, int64_t N, int64_t K, float eps,
                    int norm, int act, int dtype, void *stream)
{
    int st = ng_validate_gemm(x, gamma, beta, W, bias, y, M, N, K, eps, norm, act, dtype);
    if (st != NG_OK)
        return st;
    return run(make_args(x, gamma, beta, W, bias, y, M, N, K, eps, norm, act, dtype),
               (hipStream_t)stream);
}

size_t fused_ffn_workspace_size(int64_t M, int64_t F, int dtype)
{
    return ng_ffn_workspace_size(M, F, dtype);
}

int fused_ffn(const void *x, const void *gamma, const void *beta, const void *W1,
              const void *b1, const void *W2, const void *b2, void *y, int64_t M, int64_t K,
              int64_t F, int64_t N, float eps, int norm, int act, int dtype, void *workspace,
              size_t workspace_bytes, void *stream)
{
    int st = ng_validate_ffn(x, gamma, beta, W1, b1, W2, b2, y, M, K, F, N, eps, norm, act,
                             dtype, workspace, workspace_bytes);
    if (st != NG_OK)
        return st;
    hipStream_t s = (hipStream_t)stream;
    // phase 1: h = act(norm_affine(x) . W1^T + b1), kept in the workspace
    st = run(make_args(x, gamma, beta, W1, b1, workspace, M, F, K, eps, norm, act, dtype), s);
    if (st != NG_OK)
        return st;
    // phase 2: y = h . W2^T + b2
    return ffn_down(workspace, W2, b2, y, M, F, N, dtype, workspace, workspace_bytes, s);
}

int fused_ffn_noalloc(const void *x, const void *gamma, const void *beta, const void *W1,
                      const void *b1, const void *W2, const void *b2, void *y, int64_t M,
                      int64_t K, int64_t F, int64_t N, float eps, int norm, int act, int dtype,
                      void *stream)
{
    // every argument check that needs no device first: with no workspace
    // the FFN validation fails last, on the workspace, if all else is valid
    int st = ng_validate_ffn(x, gamma, beta, W1, b1, W2, b2, y, M, K, F, N, eps, norm, act,
                             dtype, nullptr, 0);
    if (st != NG_ERR_WORKSPACE)
        return st == NG_OK ? NG_ERR_WORKSPACE : st;
    if (ng_ffn_workspace_size(M, F, dtype) > (size_t)NG_FFN_NOALLOC_SCRATCH_BYTES)
        return NG_ERR_SCRATCH;
    void *ws = ng::scratch_ptr();
    if (!ws)
        return NG_ERR_HIP;
    return fused_ffn(x, gamma, beta, W1, b1, W2, b2, y, M, K, F, N, eps, norm, act, dtype, ws,
                     (size_t)NG_FFN_NOALLOC_SCRATCH_BYTES, stream);
}

int norm_gemm_fold_weights(const void *W, const void *gamma, const void *beta, const void *bias,
                           void *W_folded, float *c1, float *c2, int64_t N, int64_t K, int dtype,
                           void *stream)
{
    int st = ng_validate_fold(W, gamma, beta, bias, W_folded, c1, c2, N, K, dtype);
    if (st != NG_OK)
        return st;
    const bool vec = ng_vector_ok(K, W, gamma, beta, W_folded) != 0;
    return ng::launch_fold(W, gamma, beta, bias, W_folded, c1, c2, N, K, dtype, vec,
                           (hipStream_t)stream) == hipSuccess
               ? NG_OK
               : NG_ERR_HIP;
}

int fused_norm_gemm_folded(const void *x, const void *W_folded, const float *c1, const float *c2,
                           void *y, int64_t M, int64_t N, int64_t K, float eps, int norm, int act,
                           int dtype, void *stream)
{
    int st = ng_validate_folded(x, W_folded, c1, c2, y, M, N, K, eps, norm, act, dtype);
    if (st != NG_OK)
        return st;
    ng::GemmArgs a = make_args(x, nullptr, nullptr, W_folded, nullptr, y, M, N, K, eps, norm,
                               act, dtype);
    a.c1 = norm == NG_NORM_LAYERNORM ? c1 : nullptr;
    a.c2 = c2;
    // the tiled kernel with 32-bit tile offsets, for any M
    if (ng_route_gemm(NG_DECODE_MAX_M + 1, N, K, a.vec ? 1 : 0, ng::cu_count()) !=
        NG_ROUTE_PREFILL_LDS)
        return NG_ERR_UNSUPPORTED;
    return ng::launch_prefill_lds_folded(a, (hipStream_t)stream) == hipSuccess ? NG_OK
                                                                               : NG_ERR_HIP;
}

size_t fused_gemm_norm_workspace_size(int64_t M, int64_t N)
{
    return ng_gemm_norm_workspace_size(M, N);
}

int fused_gemm_norm(const void *x, const void *W, const void *bias, const void *gamma,
                    const void *beta, void *y, int64_t M, int64_t N, int64_t K, float eps,
                    int norm, int dtype, void *workspace, size_t workspace_bytes, void *stream)
{
    int st = ng_validate_gemm_norm(x, W, bias, gamma, beta, y, M, N, K, eps, norm, dtype,
                                   workspace, workspace_bytes);
    if (st != NG_OK)
        return st;
    const ng::GemmArgs a = make_args(x, nullptr, nullptr, W, nullptr, y, M, N, K, 0.0f,
                                     NG_NORM_NONE, NG_ACT_NONE, dtype);
    // the tiled kernel writes the fp32 sums, for any M
    if (ng_route_gemm(NG_DECODE_MAX_M + 1, N, K, a.vec ? 1 : 0, ng::cu_count()) !=
        NG_ROUTE_PREFILL_LDS)
        return NG_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    // K split over two workgroups per tile when the workspace holds two
    // planes and the tiles leave CUs idle: two equal ranges when the tiles
    // fill at most half of the CUs, else the skipped-slice schedule
    const size_t plane = ng_gemm_norm_workspace_size(M, N);
    const int cus = ng::cu_count();
    const bool two = workspace_bytes >= 2 * plane;
    const bool halves = two && 2 * ng::prefill_tiles(M, N) <= cus && ng::prefill_k_steps(K) >= 4;
    const bool skip = two && !halves && ng_skip_slice_plan(M, N, K, cus, nullptr, nullptr);
    const int ksplit = halves || skip ? 2 : 1;
    // the planes are M N floats apart: with ksplit 2 the partial of part s
    // starts at s M N (the sum kernel's layout), inside the two planes
    const hipError_t e = skip ? ng::launch_prefill_lds_skip_slice(a, (float *)workspace, s)
                              : ng::launch_prefill_lds_splitk(a, (float *)workspace, ksplit, s);
    if (e != hipSuccess ||
        ng::launch_postnorm((const float *)workspace, bias, gamma, beta, y, M, N, ksplit, eps,
                            norm, dtype, s) != hipSuccess)
        return NG_ERR_HIP;
    return NG_OK;
}

size_t fused_gated_ffn_workspace_size(int64_t M, int64_t F, int dtype)
{
    return ng_gated_ffn_workspace_size(M, F, dtype);
}

int fused_gated_ffn(const void *x, const void *gamma, const void *beta, const void *W1,
                    const void *b1, const void *W2, const void *b2, void *y, int64_t M,
                    int64_t K, int64_t F, int64_t N, float eps, int norm, int act, int dtype,
                    void *workspace, size_t workspace_bytes, void *stream)
{
    int st = ng_validate_gated_ffn(x, gamma, beta, W1, b1, W2, b2, y, M, K, F, N, eps, norm,
                                   act, dtype, workspace, workspace_bytes);
    if (st != NG_OK)
        return st;
    hipStream_t s = (hipStream_t)stream;
    char *h = (char *)workspace;
    // phase 1: h = act(a . W_gate^T + b_gate) * (a . W_up^T + b_up)
    ng::GemmArgs a = make_args(x, gamma, beta, W1, b1, h, M, F, K, eps, norm, act, dtype);
    if (ng_gated_tiled_fits(M, F, K, a.vec ? 1 : 0)) {
        // the [gate | up] area past h (unused by the tiled kernel, and inside
        // the size the validation checked) holds the partial sums of the
        // last round's split tiles, if any
        const size_t hbytes = (((size_t)M * (size_t)F * 2u) + 255u) & ~(size_t)255u;
        const size_t need = ng_gated_ffn_workspace_size(M, F, dtype);
        if (need > hbytes) {
            a.part = (float *)((char *)workspace + hbytes);
            a.part_bytes = need - hbytes;
        }
        if (ng::launch_prefill_lds_gated(a, s) != hipSuccess)
            return NG_ERR_HIP;
    } else {
        // the [gate | up] projections of every row, then the gating
        void *gu = h + (size_t)M * (size_t)F * 2u;
        st = run(make_args(x, gamma, beta, W1, b1, gu, M, 2 * F, K, eps, norm, NG_ACT_NONE,
                           dtype),
                 s);
        if (st != NG_OK)
            return st;
        if (ng::launch_gate(gu, h, M, F, act, dtype, s) != hipSuccess)
            return NG_ERR_HIP;
    }
    // phase 2: y = h . W2^T + b2 (the [gate | up] area is free by now)
    return ffn_down(h, W2, b2, y, M, F, N, dtype, workspace, workspace_bytes, s);
}

const char *norm_gemm_status_string(int status)
{
    switch (status) {
    case NG_OK: return "ok";
    case NG_ERR_NULL: return "a required pointer is NULL";
    case NG_ERR_SHAPE: return "invalid shape (M, N, K and F must be in [1, 2^31-1])";
    case NG_ERR_ENUM: return "norm, act or dtype out of range";
    case NG_ERR_EPS: return "eps must be finite and >= 0";
    case NG_ERR_ALIAS: return "the output overlaps an input or the workspace";
    case NG_ERR_WORKSPACE: return "workspace missing or too small";
    case NG_ERR_UNSUPPORTED: return "unsupported request";
    case NG_ERR_ALIGN: return "a pointer is not 2-byte aligned";
    case NG_ERR_HIP: return "HIP runtime error";
    case NG_ERR_SCRATCH:
        return "the request needs more workspace than the allocation-free entry point's "
               "static scratch holds (M * F * 2 bytes, rounded up to 256, at most "
               "NG_FFN_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
    }
}

int norm_gemm_abi_version(void)
{
    return NORM_GEMM_ABI_VERSION;
}

}  // extern "C"

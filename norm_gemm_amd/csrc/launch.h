// launch.h -- host-side launch descriptor shared by the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "route.h"

namespace ng {

// One validated GEMM request; pointers are device addresses.
struct GemmArgs {
    const void *x, *gamma, *beta, *W, *bias;
    void *y;
    int64_t M, N, K;
    float eps;
    int norm, act, dtype;
    bool vec;  // K % 8 == 0 and x, W, gamma, beta 16-byte aligned
    // inference-mode folding: W holds W' = W * gamma; c1 = W' 1, c2 = W beta + bias
    const float *c1 = nullptr, *c2 = nullptr;
    // gated calls: device scratch (16-byte aligned) for the fp32 partial sums
    // of the last round's tiles when their K is split (ng_gated_split_tiles)
    float *part = nullptr;
    size_t part_bytes = 0;
};

hipError_t launch_prefill(const GemmArgs &a, hipStream_t s);      // any alignment
hipError_t launch_prefill_lds(const GemmArgs &a, hipStream_t s);  // route NG_ROUTE_PREFILL_LDS
hipError_t launch_decode(const GemmArgs &a, hipStream_t s);      // any alignment
hipError_t launch_decode_lds(const GemmArgs &a, hipStream_t s);  // a.vec only
hipError_t launch_decode_wide(const GemmArgs &a, hipStream_t s); // route NG_ROUTE_DECODE_WIDE
// gated tiled kernel: a.W = [W_gate; W_up] is [2 a.N, a.K], a.bias [2 a.N]
// (only when ng_gated_tiled_fits)
hipError_t launch_prefill_lds_gated(const GemmArgs &a, hipStream_t s);
// 256 x 192 tiles for normalizing calls (ng_wide_tiles_fit, no folded
// weights, N % 8 == 0 and a 16-byte aligned y for the statistics records)
hipError_t launch_prefill_wide(const GemmArgs &a, hipStream_t s);
// row statistics (rs, -mu rs) into the first 8 bytes of each row's slice of
// every tw-column tile of y (tn tiles per row)
hipError_t launch_row_stats_to_y(const void *x, void *y, int64_t M, int64_t N, int64_t K,
                                 float eps, int norm, int tn, int tw, int dtype, hipStream_t s);
// folded weights (a.W = W', a.c1, a.c2; route NG_ROUTE_PREFILL_LDS for any M)
hipError_t launch_prefill_lds_folded(const GemmArgs &a, hipStream_t s);
// W' = W * gamma, c1 = W' 1, c2 = W beta + bias (one workgroup per row of W)
hipError_t launch_fold(const void *W, const void *gamma, const void *beta, const void *bias,
                       void *Wf, float *c1, float *c2, int64_t N, int64_t K, int dtype, bool vec,
                       hipStream_t s);
// split K of the plain tiled GEMM (a.vec, no normalization): fp32 partials
// part[ksplit][M][N] (ksplit >= 1), then y = act(sum of the partials + bias)
int prefill_tiles(int64_t M, int64_t N);
int prefill_k_steps(int64_t K);
hipError_t launch_prefill_lds_splitk(const GemmArgs &a, float *part, int ksplit, hipStream_t s);
// Plain GEMM on the skipped-slice schedule of ng_skip_slice_plan (fp32
// partials of the two parts of every tile in planes 0 and 1 of part, M N
// floats apart); hipErrorInvalidValue when the plan does not apply.
hipError_t launch_prefill_lds_skip_slice(const GemmArgs &a, float *part, hipStream_t s);
hipError_t launch_splitk_sum(const float *part, const void *bias, void *y, int64_t M, int64_t N,
                             int ksplit, int act, int dtype, hipStream_t s);
// y = norm_affine(sum of the partials + bias) over each output row
hipError_t launch_postnorm(const float *part, const void *bias, const void *gamma,
                           const void *beta, void *y, int64_t M, int64_t N, int ksplit, float eps,
                           int norm, int dtype, hipStream_t s);
// h[M, F] = act(gu[:, :F]) * gu[:, F:] for gu[M, 2F]
hipError_t launch_gate(const void *gu, void *h, int64_t M, int64_t F, int act, int dtype,
                       hipStream_t s);

constexpr int64_t kDecodeMaxM = NG_DECODE_MAX_M;

// Compute units of the current device, queried once per device and cached
// (256 if the query fails).
int cu_count();

}  // namespace ng

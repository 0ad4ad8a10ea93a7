// postnorm.hip -- the normalization of a GEMM's output rows (page
// "昇腾CANN的MatMul融合玩法，让大模型推理快3倍", section 五, optimization 3:
// the fused "MatMul(Output)_RMSNorm" of the LLaMA layer):
//
//     z[m,n] = sum_k x[m,k] W[n,k] + bias[n]
//     y[m,n] = (z[m,n] - mu_m) * rs_m * gamma[n] + beta[n]
//
// with rs_m = 1/sqrt(var_m + eps) over the N outputs of row m (RMSNorm:
// mu = 0, var = mean of z^2). The statistics need every output of a row,
// which the GEMM's tiles produce on different workgroups, so the tiled kernel
// writes its fp32 sums (per K range when K is split) to a workspace and this
// kernel finishes each row: it adds the K ranges and the bias in a fixed
// order, takes the mean and the variance in two passes over the row (fp32;
// the row is re-read from L2), and writes y rounded once. z never exists in
// the output type, so the normalization sees the unrounded sums.
#include "device_common.h"
#include "launch.h"

namespace ng {
namespace {

constexpr int PN_THREADS = 256;

// sum over this thread's columns of f(z[n]) for the row, then over the
// workgroup in a fixed order (lane, wave): deterministic
__device__ __forceinline__ float block_sum(float v, float *red)
{
    v = wave_sum(v);
    const int tid = threadIdx.x;
    __syncthreads();                      // red may still be read by a previous sum
    if ((tid & 63) == 0)
        red[tid >> 6] = v;
    __syncthreads();
    return ((red[0] + red[1]) + red[2]) + red[3];
}

template <int DT>
__global__ __launch_bounds__(PN_THREADS) void postnorm_kernel(
    const float *__restrict__ part, const uint16_t *__restrict__ bias,
    const uint16_t *__restrict__ gamma, const uint16_t *__restrict__ beta,
    uint16_t *__restrict__ y, int64_t M, int N, int ksplit, float eps, int norm)
{
    __shared__ float red[PN_THREADS / 64];
    const int64_t m = blockIdx.x;
    const int64_t plane = M * (int64_t)N;
    const float *row = part + m * N;
    auto z = [&](int n) {
        float v = row[n];
        for (int s = 1; s < ksplit; ++s)
            v += row[(int64_t)s * plane + n];
        return bias ? v + bits_to_f<DT>(bias[n]) : v;
    };
    const float invN = 1.0f / (float)N;
    float mu = 0.0f, var;
    if (norm == NORM_LAYERNORM) {
        float s1 = 0.0f;
        for (int n = threadIdx.x; n < N; n += PN_THREADS)
            s1 += z(n);
        mu = block_sum(s1, red) * invN;
        float s2 = 0.0f;
        for (int n = threadIdx.x; n < N; n += PN_THREADS) {
            const float d = z(n) - mu;
            s2 = fmaf(d, d, s2);
        }
        var = block_sum(s2, red) * invN;
    } else {
        float s2 = 0.0f;
        for (int n = threadIdx.x; n < N; n += PN_THREADS) {
            const float v = z(n);
            s2 = fmaf(v, v, s2);
        }
        var = block_sum(s2, red) * invN;
    }
    const float rs = rsqrtf(var + eps);
    uint16_t *yr = y + m * N;
    for (int n = threadIdx.x; n < N; n += PN_THREADS) {
        float v = (z(n) - mu) * rs;
        if (gamma)
            v *= bits_to_f<DT>(gamma[n]);
        if (beta)
            v += bits_to_f<DT>(beta[n]);
        yr[n] = f_to_bits<DT>(v);
    }
}

}  // namespace

hipError_t launch_postnorm(const float *part, const void *bias, const void *gamma,
                           const void *beta, void *y, int64_t M, int64_t N, int ksplit, float eps,
                           int norm, int dtype, hipStream_t s)
{
#define NG_PN_ARGS                                                                           \
    part, (const uint16_t *)bias, (const uint16_t *)gamma, (const uint16_t *)beta,           \
        (uint16_t *)y, M, (int)N, ksplit, eps, norm
    if (dtype == DT_F16)
        hipLaunchKernelGGL((postnorm_kernel<DT_F16>), dim3((unsigned)M), dim3(PN_THREADS), 0, s,
                           NG_PN_ARGS);
    else
        hipLaunchKernelGGL((postnorm_kernel<DT_BF16>), dim3((unsigned)M), dim3(PN_THREADS), 0, s,
                           NG_PN_ARGS);
#undef NG_PN_ARGS
    return hipGetLastError();
}

}  // namespace ng

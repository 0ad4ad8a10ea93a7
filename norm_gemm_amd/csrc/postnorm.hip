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
// order, takes the mean and the variance in two passes over the row (fp32),
// and writes y rounded once. Rows of up to 16384 outputs stay in registers
// between the passes; longer ones are re-read from L2. z never exists in the
// output type, so the normalization sees the unrounded sums.
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

// The same, with the row held in registers: thread t keeps the float4
// chunks c = t + 256 j (j < J) of the row, so every fp32 sum is read once
// (16-byte loads, the K ranges added in order, then the bias), the two
// statistics passes run over registers and y is written four outputs per
// store. Needs N % 4 == 0 and N <= 1024 J; `v8` says whether bias / gamma /
// beta / y allow 8-byte accesses (else 2-byte ones).
template <int DT, int J>
__global__ __launch_bounds__(PN_THREADS) void postnorm_reg_kernel(
    const float *__restrict__ part, const uint16_t *__restrict__ bias,
    const uint16_t *__restrict__ gamma, const uint16_t *__restrict__ beta,
    uint16_t *__restrict__ y, int64_t M, int N, int ksplit, float eps, int norm, int v8)
{
    __shared__ float red[PN_THREADS / 64];
    const int64_t m = blockIdx.x;
    const int tid = threadIdx.x;
    const int nc = N >> 2;
    const int64_t plane4 = (M * (int64_t)N) >> 2;
    const float4 *row = reinterpret_cast<const float4 *>(part + m * N);
    auto load4 = [&](const uint16_t *p, int c, float (&f)[4]) {
        if (v8) {
            const uint2 w = *reinterpret_cast<const uint2 *>(p + 4 * c);
            f[0] = bits_to_f<DT>((uint16_t)(w.x & 0xffffu));
            f[1] = bits_to_f<DT>((uint16_t)(w.x >> 16));
            f[2] = bits_to_f<DT>((uint16_t)(w.y & 0xffffu));
            f[3] = bits_to_f<DT>((uint16_t)(w.y >> 16));
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                f[e] = bits_to_f<DT>(p[4 * c + e]);
        }
    };
    float z[J][4];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int c = tid + PN_THREADS * j;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            z[j][e] = 0.0f;
        if (c < nc) {
            float4 v = row[c];
            for (int s = 1; s < ksplit; ++s) {
                const float4 u = row[(int64_t)s * plane4 + c];
                v.x += u.x;
                v.y += u.y;
                v.z += u.z;
                v.w += u.w;
            }
            z[j][0] = v.x;
            z[j][1] = v.y;
            z[j][2] = v.z;
            z[j][3] = v.w;
            if (bias) {
                float b[4];
                load4(bias, c, b);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    z[j][e] += b[e];
            }
        }
    }
    const float invN = 1.0f / (float)N;
    float mu = 0.0f;
    if (norm == NORM_LAYERNORM) {
        float s1 = 0.0f;
#pragma unroll
        for (int j = 0; j < J; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                s1 += z[j][e];              // zero past the row
        mu = block_sum(s1, red) * invN;
    }
    float s2 = 0.0f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
        if (tid + PN_THREADS * j < nc) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float d = z[j][e] - mu;
                s2 = fmaf(d, d, s2);
            }
        }
    }
    const float rs = rsqrtf(block_sum(s2, red) * invN + eps);
    uint16_t *yr = y + m * N;
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int c = tid + PN_THREADS * j;
        if (c >= nc)
            continue;
        float g[4] = {1.0f, 1.0f, 1.0f, 1.0f}, b[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (gamma)
            load4(gamma, c, g);
        if (beta)
            load4(beta, c, b);
        uint16_t o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float v = (z[j][e] - mu) * rs;
            if (gamma)
                v *= g[e];
            if (beta)
                v += b[e];
            o[e] = f_to_bits<DT>(v);
        }
        if (v8) {
            *reinterpret_cast<uint2 *>(yr + 4 * c) =
                make_uint2((uint32_t)o[0] | ((uint32_t)o[1] << 16),
                           (uint32_t)o[2] | ((uint32_t)o[3] << 16));
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                yr[4 * c + e] = o[e];
        }
    }
}

}  // namespace

hipError_t launch_postnorm(const float *part, const void *bias, const void *gamma,
                           const void *beta, void *y, int64_t M, int64_t N, int ksplit, float eps,
                           int norm, int dtype, hipStream_t s)
{
    // rows of up to 16384 outputs (a multiple of 4) in registers
    if (N % 4 == 0 && N <= 16 * 1024) {
        auto a8 = [](const void *p) { return ((uintptr_t)p & 7u) == 0; };
        const int v8 = a8(y) && (!bias || a8(bias)) && (!gamma || a8(gamma)) &&
                       (!beta || a8(beta));
        const int j = (int)((N + 1023) / 1024);
#define NG_PN_REG(DT, J)                                                                     \
    hipLaunchKernelGGL((postnorm_reg_kernel<DT, J>), dim3((unsigned)M), dim3(PN_THREADS), 0, s, \
                       part, (const uint16_t *)bias, (const uint16_t *)gamma,                   \
                       (const uint16_t *)beta, (uint16_t *)y, M, (int)N, ksplit, eps, norm, v8)
#define NG_PN_REG_DT(DT)                                                                     \
    do {                                                                                     \
        if (j <= 1)                                                                          \
            NG_PN_REG(DT, 1);                                                                \
        else if (j <= 2)                                                                     \
            NG_PN_REG(DT, 2);                                                                \
        else if (j <= 4)                                                                     \
            NG_PN_REG(DT, 4);                                                                \
        else if (j <= 8)                                                                     \
            NG_PN_REG(DT, 8);                                                                \
        else                                                                                 \
            NG_PN_REG(DT, 16);                                                               \
    } while (0)
        if (dtype == DT_F16)
            NG_PN_REG_DT(DT_F16);
        else
            NG_PN_REG_DT(DT_BF16);
#undef NG_PN_REG_DT
#undef NG_PN_REG
        return hipGetLastError();
    }
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

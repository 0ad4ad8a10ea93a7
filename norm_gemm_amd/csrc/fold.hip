// fold.hip -- inference-mode folding of the normalization's affine terms into
// the weights (page "LayerNorm 融合算子如何让大模型推理再快 15%？深度拆解 ATB 的实现",
// section 6.2, tip 2: with gamma and beta fixed at inference, gamma is folded
// once, ahead of time, into the weights of the MatMul that follows).
//
// One workgroup of 256 threads per row n of W:
//   W'[n,k] = round(W[n,k] * gamma[k])   one rounding to the storage type (the
//                                        product of two 16-bit values is exact
//                                        in fp32)
//   c1[n]   = sum_k W'[n,k]              of the rounded values the GEMM uses,
//                                        so that sum_k x_k W'_k - mu c1 is the
//                                        sum over the centred row
//   c2[n]   = sum_k W[n,k] beta[k] + bias[n]
// c1 and c2 are fp32 sums in a fixed order (lane, wave), so repeated calls
// give identical results. W is read once and W' written once: an HBM-bound
// kernel that runs once per weight.
#include "device_common.h"
#include "launch.h"

namespace ng {
namespace {

template <int DT, bool VEC>
__global__ __launch_bounds__(256) void fold_kernel(const uint16_t *__restrict__ W,
                                                   const uint16_t *__restrict__ gamma,
                                                   const uint16_t *__restrict__ beta,
                                                   const uint16_t *__restrict__ bias,
                                                   uint16_t *__restrict__ Wf,
                                                   float *__restrict__ c1,
                                                   float *__restrict__ c2, int K)
{
    const int n = blockIdx.x;
    const int tid = threadIdx.x;
    const uint16_t *wr = W + (int64_t)n * K;
    uint16_t *fr = Wf + (int64_t)n * K;
    float s1 = 0.0f, s2 = 0.0f;
    if constexpr (VEC) {
        const int nch = K / 8;
        for (int c = tid; c < nch; c += 256) {
            const u32x4 wv = ldg128(wr + (int64_t)c * 8);
            float w[8], g[8], b[8], f[8];
            unpack8<DT>(wv, w);
            if (gamma)
                unpack8<DT>(ldg128(gamma + (int64_t)c * 8), g);
            if (beta)
                unpack8<DT>(ldg128(beta + (int64_t)c * 8), b);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                f[e] = gamma ? w[e] * g[e] : w[e];
            const u32x4 fv = pack8<DT>(f);
            *reinterpret_cast<u32x4 *>(fr + (int64_t)c * 8) = fv;
            float fq[8];
            unpack8<DT>(fv, fq);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                s1 += fq[e];
                if (beta)
                    s2 = fmaf(w[e], b[e], s2);
            }
        }
    } else {
        for (int k = tid; k < K; k += 256) {
            const float w = bits_to_f<DT>(wr[k]);
            const float g = gamma ? bits_to_f<DT>(gamma[k]) : 1.0f;
            const uint16_t fb = f_to_bits<DT>(w * g);
            fr[k] = fb;
            s1 += bits_to_f<DT>(fb);
            if (beta)
                s2 = fmaf(w, bits_to_f<DT>(beta[k]), s2);
        }
    }
    s1 = wave_sum(s1);
    s2 = wave_sum(s2);
    __shared__ float red[2][4];
    if ((tid & 63) == 0) {
        red[0][tid >> 6] = s1;
        red[1][tid >> 6] = s2;
    }
    __syncthreads();
    if (tid == 0) {
        const float a = ((red[0][0] + red[0][1]) + red[0][2]) + red[0][3];
        const float b = ((red[1][0] + red[1][1]) + red[1][2]) + red[1][3];
        c1[n] = a;
        c2[n] = b + (bias ? bits_to_f<DT>(bias[n]) : 0.0f);
    }
}

template <int DT>
hipError_t launch_fold_dt(const void *W, const void *gamma, const void *beta, const void *bias,
                          void *Wf, float *c1, float *c2, int64_t N, int64_t K, bool vec,
                          hipStream_t s)
{
#define NG_FOLD_ARGS                                                                         \
    (const uint16_t *)W, (const uint16_t *)gamma, (const uint16_t *)beta,                     \
        (const uint16_t *)bias, (uint16_t *)Wf, c1, c2, (int)K
    if (vec)
        hipLaunchKernelGGL((fold_kernel<DT, true>), dim3((unsigned)N), dim3(256), 0, s,
                           NG_FOLD_ARGS);
    else
        hipLaunchKernelGGL((fold_kernel<DT, false>), dim3((unsigned)N), dim3(256), 0, s,
                           NG_FOLD_ARGS);
#undef NG_FOLD_ARGS
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fold(const void *W, const void *gamma, const void *beta, const void *bias,
                       void *Wf, float *c1, float *c2, int64_t N, int64_t K, int dtype, bool vec,
                       hipStream_t s)
{
    return dtype == DT_F16 ? launch_fold_dt<DT_F16>(W, gamma, beta, bias, Wf, c1, c2, N, K, vec, s)
                           : launch_fold_dt<DT_BF16>(W, gamma, beta, bias, Wf, c1, c2, N, K, vec, s);
}

}  // namespace ng

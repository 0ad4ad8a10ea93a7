// gated.hip -- elementwise kernels of the FFN paths.
//
// gate_kernel: h[m, f] = act(g[m, f]) * u[m, f] from the gate and up
// projections of every row, stored side by side as gu[M, 2F] (gate columns
// first). Used by the gated FFN (page "CANN推理加速库ascend-transformer-boost
// ATB算子融合实战…", Llama2 section: the SwiGLU FFN, a SiLU-gated linear unit)
// where the fused gated epilogue of the tiled kernel does not apply: M <= 32
// (the weight-streaming kernels) and unaligned operands. Elementwise and
// HBM-bound; g and u are read as rounded to the I/O type, the product is
// taken in fp32 and rounded once.
#include "device_common.h"
#include "launch.h"

namespace ng {
namespace {

template <int DT>
__global__ __launch_bounds__(256) void gate_kernel(const uint16_t *__restrict__ gu,
                                                   uint16_t *__restrict__ h, int64_t M,
                                                   int64_t F, int act)
{
    const int64_t total = M * F;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += stride) {
        const int64_t m = i / F, f = i - m * F;
        const float g = bits_to_f<DT>(gu[m * 2 * F + f]);
        const float u = bits_to_f<DT>(gu[m * 2 * F + F + f]);
        h[i] = f_to_bits<DT>(apply_act(g, act) * u);
    }
}

// splitk_sum_kernel: y = act(sum over s of part[s] + bias), the partial
// sums of a GEMM whose K was split over ksplit workgroups per tile, added in
// s order (deterministic), one rounding.
template <int DT>
__global__ __launch_bounds__(256) void splitk_sum_kernel(const float *__restrict__ part,
                                                         const uint16_t *__restrict__ bias,
                                                         uint16_t *__restrict__ y, int64_t M,
                                                         int64_t N, int ksplit, int act)
{
    const int64_t total = M * N;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += stride) {
        float v = 0.0f;
        for (int s = 0; s < ksplit; ++s)
            v += part[(int64_t)s * total + i];
        if (bias)
            v += bits_to_f<DT>(bias[i % N]);
        y[i] = f_to_bits<DT>(apply_act(v, act));
    }
}

}  // namespace

hipError_t launch_splitk_sum(const float *part, const void *bias, void *y, int64_t M, int64_t N,
                             int ksplit, int act, int dtype, hipStream_t s)
{
    const int64_t blocks64 = (M * N + 255) / 256;
    const unsigned blocks = (unsigned)(blocks64 < 16384 ? blocks64 : 16384);
    if (dtype == DT_F16)
        hipLaunchKernelGGL((splitk_sum_kernel<DT_F16>), dim3(blocks), dim3(256), 0, s, part,
                           (const uint16_t *)bias, (uint16_t *)y, M, N, ksplit, act);
    else
        hipLaunchKernelGGL((splitk_sum_kernel<DT_BF16>), dim3(blocks), dim3(256), 0, s, part,
                           (const uint16_t *)bias, (uint16_t *)y, M, N, ksplit, act);
    return hipGetLastError();
}

hipError_t launch_gate(const void *gu, void *h, int64_t M, int64_t F, int act, int dtype,
                       hipStream_t s)
{
    const int64_t blocks64 = (M * F + 255) / 256;
    const unsigned blocks = (unsigned)(blocks64 < 16384 ? blocks64 : 16384);
    if (dtype == DT_F16)
        hipLaunchKernelGGL((gate_kernel<DT_F16>), dim3(blocks), dim3(256), 0, s,
                           (const uint16_t *)gu, (uint16_t *)h, M, F, act);
    else
        hipLaunchKernelGGL((gate_kernel<DT_BF16>), dim3(blocks), dim3(256), 0, s,
                           (const uint16_t *)gu, (uint16_t *)h, M, F, act);
    return hipGetLastError();
}

}  // namespace ng

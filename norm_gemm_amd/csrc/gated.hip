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

// The same sum, eight consecutive outputs of one row per thread (N % 8 == 0,
// part and y 16-byte aligned): two 16-byte loads per plane, one 16-byte
// store. Threads map to 8-column chunks of a row (x) and rows (y, strided),
// so the bias chunk is read once per thread and no index is divided.
template <int DT>
__global__ __launch_bounds__(256) void splitk_sum_vec_kernel(const float *__restrict__ part,
                                                             const uint16_t *__restrict__ bias,
                                                             uint16_t *__restrict__ y, int64_t M,
                                                             int64_t N, int ksplit, int act)
{
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;   // 8-column chunk
    if (c * 8 >= N)
        return;
    const int64_t n = c * 8, plane = M * N;
    float b[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        b[e] = 0.0f;
    if (bias) {
        const uint4 bv = *reinterpret_cast<const uint4 *>(bias + n);
        const uint32_t w[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
            b[e] = bits_to_f<DT>((uint16_t)((w[e >> 1] >> ((e & 1) * 16)) & 0xffffu));
    }
    for (int64_t m = blockIdx.y; m < M; m += gridDim.y) {
        const float *p = part + m * N + n;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            v[e] = 0.0f;
        for (int s = 0; s < ksplit; ++s) {
            const float4 lo = *reinterpret_cast<const float4 *>(p + s * plane);
            const float4 hi = *reinterpret_cast<const float4 *>(p + s * plane + 4);
            v[0] += lo.x; v[1] += lo.y; v[2] += lo.z; v[3] += lo.w;
            v[4] += hi.x; v[5] += hi.y; v[6] += hi.z; v[7] += hi.w;
        }
        uint32_t o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t a = f_to_bits<DT>(apply_act(v[2 * e] + b[2 * e], act));
            const uint32_t h = f_to_bits<DT>(apply_act(v[2 * e + 1] + b[2 * e + 1], act));
            o[e] = a | (h << 16);
        }
        *reinterpret_cast<uint4 *>(y + m * N + n) = uint4{o[0], o[1], o[2], o[3]};
    }
}

}  // namespace

hipError_t launch_splitk_sum(const float *part, const void *bias, void *y, int64_t M, int64_t N,
                             int ksplit, int act, int dtype, hipStream_t s)
{
    if (N % 8 == 0 && ((uintptr_t)part & 15u) == 0 && ((uintptr_t)y & 15u) == 0 &&
        ((uintptr_t)bias & 15u) == 0) {
        const dim3 grid((unsigned)((N / 8 + 255) / 256), (unsigned)(M < 4096 ? M : 4096));
        if (dtype == DT_F16)
            hipLaunchKernelGGL((splitk_sum_vec_kernel<DT_F16>), grid, dim3(256), 0, s, part,
                               (const uint16_t *)bias, (uint16_t *)y, M, N, ksplit, act);
        else
            hipLaunchKernelGGL((splitk_sum_vec_kernel<DT_BF16>), grid, dim3(256), 0, s, part,
                               (const uint16_t *)bias, (uint16_t *)y, M, N, ksplit, act);
        return hipGetLastError();
    }
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

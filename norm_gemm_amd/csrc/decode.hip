// decode.hip -- skinny-M (M <= 32) normalization-prologue GEMM that streams
// W from HBM exactly once.
//
// With M <= 32 the work is bound by reading W[N,K] (page "华为CANN算子库如何优化
// 大模型推理性能", section 2.2 names single-token decode as the case that gains
// most from tiling with double buffering). One workgroup of 8 waves owns a
// slab of 16 * nbk consecutive rows of W; the 8 waves split K, each streaming
// its K range of every row of the slab, and the partial sums are reduced in
// LDS at the end.
//
// MFMA v_mfma_f32_16x16x32_{f16,bf16} with W as the A operand: lane l holds
// W row (l % 16), k = (l / 16) * 8 + 0..7, i.e. 16 contiguous bytes that come
// straight from HBM into the operand registers (4 lanes cover 64 contiguous
// bytes of a row); the B operand is the normalized x row (l % 16) at the
// same k, computed in registers from x (L2-resident) and the row statistics.
// Result element r of lane l is C[4 (l / 16) + r][l % 16] = y^T[n][m].
#include "device_common.h"
#include "launch.h"

namespace ng {
namespace {

constexpr int kNW = 8;       // waves per workgroup
constexpr int kNBMax = 8;    // max 16-row blocks of W per workgroup

template <int DT>
__device__ __forceinline__ floatx4 mfma16(const u32x4 &a, const u32x4 &b, const floatx4 &c)
{
    if constexpr (DT == DT_F16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a),
                                                     __builtin_bit_cast(half8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                      __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// MB = number of 16-column blocks of M (1 for M <= 16, 2 for M <= 32).
template <int DT, bool AFFINE, bool VEC, int MB>
__global__ __launch_bounds__(64 * kNW) void decode_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ gamma,
    const uint16_t *__restrict__ beta, const uint16_t *__restrict__ W,
    const uint16_t *__restrict__ bias, uint16_t *__restrict__ y, int M, int N, int K,
    float eps, int norm, int act, int nbk)
{
    __shared__ float s_rs[32], s_mu[32];
    __shared__ float red[kNBMax * 16][MB * 16 + 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int slab = nbk * 16;
    const int n0 = blockIdx.x * slab;

    const int nchunks = (K + 31) / 32;
    const int cpw = (nchunks + kNW - 1) / kNW;
    const int c_begin = wave * cpw;
    const int c_end = min(nchunks, c_begin + cpw);

    auto load_w = [&](int c, u32x4 *dst) {
        const int64_t k = (int64_t)c * 32 + lg * 8;
#pragma unroll
        for (int nb = 0; nb < kNBMax; ++nb) {
            if (nb < nbk) {
                const int n = n0 + nb * 16 + lr;
                dst[nb] = (n < N) ? load_chunk<VEC>(W + (int64_t)n * K, k, K)
                                  : u32x4{0u, 0u, 0u, 0u};
            }
        }
    };

    // Weights first: the first fragments are in flight during the statistics.
    u32x4 wcur[kNBMax];
    if (c_begin < c_end)
        load_w(c_begin, wcur);

    float rs[MB], mu[MB];
    if constexpr (AFFINE) {
        for (int m = wave; m < M; m += kNW) {
            float a, b;
            row_stats<DT, VEC>(x + (int64_t)m * K, K, eps, norm, lane, a, b);
            if (lane == 0) {
                s_rs[m] = a;
                s_mu[m] = b;
            }
        }
        __syncthreads();
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int m = mb * 16 + lr;
            rs[mb] = m < M ? s_rs[m] : 0.0f;
            mu[mb] = m < M ? s_mu[m] : 0.0f;
        }
    }

    floatx4 acc[kNBMax][MB];
#pragma unroll
    for (int nb = 0; nb < kNBMax; ++nb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
            acc[nb][mb] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

    for (int c = c_begin; c < c_end; ++c) {
        u32x4 wnext[kNBMax];
        if (c + 1 < c_end)
            load_w(c + 1, wnext);

        const int64_t k = (int64_t)c * 32 + lg * 8;
        u32x4 xf[MB];
        float g[8], bt[8];
        if constexpr (AFFINE) {
            if (gamma) {
                unpack8<DT>(load_chunk<VEC>(gamma, k, K), g);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) g[e] = 1.0f;
            }
            if (beta) {
                unpack8<DT>(load_chunk<VEC>(beta, k, K), bt);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) bt[e] = 0.0f;
            }
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int m = mb * 16 + lr;
            const u32x4 raw = (m < M) ? load_chunk<VEC>(x + (int64_t)m * K, k, K)
                                      : u32x4{0u, 0u, 0u, 0u};
            if constexpr (AFFINE) {
                float f[8];
                unpack8<DT>(raw, f);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float v = fmaf((f[e] - mu[mb]) * rs[mb], g[e], bt[e]);
                    f[e] = (k + e < K && m < M) ? v : 0.0f;
                }
                xf[mb] = pack8<DT>(f);
            } else {
                xf[mb] = raw;
            }
        }
#pragma unroll
        for (int nb = 0; nb < kNBMax; ++nb) {
            if (nb < nbk) {
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    acc[nb][mb] = mfma16<DT>(wcur[nb], xf[mb], acc[nb][mb]);
            }
        }
#pragma unroll
        for (int nb = 0; nb < kNBMax; ++nb)
            wcur[nb] = wnext[nb];
    }

    // Reduce the 8 K-partials in LDS, one wave after the other.
    for (int w = 0; w < kNW; ++w) {
        if (wave == w) {
#pragma unroll
            for (int nb = 0; nb < kNBMax; ++nb) {
                if (nb < nbk) {
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            float &dst = red[nb * 16 + lg * 4 + r][mb * 16 + lr];
                            dst = (w == 0) ? acc[nb][mb][r] : dst + acc[nb][mb][r];
                        }
                }
            }
        }
        __syncthreads();
    }

    // Epilogue: bias, activation, one rounding; consecutive threads write
    // consecutive n of one output row.
    for (int idx = tid; idx < M * slab; idx += 64 * kNW) {
        const int m = idx / slab, nl = idx % slab;
        const int n = n0 + nl;
        if (n < N) {
            float v = red[nl][m];
            if (bias)
                v += bits_to_f<DT>(bias[n]);
            y[(int64_t)m * N + n] = f_to_bits<DT>(apply_act(v, act));
        }
    }
}

template <int DT, bool AFFINE, bool VEC>
hipError_t launch_t(const GemmArgs &a, int nbk, int grid, hipStream_t s)
{
#define NG_DECODE_ARGS                                                                       \
    (const uint16_t *)a.x, (const uint16_t *)a.gamma, (const uint16_t *)a.beta,              \
        (const uint16_t *)a.W, (const uint16_t *)a.bias, (uint16_t *)a.y, (int)a.M, (int)a.N, \
        (int)a.K, a.eps, a.norm, a.act, nbk
    if (a.M <= 16)
        hipLaunchKernelGGL((decode_kernel<DT, AFFINE, VEC, 1>), dim3(grid), dim3(64 * kNW), 0, s,
                           NG_DECODE_ARGS);
    else
        hipLaunchKernelGGL((decode_kernel<DT, AFFINE, VEC, 2>), dim3(grid), dim3(64 * kNW), 0, s,
                           NG_DECODE_ARGS);
#undef NG_DECODE_ARGS
    return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const GemmArgs &a, int nbk, int grid, hipStream_t s)
{
    // element loads only: aligned skinny calls take the line or wide kernels
    const bool affine = a.norm != NORM_NONE;
    return affine ? launch_t<DT, true, false>(a, nbk, grid, s)
                  : launch_t<DT, false, false>(a, nbk, grid, s);
}

}  // namespace

hipError_t launch_decode(const GemmArgs &a, hipStream_t s)
{
    const int cus = cu_count();
    // enough 16-row blocks per workgroup for about one workgroup per CU
    const int64_t blocks = (a.N + 15) / 16;
    int nbk = (int)((blocks + cus - 1) / cus);
    nbk = nbk < 1 ? 1 : (nbk > kNBMax ? kNBMax : nbk);
    const int grid = (int)((blocks + nbk - 1) / nbk);
    if (a.dtype == DT_F16)
        return launch_dt<DT_F16>(a, nbk, grid, s);
    return launch_dt<DT_BF16>(a, nbk, grid, s);
}

}  // namespace ng

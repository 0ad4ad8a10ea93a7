// prefill.hip -- tiled MFMA kernel for the normalization-prologue GEMM,
// M > 32 (page "LayerNorm 融合算子如何让大模型推理再快 15%？深度拆解 ATB 的实现",
// sections 2.1-3.1: tile-level fusion, the normalized tile stays on chip,
// weights are fetched while the statistics are computed).
//
// One workgroup owns a BM x BN tile of y.
//   1. Prologue: the first W and x tiles are requested, then each wave
//      reduces the row statistics of BM/NWAVES rows (one pass, fp32) into
//      LDS as (mu, rs) with a_norm = (x - mu) * rs.
//   2. K loop in BK steps: x chunk -> fp32 normalize + affine -> one RNE
//      rounding -> LDS A tile; W chunk -> LDS B tile; both double-buffered,
//      with the next step's global loads in flight during the MFMAs.
//      The normalized activation exists only in registers and LDS.
//   3. Epilogue in registers: + bias, optional SiLU, one rounding, store.
//
// MFMA: v_mfma_f32_32x32x16_{f16,bf16}. Operand lanes (checked on gfx950):
// lane l holds row (l % 32), k = (l / 32) * 8 + 0..7 of both A (x rows) and
// B (W rows); result element 4*q + r of lane l is C[8q + 4(l/32) + r][l % 32].
// LDS tiles are [rows][BK] with the 16-byte chunk index XOR-swizzled by the
// row so that 8 consecutive rows read at one k land in distinct banks.
#include "device_common.h"
#include "launch.h"

namespace ng {
namespace {

template <int BM_, int BN_, int BK_, int WM_, int WN_>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
    static constexpr int NWAVES = WM * WN;
    static constexpr int THREADS = 64 * NWAVES;
    static constexpr int TM = BM / WM, TN = BN / WN;   // wave tile
    static constexpr int FM = TM / 32, FN = TN / 32;   // 32x32 MFMA blocks per wave
    static constexpr int CPR = BK / 8;                 // 16-byte chunks per tile row
    static constexpr int A_CH = BM * CPR / THREADS;    // A chunks per thread per step
    static constexpr int B_CH = BN * CPR / THREADS;
    static constexpr int ROWS_PER_PASS = THREADS / CPR;
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be 32-aligned");
    static_assert(BK % 16 == 0 && (CPR & (CPR - 1)) == 0, "BK must be 16 * 2^j");
    static_assert(BM * CPR % THREADS == 0 && BN * CPR % THREADS == 0, "chunk split");
};

template <int CPR>
__device__ __forceinline__ int swz(int row, int chunk)
{
    return chunk ^ (row & (CPR - 1));
}

template <int DT>
__device__ __forceinline__ floatx16 mfma32(const u32x4 &a, const u32x4 &b, const floatx16 &c)
{
    if constexpr (DT == DT_F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, a),
                                                     __builtin_bit_cast(half8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                      __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// AFFINE = false: norm NONE, the x chunk goes to LDS untouched.
template <class C, int DT, bool AFFINE, bool VEC>
__global__ __launch_bounds__(C::THREADS) void prefill_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ gamma,
    const uint16_t *__restrict__ beta, const uint16_t *__restrict__ W,
    const uint16_t *__restrict__ bias, uint16_t *__restrict__ y, int M, int N, int K,
    float eps, int norm, int act, int tiles_m, int tiles_n)
{
    __shared__ u32x4 As[2][C::BM * C::CPR];
    __shared__ u32x4 Bs[2][C::BN * C::CPR];
    __shared__ float s_rs[C::BM], s_mu[C::BM];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    // Workgroups are dealt to the 8 XCDs round-robin; regroup so that each
    // XCD works on a contiguous range of tiles (M fastest), which keeps the
    // W columns of that range in the XCD's own L2.
    const int G = tiles_m * tiles_n;
    int b = blockIdx.x;
    if ((G & 7) == 0)
        b = (b & 7) * (G >> 3) + (b >> 3);
    const int tm = b % tiles_m, tn = b / tiles_m;
    const int m0 = tm * C::BM, n0 = tn * C::BN;

    // per-thread chunk coordinates: fixed chunk column, rows strided
    const int cc = tid % C::CPR;
    const int r0 = tid / C::CPR;
    const int KT = (K + C::BK - 1) / C::BK;

    u32x4 ra[C::A_CH], rb[C::B_CH];
    u32x4 rg = {0u, 0u, 0u, 0u}, rbt = {0u, 0u, 0u, 0u};

    auto load_step = [&](int kt) {
        const int64_t k = (int64_t)kt * C::BK + cc * 8;
#pragma unroll
        for (int i = 0; i < C::A_CH; ++i) {
            const int m = m0 + r0 + i * C::ROWS_PER_PASS;
            ra[i] = (m < M) ? load_chunk<VEC>(x + (int64_t)m * K, k, K) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < C::B_CH; ++i) {
            const int n = n0 + r0 + i * C::ROWS_PER_PASS;
            rb[i] = (n < N) ? load_chunk<VEC>(W + (int64_t)n * K, k, K) : u32x4{0u, 0u, 0u, 0u};
        }
        if constexpr (AFFINE) {
            if (gamma)
                rg = load_chunk<VEC>(gamma, k, K);
            if (beta)
                rbt = load_chunk<VEC>(beta, k, K);
        }
    };

    // per-row (rs, mu) of this thread's A rows, filled after the prologue
    float rrs[C::A_CH], rmu[C::A_CH];

    // Normalized, affine-applied A chunk: a = (x - mu) * rs * g + b in fp32,
    // rounded once; positions k >= K are exactly zero.
    auto store_step = [&](int kt, int buf) {
        const int64_t k = (int64_t)kt * C::BK + cc * 8;
        if constexpr (AFFINE) {
            float g[8], bt[8];
            if (gamma) {
                unpack8<DT>(rg, g);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) g[e] = 1.0f;
            }
            if (beta) {
                unpack8<DT>(rbt, bt);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) bt[e] = 0.0f;
            }
#pragma unroll
            for (int i = 0; i < C::A_CH; ++i) {
                const int r = r0 + i * C::ROWS_PER_PASS;
                const float rs = rrs[i], mu = rmu[i];
                float f[8];
                unpack8<DT>(ra[i], f);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float v = fmaf((f[e] - mu) * rs, g[e], bt[e]);
                    f[e] = (k + e < K && m0 + r < M) ? v : 0.0f;
                }
                As[buf][r * C::CPR + swz<C::CPR>(r, cc)] = pack8<DT>(f);
            }
        } else {
#pragma unroll
            for (int i = 0; i < C::A_CH; ++i) {
                const int r = r0 + i * C::ROWS_PER_PASS;
                As[buf][r * C::CPR + swz<C::CPR>(r, cc)] = ra[i];
            }
        }
#pragma unroll
        for (int i = 0; i < C::B_CH; ++i) {
            const int r = r0 + i * C::ROWS_PER_PASS;
            Bs[buf][r * C::CPR + swz<C::CPR>(r, cc)] = rb[i];
        }
    };

    // 1. issue the first tile's loads, then the statistics prologue
    load_step(0);
    if constexpr (AFFINE) {
        for (int r = wave; r < C::BM; r += C::NWAVES) {
            const int m = m0 + r;
            float rs = 0.0f, mu = 0.0f;
            if (m < M)
                row_stats<DT, VEC>(x + (int64_t)m * K, K, eps, norm, lane, rs, mu);
            if (lane == 0) {
                s_rs[r] = rs;
                s_mu[r] = mu;
            }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < C::A_CH; ++i) {
            rrs[i] = s_rs[r0 + i * C::ROWS_PER_PASS];
            rmu[i] = s_mu[r0 + i * C::ROWS_PER_PASS];
        }
    }
    store_step(0, 0);
    __syncthreads();

    const int wm = wave / C::WN, wn = wave % C::WN;
    floatx16 acc[C::FM][C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    const int lrow = lane & 31, lk = lane >> 5;

    // 2. K loop
    for (int kt = 0; kt < KT; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < KT)
            load_step(kt + 1);
#pragma unroll
        for (int kk = 0; kk < C::BK / 16; ++kk) {
            const int ch = kk * 2 + lk;
            u32x4 af[C::FM], bf[C::FN];
#pragma unroll
            for (int i = 0; i < C::FM; ++i) {
                const int r = wm * C::TM + i * 32 + lrow;
                af[i] = As[buf][r * C::CPR + swz<C::CPR>(r, ch)];
            }
#pragma unroll
            for (int j = 0; j < C::FN; ++j) {
                const int r = wn * C::TN + j * 32 + lrow;
                bf[j] = Bs[buf][r * C::CPR + swz<C::CPR>(r, ch)];
            }
#pragma unroll
            for (int i = 0; i < C::FM; ++i)
#pragma unroll
                for (int j = 0; j < C::FN; ++j)
                    acc[i][j] = mfma32<DT>(af[i], bf[j], acc[i][j]);
        }
        if (kt + 1 < KT)
            store_step(kt + 1, buf ^ 1);
        __syncthreads();
    }

    // 3. epilogue: bias, activation, one rounding, masked stores
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
        const int n = n0 + wn * C::TN + j * 32 + lrow;
        if (n >= N)
            continue;
        const float bv = bias ? bits_to_f<DT>(bias[n]) : 0.0f;
#pragma unroll
        for (int i = 0; i < C::FM; ++i) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = m0 + wm * C::TM + i * 32 + q * 8 + lk * 4 + r;
                    if (m < M)
                        y[(int64_t)m * N + n] = f_to_bits<DT>(apply_act(acc[i][j][q * 4 + r] + bv, act));
                }
        }
    }
}

using Cfg128x128 = TileCfg<128, 128, 64, 2, 2>;

template <class C, int DT, bool AFFINE, bool VEC>
hipError_t launch_t(const GemmArgs &a, hipStream_t s)
{
    const int tiles_m = (int)((a.M + C::BM - 1) / C::BM);
    const int tiles_n = (int)((a.N + C::BN - 1) / C::BN);
    hipLaunchKernelGGL((prefill_kernel<C, DT, AFFINE, VEC>), dim3(tiles_m * tiles_n),
                       dim3(C::THREADS), 0, s, (const uint16_t *)a.x, (const uint16_t *)a.gamma,
                       (const uint16_t *)a.beta, (const uint16_t *)a.W,
                       (const uint16_t *)a.bias, (uint16_t *)a.y, (int)a.M, (int)a.N,
                       (int)a.K, a.eps, a.norm, a.act, tiles_m, tiles_n);
    return hipGetLastError();
}

template <class C, int DT>
hipError_t launch_dt(const GemmArgs &a, hipStream_t s)
{
    const bool affine = a.norm != NORM_NONE;
    if (a.vec)
        return affine ? launch_t<C, DT, true, true>(a, s) : launch_t<C, DT, false, true>(a, s);
    return affine ? launch_t<C, DT, true, false>(a, s) : launch_t<C, DT, false, false>(a, s);
}

}  // namespace

hipError_t launch_prefill(const GemmArgs &a, hipStream_t s)
{
    if (a.dtype == DT_F16)
        return launch_dt<Cfg128x128, DT_F16>(a, s);
    return launch_dt<Cfg128x128, DT_BF16>(a, s);
}

}  // namespace ng

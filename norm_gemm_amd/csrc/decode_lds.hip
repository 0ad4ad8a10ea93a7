// decode_lds.hip -- skinny-M (M <= 32) normalization-prologue GEMM for
// 16-byte aligned operands with K % 8 == 0: W is streamed from HBM exactly
// once, in whole 128-byte lines.
//
// With M <= 32 the work is bound by reading W[N,K] (page "华为CANN算子库如何优化
// 大模型推理性能", section 2.2: single-token decode gains most from tiling with
// double buffering). One workgroup of 8 waves owns a slab of 16 * NBK rows of
// W; the waves split K into contiguous ranges of 64-element k-blocks.
//
// W path: a block is 16 rows x 64 k (2 KB). Two direct HBM -> LDS loads fill
// it; each covers 8 rows x 128 contiguous bytes, so every request is a whole
// cache line. Each wave owns NBK block slots in LDS, one per row block of the
// slab, and keeps NBK - 1 blocks in flight ahead of the one it multiplies
// (block (kb, nb) always lives in slot nb; the load issued at a step refills
// the slot consumed at the step before). Within a slot the 16-byte chunk
// index is XOR-swizzled by (row / 2) % 8, which keeps the MFMA operand reads
// (16 rows at one chunk) free of bank conflicts. Every slot is an LDS object
// of its own, so the compiler's wait for a direct load only covers the loads
// into that slot.
//
// MFMA v_mfma_f32_16x16x32_{f16,bf16} with W as the A operand: for k-step s of
// a block, lane l holds W row (l % 16), logical chunk 4s + l / 16 (8 values);
// the B operand is the normalized x row (l % 16) at the same k, computed in
// registers from x (L2-resident) and the row statistics, once per k-block for
// all the slab's row blocks, from raw x loaded one k-block ahead. Result
// element r of lane l is C[4 (l / 16) + r][l % 16] = y^T[n][m]. The 8 waves'
// K-partials are summed in a fixed order through LDS (deterministic).
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace ng {
namespace {

// Cache policy of the W loads: non-temporal (nt), so the L2 may replace the
// streamed W lines first; every W line is read once per call, and the hint
// keeps them from crowding the L2 (M = 32: 82.6 -> 74.7 us on W[28672, 8192]).
constexpr int kWPolicy = 2;

constexpr int kNW = 8;                  // waves per workgroup
constexpr int kNBMax = 8;               // max 16-row blocks of W per workgroup
constexpr int kBlockChunks = 16 * 8;    // 16 rows x 8 chunks of 16 bytes

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

__device__ __forceinline__ int dswz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

template <int I>
using ic = std::integral_constant<int, I>;

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (I < N) {
        f(ic<I>{});
        static_for<I + 1, N>(f);
    }
}

// Normalization modes of the kernel.
enum {
    DM_NONE = 0,      // x as given
    DM_STATS = 1,     // LayerNorm / RMSNorm: row statistics first, then
                      // (x - mu) * rs * gamma + beta in registers
    DM_RMS_LATE = 2,  // RMSNorm without beta, bf16: x * gamma into the MFMA,
                      // each row's sum of x^2 on the matrix cores, rs applied
                      // per output row at the end
};

// DM = normalization mode; MB = number of 16-column blocks of M (1 for
// M <= 16, 2 for M <= 32); NBK = 16-row blocks of W per workgroup (2..8).
template <int DT, int DM, int MB, int NBK>
__global__ __launch_bounds__(64 * kNW) void decode_lds_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ gamma,
    const uint16_t *__restrict__ beta, const uint16_t *__restrict__ W,
    const uint16_t *__restrict__ bias, uint16_t *__restrict__ y, int M, int N, int K,
    float eps, int norm, int act)
{
    static_assert(NBK >= 2 && NBK <= kNBMax, "2..8 row blocks per workgroup");
    constexpr bool AFFINE = DM == DM_STATS;
    constexpr bool LATE = DM == DM_RMS_LATE;
    constexpr int D = NBK - 1;                          // blocks in flight per wave
    // loads per x group: x chunks, plus gamma and beta (statistics mode) or
    // gamma (late RMS scaling)
    constexpr int XL = 2 * MB + (AFFINE ? 4 : LATE ? 2 : 0);
    __shared__ u32x4 L0[kNW][kBlockChunks], L1[kNW][kBlockChunks], L2[kNW][kBlockChunks],
        L3[kNW][kBlockChunks], L4[kNW][kBlockChunks], L5[kNW][kBlockChunks],
        L6[kNW][kBlockChunks], L7[kNW][kBlockChunks];
    __shared__ float s_rs[32], s_mu[32];  // per row: statistics; late RMS: rs (epilogue)
    __shared__ float s_ss[kNW][32];     // late RMS: per-wave sums of x^2 per row

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const int n0 = blockIdx.x * (NBK * 16);

    // slot S of wave w
    auto slot = [&](auto S, int w) -> u32x4 * {
        constexpr int s = decltype(S)::value;
        if constexpr (s == 0) return L0[w];
        else if constexpr (s == 1) return L1[w];
        else if constexpr (s == 2) return L2[w];
        else if constexpr (s == 3) return L3[w];
        else if constexpr (s == 4) return L4[w];
        else if constexpr (s == 5) return L5[w];
        else if constexpr (s == 6) return L6[w];
        else return L7[w];
    };

    // this wave's K range in 64-element k-blocks
    const int nkb = (K + 63) / 64;
    const int kbpw = (nkb + kNW - 1) / kNW;
    const int kb0 = min(wave * kbpw, nkb);
    const int kb1 = min(kb0 + kbpw, nkb);
    // Each workgroup walks its waves' ranges from a different starting
    // k-block (logical k-block kb is physical block kp(kb)): every CU reads
    // all of x and gamma, and in lockstep all CUs would request the same
    // lines of them at once, queueing at one L2 channel per line.
    const int nrange = max(kb1 - kb0, 1);
    const int rot = (int)blockIdx.x % nrange;
    auto kp = [&](int kb) { return kb0 + (kb - kb0 + rot) % nrange; };

    // Direct loads of block (kb, NB) into slot NB: load h (0/1) puts row
    // 8h + lane/8 at chunk position lane%8, holding logical chunk
    // dswz(row, lane%8). A block past this wave's range keeps the load
    // count uniform: it re-reads the wave's most recently loaded block (the
    // last row block of its last k-block, still in L2) into a slot that is
    // never read again.
    const int drow0 = lane >> 3;
    auto issue_block = [&](auto NB, int kb) {
        int nb = decltype(NB)::value;
        if (kb >= kb1) {
            kb = kb1 - 1;
            nb = NBK - 1;
        }
        kb = kp(kb);
        u32x4 *dst = slot(NB, wave);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int row = 8 * h + drow0;
            const int n = min(n0 + nb * 16 + row, N - 1);
            const int k = kb * 64 + dswz(row, lane & 7) * 8;
            __builtin_amdgcn_global_load_lds(
                (const void *)(W + (int64_t)n * K + (k < K ? k : 0)),
                (__attribute__((address_space(3))) void *)&dst[h * 64], 16, 0, kWPolicy);
        }
    };

    // x of one k-block (chunks lg and 4 + lg of rows lr, lr + 16), loaded raw
    // into register set SET; the loads are unconditional (clamped addresses)
    // so that every x group is the same number of loads.
    u32x4 xr[2][MB][2], gr[2][2], br[2][2];
    const uint16_t *gp = gamma ? gamma : x;
    const uint16_t *bp = beta ? beta : x;
    auto load_x = [&](auto SET, int kb) {
        constexpr int set = decltype(SET)::value;
        kb = kp(min(kb, kb1 - 1));
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const int k = kb * 64 + (4 * s2 + lg) * 8;
            const int kc = k < K ? k : 0;
            if constexpr (AFFINE || LATE)
                gr[set][s2] = ldg128(gp + kc);
            if constexpr (AFFINE)
                br[set][s2] = ldg128(bp + kc);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                xr[set][mb][s2] = ldg128(x + (int64_t)min(mb * 16 + lr, M - 1) * K + kc);
        }
    };

    // x of the first k-block, then D W blocks, in flight during the statistics
    const bool has_work = kb0 < kb1;
    if (has_work) {
        load_x(ic<0>{}, kb0);
        issue_fence(x, gamma, beta);   // keep x ahead of the blocks
        static_for<0, D>([&](auto NB) { issue_block(NB, kb0); });
    }

    float rs[MB], mu[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        rs[mb] = 1.0f;
        mu[mb] = 0.0f;
    }
    if constexpr (AFFINE) {
        for (int m = wave; m < M; m += kNW) {
            float a, b;
            row_stats_wide<DT>(x + (int64_t)m * K, K, eps, norm, lane, a, b);
            if (lane == 0) {
                s_rs[m] = a;
                s_mu[m] = b;
            }
        }
        lds_barrier();
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int m = mb * 16 + lr;
            rs[mb] = m < M ? s_rs[m] : 0.0f;
            mu[mb] = m < M ? s_mu[m] : 0.0f;
        }
    }

    // B operands of k-block kb from register set SET: normalized (statistics
    // mode), times gamma with the sums of x^2 taken on the way (late RMS), or
    // x itself
    floatx4 accss[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
        accss[mb] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    auto x_frags = [&](auto SET, int kb, u32x4 (&xf)[MB][2]) {
        constexpr int set = decltype(SET)::value;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const bool kin = kb * 64 + (4 * s2 + lg) * 8 < K;
            if constexpr (LATE) {
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    const bool live = kin && mb * 16 + lr < M;
                    // x masked once. The A and B operand layouts of the
                    // 16x16x32 MFMA coincide (lane l: row l % 16, k-group
                    // l / 16), so x times itself accumulates
                    // C[i][j] = sum_k x_ik x_jk, whose diagonal holds each
                    // row's sum of squares (bf16 products are exact in fp32)
                    const u32x4 xz = live ? xr[set][mb][s2] : u32x4{0u, 0u, 0u, 0u};
                    accss[mb] = mfma16<DT>(xz, xz, accss[mb]);
                    if (gamma) {
                        float f[8], g[8];
                        unpack8<DT>(xz, f);
                        unpack8<DT>(gr[set][s2], g);
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            f[e] *= g[e];
                        xf[mb][s2] = pack8<DT>(f);
                    } else {
                        xf[mb][s2] = xz;
                    }
                }
                continue;
            }
            float g[8], bt[8];
            if constexpr (AFFINE) {
                unpack8<DT>(gr[set][s2], g);
                unpack8<DT>(br[set][s2], bt);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    g[e] = gamma ? g[e] : 1.0f;
                    bt[e] = beta ? bt[e] : 0.0f;
                }
            }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const bool live = kin && mb * 16 + lr < M;
                if constexpr (AFFINE) {
                    float f[8];
                    unpack8<DT>(xr[set][mb][s2], f);
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        f[e] = fmaf((f[e] - mu[mb]) * rs[mb], g[e], bt[e]);
                    xf[mb][s2] = live ? pack8<DT>(f) : u32x4{0u, 0u, 0u, 0u};
                } else {
                    xf[mb][s2] = live ? xr[set][mb][s2] : u32x4{0u, 0u, 0u, 0u};
                }
            }
        }
    };

    floatx4 acc[NBK][MB];
#pragma unroll
    for (int nb = 0; nb < NBK; ++nb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
            acc[nb][mb] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

    // One k-block: load x of the next one (if NEXT), normalize this one's, then
    // for each row block nb: issue block (kb, nb) + D, wait for block (kb, nb),
    // multiply it. Loads issued after block (kb, nb) at its wait: the D
    // younger blocks (2 D loads) and, for nb < D with NEXT, the x group of
    // kb + 1 (issued at the top of kb, after (kb, nb), which was issued during
    // k-block kb - 1 or before the loop). The compiler may reorder loads only
    // between two waits (the waits clobber memory), which can make a wait
    // stricter but never looser.
    auto kblock = [&](auto SET, auto NEXT, int kb) {
        constexpr int set = decltype(SET)::value;
        constexpr bool next = decltype(NEXT)::value;
        // x of kb was issued at the top of k-block kb - 1 (or before the
        // loop); younger than it are at least the blocks issued at steps
        // (kb - 1, 1 .. NBK - 1) and the x group of kb + 1: waiting down to
        // that many leaves the D prefetched blocks in flight.
        if constexpr (next) {
            load_x(ic<set ^ 1>{}, kb + 1);
            issue_fence(x, gamma, beta);
            wait_vmcnt<2 * D + XL>();
        } else {
            wait_vmcnt<2 * D>();
        }
        u32x4 xf[MB][2];
        const int kbp = kp(kb);           // physical k-block
        x_frags(SET, kbp, xf);
        static_for<0, NBK>([&](auto NB) {
            constexpr int nb = decltype(NB)::value;
            constexpr int nb_next = (nb + D) % NBK;
            // the refill of slot nb_next (read at the step before) stays
            // behind that step's MFMAs, hence behind its LDS reads
            issue_fence(x, gamma, beta);
            issue_block(ic<nb_next>{}, nb + D >= NBK ? kb + 1 : kb);
            if constexpr (next && nb < D)
                wait_vmcnt<2 * D + XL>();
            else
                wait_vmcnt<2 * D>();
            u32x4 *sl = slot(NB, wave);
            if (kbp * 64 + 64 > K) {
                // zero the chunks past K of this lane's own direct loads
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int row = 8 * h + drow0;
                    if (kbp * 64 + dswz(row, lane & 7) * 8 >= K)
                        sl[h * 64 + lane] = u32x4{0u, 0u, 0u, 0u};
                }
            }
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const u32x4 wf = sl[lr * 8 + dswz(lr, 4 * s + lg)];
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    acc[nb][mb] = mfma16<DT>(wf, xf[mb][s], acc[nb][mb]);
            }
        });
    };

    if (has_work) {
        int kb = kb0;
        for (; kb + 1 < kb1; kb += 2) {
            kblock(ic<0>{}, std::true_type{}, kb);
            kblock(ic<1>{}, std::true_type{}, kb + 1);
        }
        if (kb < kb1)
            kblock(ic<0>{}, std::false_type{}, kb);
    }
    wait_vmcnt<0>();

    // Partials: wave w writes its row block nb into its own slot nb as
    // float [16 MB m][16 n] (1 KB per 16 m, fits the 2 KB slot): lane (lr,
    // lg) holds n = 4 lg .. 4 lg + 3 of column m = lr, one 16-byte store,
    // and the epilogue's lanes read consecutive n of one m (no LDS bank
    // conflicts either way). Late RMS: the wave's sum of x^2 per row
    // (diagonal element i of a 16x16 result sits in lane i + 16 (i / 4),
    // accumulator register i % 4).
    if constexpr (LATE) {
        if (lg == (lr >> 2)) {
            const int r = lr & 3;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                s_ss[wave][mb * 16 + lr] = r == 0 ? accss[mb][0] : r == 1 ? accss[mb][1]
                                         : r == 2 ? accss[mb][2] : accss[mb][3];
        }
    }
    static_for<0, NBK>([&](auto NB) {
        constexpr int nb = decltype(NB)::value;
        floatx4 *p = reinterpret_cast<floatx4 *>(slot(NB, wave));
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
            p[(mb * 16 + lr) * 4 + lg] = acc[nb][mb];
    });
    lds_barrier();
    if constexpr (LATE) {
        // each row's scale once: sum of the waves' x^2 in wave order
        if (tid < M) {
            float q = 0.0f;
#pragma unroll
            for (int w = 0; w < kNW; ++w)
                q += s_ss[w][tid];
            s_rs[tid] = rsqrtf(q / (float)K + eps);
        }
        lds_barrier();
    }

    // Epilogue: wave w finishes row block nb = w. Lane item (m, q) sums the
    // 8 partials of outputs n = 4 q .. 4 q + 3 of row m in wave order (16-byte
    // LDS reads), scales them (late RMS), adds the bias, applies the
    // activation and rounds once; 8-byte stores where the rows allow them.
    const bool vst = (N & 3) == 0 && ((uintptr_t)y & 7u) == 0;
    static_for<0, NBK>([&](auto NB) {
        constexpr int nb = decltype(NB)::value;
        if (wave != nb)
            return;
        for (int idx = lane; idx < M * 4; idx += 64) {
            const int m = idx >> 2, q = idx & 3;
            floatx4 v = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int w = 0; w < kNW; ++w)
                v += reinterpret_cast<const floatx4 *>(slot(NB, w))[m * 4 + q];
            const int n = n0 + nb * 16 + 4 * q;
            uint16_t o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float t = v[e];
                if constexpr (LATE)
                    t *= s_rs[m];
                if (bias && n + e < N)
                    t += bits_to_f<DT>(bias[n + e]);
                o[e] = f_to_bits<DT>(apply_act(t, act));
            }
            uint16_t *yp = y + (int64_t)m * N + n;
            if (vst && n + 3 < N) {
                *reinterpret_cast<uint2 *>(yp) =
                    make_uint2((uint32_t)o[0] | ((uint32_t)o[1] << 16),
                               (uint32_t)o[2] | ((uint32_t)o[3] << 16));
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (n + e < N)
                        yp[e] = o[e];
            }
        }
    });
}

template <int DT, int DM, int NBK>
hipError_t launch_t(const GemmArgs &a, int grid, hipStream_t s)
{
#define NG_DECODE_ARGS                                                                       \
    (const uint16_t *)a.x, (const uint16_t *)a.gamma, (const uint16_t *)a.beta,              \
        (const uint16_t *)a.W, (const uint16_t *)a.bias, (uint16_t *)a.y, (int)a.M, (int)a.N, \
        (int)a.K, a.eps, a.norm, a.act
    if (a.M <= 16)
        hipLaunchKernelGGL((decode_lds_kernel<DT, DM, 1, NBK>), dim3(grid), dim3(64 * kNW), 0, s,
                           NG_DECODE_ARGS);
    else
        hipLaunchKernelGGL((decode_lds_kernel<DT, DM, 2, NBK>), dim3(grid), dim3(64 * kNW), 0, s,
                           NG_DECODE_ARGS);
#undef NG_DECODE_ARGS
    return hipGetLastError();
}

template <int DT, int DM>
hipError_t launch_nbk(const GemmArgs &a, int nbk, int grid, hipStream_t s)
{
    switch (nbk) {
    case 2: return launch_t<DT, DM, 2>(a, grid, s);
    case 3: return launch_t<DT, DM, 3>(a, grid, s);
    case 4: return launch_t<DT, DM, 4>(a, grid, s);
    case 5: return launch_t<DT, DM, 5>(a, grid, s);
    case 6: return launch_t<DT, DM, 6>(a, grid, s);
    case 7: return launch_t<DT, DM, 7>(a, grid, s);
    default: return launch_t<DT, DM, 8>(a, grid, s);
    }
}

}  // namespace

hipError_t launch_decode_lds(const GemmArgs &a, hipStream_t s)
{
    const int cus = cu_count();
    // about one workgroup per CU: the fewest row blocks per workgroup that
    // cover N in one pass over the CUs, at least 2 (one in flight), at most 8
    const int64_t blocks = (a.N + 15) / 16;
    int64_t nbk = (blocks + cus - 1) / cus;
    nbk = nbk < 2 ? 2 : (nbk > kNBMax ? kNBMax : nbk);
    const int grid = (int)((blocks + nbk - 1) / nbk);
    if (a.norm == NORM_NONE)
        return a.dtype == DT_F16 ? launch_nbk<DT_F16, DM_NONE>(a, (int)nbk, grid, s)
                                 : launch_nbk<DT_BF16, DM_NONE>(a, (int)nbk, grid, s);
    if (a.dtype == DT_F16)
        return launch_nbk<DT_F16, DM_STATS>(a, (int)nbk, grid, s);
    // bf16 RMSNorm without beta: scale after the product (x * gamma stays in
    // bf16 range, no statistics pass before the W stream)
    if (a.norm == NORM_RMSNORM && !a.beta)
        return launch_nbk<DT_BF16, DM_RMS_LATE>(a, (int)nbk, grid, s);
    return launch_nbk<DT_BF16, DM_STATS>(a, (int)nbk, grid, s);
}

}  // namespace ng

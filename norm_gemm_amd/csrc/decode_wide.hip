// decode_wide.hip -- skinny-M (M <= 16) normalization-prologue GEMM for
// 16-byte aligned operands with K % 8 == 0, streaming W in 512-byte row
// pieces.
//
// With M <= 16 the work is bound by reading W[N,K] once (page "华为CANN算子库如何
// 优化大模型推理性能", section 2.2: single-token decode gains most from tiling
// with double buffering). One workgroup of 8 waves owns a slab of 16 * NBK
// rows of W; the waves split K into contiguous ranges of 256-element k-blocks
// and walk them k-block by k-block, each k-block over all NBK row blocks.
//
// W path: a block is 16 rows x 256 k (8 KB), filled by 8 direct HBM -> LDS
// loads of 2 rows x 512 contiguous bytes each. Of the access orders measured
// on MI355X for this k-block-major walk, whole 512-byte row pieces per
// instruction streamed fastest (about 4 % above 128-byte pieces). Each wave
// owns two block slots: while it multiplies one block the next is in flight.
// Row r of a slot holds its 32 chunks of 16 bytes XOR-swizzled by r, so the
// MFMA operand reads (16 rows at one chunk) hit 16 distinct bank groups.
//
// MFMA v_mfma_f32_16x16x32_{f16,bf16}, W as the A operand: for k-step s
// (0..7) of a block, lane l holds W row l % 16, logical chunk 4 s + l / 16;
// the B operand is the normalized x row l % 16 at the same k, computed in
// registers once per k-block (for all row blocks) from raw x, gamma and beta
// loaded one k-block ahead. Result element r of lane l is
// C[4 (l / 16) + r][l % 16] = y^T[n][m]. The 8 waves' K-partials are summed in
// a fixed order through LDS (deterministic).
//
// Row statistics (LayerNorm / RMSNorm over the whole row, fp32 sums) are
// split over all 512 threads; their loads are issued before the first W
// block, so waiting for them does not drain the W stream.
#include <stdint.h>
#include <type_traits>

#include "device_common.h"
#include "launch.h"
#include "route.h"

namespace ng {
namespace {

// Cache policy of the W loads: non-temporal (nt), so the L2 may replace the
// streamed W lines first; every W line is read once per call, and the hint
// keeps them from crowding the L2 (M = 32: 82.6 -> 74.7 us on W[28672, 8192]).
constexpr int kWPolicy = 2;

constexpr int kNW = 8;                   // waves per workgroup
constexpr int kNBMax = 8;                // max 16-row blocks of W per workgroup
constexpr int kSlotChunks = 16 * 32;     // 16 rows x 32 chunks of 16 bytes = 8 KB
constexpr int kKB = 256;                 // k-block (elements)

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
    NM_NONE = 0,      // x as given
    NM_STATS = 1,     // LayerNorm / RMSNorm: statistics pass first, then
                      // (x - mu) * rs * gamma + beta in registers
    NM_RMS_LATE = 2,  // RMSNorm without beta, bf16: x * gamma into the MFMA,
                      // sum of x^2 on the way, rs applied per row at the end
};

// NM = normalization mode; GB: bit 0 gamma present, bit 1 beta present;
// NBK = 16-row blocks of W per workgroup (1..8).
template <int DT, int NM, int GB, int NBK>
__global__ __launch_bounds__(64 * kNW) void decode_wide_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ gamma,
    const uint16_t *__restrict__ beta, const uint16_t *__restrict__ W,
    const uint16_t *__restrict__ bias, uint16_t *__restrict__ y, int M, int N, int K,
    float eps, int norm, int act)
{
    static_assert(NBK >= 1 && NBK <= kNBMax, "1..8 row blocks per workgroup");
    static_assert(NM != NM_RMS_LATE || (GB & 2) == 0, "late RMS scaling has no beta");
    constexpr bool HG = NM != NM_NONE && (GB & 1);     // gamma loaded
    constexpr bool HB = NM == NM_STATS && (GB & 2);    // beta loaded
    constexpr int XL = 8 + (HG ? 8 : 0) + (HB ? 8 : 0);  // loads per x group
    constexpr int BL = 8;                          // loads per W block
    __shared__ u32x4 S0[kNW][kSlotChunks], S1[kNW][kSlotChunks];   // 128 KB
    __shared__ float s_stat[16][2];     // (rs, mu) per row; late RMS: rs (epilogue)
    __shared__ float s_ss[kNW][16];     // NM_RMS_LATE: per-wave sums of x^2

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    // slab of W rows; the last workgroup's slab is moved back to end at N
    // (N >= 16 NBK), overlapping its neighbour, which computes the shared
    // rows bit for bit alike, so every W row index below is in range
    const int n0 = min((int)blockIdx.x * (NBK * 16), N - NBK * 16);

    auto slot = [&](auto S, int w) -> u32x4 * {
        if constexpr (decltype(S)::value == 0)
            return S0[w];
        else
            return S1[w];
    };

    // this wave's K range in 256-element k-blocks
    const int nkb = (K + kKB - 1) / kKB;
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
    const bool has_work = kb0 < kb1;

    // Direct loads of block (kb, nb) into slot SL: load q (0..7) puts row
    // 2q + lane/32 at chunk position lane%32, holding logical chunk
    // (lane%32) ^ row = ((lane%32) ^ (lane/32)) ^ 2q. The row offset is
    // uniform except for lane/32, so the per-lane address part is one small
    // term. A block past this wave's range keeps the load count (and so the
    // waits) uniform: it re-reads the wave's most recently loaded block (the
    // last row block of its last k-block, still in L2) into the slot that
    // was just consumed (never read again). (Direct loads through a buffer
    // descriptor would need fewer registers, but the compiler then loses
    // which LDS slot each load writes and waits for all of them before
    // every LDS read.)
    const int dpos = lane & 31;
    const int drow = lane >> 5;
    const int lchunk = dpos ^ drow;
    const int lrowoff = drow * K;
    auto issue_block = [&](auto SL, int kb, int nb) {
        if (kb >= kb1) {
            kb = kb1 - 1;
            nb = NBK - 1;
        }
        kb = max(kb, 0);
        if (kb >= kb0 && kb < kb1)
            kb = kp(kb);
        u32x4 *dst = slot(SL, wave);
        const uint16_t *wb = W + (int64_t)(n0 + nb * 16) * K;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int k = kb * kKB + (lchunk ^ (2 * q)) * 8;
            __builtin_amdgcn_global_load_lds(
                (const void *)(wb + (int64_t)(2 * q) * K + (lrowoff + (k < K ? k : 0))),
                (__attribute__((address_space(3))) void *)&dst[q * 64], 16, 0, kWPolicy);
        }
    };

    // raw x (row lr, clamped), gamma and beta (when present) of one k-block:
    // chunk 4 s + lg for k-step s; unconditional loads (clamped addresses)
    // so that every x group is exactly XL loads. One register set: a
    // k-block's raw values are normalized before the next k-block's load.
    u32x4 xr[8], gr[8], br[8];
    const uint16_t *xrow = x + (int64_t)min(lr, M - 1) * K;
    auto load_x = [&](int kb) {
        kb = min(kb, nkb - 1);
        if (kb >= kb0 && kb < kb1)
            kb = kp(kb);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int k = kb * kKB + (4 * s + lg) * 8;
            const int kc = k < K ? k : 0;
            xr[s] = ldg128(xrow + kc);
            if constexpr (HG)
                gr[s] = ldg128(gamma + kc);
            if constexpr (HB)
                br[s] = ldg128(beta + kc);
        }
    };

    // ---- prologue: x of the first k-block, statistics loads, first W block.
    // Statistics: wave w owns row min(w, M - 1) (rows 8..15 get a second
    // pass below); each lane loads chunks lane + 64 u, u < 16, of that row
    // up front -- rows of up to 8192 elements in one round trip -- plus the
    // row's first element (the LayerNorm shift). All of these loads are
    // unconditional (clamped) and precede the first W block, so one wait
    // for all but the youngest BL loads covers them and leaves the W block
    // in flight; the first k-block's x wait is then already satisfied.
    const int nchunk = K / 8;
    const bool ln = norm == NORM_LAYERNORM;
    constexpr int kUp = 16;
    u32x4 sv[kUp];
    uint32_t shv = 0;
    const int srow = min(wave, M - 1);
    load_x(kb0);
    issue_fence(x, gamma, beta);
    if constexpr (NM == NM_STATS) {
        const uint16_t *r = x + (int64_t)srow * K;
#pragma unroll
        for (int u = 0; u < kUp; ++u)
            sv[u] = ldg128(r + (int64_t)min(lane + 64 * u, nchunk - 1) * 8);
        shv = r[0];
    }
    issue_fence(x, gamma, beta);
    issue_block(ic<0>{}, kb0, 0);
    if constexpr (NBK >= 2)
        issue_block(ic<1>{}, kb0, 1);
    else
        issue_block(ic<1>{}, kb0 + 1, 0);
    issue_fence(x, gamma, beta);
    // everything but the two W blocks has landed (x group, statistics loads)
    wait_vmcnt<2 * BL>();
    issue_fence(x, gamma, beta);

    float rs = 1.0f, mu = 0.0f;
    if constexpr (NM == NM_STATS) {
        const float invK = 1.0f / (float)K;
        // sums of one row (shifted by its first element for LayerNorm) ->
        // (rs, mu) in s_stat, written by lane 0
        auto finish_row = [&](int m, float s1, float s2, uint32_t h) {
            s1 = wave_sum(s1);
            s2 = wave_sum(s2);
            if (lane == 0) {
                if (ln) {
                    const float md = s1 * invK;
                    const float var = fmaxf(fmaf(-md, md, s2 * invK), 0.0f);
                    s_stat[m][0] = rsqrtf(var + eps);
                    s_stat[m][1] = bits_to_f<DT>((uint16_t)h) + md;
                } else {
                    s_stat[m][0] = rsqrtf(s2 * invK + eps);
                    s_stat[m][1] = 0.0f;
                }
            }
        };
        auto acc_chunk = [&](const u32x4 &v, uint32_t h, float &s1, float &s2) {
            const uint32_t sh2 = ln ? (h | (h << 16)) : 0u;
            if (ln)
                stats_chunk<DT, true>(v, sh2, s1, s2);
            else
                stats_chunk<DT, false>(v, sh2, s1, s2);
        };
        {
            float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
            for (int u = 0; u < kUp; ++u)
                if (lane + 64 * u < nchunk)
                    acc_chunk(sv[u], shv, s1, s2);
            // rows longer than 8192: the remaining chunks (drains W prefetch)
            for (int c = lane + 64 * kUp; c < nchunk; c += 64)
                acc_chunk(ldg128(x + (int64_t)srow * K + (int64_t)c * 8), shv, s1, s2);
            if (wave < M)
                finish_row(wave, s1, s2, shv);
        }
        if (wave + kNW < M) {
            // second row of this wave (M > 8; drains this wave's W prefetch)
            const int m = wave + kNW;
            const uint16_t *r = x + (int64_t)m * K;
            const uint32_t h = r[0];
            float s1 = 0.0f, s2 = 0.0f;
            for (int c = lane; c < nchunk; c += 64)
                acc_chunk(ldg128(r + (int64_t)c * 8), h, s1, s2);
            finish_row(m, s1, s2, h);
        }
        lds_barrier();
        rs = lr < M ? s_stat[lr][0] : 0.0f;
        mu = lr < M ? s_stat[lr][1] : 0.0f;
    }

    // B operands of k-block kb from the raw registers: normalized
    // (NM_STATS), times gamma with the sum of x^2 taken on the way
    // (NM_RMS_LATE), or x itself
    floatx4 accss = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    auto x_frags = [&](int kb, u32x4 (&xf)[8]) {
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const bool live = kb * kKB + (4 * s + lg) * 8 < K && lr < M;
            if constexpr (NM == NM_STATS) {
                float f[8], g[8], bt[8];
                unpack8<DT>(xr[s], f);
                if constexpr (HG)
                    unpack8<DT>(gr[s], g);
                if constexpr (HB)
                    unpack8<DT>(br[s], bt);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float v = (f[e] - mu) * rs;
                    if constexpr (HG && HB)
                        f[e] = fmaf(v, g[e], bt[e]);
                    else if constexpr (HG)
                        f[e] = v * g[e];
                    else if constexpr (HB)
                        f[e] = v + bt[e];
                    else
                        f[e] = v;
                }
                xf[s] = live ? pack8<DT>(f) : u32x4{0u, 0u, 0u, 0u};
            } else if constexpr (NM == NM_RMS_LATE) {
                // x masked once. Sum of x^2 on the matrix cores: the A and B
                // operand layouts of the 16x16x32 MFMA coincide (lane l: row
                // l % 16, k-group l / 16), so x times itself accumulates
                // C[i][j] = sum_k x_ik x_jk, whose diagonal is each row's
                // sum of squares (bf16 products are exact in fp32)
                const u32x4 xz = live ? xr[s] : u32x4{0u, 0u, 0u, 0u};
                accss = mfma16<DT>(xz, xz, accss);
                if constexpr (HG) {
                    float f[8], g[8];
                    unpack8<DT>(xz, f);
                    unpack8<DT>(gr[s], g);
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        f[e] *= g[e];
                    xf[s] = pack8<DT>(f);
                } else {
                    xf[s] = xz;
                }
            } else {
                xf[s] = live ? xr[s] : u32x4{0u, 0u, 0u, 0u};
            }
        }
    };

    floatx4 acc[NBK];
#pragma unroll
    for (int nb = 0; nb < NBK; ++nb)
        acc[nb] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

    // Pipeline: block i of this wave's sequence (k-block major) lives in slot
    // i % 2; after block i has been multiplied, block i + 2 is issued into
    // its slot, so two blocks are in flight while a wave normalizes x or
    // waits. One k-block (PH = parity of its index in this wave's range,
    // which with NBK decides the slots):
    //  - wait for x of kb: younger than it are the blocks issued during
    //    k-block kb - 1 (NBK of them, the last two (kb, 0) and (kb, 1));
    //  - normalize x of kb, then issue x of kb + 1 (if NEXT);
    //  - step nb waits for block (kb, nb): younger than it are block
    //    (kb, nb) + 1 and, for nb < 2 with NEXT, the x group of kb + 1.
    // The compiler may reorder loads only between two waits, which can make
    // a wait stricter, never looser.
    auto kblock = [&](auto PH, auto NEXT, int kb) {
        constexpr int ph = decltype(PH)::value;
        constexpr bool next = decltype(NEXT)::value;
        wait_vmcnt<BL * (NBK >= 2 ? 2 : 1)>();
        u32x4 xf[8];
        const int kbp = kp(kb);           // physical k-block
        x_frags(kbp, xf);
        // the raw registers are free only after x_frags: keep the next
        // k-block's loads behind it (else both register sets are live)
        issue_fence(x, gamma, beta);
        if constexpr (next)
            load_x(kb + 1);
        static_for<0, NBK>([&](auto NB) {
            constexpr int nb = decltype(NB)::value;
            constexpr int sl = (ph * (NBK & 1) + nb) & 1;          // slot of (kb, nb)
            issue_fence(x, gamma, beta);
            if constexpr (next && nb < 2)
                wait_vmcnt<BL + XL>();
            else
                wait_vmcnt<BL>();
            u32x4 *blk = slot(ic<sl>{}, wave);
            if (kbp * kKB + kKB > K) {
                // zero the chunks past K of this lane's own direct loads
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    if (kbp * kKB + (lchunk ^ (2 * q)) * 8 >= K)
                        blk[q * 64 + lane] = u32x4{0u, 0u, 0u, 0u};
                }
            }
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const u32x4 wf = blk[lr * 32 + ((4 * s + lg) ^ lr)];
                acc[nb] = mfma16<DT>(wf, xf[s], acc[nb]);
            }
            // refill this slot with block (kb, nb) + 2 once its reads are
            // consumed (the MFMAs above wait for them)
            issue_fence(x, gamma, beta);
            if constexpr (nb + 2 < NBK)
                issue_block(ic<sl>{}, kb, nb + 2);
            else
                issue_block(ic<sl>{}, kb + (nb + 2) / NBK, (nb + 2) % NBK);
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

    // Partials: wave w writes row block nb into its own slot 0 as
    // float [16 m][16 n] at nb * 1 KB (NBK <= 8 blocks fit in 8 KB): lane
    // (lr, lg) holds n = 4 lg .. 4 lg + 3 of column m = lr, one 16-byte
    // store, and the epilogue's lanes read consecutive n of one m (no LDS
    // bank conflicts either way). Late RMS: the wave's sum of x^2 per row.
    if constexpr (NM == NM_RMS_LATE) {
        // diagonal element i of the 16x16 result sits in lane i + 16 (i / 4),
        // accumulator register i % 4
        if (lg == (lr >> 2)) {
            const int r = lr & 3;
            s_ss[wave][lr] = r == 0 ? accss[0] : r == 1 ? accss[1] : r == 2 ? accss[2] : accss[3];
        }
    }
    {
        floatx4 *p = reinterpret_cast<floatx4 *>(S0[wave]);
#pragma unroll
        for (int nb = 0; nb < NBK; ++nb)
            p[nb * 64 + lr * 4 + lg] = acc[nb];
    }
    lds_barrier();
    if constexpr (NM == NM_RMS_LATE) {
        // each row's scale once: sum of the waves' x^2 in wave order
        if (tid < M) {
            float q = 0.0f;
#pragma unroll
            for (int w = 0; w < kNW; ++w)
                q += s_ss[w][tid];
            s_stat[tid][0] = rsqrtf(q / (float)K + eps);
        }
        lds_barrier();
    }

    // Epilogue: wave w finishes row block nb = w. Lane item (m, q) sums the
    // 8 partials of outputs n = 4 q .. 4 q + 3 of row m in wave order (16-byte
    // LDS reads), scales them (late RMS), adds the bias, applies the
    // activation and rounds once; 8-byte stores where the rows allow them.
    const bool vst = (N & 3) == 0 && ((uintptr_t)y & 7u) == 0;
    if (wave < NBK) {
        const int nb = wave;
        for (int idx = lane; idx < M * 4; idx += 64) {
            const int m = idx >> 2, q = idx & 3;
            floatx4 v = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int w = 0; w < kNW; ++w)
                v += reinterpret_cast<const floatx4 *>(S0[w])[nb * 64 + m * 4 + q];
            const int n = n0 + nb * 16 + 4 * q;
            uint16_t o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float t = v[e];
                if constexpr (NM == NM_RMS_LATE)
                    t *= s_stat[m][0];
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
    }
}

template <int DT, int NM, int GB, int NBK>
hipError_t launch_t(const GemmArgs &a, int grid, hipStream_t s)
{
    hipLaunchKernelGGL((decode_wide_kernel<DT, NM, GB, NBK>), dim3(grid), dim3(64 * kNW), 0, s,
                       (const uint16_t *)a.x, (const uint16_t *)a.gamma,
                       (const uint16_t *)a.beta, (const uint16_t *)a.W,
                       (const uint16_t *)a.bias, (uint16_t *)a.y, (int)a.M, (int)a.N, (int)a.K,
                       a.eps, a.norm, a.act);
    return hipGetLastError();
}

template <int DT, int NM, int GB>
hipError_t launch_nbk(const GemmArgs &a, int nbk, int grid, hipStream_t s)
{
    switch (nbk) {
    case 1: return launch_t<DT, NM, GB, 1>(a, grid, s);
    case 2: return launch_t<DT, NM, GB, 2>(a, grid, s);
    case 3: return launch_t<DT, NM, GB, 3>(a, grid, s);
    case 4: return launch_t<DT, NM, GB, 4>(a, grid, s);
    case 5: return launch_t<DT, NM, GB, 5>(a, grid, s);
    case 6: return launch_t<DT, NM, GB, 6>(a, grid, s);
    case 7: return launch_t<DT, NM, GB, 7>(a, grid, s);
    default: return launch_t<DT, NM, GB, 8>(a, grid, s);
    }
}

template <int DT>
hipError_t launch_dt(const GemmArgs &a, int nbk, int grid, hipStream_t s)
{
    const int gb = (a.gamma ? 1 : 0) | (a.beta ? 2 : 0);
    if (a.norm == NORM_NONE)
        return launch_nbk<DT, NM_NONE, 0>(a, nbk, grid, s);
    if constexpr (DT == DT_BF16) {
        // bf16 has the exponent range of fp32, so x * gamma cannot overflow
        // or lose precision to subnormals where x * rs * gamma would not
        if (a.norm == NORM_RMSNORM && !a.beta)
            return a.gamma ? launch_nbk<DT, NM_RMS_LATE, 1>(a, nbk, grid, s)
                           : launch_nbk<DT, NM_RMS_LATE, 0>(a, nbk, grid, s);
    }
    switch (gb) {
    case 0: return launch_nbk<DT, NM_STATS, 0>(a, nbk, grid, s);
    case 1: return launch_nbk<DT, NM_STATS, 1>(a, nbk, grid, s);
    case 2: return launch_nbk<DT, NM_STATS, 2>(a, nbk, grid, s);
    default: return launch_nbk<DT, NM_STATS, 3>(a, nbk, grid, s);
    }
}

}  // namespace

hipError_t launch_decode_wide(const GemmArgs &a, hipStream_t s)
{
    const int nbk = ng_decode_wide_row_blocks(a.N, cu_count());
    // byte offsets within a slab are 32-bit
    if (ng_route_gemm(a.M, a.N, a.K, a.vec ? 1 : 0, cu_count()) != NG_ROUTE_DECODE_WIDE)
        return hipErrorInvalidValue;
    const int64_t blocks = (a.N + 15) / 16;
    const int grid = (int)((blocks + nbk - 1) / nbk);
    return a.dtype == DT_F16 ? launch_dt<DT_F16>(a, nbk, grid, s)
                             : launch_dt<DT_BF16>(a, nbk, grid, s);
}

}  // namespace ng

// prefill_lds.hip -- the main normalization-prologue GEMM kernel for M > 32
// with 16-byte aligned operands and K % 8 == 0 (page "LayerNorm 融合算子如何让大模型
// 推理再快 15%？深度拆解 ATB 的实现", sections 2.1-3.2: tile-level fusion with the
// normalized tile kept on chip, weights fetched while the statistics are
// computed, aligned contiguous accesses).
//
// Persistent workgroups of 4 waves, one per CU, each walking a list of
// 128 x 256 output tiles that share one 128-row block of x:
//   prologue  W tiles for the first two K steps are requested straight into
//             LDS; the 4 waves reduce the statistics of the block's 128 rows
//             (one pass, packed dot products accumulating in fp32) unless the
//             previous tile had the same rows.
//   K loop    BK = 64. W: HBM -> LDS by direct 128-bit loads (no registers),
//             three stages in flight. x: HBM -> registers -> normalize + affine
//             in fp32 (x*rs + nmr, then *gamma + beta, mixed-precision FMAs)
//             -> one RNE rounding -> LDS, two stages. The normalized x lives
//             only in registers and LDS.
//   MFMA      v_mfma_f32_32x32x16 with W as the first operand and normalized
//             x as the second, so each 32x32 result block is y^T: lane l holds
//             output row m = l % 32 and four consecutive output columns.
//   epilogue  + bias, optional SiLU, one rounding, staged through LDS into
//             row-major order and written with 128-bit stores.
//
// Workgroups are dealt to the 8 XCDs round-robin. When the shape allows, the
// tiles are assigned so that the 32 workgroups of one XCD work at the same
// time on every row block of a few W column blocks: each W tile is fetched
// from HBM once into that XCD's L2 and reused by all row blocks.
//
// LDS tiles are [rows][64] 16-bit elements with the 16-byte chunk index XOR-
// swizzled by (row / 2) % 8; with the MFMA operand pattern (32 rows x one
// chunk per half-wave) this keeps ds_read_b128 free of bank conflicts.
#include <stdlib.h>

#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace ng {
namespace {

constexpr int BM = 128, BN = 256, BK = 64;
constexpr int NWAVE = 8, THREADS = 64 * NWAVE;
constexpr int CPR = BK / 8;                      // 16-byte chunks per tile row
constexpr int A_CH = BM * CPR / THREADS;         // A chunks per thread per K step (4)
constexpr int A_ROWS_PER_PASS = THREADS / CPR;   // 32
constexpr int B_DMA = BN * CPR / THREADS;        // W direct loads per lane per K step (8)
constexpr int A_TILE = BM * CPR, B_TILE = BN * CPR;   // in 16-byte chunks
static_assert(2 * A_TILE * 16 + 4 * B_TILE * 16 == 160 * 1024, "LDS budget");
constexpr int WM = 64, WN = 64;                  // wave tile (m x n)
constexpr int WGM = BM / WM, WGN = BN / WN;      // wave grid (2 x 4)
constexpr int FM = WM / 32, FN = WN / 32;        // 32x32 blocks per wave (2 x 2)
constexpr int B_RPW = BN / NWAVE;                // W rows loaded per wave per K step
static_assert(WGM * WGN == NWAVE && B_RPW % 8 == 0 && B_DMA * 8 == B_RPW, "wave split");

static_assert(A_CH * THREADS == BM * CPR && B_DMA * THREADS == BN * CPR, "tile split");
static_assert(64 * 32 <= B_TILE, "half-tile epilogue staging fits one W stage");

// ds_read_b128 is served 16 lanes (256 bytes, all 64 banks) at a time; with
// 128-byte rows the 16 rows an operand read touches at one chunk land in
// distinct 16-byte bank groups when even and odd rows fall in opposite halves
// of 256 bytes and the chunk index is XORed with (row / 2) % 8.
__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

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

// One normalized chunk: a = (x * rs + nmr) * g + b in fp32, one rounding.
template <int DT>
__device__ __forceinline__ u32x4 normalize_chunk(const u32x4 &raw, float rs, float nmr,
                                                 const float *g, const float *b)
{
    float f[8];
    unpack8<DT>(raw, f);
#pragma unroll
    for (int e = 0; e < 8; ++e)
        f[e] = fmaf(fmaf(f[e], rs, nmr), g[e], b[e]);
    return pack8<DT>(f);
}

// NORM_GEMM_STATS=prologue selects the in-kernel statistics prologue instead of
// the statistics pass (both are correct; used to compare them by measurement).
inline bool stats_in_kernel()
{
    static const bool v = [] {
        const char *e = getenv("NORM_GEMM_STATS");
        return e && e[0] == 'p';
    }();
    return v;
}

struct TileMap {
    int tm, tn, T;      // row blocks, column blocks, tiles
    int xcd;            // 1: XCD-grouped assignment (see file comment)
};

// Tile of workgroup b (one tile per workgroup, T workgroups). XCD-grouped:
// workgroup b runs on XCD b % 8, and the j-th workgroup of an XCD takes row
// block j % tm of column block (b % 8) * (tn / 8) + j / tm, so the workgroups
// an XCD runs together cover every row block of a few W column blocks.
__device__ __forceinline__ void tile_of(const TileMap &mp, int b, int &mb, int &nt)
{
    if (mp.xcd) {
        const int x = b & 7, j = b >> 3;
        mb = j % mp.tm;
        nt = x * (mp.tn >> 3) + j / mp.tm;
        return;
    }
    mb = b % mp.tm;
    nt = b / mp.tm;
}

// Statistics modes of the main kernel.
enum { ST_NONE = 0, ST_PROLOGUE = 1, ST_FROM_Y = 2 };

// Row-statistics pass for ST_FROM_Y: one wave per row of x, one pass over the
// row with 128-bit loads and packed dot products accumulating in fp32, a wave
// reduction, then (rs, nmr) as two floats written into the first 8 bytes of
// the row's slice of every 256-column output tile of y. Each tile of the main
// kernel reads these 8 bytes of its own rows before it writes its own tile,
// so y serves as per-tile scratch and no workgroup reads memory that another
// one writes. Only the statistics pass through device memory; the normalized
// activation never does.
template <int DT>
__global__ __launch_bounds__(256) void row_stats_to_y_kernel(const uint16_t *__restrict__ x,
                                                             uint16_t *__restrict__ y, int M,
                                                             int N, int K, float eps, int norm,
                                                             int tn)
{
    const int lane = threadIdx.x & 63;
    const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (m >= M)
        return;
    const uint16_t *row = x + (int64_t)m * K;
    const bool ln = norm == NORM_LAYERNORM;
    const uint32_t s0 = ln ? (uint32_t)row[0] : 0u;
    const uint32_t sh2 = s0 | (s0 << 16);
    float s1 = 0.0f, s2 = 0.0f;
    const int nch = K / 8;
    int c = lane;
    // eight 16-byte loads in flight per lane before they are consumed
    for (; c + 7 * 64 < nch; c += 8 * 64) {
        u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            v[u] = ldg128(row + (int64_t)(c + u * 64) * 8);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (ln)
                stats_chunk<DT, true>(v[u], sh2, s1, s2);
            else
                stats_chunk<DT, false>(v[u], sh2, s1, s2);
        }
    }
    for (; c < nch; c += 64) {
        const u32x4 v = ldg128(row + (int64_t)c * 8);
        if (ln)
            stats_chunk<DT, true>(v, sh2, s1, s2);
        else
            stats_chunk<DT, false>(v, sh2, s1, s2);
    }
    s1 = wave_sum(s1);
    s2 = wave_sum(s2);
    float rs, nmr;
    finish_stats(s1, s2, bits_to_f<DT>((uint16_t)s0), K, eps, ln, rs, nmr);
    const uint2 pk = make_uint2(__builtin_bit_cast(uint32_t, rs), __builtin_bit_cast(uint32_t, nmr));
    for (int t = lane; t < tn; t += 64)
        *reinterpret_cast<uint2 *>(y + (int64_t)m * N + (int64_t)t * BN) = pk;
}

template <int DT, int STATS>
__global__ __launch_bounds__(THREADS, 1) void prefill_lds_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ gamma,
    const uint16_t *__restrict__ beta, const uint16_t *__restrict__ W,
    const uint16_t *__restrict__ bias, uint16_t *__restrict__ y, int M, int N, int K,
    float eps, int norm, int act, TileMap mp, int vec_out)
{
    constexpr bool AFFINE = STATS != ST_NONE;
    // One LDS object per pipeline stage, so that the compiler can tell the
    // stage being filled by direct loads from the stages being read.
    // 2 x 16 KB (x) + 4 x 32 KB (W) = 160 KB, the whole LDS of a CU.
    __shared__ u32x4 A0[A_TILE], A1[A_TILE];
    __shared__ u32x4 B0[B_TILE], B1[B_TILE], B2[B_TILE], B3[B_TILE];
    // stage buffers by compile-time index
    auto Ast = [&](auto sc) -> u32x4 * {
        if constexpr ((decltype(sc)::value & 1) == 0)
            return A0;
        else
            return A1;
    };
    auto Bst = [&](auto sc) -> u32x4 * {
        constexpr int i = decltype(sc)::value & 3;
        if constexpr (i == 0)
            return B0;
        else if constexpr (i == 1)
            return B1;
        else if constexpr (i == 2)
            return B2;
        else
            return B3;
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    const int lrow = lane & 31, lk = lane >> 5;
    const int cc = tid % CPR, r0 = tid / CPR;      // A chunk coordinates
    // rows r0 + i * A_ROWS_PER_PASS share the swizzle (A_ROWS_PER_PASS % 16 == 0)
    static_assert(A_ROWS_PER_PASS % 16 == 0, "one swizzle for a thread's A rows");
    const int a_woff = r0 * CPR + swz(r0, cc);
    const int nk = (K + BK - 1) / BK;
    const bool k_tail = (K % BK) != 0;
    // gamma / beta are read unconditionally (a valid stand-in pointer when
    // absent) so that the K loop has no branches around its loads
    const bool has_g = gamma != nullptr, has_b = beta != nullptr;
    const uint16_t *gp = has_g ? gamma : x;
    const uint16_t *bp = has_b ? beta : x;

    // (rs, nmr) of this thread's 4 x rows; kept across tiles of one row block
    float rrs[A_CH], rnmr[A_CH];
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
        rrs[i] = 1.0f;
        rnmr[i] = 0.0f;
    }

    {
        int mb, nt;
        tile_of(mp, blockIdx.x, mb, nt);
        const int m0 = mb * BM, n0 = nt * BN;

        // ---- W: direct HBM -> LDS loads of K step kt into stage buffer dst.
        // DMA instruction i of this wave fills rows wave*B_RPW + i*8 .. +7; lane l
        // lands at chunk position l, i.e. row +l/8, physical chunk l%8, which
        // holds logical chunk swz(row, l%8). Rows past N re-read row N-1
        // (their outputs are discarded); steps past the last re-read the last
        // step (never consumed); chunks past K read the row's first chunk and
        // are zeroed once landed (fix_tail).
        const uint16_t *wrow[B_DMA];
        int wch[B_DMA];
#pragma unroll
        for (int i = 0; i < B_DMA; ++i) {
            const int row = wave * B_RPW + i * 8 + (lane >> 3);
            wch[i] = swz(row, lane & 7);
            wrow[i] = W + (int64_t)min(n0 + row, N - 1) * K;
        }
        auto issue_b = [&](int kt, u32x4 *dst) {
            kt = min(kt, nk - 1);
#pragma unroll
            for (int i = 0; i < B_DMA; ++i) {
                const int k = kt * BK + wch[i] * 8;
                __builtin_amdgcn_global_load_lds(
                    (const void *)(wrow[i] + (k < K ? k : 0)),
                    (__attribute__((address_space(3))) void *)&dst[(wave * B_RPW + i * 8) * CPR], 16,
                    0, 0);
            }
        };
        auto fix_tail = [&](u32x4 *dst) {
#pragma unroll
            for (int i = 0; i < B_DMA; ++i) {
                const int row = wave * B_RPW + i * 8 + (lane >> 3);
                if ((nk - 1) * BK + wch[i] * 8 >= K)
                    dst[row * CPR + (lane & 7)] = u32x4{0u, 0u, 0u, 0u};
            }
        };

        // ---- x chunks: registers, branch-free (clamped address, then select)
        const uint16_t *xrow[A_CH];
        bool rlive[A_CH];
#pragma unroll
        for (int i = 0; i < A_CH; ++i) {
            const int m = m0 + r0 + i * A_ROWS_PER_PASS;
            rlive[i] = m < M;
            xrow[i] = x + (int64_t)min(m, M - 1) * K;
        }
        u32x4 ra[2][A_CH], rg[2], rb[2];
        auto load_a = [&](int kt, int set) {
            kt = min(kt, nk - 1);
            const int k = kt * BK + cc * 8;
            const int kc = k < K ? k : 0;
#pragma unroll
            for (int i = 0; i < A_CH; ++i)
                ra[set][i] = ldg128(xrow[i] + kc);
            if constexpr (AFFINE) {
                rg[set] = ldg128(gp + kc);
                rb[set] = ldg128(bp + kc);
            }
        };

        // issue order A(0) B(0) A(1) B(1) B(2): the steady-state step issues
        // A(kt+2) then B(kt+3), and waits until 22 loads remain outstanding
        load_a(0, 0);
        issue_b(0, B0);
        load_a(1, 1);
        issue_b(1, B1);
        issue_b(2, B2);

        if constexpr (STATS == ST_FROM_Y) {
            // statistics left by the statistics pass in this tile's own rows
#pragma unroll
            for (int i = 0; i < A_CH; ++i) {
                const int m = min(m0 + r0 + i * A_ROWS_PER_PASS, M - 1);
                const uint2 pk = *reinterpret_cast<const uint2 *>(y + (int64_t)m * N + n0);
                rrs[i] = __builtin_bit_cast(float, pk.x);
                rnmr[i] = __builtin_bit_cast(float, pk.y);
            }
        } else if constexpr (STATS == ST_PROLOGUE) {
            {
                // one wave per row, 4 rows at a time, reduced in fp32; staged
                // through the second x stage (free until the first K step)
                float *s_rs = reinterpret_cast<float *>(A1);
                float *s_nmr = s_rs + BM;
                const bool ln = norm == NORM_LAYERNORM;
                const int nch = K / 8;
                for (int rr = wave * (BM / NWAVE); rr < (wave + 1) * (BM / NWAVE); rr += 4) {
                    float s1[4] = {0.f, 0.f, 0.f, 0.f}, s2[4] = {0.f, 0.f, 0.f, 0.f};
                    uint32_t sh2[4];
                    const uint16_t *rowp[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int m = min(m0 + rr + q, M - 1);
                        rowp[q] = x + (int64_t)m * K;
                        const uint32_t s0 = ln ? (uint32_t)rowp[q][0] : 0u;
                        sh2[q] = s0 | (s0 << 16);
                    }
                    for (int c = lane; c < nch; c += 64) {
                        u32x4 v[4];
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            v[q] = ldg128(rowp[q] + c * 8);
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            if (ln)
                                stats_chunk<DT, true>(v[q], sh2[q], s1[q], s2[q]);
                            else
                                stats_chunk<DT, false>(v[q], sh2[q], s1[q], s2[q]);
                        }
                    }
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float a1 = wave_sum(s1[q]), a2 = wave_sum(s2[q]);
                        float rs, nmr;
                        finish_stats(a1, a2, bits_to_f<DT>((uint16_t)(sh2[q] & 0xffffu)), K, eps,
                                     ln, rs, nmr);
                        if (lane == 0) {
                            s_rs[rr + q] = rs;
                            s_nmr[rr + q] = nmr;
                        }
                    }
                }
                __syncthreads();
#pragma unroll
                for (int i = 0; i < A_CH; ++i) {
                    rrs[i] = s_rs[r0 + i * A_ROWS_PER_PASS];
                    rnmr[i] = s_nmr[r0 + i * A_ROWS_PER_PASS];
                }
                __syncthreads();
            }
        }

        // normalized (or plain) x chunks of K step kt from register set `set`
        // into stage buffer dst; rows past M and chunks past K become zero
        auto store_a = [&](int kt, int set, u32x4 *dst) {
            const bool kin = kt * BK + cc * 8 < K;
            if constexpr (AFFINE) {
                float g[8], b[8];
                unpack8<DT>(rg[set], g);
                unpack8<DT>(rb[set], b);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    g[e] = has_g ? g[e] : 1.0f;
                    b[e] = has_b ? b[e] : 0.0f;
                }
#pragma unroll
                for (int i = 0; i < A_CH; ++i) {
                    const u32x4 v = normalize_chunk<DT>(ra[set][i], rrs[i], rnmr[i], g, b);
                    dst[a_woff + i * A_ROWS_PER_PASS * CPR] =
                        (kin && rlive[i]) ? v : u32x4{0u, 0u, 0u, 0u};
                }
            } else {
#pragma unroll
                for (int i = 0; i < A_CH; ++i)
                    dst[a_woff + i * A_ROWS_PER_PASS * CPR] =
                        (kin && rlive[i]) ? ra[set][i] : u32x4{0u, 0u, 0u, 0u};
            }
        };

        wait_vmcnt<0>();
        store_a(0, 0, A0);
        if (k_tail && nk == 1)
            fix_tail(B0);
        if (k_tail && nk == 2)
            fix_tail(B1);
        if (k_tail && nk == 3)
            fix_tail(B2);
        lds_barrier();

        floatx16 acc[FN][FM];
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[j][i][e] = 0.0f;

        // Operand chunk of this lane for sub-step kk: rows 32 apart share the
        // swizzle, so one offset per sub-step (plus compile-time row and
        // stage offsets) addresses every fragment of every stage.
        u32x4 wf[2][FN], xf[2][FM];
        auto read_frags = [&](const u32x4 *Ac, const u32x4 *Bc, int kk, int buf) {
            const int sw = swz(lrow, kk * 2 + lk);
            const int aoff = (wm * WM + lrow) * CPR + sw;
            const int boff = (wn * WN + lrow) * CPR + sw;
#pragma unroll
            for (int j = 0; j < FN; ++j)
                wf[buf][j] = Bc[boff + j * 32 * CPR];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                xf[buf][i] = Ac[aoff + i * 32 * CPR];
        };
        auto mfmas = [&](int buf) {
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    acc[j][i] = mfma32<DT>(wf[buf][j], xf[buf][i], acc[j][i]);
        };
        read_frags(A0, B0, 0, 0);

        // One K step (stage indices static through the 4-way unroll):
        //   issue x(kt+2) -> register set kt%2, W(kt+3) -> stage (kt+3)%4;
        //   sub-steps 0..2 of kt, reading sub-step fragments one ahead;
        //   wait until x(kt+1) and W(kt+1) arrived, write normalized x(kt+1);
        //   barrier; fragments of sub-step 0 of kt+1; sub-step 3 of kt.
        constexpr int kInflight = 2 * B_DMA + A_CH + (AFFINE ? 2 : 0);
        auto step = [&](int kt, auto sc) {
            constexpr int s = decltype(sc)::value;
            using S1 = std::integral_constant<int, (s + 1) & 3>;
            using S3 = std::integral_constant<int, (s + 3) & 3>;
            const u32x4 *Ac = Ast(sc);
            const u32x4 *Bc = Bst(sc);
            load_a(kt + 2, s & 1);
            issue_b(kt + 3, Bst(S3{}));
            read_frags(Ac, Bc, 1, 1);
            mfmas(0);
            read_frags(Ac, Bc, 2, 0);
            mfmas(1);
            read_frags(Ac, Bc, 3, 1);
            mfmas(0);
            wait_vmcnt<kInflight>();
            store_a(kt + 1, (s + 1) & 1, Ast(S1{}));
            if (k_tail && kt + 1 == nk - 1)
                fix_tail(Bst(S1{}));
            lds_barrier();
            read_frags(Ast(S1{}), Bst(S1{}), 0, 0);
            mfmas(1);
        };
        for (int kt = 0; kt < nk; kt += 4) {
            step(kt, I0{});
            if (kt + 1 < nk)
                step(kt + 1, I1{});
            if (kt + 2 < nk)
                step(kt + 2, I2{});
            if (kt + 3 < nk)
                step(kt + 3, I3{});
        }
        // drain the clamped loads issued past the last step before LDS reuse
        wait_vmcnt<0>();
        __syncthreads();

        // ---- epilogue: bias + activation in registers, staged row-major in
        // LDS (rows 0-63 in B0, 64-127 in B1; 16-byte chunks XOR-swizzled by
        // row), then written with 128-bit stores
        {
            u32x4 *stg = wm ? B1 : B0;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int nl = wn * WN + j * 32 + q * 8 + lk * 4;
                    float bv[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int n = n0 + nl + r;
                        bv[r] = (bias && n < N) ? bits_to_f<DT>(bias[n]) : 0.0f;
                    }
#pragma unroll
                    for (int i = 0; i < FM; ++i) {
                        const int ml = i * 32 + lrow;            // row within the half
                        float v[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            v[r] = apply_act(acc[j][i][q * 4 + r] + bv[r], act);
                        const int chunk = (nl >> 3) ^ (ml & 31);
                        uint32_t *dst = reinterpret_cast<uint32_t *>(&stg[ml * 32 + chunk]) + (lk * 2);
                        dst[0] = pack2<DT>(v[0], v[1]);
                        dst[1] = pack2<DT>(v[2], v[3]);
                    }
                }
            }
        }
        __syncthreads();
        constexpr int ROWS_PER_PASS = THREADS / 32;
#pragma unroll 4
        for (int p = 0; p < BM / ROWS_PER_PASS; ++p) {
            const int row = p * ROWS_PER_PASS + (tid >> 5), ch = tid & 31;
            const int m = m0 + row, n = n0 + ch * 8;
            const u32x4 *src = row < 64 ? B0 : B1;
            const int rl = row & 63;
            const u32x4 v = src[rl * 32 + (ch ^ (rl & 31))];
            if (m >= M || n >= N)
                continue;
            uint16_t *dst = y + (int64_t)m * N + n;
            if (vec_out && n + 8 <= N) {
                *reinterpret_cast<u32x4 *>(dst) = v;
            } else {
                const int cnt = min(8, N - n);
                for (int e = 0; e < cnt; ++e)
                    dst[e] = (uint16_t)((v[e >> 1] >> ((e & 1) * 16)) & 0xffffu);
            }
        }
        __syncthreads();
    }
}

template <int DT, int STATS>
hipError_t launch_t(const GemmArgs &a, hipStream_t s)
{
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (cus < 1)
        cus = 256;
    TileMap mp;
    mp.tm = (int)((a.M + BM - 1) / BM);
    mp.tn = (int)((a.N + BN - 1) / BN);
    mp.T = mp.tm * mp.tn;
    mp.xcd = (cus % 8 == 0 && mp.tn % 8 == 0) ? 1 : 0;
    const int vec_out = (a.N % 8 == 0 && ((uintptr_t)a.y & 15u) == 0) ? 1 : 0;
    if constexpr (STATS == ST_FROM_Y) {
        hipLaunchKernelGGL((row_stats_to_y_kernel<DT>), dim3((unsigned)((a.M + 3) / 4)), dim3(256),
                           0, s, (const uint16_t *)a.x, (uint16_t *)a.y, (int)a.M, (int)a.N,
                           (int)a.K, a.eps, a.norm, mp.tn);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL((prefill_lds_kernel<DT, STATS>), dim3(mp.T), dim3(THREADS), 0, s,
                       (const uint16_t *)a.x, (const uint16_t *)a.gamma, (const uint16_t *)a.beta,
                       (const uint16_t *)a.W, (const uint16_t *)a.bias, (uint16_t *)a.y, (int)a.M,
                       (int)a.N, (int)a.K, a.eps, a.norm, a.act, mp, vec_out);
    return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const GemmArgs &a, hipStream_t s)
{
    if (a.norm == NORM_NONE)
        return launch_t<DT, ST_NONE>(a, s);
    // The statistics pass needs 8 bytes of y in every tile's rows: every
    // tile (including the last, partial one) must have at least 4 columns
    // and the rows must be 8-byte aligned.
    const bool y_scratch = a.N % 8 == 0 && ((uintptr_t)a.y & 15u) == 0 && !stats_in_kernel();
    return y_scratch ? launch_t<DT, ST_FROM_Y>(a, s) : launch_t<DT, ST_PROLOGUE>(a, s);
}

}  // namespace

hipError_t launch_prefill_lds(const GemmArgs &a, hipStream_t s)
{
    return a.dtype == DT_F16 ? launch_dt<DT_F16>(a, s) : launch_dt<DT_BF16>(a, s);
}

}  // namespace ng

// prefill_lds.hip -- the main normalization-prologue GEMM kernel for M > 32
// with 16-byte aligned operands and K % 8 == 0 (page "LayerNorm 融合算子如何让大模型
// 推理再快 15%？深度拆解 ATB 的实现", sections 2.1-3.2: tile-level fusion with the
// normalized tile kept on chip, weights fetched while the statistics are
// computed, aligned contiguous accesses).
//
// One workgroup of 8 waves per 128 x 256 output tile, one workgroup per CU
// (150 KB of LDS). Each wave computes a 64 x 64 block of the tile.
//   statistics  a separate pass reduces each row of x once (one pass, fp32
//               sum and sum of squares) and leaves (1/sigma, -mu/sigma) in
//               the tile's own rows of y, which the main kernel reads before
//               it writes them (an in-kernel prologue is used when y cannot
//               serve as scratch).
//   K loop      BK = 64, three LDS stages, W loads two steps ahead. W goes
//               HBM -> LDS by direct 128-bit loads (no registers), one after
//               each pair of MFMAs so that the load unit stays busy while the
//               matrix cores run; so does x when it is not normalized. With
//               normalization each lane loads its x chunks of step k + 1
//               into registers at the start of step k, normalizes them in its
//               last sub-step (fp32 arithmetic, one rounding to the operand
//               type) and writes them once into the next stage, so the normalized x
//               lives only in registers and LDS. gamma and beta come with x,
//               or, when both are given, through small LDS slots loaded by
//               one wave per workgroup two steps ahead.
//   gated       (GT) a tile's 256 W rows are the gate and up rows of 128
//               output columns; the epilogue forms act(gate) * up.
//   split K     (SK) workgroups split the K steps of a tile in two and write
//               fp32 partials, summed in order by a second kernel.
//   MFMA        v_mfma_f32_32x32x16 with W as the first operand and normalized
//               x as the second, so each 32x32 result block is y^T: lane l
//               holds output row m = l % 32 and four consecutive columns.
//               Fragments of the next sub-step are read ahead.
//   epilogue    + bias, optional activation, one rounding, staged through LDS into
//               row-major order and written with 128-bit stores.
//
// Workgroups are dealt to the 8 XCDs round-robin. When the shape allows, the
// tiles are assigned so that the 32 workgroups of one XCD work at the same
// time on every row block of a few W column blocks: each W tile is fetched
// from HBM once into that XCD's L2 and reused by all row blocks.
//
// LDS tiles are [rows][64] 16-bit elements with the 16-byte chunk index XOR-
// swizzled by (row / 2) % 8; with the MFMA operand pattern (32 rows x one
// chunk per half-wave) this keeps ds_read_b128 free of bank conflicts.
#include <type_traits>

#include "device_common.h"
#include "launch.h"
#include "route.h"

namespace ng {
namespace {

constexpr int BM = 128, BN = 256, BK = 64;
constexpr int NWAVE = 8, THREADS = 64 * NWAVE;
constexpr int CPR = BK / 8;                      // 16-byte chunks per tile row
constexpr int B_DMA = BN * CPR / THREADS;        // W direct loads per lane per K step (4)
constexpr int A_TILE = BM * CPR, B_TILE = BN * CPR;   // in 16-byte chunks
constexpr int NSTAGE = 3;                        // pipeline stages (loads 2 steps ahead)
constexpr int A_DMA = BM * CPR / THREADS;        // x direct loads per lane per K step (2)
constexpr int A_RPW = BM / NWAVE;                // x rows loaded per wave per K step
constexpr int A_IST = BM / A_DMA;                // rows between a lane's x rows (64)
static_assert(NSTAGE * (A_TILE + B_TILE) * 16 <= 160 * 1024, "LDS budget");
static_assert(A_DMA * 8 == A_RPW && A_IST % 16 == 0, "x rows per wave; one swizzle per lane");
constexpr int WM = 64, WN = 64;                  // wave tile (m x n)
constexpr int WGM = BM / WM, WGN = BN / WN;      // wave grid (2 x 4)
constexpr int FM = WM / 32, FN = WN / 32;        // 32x32 blocks per wave (2 x 2)
constexpr int B_RPW = BN / NWAVE;                // W rows loaded per wave per K step
static_assert(WGM * WGN == NWAVE && B_RPW % 8 == 0 && B_DMA * 8 == B_RPW, "wave split");

static_assert(B_DMA * THREADS == BN * CPR, "tile split");
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
// the row's slice of every tw-column output tile of y. Each tile of the main
// kernel reads these 8 bytes of its own rows before it writes its own tile,
// so y serves as per-tile scratch and no workgroup reads memory that another
// one writes. Only the statistics pass through device memory; the normalized
// activation never does.
template <int DT>
__global__ __launch_bounds__(256) void row_stats_to_y_kernel(const uint16_t *__restrict__ x,
                                                             uint16_t *__restrict__ y, int M,
                                                             int N, int K, float eps, int norm,
                                                             int tn, int tw)
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
        *reinterpret_cast<uint2 *>(y + (int64_t)m * N + (int64_t)t * tw) = pk;
}

// GB: bit 0 gamma present, bit 1 beta present (with STATS != ST_NONE);
// KT: K % 64 != 0 (the last K step is ragged); LN: LayerNorm (else RMSNorm,
// with STATS != ST_NONE); GT: gated output (see the gated epilogue): W is
// [2N, K] = [W_gate; W_up], bias [2N], and a tile covers 128 output columns;
// SK: split K (no normalization): workgroup b computes tile b % T over the
// b / T-th of ksplit contiguous K ranges and writes its fp32 partial sums to
// part[b / T][M][N] (bias and activation are applied by the sum of the
// partials).
template <int DT, int STATS, int GB, bool KT, bool LN, bool GT, bool SK>
__global__ __launch_bounds__(THREADS, 1) void prefill_lds_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ gamma,
    const uint16_t *__restrict__ beta, const uint16_t *__restrict__ W,
    const uint16_t *__restrict__ bias, uint16_t *__restrict__ y, int M, int N, int K,
    float eps, int norm, int act, TileMap mp, int vec_out, float *__restrict__ part, int ksplit)
{
    static_assert(!SK || (STATS == ST_NONE && !GT), "split K only for the plain GEMM");
    constexpr bool AFFINE = STATS != ST_NONE;
    constexpr bool HG = AFFINE && (GB & 1), HB = AFFINE && (GB & 2);
    // direct loads per lane per K step: W, plus x when it is not normalized
    // (normalized x, gamma and beta come through registers)
    constexpr int LPS = AFFINE ? B_DMA : B_DMA + A_DMA;
    static_assert(A_DMA == 2, "two x chunks per lane");
    // One LDS object per pipeline stage and operand
    __shared__ u32x4 A0[A_TILE], A1[A_TILE], A2[A_TILE];
    __shared__ u32x4 B0[B_TILE], B1[B_TILE], B2[B_TILE];
    // gamma (chunks 0-7) and beta (chunks 8-15) of one K step, in three slots
    // used like the stages (see the K step); one chunk per lane of a wave
    __shared__ u32x4 G0[64], G1[64], G2[64];
    auto Ast = [&](auto sc) -> u32x4 * {
        constexpr int i = decltype(sc)::value % NSTAGE;
        if constexpr (i == 0)
            return A0;
        else if constexpr (i == 1)
            return A1;
        else
            return A2;
    };
    auto Bst = [&](auto sc) -> u32x4 * {
        constexpr int i = decltype(sc)::value % NSTAGE;
        if constexpr (i == 0)
            return B0;
        else if constexpr (i == 1)
            return B1;
        else
            return B2;
    };
    auto Gst = [&](auto sc) -> u32x4 * {
        constexpr int i = decltype(sc)::value % NSTAGE;
        if constexpr (i == 0)
            return G0;
        else if constexpr (i == 1)
            return G1;
        else
            return G2;
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WGN, wn = wave % WGN;
    const int lrow = lane & 31, lk = lane >> 5;
    // K range of this workgroup: all of K, or with split K the ks-th of
    // ksplit ranges of whole K steps (the host gives every range a step).
    // Ke is the extent of the range; K stays the row stride.
    const int ks = SK ? (int)blockIdx.x / mp.T : 0;
    const int nks = SK ? ((K + BK - 1) / BK + ksplit - 1) / ksplit : 0;
    const int kbase = SK ? ks * nks * BK : 0;
    const int Ke = SK ? min(K - kbase, nks * BK) : K;
    const int nk = (Ke + BK - 1) / BK;
    constexpr bool k_tail = KT;

    // output columns per tile: 256, or 128 gated (the 256 W rows of a tile are
    // the gate and up rows of the same 128 columns)
    constexpr int BNO = GT ? BN / 2 : BN;
    int mb, nt;
    tile_of(mp, SK ? (int)blockIdx.x % mp.T : (int)blockIdx.x, mb, nt);
    const int m0 = mb * BM, n0 = nt * BNO;

    // ---- direct HBM -> LDS loads. Instruction i of a wave fills 8 tile rows
    // (x: i*A_IST + wave*8 .., W: wave*B_RPW + i*8 ..); lane l lands at chunk
    // position l, i.e. row +l/8, physical chunk l%8, which holds logical chunk
    // swz(row, l%8). Rows past M or N re-read the last row (x rows are zeroed
    // when normalized, W rows' outputs are discarded); steps past the last
    // re-read the last step (never consumed).
    // Addressing: a uniform base (tile origin + K step, scalar registers)
    // plus a per-lane 32-bit byte offset that is fixed for the whole tile, so
    // no address register is rewritten while its load is in flight (the
    // compiler would wait for the load before reusing it). The last K step
    // of a ragged K has its own fixed offsets: chunks past K re-read the
    // row's last valid chunk (in bounds) and are zeroed once landed.
    const int kl = (nk - 1) * BK;                     // first k of the last step
    const int clast = (Ke - kl + 7) / 8 - 1;          // last valid chunk in it
    auto tail_chunk = [&](int c) { return kl + c * 8 < Ke ? c : clast; };
    int wch[B_DMA], ach[A_DMA];
    uint32_t woff[B_DMA], woff_t[B_DMA], aoff_g[A_DMA], aoff_t[A_DMA];
    bool alive[A_DMA];
    const uint16_t *wtile = W + (int64_t)n0 * K + kbase;
    const uint16_t *xtile = x + (int64_t)m0 * K + kbase;
#pragma unroll
    for (int i = 0; i < B_DMA; ++i) {
        const int row = wave * B_RPW + i * 8 + (lane >> 3);
        wch[i] = swz(row, lane & 7);
        // W row of tile row `row`, relative to n0. Gated: tile rows 64 w + r
        // (r < 32) hold the gate row of output column 32 w + r and rows
        // 64 w + 32 + r the up row of the same column, so that each wave's
        // two 32-row MFMA blocks are the gate and up halves of its columns.
        int src;
        if constexpr (GT) {
            const int f = min(n0 + (row >> 6) * 32 + (row & 31), N - 1) - n0;
            src = (row & 32) ? N + f : f;
        } else {
            src = min(n0 + row, N - 1) - n0;
        }
        const uint32_t rb = (uint32_t)src * (uint32_t)K;
        woff[i] = (rb + wch[i] * 8) * 2u;
        woff_t[i] = (rb + tail_chunk(wch[i]) * 8) * 2u;
    }
#pragma unroll
    for (int i = 0; i < A_DMA; ++i) {
        const int row = i * A_IST + wave * 8 + (lane >> 3);
        ach[i] = swz(row, lane & 7);
        alive[i] = m0 + row < M;
        const uint32_t rb = (uint32_t)(min(m0 + row, M - 1) - m0) * (uint32_t)K;
        aoff_g[i] = (rb + ach[i] * 8) * 2u;
        aoff_t[i] = (rb + tail_chunk(ach[i]) * 8) * 2u;
    }
    // gamma / beta chunk of this lane's x chunks (tail: clamped in bounds)
    const uint32_t goff = ach[0] * 16u, goff_t = tail_chunk(ach[0]) * 16u;
    auto issue = [&](int kt, u32x4 *As, u32x4 *Bs) {
        kt = min(kt, nk - 1);
        const bool tl = KT && kt == nk - 1;
        const char *wb = reinterpret_cast<const char *>(wtile) + (size_t)kt * (BK * 2);
        const char *xb = reinterpret_cast<const char *>(xtile) + (size_t)kt * (BK * 2);
        if constexpr (!AFFINE) {
#pragma unroll
            for (int i = 0; i < A_DMA; ++i)
                dma16(xb, tl ? aoff_t[i] : aoff_g[i], lds_addr(&As[(i * A_IST + wave * 8) * CPR]));
        }
#pragma unroll
        for (int i = 0; i < B_DMA; ++i)
            dma16(wb, tl ? woff_t[i] : woff[i], lds_addr(&Bs[(wave * B_RPW + i * 8) * CPR]));
    };

    // (rs, nmr) of the rows of this lane's x chunks
    float rrs[A_DMA], rnmr[A_DMA];
#pragma unroll
    for (int i = 0; i < A_DMA; ++i) {
        rrs[i] = 1.0f;
        rnmr[i] = 0.0f;
    }
    if constexpr (STATS == ST_FROM_Y) {
        // statistics left by the statistics pass in this tile's own rows
#pragma unroll
        for (int i = 0; i < A_DMA; ++i) {
            const int m = min(m0 + i * A_IST + wave * 8 + (lane >> 3), M - 1);
            const uint2 pk = *reinterpret_cast<const uint2 *>(y + (int64_t)m * N + n0);
            rrs[i] = __builtin_bit_cast(float, pk.x);
            rnmr[i] = __builtin_bit_cast(float, pk.y);
        }
        // complete them before the direct loads start: the compiler does not
        // count those, so only an empty queue tells it these have landed
        wait_vmcnt<0>();
    } else if constexpr (STATS == ST_PROLOGUE) {
        // one wave per row, 4 rows at a time, reduced in fp32; exchanged
        // through the third x stage (not loaded before the first K step)
        float *s_rs = reinterpret_cast<float *>(A2);
        float *s_nmr = s_rs + BM;
        const bool ln = LN;
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
                finish_stats(a1, a2, bits_to_f<DT>((uint16_t)(sh2[q] & 0xffffu)), K, eps, ln, rs,
                             nmr);
                if (lane == 0) {
                    s_rs[rr + q] = rs;
                    s_nmr[rr + q] = nmr;
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < A_DMA; ++i) {
            const int row = i * A_IST + wave * 8 + (lane >> 3);
            rrs[i] = s_rs[row];
            rnmr[i] = s_nmr[row];
        }
        __syncthreads();
    }

    // x chunks of K step kt that this lane loaded: normalized + affine in
    // fp32, x * rs + nmr, then * gamma + beta, rounded once to the operand
    // type (fp16: mixed-precision FMAs read the fp16 inputs directly and the
    // last one rounds to fp16), written back in place; rows past M and chunks past K become
    // zero. A lane's x rows are A_IST apart: one swizzle, so one logical
    // chunk and one gamma / beta chunk for all of them. Split into the LDS
    // reads and the arithmetic + write so that MFMAs can run in between.
    struct NormRaw {
        u32x4 v[A_DMA], g, b;
    };
    // x / gamma / beta chunks of K step kt into registers (asynchronous: see
    // ldg16_async; NXL loads, completed by wait_vmcnt_tied)
    constexpr int NXL = A_DMA + (HG ? 1 : 0) + (HB ? 1 : 0);
    // With both gamma and beta they come through LDS slots (issue_gb), read
    // at the start of the step before the one that uses them; with one of
    // them, straight into registers with x (measured faster there).
    constexpr bool RING = HG && HB;
    auto load_gb_regs = [&](int kt, NormRaw &r) {
        kt = min(kt, nk - 1);
        const bool tl = KT && kt == nk - 1;
        const char *gb = reinterpret_cast<const char *>(gamma) + (size_t)kt * (BK * 2);
        const char *bb = reinterpret_cast<const char *>(beta) + (size_t)kt * (BK * 2);
        if constexpr (HG)
            r.g = ldg16_async(gb, tl ? goff_t : goff);
        if constexpr (HB)
            r.b = ldg16_async(bb, tl ? goff_t : goff);
    };
    auto load_raw = [&](int kt, NormRaw &r) {
        kt = min(kt, nk - 1);
        const bool tl = KT && kt == nk - 1;
        const char *xb = reinterpret_cast<const char *>(xtile) + (size_t)kt * (BK * 2);
#pragma unroll
        for (int i = 0; i < A_DMA; ++i)
            r.v[i] = ldg16_async(xb, tl ? aoff_t[i] : aoff_g[i]);
        r.g = r.b = u32x4{0u, 0u, 0u, 0u};
        if constexpr (!RING)
            load_gb_regs(kt, r);
    };
    // gamma / beta of K step kt into a slot: one direct load by wave 0 alone,
    // lanes 0-7 the gamma chunks and 8-15 the beta chunks (past K: the last
    // valid chunk; the other lanes repeat them). All waves of all CUs loading
    // the same two lines every step would queue their requests at one L2
    // channel; this is one request per line per CU and step. Issued two steps
    // ahead: wave 0's waits on its x loads of the same step cover it, and the
    // step's barrier publishes it.
    auto issue_gb = [&](int kt, u32x4 *Gs) {
        if constexpr (RING) {
            if (wave == 0) {
                kt = min(kt, nk - 1);
                const int c = lane & 7;
                const int k = (kt * BK + c * 8 < K) ? kt * BK + c * 8 : kl + clast * 8;
                dma16_ptr(((lane & 8) == 0 ? gamma : beta) + k, lds_addr(Gs));
            }
        }
    };
    // (only with RING: otherwise the slots are never written and gamma / beta
    // came into registers with x)
    auto read_gb = [&](const u32x4 *Gs, NormRaw &r) {
        if constexpr (RING) {
            r.g = Gs[ach[0]];
            r.b = Gs[CPR + ach[0]];
        }
    };
    auto nrm_store = [&](int kt, u32x4 *As, const NormRaw &r) {
        const bool kin = kt * BK + ach[0] * 8 < K;
        float g[8], bt[8];
        if constexpr (HG)
            unpack8<DT>(r.g, g);
        if constexpr (HB)
            unpack8<DT>(r.b, bt);
#pragma unroll
        for (int i = 0; i < A_DMA; ++i) {
            const bool live = alive[i] && kin;
            float f[8];
            unpack8<DT>(r.v[i], f);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float v = fmaf(f[e], rrs[i], rnmr[i]);
                if constexpr (HG && HB)
                    f[e] = fmaf(v, g[e], bt[e]);
                else if constexpr (HG)
                    f[e] = v * g[e];
                else if constexpr (HB)
                    f[e] = v + bt[e];
                else
                    f[e] = v;
            }
            As[(i * A_IST + wave * 8) * CPR + lane] =
                live ? pack8<DT>(f) : u32x4{0u, 0u, 0u, 0u};
        }
    };
    // without normalization only the chunks past K of the last step need
    // zeroing (rows past M re-read row M - 1 and their outputs are dropped)
    auto zero_tail_x = [&](u32x4 *As) {
        if ((nk - 1) * BK + ach[0] * 8 >= Ke) {
#pragma unroll
            for (int i = 0; i < A_DMA; ++i)
                As[(i * A_IST + wave * 8) * CPR + lane] = u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto fix_tail = [&](u32x4 *Bs) {
#pragma unroll
        for (int i = 0; i < B_DMA; ++i) {
            const int row = wave * B_RPW + i * 8 + (lane >> 3);
            if ((nk - 1) * BK + wch[i] * 8 >= Ke)
                Bs[row * CPR + (lane & 7)] = u32x4{0u, 0u, 0u, 0u};
        }
    };

    // ---- prologue: K steps 0 and 1 in flight; step 0 normalized
    issue_fence(x, gamma, beta);
    if constexpr (AFFINE) {
        NormRaw r0;
        load_raw(0, r0);
        if constexpr (RING)
            load_gb_regs(0, r0);
        issue_gb(1, G1);
        issue(0, A0, B0);
        issue(1, A1, B1);
        wait_vmcnt_tied<2 * LPS>(r0.v[0], r0.v[1], r0.g, r0.b);
        nrm_store(0, A0, r0);
    } else {
        issue(0, A0, B0);
        issue(1, A1, B1);
    }
    issue_fence(x, gamma, beta);
    wait_vmcnt<LPS>();                 // this wave's loads of step 0 have landed
    issue_fence(x, gamma, beta);
    if (k_tail && nk == 1) {
        if constexpr (!AFFINE)
            zero_tail_x(A0);
        fix_tail(B0);
    }
    lds_barrier();

    floatx16 acc[FN][FM];
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[j][i][e] = 0.0f;

    // Operand chunks of this lane for sub-step kk: rows 32 apart share the
    // swizzle, so one offset per sub-step (plus compile-time row and stage
    // offsets) addresses every fragment of every stage.
    struct Frag {
        u32x4 w[FN], a[FM];
    };
    auto rdfrag = [&](const u32x4 *Ac, const u32x4 *Bc, int kk, Frag &f) {
        const int sw = swz(lrow, kk * 2 + lk);
        const int aoff = (wm * WM + lrow) * CPR + sw;
        const int boff = (wn * WN + lrow) * CPR + sw;
#pragma unroll
        for (int j = 0; j < FN; ++j)
            f.w[j] = Bc[boff + j * 32 * CPR];
#pragma unroll
        for (int i = 0; i < FM; ++i)
            f.a[i] = Ac[aoff + i * 32 * CPR];
    };
    auto mm = [&](const Frag &f, int j) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
            acc[j][i] = mfma32<DT>(f.w[j], f.a[i], acc[j][i]);
    };
    auto sb = [] { __builtin_amdgcn_sched_barrier(0); };

    // One K step on stage kt % 3. The direct loads of step kt + 2 go into the
    // stage read in step kt - 1 (free since that step's barrier), one after
    // a pair of MFMAs, so that the load unit is fed while the matrix cores
    // run; fragments of the next sub-step are read before the MFMAs of the
    // current one.
    //   normalized x: the x / gamma / beta chunks of step kt + 1 are loaded
    //   into registers at the start of the step; in sub-step 3 (younger are
    //   only the three W loads issued since) they are normalized and written
    //   once into stage (kt + 1) % 3, last read in step kt - 2. W goes one
    //   load per sub-step.
    //   plain x: x and W of step kt + 2 both go direct, in the first six
    //   slots.
    // At the end this wave's loads of step kt + 1 have landed (the LPS of
    // step kt + 2 are the only younger ones); the barrier makes step kt + 1
    // complete for every wave and frees stage kt % 3.
    auto step = [&](int kt, auto sc) {
        constexpr int s = decltype(sc)::value;
        using S1 = std::integral_constant<int, s + 1>;
        using S2 = std::integral_constant<int, s + 2>;
        const u32x4 *Ac = Ast(sc);
        const u32x4 *Bc = Bst(sc);
        u32x4 *An = Ast(S2{}), *Bn = Bst(S2{});
        const int kn = min(kt + 2, nk - 1);
        const bool tl = KT && kn == nk - 1;
        const char *wb = reinterpret_cast<const char *>(wtile) + (size_t)kn * (BK * 2);
        const char *xb = reinterpret_cast<const char *>(xtile) + (size_t)kn * (BK * 2);
        // load slot d: x chunks first when x goes direct, then W
        auto slot = [&](auto dc) {
            constexpr int d = decltype(dc)::value;
            constexpr int NA = AFFINE ? 0 : A_DMA;
            if constexpr (d < NA) {
                dma16(xb, tl ? aoff_t[d] : aoff_g[d],
                      lds_addr(&An[(d * A_IST + wave * 8) * CPR]));
            } else if constexpr (d < LPS) {
                constexpr int i = d - NA;
                dma16(wb, tl ? woff_t[i] : woff[i],
                      lds_addr(&Bn[(wave * B_RPW + i * 8) * CPR]));
            }
            sb();
        };
        using D0 = std::integral_constant<int, 0>;
        using D1 = std::integral_constant<int, 1>;
        using D2 = std::integral_constant<int, 2>;
        using D3 = std::integral_constant<int, 3>;
        using D4 = std::integral_constant<int, 4>;
        using D5 = std::integral_constant<int, 5>;
        Frag f0, f1;
        issue_fence(x, gamma, beta);
        if constexpr (AFFINE) {
            static_assert(LPS == 4, "one W load per sub-step");
            issue_gb(kt + 2, Gst(S2{}));
            NormRaw raw;
            load_raw(kt + 1, raw);
            // published by the barrier that ended step kt - 1
            read_gb(Gst(S1{}), raw);
            sb();
            rdfrag(Ac, Bc, 0, f0);
            sb();
            rdfrag(Ac, Bc, 1, f1);
            sb();
            mm(f0, 0);
            sb();
            slot(D0{});
            mm(f0, 1);
            sb();
            rdfrag(Ac, Bc, 2, f0);
            sb();
            mm(f1, 0);
            sb();
            slot(D1{});
            mm(f1, 1);
            sb();
            rdfrag(Ac, Bc, 3, f1);
            sb();
            mm(f0, 0);
            sb();
            slot(D2{});
            mm(f0, 1);
            sb();
            wait_vmcnt_tied<3>(raw.v[0], raw.v[1], raw.g, raw.b);
            mm(f1, 0);
            // (in the last step this normalizes a stage that is never read)
            nrm_store(kt + 1, Ast(S1{}), raw);
            sb();
            slot(D3{});
            mm(f1, 1);
            sb();
        } else {
            static_assert(LPS == 6, "six direct loads per K step");
            rdfrag(Ac, Bc, 0, f0);
            sb();
            rdfrag(Ac, Bc, 1, f1);
            sb();
            mm(f0, 0);
            sb();
            slot(D0{});
            mm(f0, 1);
            sb();
            slot(D1{});
            rdfrag(Ac, Bc, 2, f0);
            sb();
            mm(f1, 0);
            sb();
            slot(D2{});
            mm(f1, 1);
            sb();
            slot(D3{});
            rdfrag(Ac, Bc, 3, f1);
            sb();
            mm(f0, 0);
            sb();
            slot(D4{});
            mm(f0, 1);
            sb();
            slot(D5{});
            mm(f1, 0);
            sb();
            mm(f1, 1);
            sb();
        }
        wait_vmcnt<LPS>();
        issue_fence(x, gamma, beta);
        if (k_tail && kt + 1 == nk - 1) {
            if constexpr (!AFFINE)
                zero_tail_x(Ast(S1{}));
            fix_tail(Bst(S1{}));
        }
        lds_barrier();
    };
    for (int kt = 0; kt < nk; kt += NSTAGE) {
        step(kt, I0{});
        if (kt + 1 < nk)
            step(kt + 1, I1{});
        if (kt + 2 < nk)
            step(kt + 2, I2{});
    }
    // drain the clamped loads issued past the last step before LDS reuse
    wait_vmcnt<0>();
    __syncthreads();

    if constexpr (SK) {
        // ---- split-K epilogue: fp32 partials straight from the accumulators,
        // four consecutive columns (16 bytes) per lane and 32x32 block row
        float *pp = part + (size_t)ks * M * N;
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + wn * WN + j * 32 + q * 8 + lk * 4;
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    const int m = m0 + wm * WM + i * 32 + lrow;
                    if (m >= M || n >= N)
                        continue;
                    float *dst = pp + (size_t)m * N + n;
                    if (n + 4 <= N && (N & 3) == 0) {
                        *reinterpret_cast<floatx4 *>(dst) =
                            floatx4{acc[j][i][q * 4], acc[j][i][q * 4 + 1], acc[j][i][q * 4 + 2],
                                    acc[j][i][q * 4 + 3]};
                    } else {
                        for (int r = 0; r < 4 && n + r < N; ++r)
                            dst[r] = acc[j][i][q * 4 + r];
                    }
                }
            }
        return;
    }
    if constexpr (GT) {
        // ---- gated epilogue: each lane holds the gate (j = 0) and up (j = 1)
        // sums of the same output elements; h = act(gate + b_gate) *
        // (up + b_up) in fp32, one rounding, staged row-major in B0 (128 rows
        // x 16 chunks, 16-byte chunks XOR-swizzled by row), then written with
        // 128-bit stores
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int nl = wn * 32 + q * 8 + lk * 4;          // column within the tile
            float bg[4], bu[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int n = n0 + nl + r;
                const bool ok = bias && n < N;
                bg[r] = ok ? bits_to_f<DT>(bias[n]) : 0.0f;
                bu[r] = ok ? bits_to_f<DT>(bias[N + n]) : 0.0f;
            }
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int ml = wm * WM + i * 32 + lrow;       // row within the tile
                float v[4];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    v[r] = apply_act(acc[0][i][q * 4 + r] + bg[r], act) *
                           (acc[1][i][q * 4 + r] + bu[r]);
                const int chunk = (nl >> 3) ^ (ml & 15);
                uint32_t *dst = reinterpret_cast<uint32_t *>(&B0[ml * 16 + chunk]) + (lk * 2);
                dst[0] = pack2<DT>(v[0], v[1]);
                dst[1] = pack2<DT>(v[2], v[3]);
            }
        }
        __syncthreads();
#pragma unroll 4
        for (int p = 0; p < BM / 32; ++p) {
            const int row = p * 32 + (tid >> 4), ch = tid & 15;
            const int m = m0 + row, n = n0 + ch * 8;
            const u32x4 v = B0[row * 16 + (ch ^ (row & 15))];
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
        return;
    }
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
}

template <int DT, int STATS, int GB, bool KT, bool LN, bool GT, bool SK = false>
hipError_t launch_k(const GemmArgs &a, hipStream_t s, float *part = nullptr, int ksplit = 1)
{
    const int cus = cu_count();
    constexpr int BNO = GT ? BN / 2 : BN;
    TileMap mp;
    mp.tm = (int)((a.M + BM - 1) / BM);
    mp.tn = (int)((a.N + BNO - 1) / BNO);
    mp.T = mp.tm * mp.tn;
    mp.xcd = (cus % 8 == 0 && mp.tn % 8 == 0) ? 1 : 0;
    const int vec_out = (a.N % 8 == 0 && ((uintptr_t)a.y & 15u) == 0) ? 1 : 0;
    if constexpr (STATS == ST_FROM_Y) {
        hipLaunchKernelGGL((row_stats_to_y_kernel<DT>), dim3((unsigned)((a.M + 3) / 4)), dim3(256),
                           0, s, (const uint16_t *)a.x, (uint16_t *)a.y, (int)a.M, (int)a.N,
                           (int)a.K, a.eps, a.norm, mp.tn, BNO);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL((prefill_lds_kernel<DT, STATS, GB, KT, LN, GT, SK>), dim3(mp.T * ksplit),
                       dim3(THREADS), 0, s,
                       (const uint16_t *)a.x, (const uint16_t *)a.gamma, (const uint16_t *)a.beta,
                       (const uint16_t *)a.W, (const uint16_t *)a.bias, (uint16_t *)a.y, (int)a.M,
                       (int)a.N, (int)a.K, a.eps, a.norm, a.act, mp, vec_out, part, ksplit);
    return hipGetLastError();
}

template <int DT, int STATS, int GB, bool LN, bool GT>
hipError_t launch_t(const GemmArgs &a, hipStream_t s)
{
    return a.K % BK ? launch_k<DT, STATS, GB, true, LN, GT>(a, s)
                    : launch_k<DT, STATS, GB, false, LN, GT>(a, s);
}

template <int DT, int STATS, bool LN, bool GT>
hipError_t launch_gb(const GemmArgs &a, hipStream_t s)
{
    switch ((a.gamma ? 1 : 0) | (a.beta ? 2 : 0)) {
    case 0: return launch_t<DT, STATS, 0, LN, GT>(a, s);
    case 1: return launch_t<DT, STATS, 1, LN, GT>(a, s);
    case 2: return launch_t<DT, STATS, 2, LN, GT>(a, s);
    default: return launch_t<DT, STATS, 3, LN, GT>(a, s);
    }
}

template <int DT, int STATS, bool GT>
hipError_t launch_norm(const GemmArgs &a, hipStream_t s)
{
    return a.norm == NORM_LAYERNORM ? launch_gb<DT, STATS, true, GT>(a, s)
                                    : launch_gb<DT, STATS, false, GT>(a, s);
}

template <int DT, bool GT>
hipError_t launch_dt(const GemmArgs &a, hipStream_t s)
{
    if (a.norm == NORM_NONE)
        return launch_t<DT, ST_NONE, 0, false, GT>(a, s);
    // The statistics pass needs 8 bytes of y in every tile's rows: every
    // tile (including the last, partial one) must have at least 4 columns
    // and the rows must be 8-byte aligned.
    const bool y_scratch = a.N % 8 == 0 && ((uintptr_t)a.y & 15u) == 0;
    return y_scratch ? launch_norm<DT, ST_FROM_Y, GT>(a, s) : launch_norm<DT, ST_PROLOGUE, GT>(a, s);
}

}  // namespace

hipError_t launch_prefill_lds(const GemmArgs &a, hipStream_t s)
{
    // tile offsets are 32-bit (see ng_tile_offsets_fit)
    static_assert(BN == NG_TILE_ROWS && BM <= BN, "tile rows");
    if (ng_route_gemm(a.M, a.N, a.K, a.vec ? 1 : 0, cu_count()) != NG_ROUTE_PREFILL_LDS)
        return hipErrorInvalidValue;
    return a.dtype == DT_F16 ? launch_dt<DT_F16, false>(a, s) : launch_dt<DT_BF16, false>(a, s);
}

int prefill_tiles(int64_t M, int64_t N)
{
    return (int)(((M + BM - 1) / BM) * ((N + BN - 1) / BN));
}

int prefill_k_steps(int64_t K)
{
    return (int)((K + BK - 1) / BK);
}

hipError_t launch_prefill_lds_splitk(const GemmArgs &a, float *part, int ksplit,
                                     hipStream_t s)
{
    // plain GEMM only; every K range must get at least one step
    if (ng_route_gemm(a.M, a.N, a.K, a.vec ? 1 : 0, cu_count()) != NG_ROUTE_PREFILL_LDS ||
        a.norm != NORM_NONE || ksplit < 2 || prefill_k_steps(a.K) < 2 * ksplit)
        return hipErrorInvalidValue;
    const bool kt = a.K % BK != 0;
    if (a.dtype == DT_F16)
        return kt ? launch_k<DT_F16, ST_NONE, 0, true, false, false, true>(a, s, part, ksplit)
                  : launch_k<DT_F16, ST_NONE, 0, false, false, false, true>(a, s, part, ksplit);
    return kt ? launch_k<DT_BF16, ST_NONE, 0, true, false, false, true>(a, s, part, ksplit)
              : launch_k<DT_BF16, ST_NONE, 0, false, false, false, true>(a, s, part, ksplit);
}

hipError_t launch_prefill_lds_gated(const GemmArgs &a, hipStream_t s)
{
    // W row offsets within a tile (up to N + 127 rows past its first gate
    // row) are 32-bit byte offsets
    if (!ng_gated_tiled_fits(a.M, a.N, a.K, a.vec ? 1 : 0))
        return hipErrorInvalidValue;
    return a.dtype == DT_F16 ? launch_dt<DT_F16, true>(a, s) : launch_dt<DT_BF16, true>(a, s);
}

}  // namespace ng

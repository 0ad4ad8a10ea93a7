// prefill_lds.hip -- the main normalization-prologue GEMM kernel for M > 32
// with 16-byte aligned operands and K % 8 == 0 (page "LayerNorm 融合算子如何让大模型
// 推理再快 15%？深度拆解 ATB 的实现", sections 2.1-3.2: tile-level fusion with the
// normalized tile kept on chip, weights fetched while the statistics are
// computed, aligned contiguous accesses).
//
// One workgroup of 8 waves per 128 x 256 output tile, one workgroup per CU
// (144 KB of LDS: three stages of a 128 x 64 x tile and a 256 x 64 W tile).
// Each wave computes a 64 x 64 block of the tile.
//   statistics  a separate pass reduces each row of x once (one pass, fp32
//               sum and sum of squares) and leaves (1/sigma, -mu/sigma) in
//               the tile's own rows of y, which the main kernel reads before
//               it writes them (an in-kernel prologue is used when y cannot
//               serve as scratch).
//   K loop      BK = 64, three LDS stages, loads two steps ahead. W goes
//               HBM -> LDS by direct 128-bit loads (no registers); so does x
//               when it is not normalized. With normalization each lane
//               loads its x chunks (and its gamma / beta chunk) into
//               registers two steps ahead, normalizes them between its own
//               MFMAs of the step before they are needed (fp32 arithmetic,
//               one rounding to the operand type) and writes them once into
//               their stage, so the normalized x lives only in registers and
//               LDS.
//   schedule    the two waves of each SIMD alternate a memory phase (LDS
//               fragment reads, load issue) and an MFMA phase, so the matrix
//               core of every SIMD always has a wave with operands ready
//               (see the kernel).
//   gated       (GT) a tile's 256 W rows are the gate and up rows of 128
//               output columns; the epilogue forms act(gate) * up. When the
//               tiles take more than one round and the last holds at most
//               half of the CUs, that round's tiles run as two K halves whose
//               fp32 gate / up sums a small kernel combines.
//   split K     (SK) workgroups split the K steps of a tile into ksplit
//               ranges, or (skipped slice) one workgroup per tile skips one
//               slice of K steps that a spare workgroup computes; each part
//               is written as fp32 partials, summed in order by a second
//               kernel.
//   folding     (FOLD) W holds gamma folded in, x goes to the MFMAs raw and
//               the epilogue applies the row statistics and two folded
//               vectors (see the kernel).
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
    int tails, len;     // skipped-slice split K: spare workgroups per XCD and
                        // slice length in K steps (tails 0: not used)
    int split_from;     // gated: workgroups from this index on compute K halves
                        // of the last tiles (split_from = T: none)
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
// ST_FROM_Y_PS: statistics from y, fp16 RMSNorm without beta, power-of-two
// prescaled operand (see the kernel).
enum { ST_NONE = 0, ST_PROLOGUE = 1, ST_FROM_Y = 2, ST_FROM_Y_PS = 3 };

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
// KT: K % 64 != 0 (the last K step is ragged); GT: gated output (see the
// gated epilogue): W is [2N, K] = [W_gate; W_up], bias [2N], and a tile
// covers 128 output columns; SK: split K (no normalization): the tile's K
// range is one part of its K steps (the kernel below says which) and its fp32
// partial sums go to one plane part[p][M][N] (bias and activation are applied
// by the sum of the partials). norm selects LayerNorm or RMSNorm for
// the in-kernel statistics (STATS == ST_PROLOGUE). FOLD: inference-mode
// folding (page "LayerNorm 融合算子如何让大模型推理再快 15%？深度拆解 ATB 的实现",
// section 6.2, tip 2): W holds W' = W * gamma, x goes to the MFMAs unnormalized
// (direct loads, as without normalization), and the epilogue applies the row
// statistics and the folded vectors: act(rs acc + (-mu rs) c1 + c2), which is
// rs (x W'^T - mu c1) + c2 (c1 = W' 1, c2 = W beta + bias, both fp32; c1 is
// not read for RMSNorm).
//
// Schedule ("ping-pong"). Waves w and w + 4 of a workgroup run on the same
// SIMD (workgroups are dealt to SIMDs that way), and the two groups of four
// waves alternate between two phases separated by workgroup barriers:
//   memory phase of step kt: read all of this wave's MFMA fragments of step
//     kt from LDS into registers; issue the x / gamma / beta register loads
//     of a later step and (first group) the direct loads of step kt + 2;
//   compute phase of step kt: the 16 MFMAs of step kt, with this wave's x
//     chunks of a later step normalized into their stage between them
//     (second group: the direct loads of step kt + 3 first).
// Waves 4-7 start one phase later, so while one wave of a SIMD runs its
// MFMAs the other runs its memory phase (LDS reads, load issue), and the
// matrix core of every SIMD always has a wave with operands ready. Each
// stage is read by the first group in phase 2 kt and by the second in phase
// 2 kt + 1, so a stage is rewritten (direct loads of kt + 3, normalized x of
// kt + 3) only from phase 2 kt + 2 on. The exact load order and waits are
// given with the prologue below.
//
// One output tile (row block mb, column block nt) over Ke elements of K from
// kbase; with split K its fp32 sums go to plane `plane` of part, and K steps
// gap_at on are taken gap_len steps further on (a skipped slice).
template <int DT, int STATS, int GB, bool KT, bool GT, bool SK, bool FOLD>
__device__ __forceinline__ void prefill_tile(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ gamma,
    const uint16_t *__restrict__ beta, const uint16_t *__restrict__ W,
    const uint16_t *__restrict__ bias, uint16_t *__restrict__ y, int M, int N, int K,
    float eps, int norm, int act, int vec_out, float *__restrict__ part,
    const float *__restrict__ c1, const float *__restrict__ c2, int mb, int nt, int kbase,
    int Ke, int plane, int gap_at, int gap_len)
{
    static_assert(!SK || (STATS == ST_NONE && !GT), "split K only for the plain GEMM");
    static_assert(!FOLD || (STATS == ST_FROM_Y || STATS == ST_PROLOGUE) && !GT && !SK && GB == 0,
                  "folding: plain GEMM on raw x with row statistics");
    // normalization inside the K loop (not with folding: x stays raw)
    constexpr bool AFFINE = STATS != ST_NONE && !FOLD;
    // Prescaled fp16 RMSNorm (no beta): the A operand is x * 2^e * gamma,
    // rounded once to fp16, with 2^e the power of two at or below the row's
    // rs = 1/sqrt(mean(x^2) + eps) (e clamped to the fp16 normal exponents
    // -14..15, so 2^e is an fp16 value and x * 2^e is exact). The epilogue
    // multiplies the fp32 sum by rs * 2^-e, which is exact scaling of the
    // same sum: y = rs 2^-e sum_k fp16(x_k 2^e gamma_k) W_k. Two packed fp16
    // products per two elements replace the fp32 normalization, and the
    // operand values keep the range of the normalized row (|x 2^e| <= |x rs|).
    constexpr bool PS = STATS == ST_FROM_Y_PS;
    static_assert(!PS || (DT == DT_F16 && !(GB & 2)), "prescale: fp16 without beta");
    constexpr bool HG = AFFINE && (GB & 1), HB = AFFINE && (GB & 2);
    // direct loads per lane per K step: W, plus x when it is not normalized
    // (normalized x, gamma and beta come through registers)
    constexpr int LPS = AFFINE ? B_DMA : B_DMA + A_DMA;
    static_assert(A_DMA == 2, "two x chunks per lane");
    // One LDS object per pipeline stage and operand
    __shared__ u32x4 A0[A_TILE], A1[A_TILE], A2[A_TILE];
    __shared__ u32x4 B0[B_TILE], B1[B_TILE], B2[B_TILE];
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
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WGN, wn = wave % WGN;   // wm is also the phase group
    const int lrow = lane & 31, lk = lane >> 5;
    // K range of this tile: Ke elements from kbase (K stays the row stride)
    const int nk = (Ke + BK - 1) / BK;

    // output columns per tile: 256, or 128 gated (the 256 W rows of a tile are
    // the gate and up rows of the same 128 columns)
    constexpr int BNO = GT ? BN / 2 : BN;
    const int m0 = mb * BM, n0 = nt * BNO;

    // ---- direct HBM -> LDS loads. Instruction i of a wave fills 8 tile rows
    // (x: i*A_IST + wave*8 .., W: wave*B_RPW + i*8 ..); lane l lands at chunk
    // position l, i.e. row +l/8, physical chunk l%8, which holds logical chunk
    // swz(row, l%8). Rows past M or N re-read the last row (x rows are zeroed
    // when normalized, W rows' outputs are discarded); steps past the last
    // re-read the last step (never consumed).
    // Addressing: a uniform base (tile origin + K step, scalar registers)
    // plus a per-lane 32-bit byte offset that is fixed for the whole tile
    // (the host routes shapes whose offsets would reach 2^32 elsewhere), so
    // no address register is rewritten while its load is in flight. The last
    // K step of a ragged K has its own fixed offsets: chunks past K re-read
    // the row's last valid chunk (in bounds) and are zeroed once landed.
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
    auto issue_dma = [&](int kt, u32x4 *As, u32x4 *Bs) {
        kt = min(kt, nk - 1);
        const bool tl = KT && kt == nk - 1;
        const int kg = SK && kt >= gap_at ? kt + gap_len : kt;   // step within K
        const char *wb = reinterpret_cast<const char *>(wtile) + (size_t)kg * (BK * 2);
        const char *xb = reinterpret_cast<const char *>(xtile) + (size_t)kg * (BK * 2);
        if constexpr (!AFFINE) {
#pragma unroll
            for (int i = 0; i < A_DMA; ++i)
                dma16(xb, tl ? aoff_t[i] : aoff_g[i], lds_addr(&As[(i * A_IST + wave * 8) * CPR]));
        }
#pragma unroll
        for (int i = 0; i < B_DMA; ++i)
            dma16(wb, tl ? woff_t[i] : woff[i], lds_addr(&Bs[(wave * B_RPW + i * 8) * CPR]));
    };

    // (rs, nmr) of the rows of this lane's x chunks: normalized = x rs + nmr
    float rrs[A_DMA], rnmr[A_DMA];
#pragma unroll
    for (int i = 0; i < A_DMA; ++i) {
        rrs[i] = 1.0f;
        rnmr[i] = 0.0f;
    }
    // prescale: 2^e of this lane's x rows (packed fp16) and rs 2^-e of the
    // output rows of its accumulators (rows wm * 64 + 32 i + lrow)
    half2_t ps2[A_DMA];
    // epilogue factors of the output rows of this lane's accumulators (rows
    // wm * 64 + 32 i + lrow): v = osc acc + onm c1 + (c2 or bias)
    float osc[FM], onm[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        osc[i] = 1.0f;
        onm[i] = 0.0f;
    }
    auto pow2_below = [](float rs) {
        // 2^e <= rs, e = floor(log2 rs) clamped to -14..15 (rs > 0, finite)
        int e = (int)((__builtin_bit_cast(uint32_t, rs) >> 23) & 0xffu) - 127;
        e = e < -14 ? -14 : (e > 15 ? 15 : e);
        return __builtin_bit_cast(float, (uint32_t)(e + 127) << 23);
    };
    if constexpr (STATS == ST_FROM_Y || PS) {
        // statistics left by the statistics pass in this tile's own rows
#pragma unroll
        for (int i = 0; i < A_DMA; ++i) {
            const int m = min(m0 + i * A_IST + wave * 8 + (lane >> 3), M - 1);
            const uint2 pk = *reinterpret_cast<const uint2 *>(y + (int64_t)m * N + n0);
            rrs[i] = __builtin_bit_cast(float, pk.x);
            rnmr[i] = __builtin_bit_cast(float, pk.y);
        }
        if constexpr (PS || FOLD) {
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int m = min(m0 + wm * WM + i * 32 + lrow, M - 1);
                const uint2 pk = *reinterpret_cast<const uint2 *>(y + (int64_t)m * N + n0);
                const float rs = __builtin_bit_cast(float, pk.x);
                if constexpr (PS) {
                    osc[i] = rs / pow2_below(rs);
                } else {
                    osc[i] = rs;
                    onm[i] = __builtin_bit_cast(float, pk.y);
                }
            }
        }
        // complete them before the direct loads start: the compiler does not
        // count those, so only an empty queue tells it these have landed
        wait_vmcnt<0>();
        if constexpr (PS) {
#pragma unroll
            for (int i = 0; i < A_DMA; ++i) {
                const _Float16 sh = (_Float16)pow2_below(rrs[i]);
                ps2[i] = half2_t{sh, sh};
            }
        }
    } else if constexpr (STATS == ST_PROLOGUE) {
        // one wave per row, 4 rows at a time, reduced in fp32; exchanged
        // through the third x stage (not loaded before the first K step)
        float *s_rs = reinterpret_cast<float *>(A2);
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
        if constexpr (FOLD) {
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                osc[i] = s_rs[wm * WM + i * 32 + lrow];
                onm[i] = s_nmr[wm * WM + i * 32 + lrow];
            }
        }
        __syncthreads();
    }

    // x chunks of one K step that this lane loads, with its gamma / beta
    // chunk: loaded asynchronously into registers (ldg16_async), completed by
    // wait_vmcnt_tied, then normalized + affine in fp32, x * rs + nmr, then
    // * gamma + beta, rounded once to the operand type (fp16: mixed-precision
    // FMAs read the fp16 inputs directly and the last one rounds to fp16),
    // and written once into the step's stage; rows past M and chunks past K
    // become zero. A lane's x rows are A_IST apart: one swizzle, so one
    // logical chunk and one gamma / beta chunk for all of them.
    struct NormRaw {
        u32x4 v[A_DMA], g, b;
    };
    // two register buffers: the x chunks of step kt go to buffer kt % 2 and
    // are loaded two steps before they are normalized
    NormRaw raw[2];
    auto load_raw = [&](int kt, NormRaw &r) {
        kt = min(kt, nk - 1);
        const bool tl = KT && kt == nk - 1;
        const char *xb = reinterpret_cast<const char *>(xtile) + (size_t)kt * (BK * 2);
#pragma unroll
        for (int i = 0; i < A_DMA; ++i)
            r.v[i] = ldg16_async(xb, tl ? aoff_t[i] : aoff_g[i]);
        const char *gb = reinterpret_cast<const char *>(gamma) + (size_t)(kbase + kt * BK) * 2;
        const char *bb = reinterpret_cast<const char *>(beta) + (size_t)(kbase + kt * BK) * 2;
        if constexpr (HG)
            r.g = ldg16_async(gb, tl ? goff_t : goff);
        else
            r.g = u32x4{0u, 0u, 0u, 0u};
        if constexpr (HB)
            r.b = ldg16_async(bb, tl ? goff_t : goff);
        else
            r.b = u32x4{0u, 0u, 0u, 0u};
    };
    // one of this lane's x chunks of step kt
    auto nrm_chunk = [&](int kt, u32x4 *As, const NormRaw &r, int i) {
        const bool live = alive[i] && kt * BK + ach[0] * 8 < Ke;
        if constexpr (PS) {
            u32x4 v = r.v[i];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                // copy the elements first (bit_cast of a vector element
                // reference is miscompiled)
                const uint32_t xw = v[d], gw = r.g[d];
                half2_t t = __builtin_bit_cast(half2_t, xw) * ps2[i];   // exact
                if constexpr (HG)
                    t = t * __builtin_bit_cast(half2_t, gw);            // one rounding
                v[d] = __builtin_bit_cast(uint32_t, t);
            }
            As[(i * A_IST + wave * 8) * CPR + lane] = live ? v : u32x4{0u, 0u, 0u, 0u};
            return;
        }
        float g[8], bt[8];
        if constexpr (HG)
            unpack8<DT>(r.g, g);
        if constexpr (HB)
            unpack8<DT>(r.b, bt);
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
        const u32x4 pk = pack8<DT>(f);
        As[(i * A_IST + wave * 8) * CPR + lane] = live ? pk : u32x4{0u, 0u, 0u, 0u};
    };
    auto nrm_store = [&](int kt, u32x4 *As, const NormRaw &r) {
#pragma unroll
        for (int i = 0; i < A_DMA; ++i)
            nrm_chunk(kt, As, r, i);
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
    auto sb = [] { __builtin_amdgcn_sched_barrier(0); };
    // plain workgroup barrier of the compute phase (no LDS access to wait for)
    auto phase_barrier = [&] {
        sb();
        asm volatile("s_barrier" ::: "memory");
        sb();
    };

    // ---- load order and waits. Loads complete in issue order, so a wait
    // for one load is a wait for every older one; the orders below let each
    // wait name only what is due (NXL = x / gamma / beta register loads of a
    // step, LPS = direct loads of a step). The normalization runs in the
    // compute phases, between a wave's own MFMAs, so that the memory phase
    // (the one on the LDS) holds only fragment reads and load issue:
    //   group 0: memory phase kt issues x of kt + 2, then the direct loads of
    //            kt + 2; compute phase kt normalizes x of kt + 1 into its
    //            stage and ends by awaiting the direct loads of kt + 1;
    //   group 1: memory phase kt issues x of kt + 3 and awaits the direct
    //            loads of kt + 1; compute phase kt starts with the direct
    //            loads of kt + 3 (their stage was last read in the phase
    //            before) and normalizes x of kt + 2 into its stage.
    // Every stage is complete one barrier before the first group reads it;
    // x gets three phases to arrive, the direct loads three to four.
    constexpr int NXL = AFFINE ? A_DMA + (HG ? 1 : 0) + (HB ? 1 : 0) : 0;
    auto tied_wait = [&](auto nc, NormRaw &r) {
        wait_vmcnt_tied<decltype(nc)::value>(r.v[0], r.v[1], r.g, r.b);
    };
    using C0 = std::integral_constant<int, 0>;
    using CX = std::integral_constant<int, NXL + 2 * LPS>;    // x of the step due
    constexpr int CL = NXL + LPS;                             // group 0: loads of kt + 1
    constexpr int CW = 2 * NXL + LPS;                         // group 1: loads of kt + 1

    // ---- prologue: step 0 complete in its stage, the loads of steps 1-2
    // in flight in each group's steady-state order. The x chunks of step j
    // go to register buffer j % 2 in group 0 and (j + 1) % 2 in group 1, so
    // that in every K step both groups load into buffer kt % 2 and
    // normalize from the other one.
    issue_fence(x, gamma, beta);
    if constexpr (AFFINE) {
        if (wm == 0) {
            load_raw(0, raw[0]);
            issue_dma(0, A0, B0);
            load_raw(1, raw[1]);
            issue_dma(1, A1, B1);
            tied_wait(std::integral_constant<int, NXL + 2 * LPS>{}, raw[0]);
            nrm_store(0, A0, raw[0]);
            issue_fence(x, gamma, beta);
            wait_vmcnt<NXL + LPS>();          // the direct loads of step 0
        } else {
            load_raw(0, raw[1]);
            issue_dma(0, A0, B0);
            load_raw(1, raw[0]);
            issue_dma(1, A1, B1);
            tied_wait(std::integral_constant<int, NXL + 2 * LPS>{}, raw[1]);
            nrm_store(0, A0, raw[1]);
            issue_fence(x, gamma, beta);
            load_raw(2, raw[1]);
            wait_vmcnt<2 * NXL + LPS>();      // the direct loads of step 0
        }
    } else {
        issue_dma(0, A0, B0);
        issue_dma(1, A1, B1);
        wait_vmcnt<LPS>();
    }
    issue_fence(x, gamma, beta);
    if (KT && nk == 1) {
        if constexpr (!AFFINE)
            zero_tail_x(A0);
        fix_tail(B0);
    }
    lds_barrier();
    if (wm == 1) {
        // the second group starts one phase later; its first phase does what
        // each of its compute phases does for kt + 3 and kt + 2: the direct
        // loads of step 2, and its x rows of step 1
        issue_dma(2, A2, B2);
        if constexpr (AFFINE) {
            tied_wait(CX{}, raw[0]);
            nrm_store(1, A1, raw[0]);
            lds_barrier();
        } else {
            phase_barrier();
        }
    }

    floatx16 acc[FN][FM];
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[j][i][e] = 0.0f;

    // this wave's fragments of one K step: [sub-step][32-row block]; rows
    // 32 apart share the swizzle, so one offset per sub-step addresses every
    // fragment of a stage
    u32x4 fa[4][FM], fb[4][FN];
    auto read_frags = [&](const u32x4 *Ac, const u32x4 *Bc) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int sw = swz(lrow, kk * 2 + lk);
            const int aoff = (wm * WM + lrow) * CPR + sw;
            const int boff = (wn * WN + lrow) * CPR + sw;
#pragma unroll
            for (int j = 0; j < FN; ++j)
                fb[kk][j] = Bc[boff + j * 32 * CPR];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                fa[kk][i] = Ac[aoff + i * 32 * CPR];
        }
    };
    auto mfma_kk = [&](int kk) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int i = 0; i < FM; ++i)
                acc[j][i] = mfma32<DT>(fb[kk][j], fa[kk][i], acc[j][i]);
    };
    // the step's MFMAs; with normalization, x of step kn from buffer r is
    // normalized into stage As between them, a few VALU instructions after
    // each MFMA (scheduling groups), so the VALU work issues while the matrix
    // core runs the MFMAs before it instead of holding the next one back
    auto compute = [&](int kn, u32x4 *As, NormRaw &r) {
        if constexpr (AFFINE) {
            mfma_kk(0);
            nrm_chunk(kn, As, r, 0);
            mfma_kk(1);
            nrm_chunk(kn, As, r, 1);
            mfma_kk(2);
            mfma_kk(3);
#pragma unroll
            for (int i = 0; i < 4 * FM * FN; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);   // up to five VALU
            }
            sb();
        } else {
            mfma_kk(0);
            sb();
            mfma_kk(1);
            sb();
            mfma_kk(2);
            sb();
            mfma_kk(3);
            sb();
        }
    };
    auto tail_fix = [&](int kt, auto s1) {
        if (KT && kt + 1 == nk - 1) {
            if constexpr (!AFFINE)
                zero_tail_x(Ast(s1));
            fix_tail(Bst(s1));
        }
    };

    // one K step (memory phase, then compute phase) of this wave; J = kt % 6
    // gives the stages (J % 3, + 1, + 2) and the x buffers. The MFMAs are one
    // code path for both groups (so the accumulators stay in place); the
    // groups differ only in which loads they issue and await where, and in
    // the step they normalize (group 0: kt + 1, group 1: kt + 2).
    auto kstep = [&](int kt, auto jc) {
        constexpr int J = decltype(jc)::value;
        using S0 = std::integral_constant<int, J % 3>;
        using S1 = std::integral_constant<int, J % 3 + 1>;
        using S2 = std::integral_constant<int, J % 3 + 2>;
        NormRaw &rl = raw[J % 2];           // loaded in this memory phase
        NormRaw &rn = raw[(J + 1) % 2];     // normalized in this compute phase
        issue_fence(x, gamma, beta);
        // memory phase
        read_frags(Ast(S0{}), Bst(S0{}));
        sb();
        if constexpr (AFFINE)
            load_raw(kt + 2 + wm, rl);
        if (wm == 0) {
            issue_dma(kt + 2, Ast(S2{}), Bst(S2{}));
        } else {
            wait_vmcnt<AFFINE ? CW : LPS>();   // the direct loads of kt + 1
            issue_fence(x, gamma, beta);
            tail_fix(kt, S1{});
        }
        lds_barrier();
        // compute phase
        sb();
        if (wm == 1)
            issue_dma(kt + 3, Ast(S0{}), Bst(S0{}));
        if constexpr (AFFINE)
            tied_wait(CX{}, rn);
        sb();
        compute(kt + 1 + wm, wm ? Ast(S2{}) : Ast(S1{}), rn);
        if (wm == 0) {
            wait_vmcnt<AFFINE ? CL : LPS>();   // the direct loads of kt + 1
            issue_fence(x, gamma, beta);
            tail_fix(kt, S1{});
        }
        lds_barrier();
    };
    using J0 = std::integral_constant<int, 0>;
    using J1 = std::integral_constant<int, 1>;
    using J2 = std::integral_constant<int, 2>;
    using J3 = std::integral_constant<int, 3>;
    using J4 = std::integral_constant<int, 4>;
    using J5 = std::integral_constant<int, 5>;
    for (int kt = 0; kt < nk; kt += 6) {
        kstep(kt, J0{});
        if (kt + 1 < nk)
            kstep(kt + 1, J1{});
        if (kt + 2 < nk)
            kstep(kt + 2, J2{});
        if (kt + 3 < nk)
            kstep(kt + 3, J3{});
        if (kt + 4 < nk)
            kstep(kt + 4, J4{});
        if (kt + 5 < nk)
            kstep(kt + 5, J5{});
    }
    if (wm == 0)
        phase_barrier();        // the second group's last compute phase
    // drain the clamped loads issued past the last step before LDS reuse; the
    // x registers of the last (unused) loads stay live until they have landed
    if constexpr (AFFINE) {
        tied_wait(C0{}, raw[0]);
        tied_wait(C0{}, raw[1]);
    } else {
        wait_vmcnt<0>();
    }
    __syncthreads();

    if constexpr (SK) {
        // ---- split-K epilogue: fp32 partials straight from the accumulators,
        // four consecutive columns (16 bytes) per lane and 32x32 block row
        float *pp = part + (size_t)plane * M * N;
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
        if (plane >= 0) {
            // ---- a K half of a split tile: the fp32 gate (j = 0) and up
            // (j = 1) sums times the row factor, stored as the tile's block
            // [128 rows][gate 128 | up 128] (no bias, no activation)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int nl = wn * 32 + q * 8 + lk * 4;
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    const int ml = wm * WM + i * 32 + lrow;
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        *reinterpret_cast<floatx4 *>(part + ml * 256 + j * 128 + nl) =
                            floatx4{acc[j][i][q * 4] * osc[i], acc[j][i][q * 4 + 1] * osc[i],
                                    acc[j][i][q * 4 + 2] * osc[i], acc[j][i][q * 4 + 3] * osc[i]};
                }
            }
            return;
        }
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
                    v[r] = apply_act(fmaf(acc[0][i][q * 4 + r], osc[i], bg[r]), act) *
                           fmaf(acc[1][i][q * 4 + r], osc[i], bu[r]);
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
                float bv[4], cv[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int n = n0 + nl + r;
                    if constexpr (FOLD) {
                        bv[r] = n < N ? c2[n] : 0.0f;
                        cv[r] = (c1 && n < N) ? c1[n] : 0.0f;
                    } else {
                        bv[r] = (bias && n < N) ? bits_to_f<DT>(bias[n]) : 0.0f;
                        cv[r] = 0.0f;
                    }
                }
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    const int ml = i * 32 + lrow;            // row within the half
                    float v[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        v[r] = apply_act(
                            fmaf(acc[j][i][q * 4 + r], osc[i], fmaf(onm[i], cv[r], bv[r])), act);
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

// Workgroup b computes one tile over the whole K, except with split K (SK):
//   uniform (mp.tails == 0): tile b % T over the b / T-th of ksplit
//     contiguous K ranges of whole steps, partial sums to plane b / T;
//   skipped slice (mp.tails > 0, tn % 8 == 0): on XCD b % 8 the j-th
//     workgroup (j = b / 8) with j < T / 8 computes local tile j (the
//     XCD-grouped tile order) over all K steps but those of slot j / tails
//     (steps [slot len, slot len + len)) into plane 0; workgroup T / 8 + e
//     computes, for slot i = 0, 1, ..., the skipped slice of local tile
//     i tails + e into plane 1. The workgroups that skip a slice at a given
//     slot run it at the same time as the spare workgroups, which so read
//     the same x steps as the tiles that have not reached their own slice.
template <int DT, int STATS, int GB, bool KT, bool GT, bool SK, bool FOLD>
__global__ __launch_bounds__(THREADS, 1) void prefill_lds_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ gamma,
    const uint16_t *__restrict__ beta, const uint16_t *__restrict__ W,
    const uint16_t *__restrict__ bias, uint16_t *__restrict__ y, int M, int N, int K,
    float eps, int norm, int act, TileMap mp, int vec_out, float *__restrict__ part, int ksplit,
    const float *__restrict__ c1, const float *__restrict__ c2)
{
    const int b = blockIdx.x;
    int nseg = 1;                 // tiles (segments) of this workgroup
    if constexpr (SK) {
        if (mp.tails > 0 && (b >> 3) >= (mp.T >> 3))
            nseg = (mp.T >> 3) / mp.tails;
    }
    for (int sg = 0; sg < nseg; ++sg) {
        // plane: the partial-sum plane of a split K (every split path sets
        // it), -1 for a whole tile
        int mb, nt, kbase = 0, Ke = K, plane = -1, gap_at = 1 << 30, gap_len = 0;
        float *pt = part;
        if constexpr (SK) {
            if (mp.tails > 0) {
                const int xc = b & 7, j = b >> 3, tx = mp.T >> 3;
                const int u = j < tx ? j : sg * mp.tails + (j - tx);   // local tile
                mb = u % mp.tm;
                nt = xc * (mp.tn >> 3) + u / mp.tm;
                if (j < tx) {
                    Ke = K - mp.len * BK;
                    gap_at = (u / mp.tails) * mp.len;
                    gap_len = mp.len;
                    plane = 0;
                } else {
                    kbase = sg * mp.len * BK;
                    Ke = mp.len * BK;
                    plane = 1;
                }
            } else {
                // every range gets at least one step (checked by the host)
                const int ks = b / mp.T;
                const int nks = ((K + BK - 1) / BK + ksplit - 1) / ksplit;
                kbase = ks * nks * BK;
                Ke = min(K - kbase, nks * BK);
                plane = ks;
                tile_of(mp, b % mp.T, mb, nt);
            }
        } else if (GT && b >= mp.split_from) {
            // gated, last round: workgroup split_from + 2 s + h computes K half
            // h of tile split_from + s (first half: the first ceil(nkt / 2)
            // steps) into plane h of that tile's partial block
            const int hw = b - mp.split_from, st = hw >> 1, S = mp.T - mp.split_from;
            tile_of(mp, mp.split_from + st, mb, nt);
            const int k1 = ((K + BK - 1) / BK + 1) / 2 * BK;
            kbase = (hw & 1) ? k1 : 0;
            Ke = (hw & 1) ? K - k1 : k1;
            plane = hw & 1;
            pt = part + ((size_t)plane * S + st) * (BM * 256);
        } else {
            tile_of(mp, b, mb, nt);
        }
        prefill_tile<DT, STATS, GB, KT, GT, SK, FOLD>(x, gamma, beta, W, bias, y, M, N, K, eps,
                                                       norm, act, vec_out, pt, c1, c2, mb, nt,
                                                       kbase, Ke, plane, gap_at, gap_len);
    }
}

// The gated outputs of the split tiles from the two partial blocks of each:
// h = act(g0 + g1 + b_gate) * (u0 + u1 + b_up) in fp32, the halves added in
// order, one rounding. Workgroup 16 s + g covers rows 8 g .. 8 g + 7 of split
// tile s (tile split_from + s); each thread four consecutive outputs of one
// row, stored as one 8-byte write when they are whole and aligned.
template <int DT>
__global__ __launch_bounds__(256) void gated_split_sum_kernel(const float *__restrict__ part,
                                                              const uint16_t *__restrict__ bias,
                                                              uint16_t *__restrict__ h, int M,
                                                              int F, int act, TileMap mp)
{
    const int st = blockIdx.x >> 4, S = mp.T - mp.split_from;
    int mb, nt;
    tile_of(mp, mp.split_from + st, mb, nt);
    const int r = (blockIdx.x & 15) * 8 + (threadIdx.x >> 5), c = (threadIdx.x & 31) * 4;
    const int m = mb * BM + r, n0 = nt * 128 + c;
    if (m >= M || n0 >= F)
        return;
    const float *p0 = part + (size_t)st * (BM * 256) + r * 256 + c;
    const float *p1 = part + ((size_t)S + st) * (BM * 256) + r * 256 + c;
    const floatx4 g0 = *reinterpret_cast<const floatx4 *>(p0);
    const floatx4 g1 = *reinterpret_cast<const floatx4 *>(p1);
    const floatx4 u0 = *reinterpret_cast<const floatx4 *>(p0 + 128);
    const floatx4 u1 = *reinterpret_cast<const floatx4 *>(p1 + 128);
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int n = n0 + q;
        const bool ok = n < F;
        const float bg = (bias && ok) ? bits_to_f<DT>(bias[n]) : 0.0f;
        const float bu = (bias && ok) ? bits_to_f<DT>(bias[F + n]) : 0.0f;
        const float g = (g0[q] + g1[q]) + bg, u = (u0[q] + u1[q]) + bu;
        o[q] = f_to_bits<DT>(apply_act(g, act) * u);
    }
    uint16_t *dst = h + (int64_t)m * F + n0;
    if (n0 + 4 <= F && ((uintptr_t)dst & 7u) == 0) {
        *reinterpret_cast<uint2 *>(dst) = make_uint2(o[0] | (o[1] << 16), o[2] | (o[3] << 16));
    } else {
        for (int q = 0; q < 4 && n0 + q < F; ++q)
            dst[q] = (uint16_t)o[q];
    }
}

template <int DT, int STATS, int GB, bool KT, bool GT, bool SK = false, bool FOLD = false>
hipError_t launch_k(const GemmArgs &a, hipStream_t s, float *part = nullptr, int ksplit = 1,
                    int tails = 0, int len = 0)
{
    const int cus = cu_count();
    constexpr int BNO = GT ? BN / 2 : BN;
    TileMap mp;
    mp.tm = (int)((a.M + BM - 1) / BM);
    mp.tn = (int)((a.N + BNO - 1) / BNO);
    mp.T = mp.tm * mp.tn;
    mp.xcd = (cus % 8 == 0 && mp.tn % 8 == 0) ? 1 : 0;
    mp.tails = tails;
    mp.len = len;
    mp.split_from = mp.T;
    // gated: the last round's tiles in two K halves when it holds at most half
    // of the CUs and the caller's scratch holds their partial sums
    int nsplit = 0;
    if constexpr (GT) {
        // the host plan counts 128 x 128-column gated tiles of 64-element steps
        static_assert(BM == 128 && BNO == 128 && BK == 64, "tile shape of the gated split plan");
        nsplit = ng_gated_split_tiles(a.M, a.N, a.K, cus);
        if (nsplit > 0 && a.part && ((uintptr_t)a.part & 15u) == 0 &&
            (size_t)nsplit * (BM * 256) * 2 * sizeof(float) <= a.part_bytes) {
            mp.split_from = mp.T - nsplit;
            part = a.part;
        } else {
            nsplit = 0;
        }
    }
    const int vec_out = (a.N % 8 == 0 && ((uintptr_t)a.y & 15u) == 0) ? 1 : 0;
    if constexpr (STATS == ST_FROM_Y || STATS == ST_FROM_Y_PS) {
        hipLaunchKernelGGL((row_stats_to_y_kernel<DT>), dim3((unsigned)((a.M + 3) / 4)), dim3(256),
                           0, s, (const uint16_t *)a.x, (uint16_t *)a.y, (int)a.M, (int)a.N,
                           (int)a.K, a.eps, a.norm, mp.tn, BNO);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    const int grid = tails > 0 ? mp.T + 8 * tails : mp.T * ksplit + nsplit;
    hipLaunchKernelGGL((prefill_lds_kernel<DT, STATS, GB, KT, GT, SK, FOLD>), dim3(grid),
                       dim3(THREADS), 0, s,
                       (const uint16_t *)a.x, (const uint16_t *)a.gamma, (const uint16_t *)a.beta,
                       (const uint16_t *)a.W, (const uint16_t *)a.bias, (uint16_t *)a.y, (int)a.M,
                       (int)a.N, (int)a.K, a.eps, a.norm, a.act, mp, vec_out, part, ksplit, a.c1,
                       a.c2);
    if constexpr (GT) {
        if (nsplit > 0) {
            hipError_t e = hipGetLastError();
            if (e != hipSuccess)
                return e;
            hipLaunchKernelGGL((gated_split_sum_kernel<DT>), dim3(16 * nsplit), dim3(256), 0, s,
                               (const float *)part, (const uint16_t *)a.bias, (uint16_t *)a.y,
                               (int)a.M, (int)a.N, a.act, mp);
        }
    }
    return hipGetLastError();
}

template <int DT, int STATS, int GB, bool GT>
hipError_t launch_t(const GemmArgs &a, hipStream_t s)
{
    return a.K % BK ? launch_k<DT, STATS, GB, true, GT>(a, s)
                    : launch_k<DT, STATS, GB, false, GT>(a, s);
}

template <int DT, int STATS, bool GT>
hipError_t launch_norm(const GemmArgs &a, hipStream_t s)
{
    switch ((a.gamma ? 1 : 0) | (a.beta ? 2 : 0)) {
    case 0: return launch_t<DT, STATS, 0, GT>(a, s);
    case 1: return launch_t<DT, STATS, 1, GT>(a, s);
    case 2: return launch_t<DT, STATS, 2, GT>(a, s);
    default: return launch_t<DT, STATS, 3, GT>(a, s);
    }
}

template <int DT, bool GT>
hipError_t launch_dt(const GemmArgs &a, hipStream_t s)
{
    if (a.norm == NORM_NONE)
        return launch_t<DT, ST_NONE, 0, GT>(a, s);
    // The statistics pass needs 8 bytes of y in every tile's rows: every
    // tile (including the last, partial one) must have at least 4 columns
    // and the rows must be 8-byte aligned.
    const bool y_scratch = a.N % 8 == 0 && ((uintptr_t)a.y & 15u) == 0;
    if (!y_scratch)
        return launch_norm<DT, ST_PROLOGUE, GT>(a, s);
    // fp16 RMSNorm without beta: power-of-two prescaled operand
    if constexpr (DT == DT_F16) {
        if (a.norm == NORM_RMSNORM && !a.beta)
            return a.gamma ? launch_t<DT, ST_FROM_Y_PS, 1, GT>(a, s)
                           : launch_t<DT, ST_FROM_Y_PS, 0, GT>(a, s);
    }
    return launch_norm<DT, ST_FROM_Y, GT>(a, s);
}

}  // namespace

hipError_t launch_row_stats_to_y(const void *x, void *y, int64_t M, int64_t N, int64_t K,
                                 float eps, int norm, int tn, int tw, int dtype, hipStream_t s)
{
    const dim3 grid((unsigned)((M + 3) / 4)), block(256);
    if (dtype == DT_F16)
        hipLaunchKernelGGL((row_stats_to_y_kernel<DT_F16>), grid, block, 0, s,
                           (const uint16_t *)x, (uint16_t *)y, (int)M, (int)N, (int)K, eps, norm,
                           tn, tw);
    else
        hipLaunchKernelGGL((row_stats_to_y_kernel<DT_BF16>), grid, block, 0, s,
                           (const uint16_t *)x, (uint16_t *)y, (int)M, (int)N, (int)K, eps, norm,
                           tn, tw);
    return hipGetLastError();
}

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
    // plain GEMM only, any M; every K range must get at least one step (one
    // range writes the fp32 sums of the whole K)
    if (ng_route_gemm(NG_DECODE_MAX_M + 1, a.N, a.K, a.vec ? 1 : 0, cu_count()) !=
            NG_ROUTE_PREFILL_LDS ||
        a.norm != NORM_NONE || ksplit < 1 || (ksplit > 1 && prefill_k_steps(a.K) < 2 * ksplit))
        return hipErrorInvalidValue;
    const bool kt = a.K % BK != 0;
    if (a.dtype == DT_F16)
        return kt ? launch_k<DT_F16, ST_NONE, 0, true, false, true>(a, s, part, ksplit)
                  : launch_k<DT_F16, ST_NONE, 0, false, false, true>(a, s, part, ksplit);
    return kt ? launch_k<DT_BF16, ST_NONE, 0, true, false, true>(a, s, part, ksplit)
              : launch_k<DT_BF16, ST_NONE, 0, false, false, true>(a, s, part, ksplit);
}

hipError_t launch_prefill_lds_skip_slice(const GemmArgs &a, float *part, hipStream_t s)
{
    // the host plan assumes 128 x 256 tiles of 64-element K steps
    static_assert(BM == 128 && BN == 256 && BK == 64, "tile shape of the skipped-slice plan");
    int tails = 0, len = 0;
    const int cus = cu_count();
    if (ng_route_gemm(NG_DECODE_MAX_M + 1, a.N, a.K, a.vec ? 1 : 0, cus) != NG_ROUTE_PREFILL_LDS ||
        a.norm != NORM_NONE || !ng_skip_slice_plan(a.M, a.N, a.K, cus, &tails, &len))
        return hipErrorInvalidValue;
    // every workgroup's tiles exist: T / 8 tiles per XCD in whole slots
    const int T = prefill_tiles(a.M, a.N);
    if (T % 8 != 0 || (T / 8) % tails != 0 || ((a.N + BN - 1) / BN) % 8 != 0 ||
        (int64_t)(T / 8 / tails + 1) * len > prefill_k_steps(a.K))
        return hipErrorInvalidValue;
    const bool kt = a.K % BK != 0;
    if (a.dtype == DT_F16)
        return kt ? launch_k<DT_F16, ST_NONE, 0, true, false, true>(a, s, part, 2, tails, len)
                  : launch_k<DT_F16, ST_NONE, 0, false, false, true>(a, s, part, 2, tails, len);
    return kt ? launch_k<DT_BF16, ST_NONE, 0, true, false, true>(a, s, part, 2, tails, len)
              : launch_k<DT_BF16, ST_NONE, 0, false, false, true>(a, s, part, 2, tails, len);
}

hipError_t launch_prefill_lds_folded(const GemmArgs &a, hipStream_t s)
{
    // a.W = W', a.c1 / a.c2 the folded vectors; statistics from the pass
    // through y when y can hold them, else in the kernel
    if (ng_route_gemm(NG_DECODE_MAX_M + 1, a.N, a.K, a.vec ? 1 : 0, cu_count()) !=
            NG_ROUTE_PREFILL_LDS ||
        a.norm == NORM_NONE || !a.c2 || (a.norm == NORM_LAYERNORM && !a.c1))
        return hipErrorInvalidValue;
    const bool y_scratch = a.N % 8 == 0 && ((uintptr_t)a.y & 15u) == 0;
    const bool kt = a.K % BK != 0;
#define NG_FOLD_K(DT, ST) \
    (kt ? launch_k<DT, ST, 0, true, false, false, true>(a, s) \
        : launch_k<DT, ST, 0, false, false, false, true>(a, s))
    if (a.dtype == DT_F16)
        return y_scratch ? NG_FOLD_K(DT_F16, ST_FROM_Y) : NG_FOLD_K(DT_F16, ST_PROLOGUE);
    return y_scratch ? NG_FOLD_K(DT_BF16, ST_FROM_Y) : NG_FOLD_K(DT_BF16, ST_PROLOGUE);
#undef NG_FOLD_K
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

// prefill_wide.hip -- the normalization-prologue GEMM on 256 x 192 output tiles
// (page "LayerNorm 融合算子如何让大模型推理再快 15%？深度拆解 ATB 的实现",
// sections 2.1-3.2: tile-level fusion with the normalized tile kept on chip,
// weights fetched while the statistics are computed, aligned contiguous
// accesses).
//
// What bounds the 128 x 256 kernel's K step on MI355X is the L2 -> CU path:
// each CU keeps about a hundred 128-byte L2 reads in flight, so its bytes per
// step set the step time, not its MFMA work. A 256 x 192 tile moves 56 KB per
// 64-k step for 1.5 times the FLOPs of a 128 x 256 tile (48 KB), and where the
// tile count fills the CUs evenly (512 tiles of x[512,*] W[49152,*] on 256
// CUs: two rounds against three) each CU moves 22 % fewer bytes for the
// whole call. Measured on the RMSNorm + MatMul + SiLU 512 x 14336 x 49152
// call: 742-746 us against 772-786 us on 128 x 256 tiles (the per-CU L2 rate
// drops with the larger tile, so the gain is smaller than the byte count
// suggests); without normalization the 128 x 256 kernel, which loads x
// straight into the LDS, stays ahead, so only normalizing calls come here.
//
// One workgroup of 8 waves per tile, one workgroup per CU (136 KB of LDS).
// Wave w computes rows 64 (w % 4) .. + 63 and columns 96 (w / 4) .. + 95
// (2 x 3 MFMA blocks of 32 x 32).
//   x           every lane loads its 4 chunks of a step (rows 64 apart, one
//               logical chunk) into registers in a memory phase, normalizes
//               them between its own MFMAs of the compute phase that follows
//               and writes them once into their stage: two x stages (32 KB
//               each) suffice (one register buffer: two would not fit the
//               256 registers a wave has at two waves per SIMD).
//   W           HBM -> LDS by direct 128-bit loads, three stages (24 KB each).
//   schedule    the two waves of each SIMD (w and w + 4) alternate a memory
//               phase (fragment reads, load issue) and an MFMA phase,
//               separated by workgroup barriers, one phase apart, as in the
//               128 x 256 kernel; the load order and waits are the same with
//               4 x loads and 3 W loads per lane and step.
//   epilogue    the prescale factor, bias, activation, one rounding, staged
//               row-major in LDS, 128-bit stores.
// K must be a multiple of 64 (whole steps); the host routes other shapes to
// the 128 x 256 kernel.
#include <type_traits>

#include "device_common.h"
#include "launch.h"
#include "route.h"

namespace ng {
namespace {

constexpr int BM = 256, BN = 192, BK = 64;
constexpr int NWAVE = 8, THREADS = 64 * NWAVE;
constexpr int CPR = BK / 8;                      // 16-byte chunks per tile row
constexpr int A_TILE = BM * CPR, B_TILE = BN * CPR;   // in 16-byte chunks
constexpr int A_DMA = BM * CPR / THREADS;        // x chunks per lane per step (4)
constexpr int B_DMA = BN * CPR / THREADS;        // W direct loads per lane per step (3)
constexpr int A_IST = BM / A_DMA;                // rows between a lane's x rows (64)
constexpr int B_RPW = BN / NWAVE;                // W rows loaded per wave per step (24)
constexpr int WM = 64, WN = 96;                  // wave tile
constexpr int WGM = BM / WM, WGN = BN / WN;      // wave grid (4 x 2)
constexpr int FM = WM / 32, FN = WN / 32;        // 32x32 blocks per wave (2 x 3)
static_assert(A_DMA == 4 && B_DMA == 3 && B_RPW == 8 * B_DMA, "loads per lane");
static_assert(WGM * WGN == NWAVE && A_IST % 16 == 0, "wave split");
static_assert((2 * A_TILE + 3 * B_TILE) * 16 <= 160 * 1024, "LDS budget");
static_assert(64 * 24 <= B_TILE && 64 * 24 <= A_TILE, "epilogue staging: 64 rows per stage");

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

// What happens to x on its way to the LDS.
enum {
    XM_PS = 1,      // fp16 RMSNorm without beta: x * 2^e * gamma (prescaled)
    XM_AFFINE = 2,  // (x rs + nmr) * gamma + beta in fp32, one rounding
};

// GB: bit 0 gamma present, bit 1 beta present (XM_PS: bit 0 only). The
// statistics records (rs, -mu rs) written by the statistics pass into this
// tile's rows of y are read first.
template <int DT, int XM, int GB>
__global__ __launch_bounds__(THREADS, 1) void prefill_wide_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ gamma,
    const uint16_t *__restrict__ beta, const uint16_t *__restrict__ W,
    const uint16_t *__restrict__ bias, uint16_t *__restrict__ y, int M, int N, int K, int act,
    int tm, int tn, int xcd, int vec_out)
{
    constexpr bool PS = XM == XM_PS, AFF = XM == XM_AFFINE;
    static_assert(PS || AFF, "normalizing modes");
    constexpr bool HG = GB & 1, HB = AFF && (GB & 2);
    constexpr int LPS = B_DMA;                                   // direct loads per step
    constexpr int NXL = A_DMA + (HG ? 1 : 0) + (HB ? 1 : 0);     // register loads per step
    __shared__ u32x4 A0[A_TILE], A1[A_TILE];
    __shared__ u32x4 B0[B_TILE], B1[B_TILE], B2[B_TILE];
    auto Ast = [&](auto sc) -> u32x4 * {
        if constexpr (decltype(sc)::value % 2 == 0)
            return A0;
        else
            return A1;
    };
    auto Bst = [&](auto sc) -> u32x4 * {
        constexpr int i = decltype(sc)::value % 3;
        if constexpr (i == 0)
            return B0;
        else if constexpr (i == 1)
            return B1;
        else
            return B2;
    };

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;                      // phase group (waves w, w + 4 share a SIMD)
    const int wm = wave & 3, wn = grp;              // wave tile position
    const int lrow = lane & 31, lk = lane >> 5;
    const int nk = K / BK;

    // tile of this workgroup: XCD-grouped when the column blocks split evenly
    // over the 8 XCDs (workgroup b runs on XCD b % 8; the j-th workgroup of an
    // XCD takes row block j % tm of column block (b % 8) (tn / 8) + j / tm)
    int mb, nt;
    {
        const int b = blockIdx.x;
        if (xcd) {
            const int xi = b & 7, j = b >> 3;
            mb = j % tm;
            nt = xi * (tn >> 3) + j / tm;
        } else {
            mb = b % tm;
            nt = b / tm;
        }
    }
    const int m0 = mb * BM, n0 = nt * BN;

    // ---- loads. W: instruction i of wave w fills tile rows w B_RPW + 8 i ..,
    // lane l at chunk position l % 8 (row + l / 8), holding logical chunk
    // swz(row, l % 8). x: chunk i of lane l of wave w is row i A_IST + 8 w +
    // l / 8, logical chunk swz(row, l % 8) (one swizzle for all four rows).
    // Rows past M or N re-read the last row (x rows past M are zeroed, W
    // rows' outputs dropped); steps past the last re-read the last step.
    // Offsets are 32-bit bytes from the tile origin (the host checks that
    // they fit), fixed for the whole tile.
    uint32_t woff[B_DMA], aoff[A_DMA];
    bool alive[A_DMA];
    const int ach = swz(wave * 8 + (lane >> 3), lane & 7);
#pragma unroll
    for (int i = 0; i < B_DMA; ++i) {
        const int row = wave * B_RPW + i * 8 + (lane >> 3);
        const uint32_t rb = (uint32_t)(min(n0 + row, N - 1) - n0) * (uint32_t)K;
        woff[i] = (rb + swz(row, lane & 7) * 8) * 2u;
    }
#pragma unroll
    for (int i = 0; i < A_DMA; ++i) {
        const int row = i * A_IST + wave * 8 + (lane >> 3);
        alive[i] = m0 + row < M;
        const uint32_t rb = (uint32_t)(min(m0 + row, M - 1) - m0) * (uint32_t)K;
        aoff[i] = (rb + ach * 8) * 2u;
    }
    const uint32_t goff = ach * 16u;
    const uint16_t *wtile = W + (int64_t)n0 * K;
    const uint16_t *xtile = x + (int64_t)m0 * K;
    auto issue_dma = [&](int kt, u32x4 *Bs) {
        kt = min(kt, nk - 1);
        const char *wb = reinterpret_cast<const char *>(wtile) + (size_t)kt * (BK * 2);
#pragma unroll
        for (int i = 0; i < B_DMA; ++i)
            dma16_nt(wb, woff[i], lds_addr(&Bs[(wave * B_RPW + i * 8) * CPR]));
    };

    // row statistics: of this lane's x rows (normalization) and of the
    // output rows of its accumulators (epilogue: rows wm 64 + 32 i + lrow)
    float rrs[A_DMA], rnmr[A_DMA];
    half2_t ps2[A_DMA];
    float osc[FM], onm[FM];
#pragma unroll
    for (int i = 0; i < A_DMA; ++i) {
        rrs[i] = 1.0f;
        rnmr[i] = 0.0f;
    }
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
    {
        // (rs, -mu rs) left by the statistics pass in the first 8 bytes of
        // each row's slice of this tile of y
#pragma unroll
        for (int i = 0; i < A_DMA; ++i) {
            const int m = min(m0 + i * A_IST + wave * 8 + (lane >> 3), M - 1);
            const uint2 pk = *reinterpret_cast<const uint2 *>(y + (int64_t)m * N + n0);
            rrs[i] = __builtin_bit_cast(float, pk.x);
            rnmr[i] = __builtin_bit_cast(float, pk.y);
        }
        if constexpr (PS) {
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int m = min(m0 + wm * WM + i * 32 + lrow, M - 1);
                const uint2 pk = *reinterpret_cast<const uint2 *>(y + (int64_t)m * N + n0);
                const float rs = __builtin_bit_cast(float, pk.x);
                osc[i] = rs / pow2_below(rs);
            }
        }
        // complete these before the asynchronous loads start (the compiler
        // does not count those, so only an empty queue tells it these landed)
        wait_vmcnt<0>();
        if constexpr (PS) {
#pragma unroll
            for (int i = 0; i < A_DMA; ++i) {
                const _Float16 sh = (_Float16)pow2_below(rrs[i]);
                ps2[i] = half2_t{sh, sh};
            }
        }
    }

    // x chunks (and gamma / beta chunk) of one step, loaded asynchronously
    // into one register buffer in a memory phase and written into their
    // stage in the compute phase that follows; completed by a tied wait
    struct Raw {
        u32x4 v[A_DMA], g, b;
    };
    Raw raw;
    auto load_raw = [&](int kt, Raw &r) {
        kt = min(kt, nk - 1);
        const char *xb = reinterpret_cast<const char *>(xtile) + (size_t)kt * (BK * 2);
#pragma unroll
        for (int i = 0; i < A_DMA; ++i)
            r.v[i] = ldg16_async(xb, aoff[i]);
        if constexpr (HG)
            r.g = ldg16_async(reinterpret_cast<const char *>(gamma) + (size_t)kt * (BK * 2), goff);
        else
            r.g = u32x4{0u, 0u, 0u, 0u};
        if constexpr (HB)
            r.b = ldg16_async(reinterpret_cast<const char *>(beta) + (size_t)kt * (BK * 2), goff);
        else
            r.b = u32x4{0u, 0u, 0u, 0u};
    };
    auto tied_wait = [&](auto nc, Raw &r) {
        constexpr int n = decltype(nc)::value;
        wait_vmcnt_tied<n>(r.v[0], r.v[1], r.v[2], r.v[3]);
        wait_vmcnt_tied<n>(r.g, r.b, r.v[0], r.v[1]);
    };
    // one of this lane's x chunks into stage As: prescaled or normalized;
    // rows past M become zero
    auto nrm_chunk = [&](u32x4 *As, const Raw &r, int i) {
        u32x4 v = r.v[i];
        if constexpr (PS) {
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
        } else if constexpr (AFF) {
            float g[8], bt[8], f[8];
            if constexpr (HG)
                unpack8<DT>(r.g, g);
            if constexpr (HB)
                unpack8<DT>(r.b, bt);
            unpack8<DT>(v, f);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float t = fmaf(f[e], rrs[i], rnmr[i]);
                if constexpr (HG && HB)
                    f[e] = fmaf(t, g[e], bt[e]);
                else if constexpr (HG)
                    f[e] = t * g[e];
                else if constexpr (HB)
                    f[e] = t + bt[e];
                else
                    f[e] = t;
            }
            v = pack8<DT>(f);
        }
        As[(i * A_IST + wave * 8) * CPR + lane] = alive[i] ? v : u32x4{0u, 0u, 0u, 0u};
    };
    auto nrm_store = [&](u32x4 *As, const Raw &r) {
#pragma unroll
        for (int i = 0; i < A_DMA; ++i)
            nrm_chunk(As, r, i);
    };
    auto sb = [] { __builtin_amdgcn_sched_barrier(0); };
    auto phase_barrier = [&] {
        sb();
        asm volatile("s_barrier" ::: "memory");
        sb();
    };

    // ---- load order and waits (loads complete in issue order, so a wait for
    // one is a wait for every older one). Per step a lane issues NXL register
    // loads (x, gamma, beta) and LPS direct loads (W):
    //   group 0: memory phase kt issues x of kt + 1, then the direct loads of
    //            kt + 2; compute phase kt writes x of kt + 1 into its stage
    //            and ends by awaiting the direct loads of kt + 1;
    //   group 1: memory phase kt issues x of kt + 2 and awaits the direct
    //            loads of kt + 1; compute phase kt starts with the direct
    //            loads of kt + 3 (their stage was last read in the phase
    //            before) and writes x of kt + 2 into its stage.
    // x stage s % 2 of step s is written in phases 2 s - 2 (group 1) and
    // 2 s - 1 (group 0) and read in phases 2 s and 2 s + 1; W stage s % 3 is
    // filled from phase 2 s - 4 on and read in the same two phases.
    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, LPS>;              // x of this phase's step
    constexpr int CL = NXL + LPS;                             // group 0: loads of kt + 1
    constexpr int CW = 2 * NXL + LPS;                         // group 1: loads of kt + 1

    // ---- prologue: step 0 complete in its stage, the direct loads of steps
    // 1 (and 2 for group 1) in flight, group 1's x of step 1 in its stage
    issue_fence(x, gamma, beta);
    load_raw(0, raw);
    issue_dma(0, B0);
    issue_dma(1, B1);
    tied_wait(std::integral_constant<int, 2 * LPS>{}, raw);
    nrm_store(A0, raw);
    issue_fence(x, gamma, beta);
    if (grp == 0) {
        wait_vmcnt<LPS>();                // the direct loads of step 0
    } else {
        load_raw(1, raw);
        wait_vmcnt<NXL + LPS>();          // the direct loads of step 0
    }
    issue_fence(x, gamma, beta);
    lds_barrier();
    if (grp == 1) {
        // the second group starts one phase later; its first phase does what
        // each of its compute phases does for kt + 3 and kt + 2: the direct
        // loads of step 2, and its x rows of step 1
        issue_dma(2, B2);
        tied_wait(C1{}, raw);
        nrm_store(A1, raw);
        lds_barrier();
    }

    floatx16 acc[FN][FM];
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[j][i][e] = 0.0f;

    // fragments of one step: [sub-step][32-row block]; rows 32 apart share
    // the swizzle, so one offset per sub-step addresses every fragment
    u32x4 fa[4][FM], fb[4][FN];
    auto read_frags = [&](const u32x4 *Ac, const u32x4 *Bc) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int sw = swz(lrow, kk * 2 + lk);
            const int aoffs = (wm * WM + lrow) * CPR + sw;
            const int boffs = (wn * WN + lrow) * CPR + sw;
#pragma unroll
            for (int j = 0; j < FN; ++j)
                fb[kk][j] = Bc[boffs + j * 32 * CPR];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                fa[kk][i] = Ac[aoffs + i * 32 * CPR];
        }
    };
    auto mfma_kk = [&](int kk) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int i = 0; i < FM; ++i)
                acc[j][i] = mfma32<DT>(fb[kk][j], fa[kk][i], acc[j][i]);
    };
    // the step's MFMAs with this lane's x chunks of a later step written
    // into As between them, a few VALU instructions after each MFMA
    auto compute = [&](u32x4 *As, int g) {
        Raw &r = raw;
        mfma_kk(0);
        // x of the step this phase writes: younger than it only the direct
        // loads issued after it (group 0: of kt + 2 in the memory phase;
        // group 1: of kt + 3 at the start of this phase)
        (void)g;
        tied_wait(C1{}, r);
        nrm_chunk(As, r, 0);
        mfma_kk(1);
        nrm_chunk(As, r, 1);
        mfma_kk(2);
        nrm_chunk(As, r, 2);
        mfma_kk(3);
        nrm_chunk(As, r, 3);
#pragma unroll
        for (int i = 0; i < 4 * FM * FN; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);   // up to three VALU
        }
        sb();
    };

    // one K step (memory phase, then compute phase); J = kt % 6 gives the x
    // stages (J % 2, + 1), the W stages (J % 3, + 1, + 2) and the x buffers
    auto kstep = [&](int kt, auto jc) {
        constexpr int J = decltype(jc)::value;
        using SA = std::integral_constant<int, J>;
        using SA1 = std::integral_constant<int, J + 1>;
        using SB = std::integral_constant<int, J>;
        using SB2 = std::integral_constant<int, J + 2>;
        issue_fence(x, gamma, beta);
        // memory phase
        read_frags(Ast(SA{}), Bst(SB{}));
        sb();
        load_raw(kt + 1 + grp, raw);
        if (grp == 0) {
            issue_dma(kt + 2, Bst(SB2{}));
        } else {
            wait_vmcnt<CW>();            // the direct loads of kt + 1
            issue_fence(x, gamma, beta);
        }
        lds_barrier();
        // compute phase (group 0: x of kt + 1 into stage (kt + 1) % 2;
        // group 1: x of kt + 2 into stage kt % 2)
        sb();
        if (grp == 1)
            issue_dma(kt + 3, Bst(SB{}));
        compute(grp ? Ast(SA{}) : Ast(SA1{}), grp);
        if (grp == 0) {
            wait_vmcnt<CL>();            // the direct loads of kt + 1
            issue_fence(x, gamma, beta);
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
    if (grp == 0)
        phase_barrier();        // the second group's last compute phase
    // drain the clamped loads issued past the last step before LDS reuse;
    // the x registers of the last (unused) loads stay live until landed
    tied_wait(C0{}, raw);
    __syncthreads();

    // ---- epilogue: rs (prescale), bias, activation, one rounding; the tile staged row-major in LDS (rows 64 r .. 64 r + 63
    // in B0, B1, B2, A0 for r = 0..3; 24 chunks of 16 bytes per row, the chunk
    // index XOR-swizzled by row % 8), then written with 128-bit stores
    auto stg = [&](int r) -> u32x4 * { return r == 0 ? B0 : r == 1 ? B1 : r == 2 ? B2 : A0; };
    {
        u32x4 *st = stg(wm);
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
                    const int ml = i * 32 + lrow;            // row within the 64-row group
                    float v[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        v[r] = apply_act(fmaf(acc[j][i][q * 4 + r], osc[i], bv[r]), act);
                    const int chunk = (nl >> 3) ^ (ml & 7);
                    uint32_t *dst = reinterpret_cast<uint32_t *>(&st[ml * 24 + chunk]) + (lk * 2);
                    dst[0] = pack2<DT>(v[0], v[1]);
                    dst[1] = pack2<DT>(v[2], v[3]);
                }
            }
        }
    }
    __syncthreads();
    for (int idx = tid; idx < BM * 24; idx += THREADS) {
        const int row = idx / 24, ch = idx - row * 24;
        const int m = m0 + row, n = n0 + ch * 8;
        const int rl = row & 63;
        const u32x4 v = stg(row >> 6)[rl * 24 + (ch ^ (rl & 7))];
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

template <int DT, int XM, int GB>
hipError_t launch_k(const GemmArgs &a, hipStream_t s)
{
    const int cus = cu_count();
    const int tm = (int)((a.M + BM - 1) / BM), tn = (int)((a.N + BN - 1) / BN);
    const int xcd = (cus % 8 == 0 && tn % 8 == 0) ? 1 : 0;
    const int vec_out = (a.N % 8 == 0 && ((uintptr_t)a.y & 15u) == 0) ? 1 : 0;
    const hipError_t e =
        launch_row_stats_to_y(a.x, a.y, a.M, a.N, a.K, a.eps, a.norm, tn, BN, a.dtype, s);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL((prefill_wide_kernel<DT, XM, GB>), dim3(tm * tn), dim3(THREADS), 0, s,
                       (const uint16_t *)a.x, (const uint16_t *)a.gamma,
                       (const uint16_t *)a.beta, (const uint16_t *)a.W, (const uint16_t *)a.bias,
                       (uint16_t *)a.y, (int)a.M, (int)a.N, (int)a.K, a.act, tm, tn, xcd,
                       vec_out);
    return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const GemmArgs &a, hipStream_t s)
{
    if constexpr (DT == DT_F16) {
        if (a.norm == NORM_RMSNORM && !a.beta)
            return a.gamma ? launch_k<DT, XM_PS, 1>(a, s) : launch_k<DT, XM_PS, 0>(a, s);
    }
    switch ((a.gamma ? 1 : 0) | (a.beta ? 2 : 0)) {
    case 0: return launch_k<DT, XM_AFFINE, 0>(a, s);
    case 1: return launch_k<DT, XM_AFFINE, 1>(a, s);
    case 2: return launch_k<DT, XM_AFFINE, 2>(a, s);
    default: return launch_k<DT, XM_AFFINE, 3>(a, s);
    }
}

}  // namespace

hipError_t launch_prefill_wide(const GemmArgs &a, hipStream_t s)
{
    // normalizing calls with whole K steps, 32-bit tile offsets and room in y
    // for the statistics records
    if (a.norm == NORM_NONE || a.c2 || !ng_wide_tiles_fit(a.M, a.N, a.K, a.vec ? 1 : 0) ||
        a.N % 8 != 0 || ((uintptr_t)a.y & 15u) != 0)
        return hipErrorInvalidValue;
    return a.dtype == DT_F16 ? launch_dt<DT_F16>(a, s) : launch_dt<DT_BF16>(a, s);
}

}  // namespace ng

// device_common.h -- gfx950 device helpers shared by the prefill and decode
// kernels: 16-bit storage formats, 128-bit chunk conversion, wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ng {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum { DT_F16 = 0, DT_BF16 = 1 };

// ---------------------------------------------------------------- scalars
template <int DT> __device__ __forceinline__ float lo_to_f(uint32_t w);
template <int DT> __device__ __forceinline__ float hi_to_f(uint32_t w);

template <> __device__ __forceinline__ float lo_to_f<DT_F16>(uint32_t w)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
template <> __device__ __forceinline__ float hi_to_f<DT_F16>(uint32_t w)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}
// bf16 is the upper half of a binary32: widening is a shift.
template <> __device__ __forceinline__ float lo_to_f<DT_BF16>(uint32_t w)
{
    return __builtin_bit_cast(float, w << 16);
}
template <> __device__ __forceinline__ float hi_to_f<DT_BF16>(uint32_t w)
{
    return __builtin_bit_cast(float, w & 0xffff0000u);
}

template <int DT> __device__ __forceinline__ float bits_to_f(uint16_t b)
{
    return lo_to_f<DT>((uint32_t)b);
}

// Round two floats to the storage type (round-to-nearest-even) and pack
// them into one dword, low half first.
template <int DT> __device__ __forceinline__ uint32_t pack2(float a, float b);

template <> __device__ __forceinline__ uint32_t pack2<DT_F16>(float a, float b)
{
    uint32_t lo = __builtin_bit_cast(uint16_t, (_Float16)a);
    uint32_t hi = __builtin_bit_cast(uint16_t, (_Float16)b);
    return lo | (hi << 16);
}
template <> __device__ __forceinline__ uint32_t pack2<DT_BF16>(float a, float b)
{
    uint32_t lo = __builtin_bit_cast(uint16_t, (__bf16)a);
    uint32_t hi = __builtin_bit_cast(uint16_t, (__bf16)b);
    return lo | (hi << 16);
}

template <int DT> __device__ __forceinline__ uint16_t f_to_bits(float a)
{
    return (uint16_t)(pack2<DT>(a, 0.0f) & 0xffffu);
}

// ------------------------------------------------------- 128-bit chunks
// A chunk is 8 consecutive elements (16 bytes) of one row.
template <int DT> __device__ __forceinline__ void unpack8(const u32x4 &c, float *f)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = lo_to_f<DT>(c[i]);
        f[2 * i + 1] = hi_to_f<DT>(c[i]);
    }
}

template <int DT> __device__ __forceinline__ u32x4 pack8(const float *f)
{
    u32x4 c;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        c[i] = pack2<DT>(f[2 * i], f[2 * i + 1]);
    return c;
}

__device__ __forceinline__ u32x4 ldg128(const uint16_t *p)
{
    return *reinterpret_cast<const u32x4 *>(p);
}

// Element-wise chunk load with bounds: elements k0..k0+7 of a row of length
// `len`; positions at or beyond `len` read as +0.
__device__ __forceinline__ u32x4 ldg_elems(const uint16_t *row, int64_t k0, int64_t len)
{
    uint16_t e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        e[i] = (k0 + i < len) ? row[k0 + i] : (uint16_t)0;
    u32x4 c;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        c[i] = (uint32_t)e[2 * i] | ((uint32_t)e[2 * i + 1] << 16);
    return c;
}

// Chunk of 8 elements starting at k0 of a row of length `len`:
// VEC (len % 8 == 0, 16-byte aligned) -> one 128-bit load or zeros.
template <bool VEC>
__device__ __forceinline__ u32x4 load_chunk(const uint16_t *row, int64_t k0, int64_t len)
{
    if constexpr (VEC) {
        if (k0 < len)
            return ldg128(row + k0);
        return u32x4{0u, 0u, 0u, 0u};
    } else {
        return ldg_elems(row, k0, len);
    }
}

// ---------------------------------------------------------- reductions
__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v += __shfl_xor(v, off, 64);
    return v;
}

// ----------------------------------------------------------- epilogue
enum { ACT_NONE = 0, ACT_SILU = 1, ACT_RELU = 2, ACT_GELU = 3 };

// SiLU(z) = z * sigmoid(z) = z / (1 + e^-z); ReLU(z) = max(z, 0) (NaN stays
// NaN); GELU(z) = z * Phi(z) = z / 2 * (1 + erf(z / sqrt 2)), the exact form.
// exp and erf from the device library.
__device__ __forceinline__ float apply_act(float z, int act)
{
    if (act == ACT_SILU)
        return z / (1.0f + __expf(-z));
    if (act == ACT_RELU)
        return z < 0.0f ? 0.0f : z;
    if (act == ACT_GELU)
        return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f));
    return z;
}

// Row statistics -> (rs, mu) such that the normalized value is
// (x - mu) * rs: LayerNorm mu = mean, rs = 1/sqrt(var+eps);
// RMSNorm mu = 0, rs = 1/sqrt(mean(x^2)+eps). Subtracting the mean before
// scaling keeps x == mean exactly zero (a constant row normalizes to 0).
enum { NORM_NONE = 0, NORM_LAYERNORM = 1, NORM_RMSNORM = 2 };

// One-pass statistics of a row with the shifted-data algorithm (Chan, Golub
// and LeVeque, "Algorithms for computing the sample variance", 1983): sums of
// d = x - x[0] and d^2 in fp32, so that a large common offset does not cancel
// in var = E[d^2] - E[d]^2.  One wave per row; VEC uses 128-bit loads.
template <int DT, bool VEC>
__device__ __forceinline__ void row_stats(const uint16_t *row, int64_t K, float eps,
                                          int norm, int lane, float &rs, float &mu)
{
    const float shift = (norm == NORM_LAYERNORM) ? bits_to_f<DT>(row[0]) : 0.0f;
    float s1 = 0.0f, s2 = 0.0f;
    const int64_t nchunk = (K + 7) / 8;
    for (int64_t c = lane; c < nchunk; c += 64) {
        u32x4 raw = load_chunk<VEC>(row, c * 8, K);
        float f[8];
        unpack8<DT>(raw, f);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            // padded positions (k >= K) read as 0 and must not contribute
            float d = (c * 8 + i < K) ? f[i] - shift : 0.0f;
            s1 += d;
            s2 = fmaf(d, d, s2);
        }
    }
    s1 = wave_sum(s1);
    s2 = wave_sum(s2);
    const float invK = 1.0f / (float)K;
    if (norm == NORM_LAYERNORM) {
        float md = s1 * invK;
        float var = fmaxf(fmaf(-md, md, s2 * invK), 0.0f);
        rs = rsqrtf(var + eps);
        mu = shift + md;
    } else if (norm == NORM_RMSNORM) {
        rs = rsqrtf(s2 * invK + eps);
        mu = 0.0f;
    } else {
        rs = 1.0f;
        mu = 0.0f;
    }
}


// ------------------------------------------------------- wait counters
// s_waitcnt with only vmcnt constrained (expcnt and lgkmcnt left at max);
// gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14].
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

// ------------------------------------------------- explicit direct load
// One 16-byte-per-lane direct load HBM -> LDS (global_load_lds_dwordx4,
// address = scalar base + 32-bit vector offset; lane l writes LDS byte
// address lds + 16 l through M0), issued as inline asm. The compiler does
// not see it as a load: it inserts no waits for it, and its own waits for
// other loads only get stricter. The caller orders it with explicit vmcnt
// waits and barriers; the "memory" clobber keeps other memory accesses on
// their side of it. M0 is only used by these statements in the kernels
// that call it.
__device__ __forceinline__ void dma16(const void *sbase, uint32_t voff, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "s"(lds)
                 : "memory", "m0");
}

// The same direct load with the non-temporal hint: the L2 may replace the
// lines first. For operand tiles with few readers (each W line of a 256-row
// tile is read by the two workgroups of its column block and then never
// again), so that the lines other workgroups still share stay resident.
__device__ __forceinline__ void dma16_nt(const void *sbase, uint32_t voff, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 :
                 : "v"(voff), "s"(sbase), "s"(lds)
                 : "memory", "m0");
}

// The same direct load with a per-lane 64-bit address (lanes may read from
// different arrays); inactive lanes neither read nor write LDS.
__device__ __forceinline__ void dma16_ptr(const void *p, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(p), "s"(lds)
                 : "memory", "m0");
}

// ------------------------------------------------ explicit register load
// One 16-byte-per-lane load into registers (global_load_dwordx4, scalar base
// + 32-bit vector offset) issued as inline asm: the compiler's own vmcnt
// accounting does not see the direct loads, so for a load it can see it
// would drain every direct load issued after it. The value arrives
// asynchronously: it may only be read after wait_vmcnt_tied has taken it as
// an in/out operand, which is where the compiler sees it defined.
__device__ __forceinline__ u32x4 ldg16_async(const void *sbase, uint32_t voff)
{
    u32x4 r;
    asm volatile("global_load_dwordx4 %0, %1, %2" : "=v"(r) : "v"(voff), "s"(sbase) : "memory");
    return r;
}

// s_waitcnt vmcnt(N) that also hands the four registers through, so no read
// of them can be placed before it
template <int N>
__device__ __forceinline__ void wait_vmcnt_tied(u32x4 &a, u32x4 &b, u32x4 &c, u32x4 &d)
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%4)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d) : "n"(N) : "memory");
}

// LDS byte address of a __shared__ object element, as a wave-uniform value
__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p);
}

// --------------------------------------------------------- issue fence
// Keeps loads through the given pointers, and all other memory operations,
// on their side of this point in program order. The pointers go into a
// volatile asm that clobbers memory, so at the IR level that asm may write
// through them and loads cannot be sunk or hoisted across it (a memory
// clobber alone does not bind __restrict__ arguments that never escape, and
// sched_barrier does not touch memory at the IR level); sched_barrier then
// stops the machine scheduler. Kernels whose explicit vmcnt waits count the
// loads issued between two points rely on it.
__device__ __forceinline__ void issue_fence(const void *a, const void *b = nullptr,
                                            const void *c = nullptr)
{
    asm volatile("" ::"s"(a), "s"(b), "s"(c) : "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// -------------------------------------------------------- LDS barrier
// Workgroup barrier for kernels with direct global->LDS loads in flight:
// each wave first waits for its own LDS operations (lgkmcnt), then all
// waves meet. No memory fence on purpose: a workgroup release fence on LDS
// also waits for every direct load still in flight (they write LDS), which
// would drain a W prefetch pipeline. Callers that need their own direct
// loads landed wait on vmcnt before calling. The "memory" clobber keeps the
// compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ------------------------------------------- packed-dot row statistics
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef short short2_t __attribute__((ext_vector_type(2)));

// Partial sums of one 8-element chunk for the row statistics, in fp32:
//   LayerNorm: d = x - shift (shift = the row's first element), s1 += sum d,
//              s2 += sum d^2;  RMSNorm: s2 += sum x^2.
// LayerNorm: the shifted difference x - shift is formed in fp32 (exact for
// both formats, and no overflow for fp16 rows spanning more than its range);
// RMSNorm: the packed dot products of gfx950 (v_dot2_f32_f16 / _bf16) of x
// with itself (the products are exact in fp32).
template <int DT, bool LN>
__device__ __forceinline__ void stats_chunk(const u32x4 &c, uint32_t shift2, float &s1, float &s2)
{
    if constexpr (LN) {
        const float sh = lo_to_f<DT>(shift2);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // copy the element first: hipcc mis-lowers __builtin_bit_cast of an
            // element of a vector reference (it re-reads element 0)
            const uint32_t w = c[i];
            const float d0 = lo_to_f<DT>(w) - sh, d1 = hi_to_f<DT>(w) - sh;
            s1 += d0 + d1;
            s2 = fmaf(d0, d0, fmaf(d1, d1, s2));
        }
    } else if constexpr (DT == DT_F16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t w = c[i];
            half2_t x = __builtin_bit_cast(half2_t, w);
            s2 = __builtin_amdgcn_fdot2(x, x, s2, false);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t w = c[i];
            short2_t x = __builtin_bit_cast(short2_t, w);
            s2 = __builtin_amdgcn_fdot2_f32_bf16(x, x, s2, false);
        }
    }
}

// (rs, nmr) from the sums: normalized = x * rs + nmr. LayerNorm:
// mean = shift + s1/K, var = max(s2/K - (s1/K)^2, 0), rs = 1/sqrt(var+eps),
// nmr = -mean*rs. RMSNorm: rs = 1/sqrt(s2/K + eps), nmr = 0.
__device__ __forceinline__ void finish_stats(float s1, float s2, float shift, int64_t K,
                                             float eps, bool ln, float &rs, float &nmr)
{
    const float invK = 1.0f / (float)K;
    if (ln) {
        const float md = s1 * invK;
        const float var = fmaxf(fmaf(-md, md, s2 * invK), 0.0f);
        rs = rsqrtf(var + eps);
        nmr = -(shift + md) * rs;
    } else {
        rs = rsqrtf(s2 * invK + eps);
        nmr = 0.0f;
    }
}

// Statistics of one row in the (rs, mu) form -- normalized = (x - mu) * rs --
// for 16-byte aligned rows with K % 8 == 0, one wave per row. Each lane
// issues its 16 chunks of every 1024-chunk stretch of the row before
// accumulating any, so a row of up to 8192 elements costs one memory round
// trip (the plain loop of row_stats waits for each chunk in turn). Sums as in
// stats_chunk (shift = the row's first element for LayerNorm).
template <int DT>
__device__ __forceinline__ void row_stats_wide(const uint16_t *row, int K, float eps, int norm,
                                               int lane, float &rs, float &mu)
{
    constexpr int UNR = 16;
    const bool ln = norm == NORM_LAYERNORM;
    const uint32_t s0 = row[0];
    const uint32_t shift2 = ln ? (s0 | (s0 << 16)) : 0u;
    float s1 = 0.0f, s2 = 0.0f;
    const int nchunk = K / 8;
    for (int c0 = 0; c0 < nchunk; c0 += 64 * UNR) {
        u32x4 v[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u)
            v[u] = ldg128(row + (int64_t)min(c0 + u * 64 + lane, nchunk - 1) * 8);
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            if (c0 + u * 64 + lane < nchunk) {
                if (ln)
                    stats_chunk<DT, true>(v[u], shift2, s1, s2);
                else
                    stats_chunk<DT, false>(v[u], shift2, s1, s2);
            }
        }
    }
    s1 = wave_sum(s1);
    s2 = wave_sum(s2);
    const float invK = 1.0f / (float)K;
    if (ln) {
        const float md = s1 * invK;
        const float var = fmaxf(fmaf(-md, md, s2 * invK), 0.0f);
        rs = rsqrtf(var + eps);
        mu = bits_to_f<DT>((uint16_t)s0) + md;
    } else {
        rs = rsqrtf(s2 * invK + eps);
        mu = 0.0f;
    }
}

}  // namespace ng

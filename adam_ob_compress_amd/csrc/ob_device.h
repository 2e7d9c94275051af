// ob_device.h -- device helpers shared by the kernel translation units (loads and stores, wave and
// block reductions, DPP bit packing, and the per-element rules of the compressed step).
#pragma once

#include "ob_internal.h"

#include <math.h>

namespace ob {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned int u2 __attribute__((ext_vector_type(2)));


// Tuning knobs (compile-time; every setting computes the same results):
//   OB_P1_UNROLL / OB_P2_UNROLL   tiles in flight per loop trip in pass 1 / pass 2
//   OB_NT_P2                      nontemporal loads of the pass-2 inputs (read once more, then dead)
//   OB_NT_ST                      nontemporal stores of the pass-2 outputs
#ifndef OB_P1_UNROLL
#define OB_P1_UNROLL 4
#endif
#ifndef OB_P2_UNROLL
#define OB_P2_UNROLL 4
#endif
#ifndef OB_NT_P2
#define OB_NT_P2 1
#endif
#ifndef OB_NT_ST
#define OB_NT_ST 1
#endif
//   OB_NT_SRV                     nontemporal loads in server pass 1
//   OB_NT_UNPACK                  nontemporal stores in unpack
//   OB_NT_DENSE                   nontemporal loads and stores in the dense step
#ifndef OB_NT_SRV
#define OB_NT_SRV 1
#endif
#ifndef OB_NT_UNPACK
#define OB_NT_UNPACK 1
#endif
#ifndef OB_NT_DENSE
#define OB_NT_DENSE 1
#endif
//   OB_SRV_UNROLL / OB_SRV2_UNROLL / OB_UNPACK_UNROLL  tiles in flight per loop trip in server
//                                 pass 1 / server pass 2 / unpack
//   OB_NT_SRV_WORDS               nontemporal loads of the worker words in server pass 1
#ifndef OB_SRV_UNROLL
#define OB_SRV_UNROLL 8
#endif
#ifndef OB_SRV2_UNROLL
#define OB_SRV2_UNROLL 4
#endif
#ifndef OB_NT_SRV_WORDS
#define OB_NT_SRV_WORDS OB_NT_SRV
#endif
#ifndef OB_UNPACK_UNROLL
#define OB_UNPACK_UNROLL 4
#endif
//   OB_NT_SRV2                    nontemporal loads and stores in server pass 2
//   OB_NT_BITS                    nontemporal stores of the compressed step's packed words and int8
//                                 signs (on: lines written with ordinary stores stay in the caches and
//                                 are written back while the next chunk group's pass 1 reads)
#ifndef OB_NT_SRV2
#define OB_NT_SRV2 0
#endif
//   OB_SRV_LINES                  server pass 1 with whole-line word loads where the layout allows
//   OB_SRV_LINES_UNROLL           wave tiles (1024 elements) in flight per wave in that kernel
#ifndef OB_SRV_LINES
#define OB_SRV_LINES 1
#endif
#ifndef OB_SRV_LINES_UNROLL
#define OB_SRV_LINES_UNROLL 4
#endif
#ifndef OB_NT_BITS
#define OB_NT_BITS 1
#endif

// ------------------------------------------------------------------------------------------------
// loads and stores
// ------------------------------------------------------------------------------------------------

template <bool NT, class V>
__device__ __forceinline__ V ldv(const V* __restrict__ p)
{
    if (NT) return __builtin_nontemporal_load(p);
    return *p;
}

struct GradF32 {
    using T = float;
    template <bool NT = false, class I>
    static __device__ __forceinline__ f4 load4(const float* __restrict__ g, I i)
    {
        return ldv<NT>(reinterpret_cast<const f4*>(g + i));
    }
    template <class I>
    static __device__ __forceinline__ float load1(const float* __restrict__ g, I i) { return g[i]; }
};

// bf16 -> fp32 is exact: the bf16 bits are the high half of the fp32 bits.
struct GradBF16 {
    using T = uint16_t;
    template <bool NT = false, class I>
    static __device__ __forceinline__ f4 load4(const uint16_t* __restrict__ g, I i)
    {
        const u2 u = ldv<NT>(reinterpret_cast<const u2*>(g + i));
        f4 r;
        r.x = __uint_as_float(u.x << 16);
        r.y = __uint_as_float(u.x & 0xffff0000u);
        r.z = __uint_as_float(u.y << 16);
        r.w = __uint_as_float(u.y & 0xffff0000u);
        return r;
    }
    template <class I>
    static __device__ __forceinline__ float load1(const uint16_t* __restrict__ g, I i)
    {
        return __uint_as_float(static_cast<uint32_t>(g[i]) << 16);
    }
};

// ------------------------------------------------------------------------------------------------
// storage formats of the error buffer ([P3] Q&A on the memory cost of error feedback: the fp32 error
// term may be kept in a 16-bit format).  A stored value is widened exactly; a new error is computed
// in fp32 and `rounded` to the format (nearest, ties to even, overflow to +-Inf) before it is stored
// and before the non-finite check sees it; store4/store1 take already rounded values.
// ------------------------------------------------------------------------------------------------

struct ErrF32 {
    using T = float;
    template <bool NT = false, class I>
    static __device__ __forceinline__ f4 load4(const float* __restrict__ p, I i)
    {
        return ldv<NT>(reinterpret_cast<const f4*>(p + i));
    }
    template <class I>
    static __device__ __forceinline__ float load1(const float* __restrict__ p, I i) { return p[i]; }
    static __device__ __forceinline__ float rounded(float e) { return e; }
    static __device__ __forceinline__ float rounded_sr(float e, uint32_t) { return e; }
    template <bool NT = false, class I>
    static __device__ __forceinline__ void store4(float* __restrict__ p, I i, f4 v)
    {
        if (NT)
            __builtin_nontemporal_store(v, reinterpret_cast<f4*>(p + i));
        else
            *reinterpret_cast<f4*>(p + i) = v;
    }
    template <class I>
    static __device__ __forceinline__ void store1(float* __restrict__ p, I i, float e) { p[i] = e; }
};

// bf16 = the high half of the fp32 bits; rounding adds just under half a bf16 ulp plus the low bit
// of the kept half (ties to even), which carries into the exponent where it must (up to Inf).
struct ErrBF16 {
    using T = uint16_t;
    template <bool NT = false, class I>
    static __device__ __forceinline__ f4 load4(const uint16_t* __restrict__ p, I i)
    {
        return GradBF16::load4<NT>(p, i);
    }
    template <class I>
    static __device__ __forceinline__ float load1(const uint16_t* __restrict__ p, I i)
    {
        return GradBF16::load1(p, i);
    }
    static __device__ __forceinline__ float rounded(float e)
    {
        const uint32_t u = __float_as_uint(e);
        if ((u & 0x7fffffffu) > 0x7f800000u) return __uint_as_float((u & 0x80000000u) | 0x7fc00000u);
        return __uint_as_float((u + 0x7fffu + ((u >> 16) & 1u)) & 0xffff0000u);
    }
    // stochastic: the magnitude's low 16 bits are the distance to the lower neighbour in units of
    // 2^-16 quanta, so it rounds up iff r < them (a carry moves to the next binade, or to Inf)
    static __device__ __forceinline__ float rounded_sr(float e, uint32_t r)
    {
        const uint32_t u = __float_as_uint(e), mag = u & 0x7fffffffu;
        if (mag > 0x7f800000u) return __uint_as_float((u & 0x80000000u) | 0x7fc00000u);
        if (mag == 0x7f800000u) return e;
        const uint32_t res = (mag & 0xffff0000u) + (r < (mag & 0xffffu) ? 0x10000u : 0u);
        return __uint_as_float(res | (u & 0x80000000u));
    }
    template <bool NT = false, class I>
    static __device__ __forceinline__ void store4(uint16_t* __restrict__ p, I i, f4 v)
    {
        u2 r;
        r.x = (__float_as_uint(v.x) >> 16) | (__float_as_uint(v.y) & 0xffff0000u);
        r.y = (__float_as_uint(v.z) >> 16) | (__float_as_uint(v.w) & 0xffff0000u);
        if (NT)
            __builtin_nontemporal_store(r, reinterpret_cast<u2*>(p + i));
        else
            *reinterpret_cast<u2*>(p + i) = r;
    }
    template <class I>
    static __device__ __forceinline__ void store1(uint16_t* __restrict__ p, I i, float e)
    {
        p[i] = static_cast<uint16_t>(__float_as_uint(e) >> 16);
    }
};

// IEEE binary16 through the hardware conversions (round to nearest even; fp16 denormals kept).
struct ErrF16 {
    using T = uint16_t;
    static __device__ __forceinline__ float widen(uint32_t h)
    {
        return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
    }
    static __device__ __forceinline__ uint32_t bits(float e)
    {
        return __builtin_bit_cast(uint16_t, static_cast<_Float16>(e));
    }
    template <bool NT = false, class I>
    static __device__ __forceinline__ f4 load4(const uint16_t* __restrict__ p, I i)
    {
        const u2 u = ldv<NT>(reinterpret_cast<const u2*>(p + i));
        f4 r;
        r.x = widen(u.x & 0xffffu);
        r.y = widen(u.x >> 16);
        r.z = widen(u.y & 0xffffu);
        r.w = widen(u.y >> 16);
        return r;
    }
    template <class I>
    static __device__ __forceinline__ float load1(const uint16_t* __restrict__ p, I i) { return widen(p[i]); }
    // e is the fp32 value of a line evaluated in double.  The empty asm keeps it an fp32 register:
    // without it the compiler fuses the two roundings (double -> fp32 -> fp16) into one software
    // double -> fp16 rounding, which differs where the fp32 value is an fp16 midpoint that the double
    // value misses by less than half an fp32 ulp (nearest-even of the fp32 value is the rule here).
    static __device__ __forceinline__ float rounded(float e)
    {
        __asm__ volatile("" : "+v"(e));
        return static_cast<float>(static_cast<_Float16>(e));
    }
    // stochastic: lo = |e| truncated to fp16, q its quantum; hi = lo + q iff r*q < (|e| - lo)*65536,
    // taken on the fp32 bits.  |e| >= 2^-14 (fp16 normal): q is 2^13 fp32 quanta, so the fraction is
    // the low 13 significand bits f and the test is r < 8f; the carry of lo + q moves into the next
    // binade, and above 65504 (0x477fe000) is Inf.  Below: q = 2^-24; with the 24-bit significand S
    // and |e| = S * 2^-(24 + s), lo = (S >> s) q and the test is r * 2^s < frac * 2^16 (s >= 14; past
    // s = 47 only r = 0 rounds up, as r * 2^s > frac * 2^16 for r >= 1).
    static __device__ __forceinline__ float rounded_sr(float e, uint32_t r)
    {
        const uint32_t u = __float_as_uint(e), mag = u & 0x7fffffffu;
        if (mag >= 0x7f800000u) return e;
        uint32_t res;
        if (mag >= 0x38800000u) {
            res = (mag & ~0x1fffu) + (r < ((mag & 0x1fffu) << 3) ? 0x2000u : 0u);
            if (res > 0x477fe000u) res = 0x7f800000u;
        } else {
            const uint32_t ex = mag >> 23;
            const uint32_t S = ex ? ((mag & 0x7fffffu) | 0x800000u) : mag;
            const uint32_t s = ex ? 126u - ex : 125u;
            const uint32_t k = s < 32u ? (S >> s) : 0u;
            const uint64_t frac = s < 32u ? (S & ((1u << s) - 1u)) : S;
            const uint32_t sc = s < 47u ? s : 47u;
            const uint32_t up = (static_cast<uint64_t>(r) << sc) < (frac << 16) ? 1u : 0u;
            res = __float_as_uint(static_cast<float>(k + up) * 5.9604644775390625e-8f);
        }
        return __uint_as_float(res | (u & 0x80000000u));
    }
    template <bool NT = false, class I>
    static __device__ __forceinline__ void store4(uint16_t* __restrict__ p, I i, f4 v)
    {
        u2 r;
        r.x = bits(v.x) | (bits(v.y) << 16);
        r.y = bits(v.z) | (bits(v.w) << 16);
        if (NT)
            __builtin_nontemporal_store(r, reinterpret_cast<u2*>(p + i));
        else
            *reinterpret_cast<u2*>(p + i) = r;
    }
    template <class I>
    static __device__ __forceinline__ void store1(uint16_t* __restrict__ p, I i, float e)
    {
        p[i] = static_cast<uint16_t>(bits(e));
    }
};

// ------------------------------------------------------------------------------------------------
// stochastic rounding of the error buffer: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC 2011), a counter-based generator, gives element i the high 16 bits
// of output word i & 3 at the 128-bit counter (i >> 2, step) under the 64-bit key seed (each split
// into 32-bit words, low word first).  One block serves the 4 elements of a lane (i a multiple of 4);
// its multiplies are native 32 x 32 -> 64-bit products.
// ------------------------------------------------------------------------------------------------

struct u4 {
    uint32_t x[4];
};

__device__ __forceinline__ u4 philox_block(uint64_t seed, uint64_t step, int64_t i)
{
    const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u, W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
    const uint64_t blk = static_cast<uint64_t>(i) >> 2;
    uint32_t c0 = static_cast<uint32_t>(blk), c1 = static_cast<uint32_t>(blk >> 32);
    uint32_t c2 = static_cast<uint32_t>(step), c3 = static_cast<uint32_t>(step >> 32);
    uint32_t k0 = static_cast<uint32_t>(seed), k1 = static_cast<uint32_t>(seed >> 32);
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += W0;
            k1 += W1;
        }
        const uint64_t p0 = static_cast<uint64_t>(M0) * c0, p1 = static_cast<uint64_t>(M1) * c2;
        const uint32_t n0 = static_cast<uint32_t>(p1 >> 32) ^ c1 ^ k0;
        const uint32_t n2 = static_cast<uint32_t>(p0 >> 32) ^ c3 ^ k1;
        c1 = static_cast<uint32_t>(p1);
        c3 = static_cast<uint32_t>(p0);
        c0 = n0;
        c2 = n2;
    }
    return u4{{c0, c1, c2, c3}};
}

// ob_dtype code of the error buffer -> its format
template <int EF> struct ErrOf;
template <> struct ErrOf<0> { using type = ErrF32; };
template <> struct ErrOf<1> { using type = ErrBF16; };
template <> struct ErrOf<2> { using type = ErrF16; };

template <bool NT = false, class I>
__device__ __forceinline__ f4 ld4(const float* __restrict__ p, I i)
{
    return ldv<NT>(reinterpret_cast<const f4*>(p + i));
}

template <bool NT = false, class I>
__device__ __forceinline__ void st4(float* __restrict__ p, I i, f4 v)
{
    if (NT)
        __builtin_nontemporal_store(v, reinterpret_cast<f4*>(p + i));
    else
        *reinterpret_cast<f4*>(p + i) = v;
}

// ------------------------------------------------------------------------------------------------
// reductions and bit packing
// ------------------------------------------------------------------------------------------------

// Butterfly over the 64 lanes: each step adds two equal-content partial sums, so every lane ends
// with the same bits.
__device__ __forceinline__ double wave_sum(double v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Sum over the block in a fixed order; every thread returns the same value.
__device__ __forceinline__ double block_sum(double v, double* lds)
{
    v = wave_sum(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = v;
    __syncthreads();
    double s = lds[0];
#pragma unroll
    for (int w = 1; w < kBlock / 64; ++w) s += lds[w];
    return s;
}

__device__ __forceinline__ uint32_t block_sum_u32(uint32_t v, uint32_t* lds)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = v;
    __syncthreads();
    uint32_t s = 0;
#pragma unroll
    for (int w = 0; w < kBlock / 64; ++w) s += lds[w];
    return s;
}

// OR of a value across each group of 8 consecutive lanes, via DPP:
// quad_perm[1,0,3,2], quad_perm[2,3,0,1], then row_half_mirror (lane j <-> 7-j in each 8-lane half
// row).  After the call every lane of the group holds the group's OR.  Must run with all lanes active.
__device__ __forceinline__ uint32_t or8(uint32_t v)
{
    v |= static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0xB1, 0xF, 0xF, false));
    v |= static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x4E, 0xF, 0xF, false));
    v |= static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x141, 0xF, 0xF, false));
    return v;
}

// Lane tid holds the 4 sign bits of elements i..i+3 (i = tile start + 4*tid, tile start a multiple of
// 32).  Lanes 8k..8k+7 together hold the 32 bits of one word; lane 8k writes it if `valid`, with a
// nontemporal store when NT.
template <bool NT, class I>
__device__ __forceinline__ void store_word(uint32_t* __restrict__ words, I i, uint32_t nib, bool valid)
{
    const uint32_t w = or8(nib << (4 * (threadIdx.x & 7)));
    if ((threadIdx.x & 7) == 0 && valid) {
        if (NT)
            __builtin_nontemporal_store(w, words + (i >> 5));
        else
            words[i >> 5] = w;
    }
}

__device__ __forceinline__ uint32_t signs4(uint32_t nib)
{
    // byte k = +1 (0x01) or -1 (0xFF) by bit k
    uint32_t r = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) r |= ((nib >> k) & 1u ? 0x01u : 0xFFu) << (8 * k);
    return r;
}

// ------------------------------------------------------------------------------------------------
// element rules
// ------------------------------------------------------------------------------------------------

// compensated = clip(g) + err ([P2] 1-bit Adam; clip of [P1] sec. 3.2).  NaN passes the clip.
template <bool CLIP>
__device__ __forceinline__ float compensate(float g, float e, float clip)
{
    if (CLIP) g = g > clip ? clip : (g < -clip ? -clip : g);
    return g + e;
}

// The sign bit of one element (1 <=> +1) and its new error from g_hat = +-scale: x, g_hat and delta
// are single fp32 operations, the EMA line is evaluated in double and rounded once.
template <bool EMA>
__device__ __forceinline__ uint32_t error_elem(float x, float& e, float scale, const CompressParams& cp)
{
    const bool b = x >= 0.0f;
    const float gh = b ? scale : -scale;              // the value the bit stands for
    const float delta = x - gh;                       // what it failed to carry
    if (EMA)
        e = static_cast<float>(cp.ef_beta * static_cast<double>(e) + cp.one_m_ef_beta * static_cast<double>(delta));
    else
        e = delta;
    return b ? 1u : 0u;
}

// m on g_hat ([P1] sec. 2.2; [P2]) and the frozen-v update with the stored (new) m ([P2]); both lines in
// double, rounded once, so a large update that nearly cancels p keeps full fp32 accuracy.
__device__ __forceinline__ void update_elem(float gh, float& mm, float vv, float& pp, const CompressParams& cp)
{
    mm = static_cast<float>(cp.beta1 * static_cast<double>(mm) + cp.one_m_beta1 * static_cast<double>(gh));
    const double den = sqrt(static_cast<double>(vv)) + cp.eps;
    pp = static_cast<float>(static_cast<double>(pp) - cp.lr * (static_cast<double>(mm) / den));
}

// One element of the compressed step; returns the sign bit (1 <=> +1).
// LAMB: p is left alone; u = m / (sqrt(v) + eps) (double, not stored) adds u^2 to usq for the layer's
// trust ratio.
template <bool EMA, bool LAMB>
__device__ __forceinline__ uint32_t compress_elem(float x, float& e, float& mm, float vv, float& pp, double& usq,
                                                  float scale, const CompressParams& cp)
{
    const uint32_t b = error_elem<EMA>(x, e, scale, cp);
    const float gh = b ? scale : -scale;
    if (!LAMB) {
        update_elem(gh, mm, vv, pp, cp);
        return b;
    }
    mm = static_cast<float>(cp.beta1 * static_cast<double>(mm) + cp.one_m_beta1 * static_cast<double>(gh));
    const double den = sqrt(static_cast<double>(vv)) + cp.eps;
    const double u = static_cast<double>(mm) / den;
    usq = fma(u, u, usq);
    return b;
}

// Chunk scale from the chunk's pass-1 partials, reduced in a fixed order (so every pass-2 block of
// the chunk computes the same bits).
__device__ __forceinline__ float chunk_scale(const PlanDev& pd, int c, double* lds)
{
    const int f0 = pd.p1_first[c], f1 = pd.p1_first[c + 1];
    double s = 0.0;
    for (int i = f0 + static_cast<int>(threadIdx.x); i < f1; i += kBlock) s += pd.partials[i];
    s = block_sum(s, lds);
    const int64_t nc = pd.chunk_off[c + 1] - pd.chunk_off[c];
    return static_cast<float>(sqrt(s / static_cast<double>(nc)));
}

// chunk_scale with the first group of tile loads overlapped: the chunk's partials are loaded, then
// `load_first()` issues the block's first tile loads (only when the block has a whole group), and
// only then are the partials reduced.  The partial loads precede the tile loads, so the in-order load
// counter lets the reduction wait for the partials alone.  The sum order, and so every block's scale
// bits, are those of chunk_scale.
template <class F>
__device__ __forceinline__ float chunk_scale_overlapped(const PlanDev& pd, int c, double* lds, bool whole_group,
                                                        F&& load_first)
{
    const int f0 = pd.p1_first[c], f1 = pd.p1_first[c + 1];
    double s = f0 + static_cast<int>(threadIdx.x) < f1 ? pd.partials[f0 + threadIdx.x] : 0.0;
    if (f1 - f0 > kBlock)
        for (int j = f0 + static_cast<int>(threadIdx.x) + kBlock; j < f1; j += kBlock) s += pd.partials[j];
    const int64_t nc = pd.chunk_off[c + 1] - pd.chunk_off[c];
    auto reduce = [&]() { return static_cast<float>(sqrt(block_sum(s, lds) / static_cast<double>(nc))); };
    // (two copies of the reduction, so that the load counter's wait on the path with the tile loads in
    // flight covers the partials alone)
    if (whole_group) {
        load_first();
        return reduce();
    }
    return reduce();
}

}  // namespace
}  // namespace ob

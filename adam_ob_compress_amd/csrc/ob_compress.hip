// ob_compress.hip -- the compressed step (pass 1: per-block sums of squares; pass 2: the fused
// streaming update) for one storage format of the error buffer.  Built once per format with
// -DOB_ERR_FMT=0 (fp32), 1 (bf16) or 2 (fp16); each build defines that format's launchers.
//
// Pages cited (title and section):
//   [P1] "1bit Adam" tutorial (intelliparadigm.com article 2150495): sec. 2.1 (sign quantization and
//        EMA error compensation), sec. 2.2 (first moment on the compressed gradient), sec. 3.2
//        (clip before quantizing, NaN check, int8 signs).
//   [P2] "DeepSpeed Communication Compression and Hiding": "1-bit Adam: warmup, frozen variance,
//        error feedback" (compressed branch of the two-phase step, dequantize).
//        "1-bit LAMB: also protect the layer-wise trust ratio" (the LAMB variant: the layer's
//        norms are taken on the reconstructed direction; the update itself is in ob_kernels.hip).
//   [P3] gradient-compression survey (bmjup.com post 14450): Q&A on the memory cost of error
//        feedback (a 16-bit error term).
//
// Design (memory bound: ~30 bytes and a few dozen ALU ops per element, no dense contraction, so no
// MFMA):
//   * every kernel walks work blocks ("items") of one chunk each; a block of 256 threads = four
//     wave64s; each lane owns 4 consecutive elements per 1024-element tile, so each fp32 array moves
//     as one 16-byte access per lane (8 bytes for 16-bit arrays) and a wave covers a contiguous run;
//   * the per-chunk scale needs the whole chunk before any element can be finished, hence two
//     passes: pass 1 writes one double partial sum of squares per block (wave butterfly in registers,
//     LDS across the four waves); pass 2 reduces the chunk's partials in a fixed order at its start
//     (every block of the chunk gets bit-identical scales), then does the fused streaming update;
//   * the host runs the two passes over groups of consecutive chunks sized to the Infinity Cache, so
//     that pass 2's re-read of g and err comes from the cache: pass 1 then loads with ordinary
//     (allocating) loads (nontemporal ones when a single launch covers all chunks), pass 2 with
//     nontemporal ones; a launch covers blocks [item0, item0 + n_items) of the plan-wide table and
//     writes its per-block results at their plan-wide index, so the results do not depend on the
//     grouping;
//   * sign bits: each lane forms a 4-bit nibble; an OR across 8 neighbouring lanes with DPP row
//     permutes (no LDS) builds the 32-bit word of 32 consecutive elements, written by one lane;
//   * all fp32 arithmetic is plain IEEE (no fast-math, denormals kept: a negative denormal must give
//     sign -1).
#include "ob_device.h"

#include <type_traits>

#ifndef OB_ERR_FMT
#error "build with -DOB_ERR_FMT=0 (fp32), 1 (bf16) or 2 (fp16)"
#endif

namespace ob {
namespace {

// ------------------------------------------------------------------------------------------------
// compressed step, pass 1: per-block sum of squares of x = clip(g) + err
// (LAMB: and of the parameters, for the layer's ||w||; DIAG: and of the error buffer read)
// ------------------------------------------------------------------------------------------------

// NT: nontemporal loads (a single launch over the whole buffer, whose reads pass 2 gets from HBM anyway);
// ordinary ones when the launch covers one chunk group, so that pass 2 finds its lines in the cache.
template <class G, class E, bool CLIP, bool LAMB, bool DIAG, bool NT>
__global__ __launch_bounds__(kBlock) void k_chunk_sumsq(PlanDev pd, const typename G::T* __restrict__ g,
                                                        const typename E::T* __restrict__ err, float clip,
                                                        const float* __restrict__ p)
{
    __shared__ double lds[kBlock / 64];
    const int blk = pd.item0 + static_cast<int>(blockIdx.x);
    const Item it = pd.items[blk];
    const int tid = threadIdx.x;
    double acc = 0.0, accw = 0.0, acce = 0.0;
    constexpr int U = OB_P1_UNROLL;
    int base = 0;
    for (; base + U * kTile <= it.len; base += U * kTile) {
        f4 gv[U], ev[U], pv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = it.start + base + u * kTile + kVec * tid;
            gv[u] = G::template load4<NT>(g, i);
            ev[u] = E::template load4<NT>(err, i);
            if (LAMB) pv[u] = ld4<NT>(p, i);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int k = 0; k < kVec; ++k) {
                const double x = compensate<CLIP>(gv[u][k], ev[u][k], clip);
                acc = fma(x, x, acc);
                if (LAMB) accw = fma(static_cast<double>(pv[u][k]), static_cast<double>(pv[u][k]), accw);
                if (DIAG) acce = fma(static_cast<double>(ev[u][k]), static_cast<double>(ev[u][k]), acce);
            }
        }
    }
    for (; base < it.len; base += kTile) {
        const int cnt = it.len - base - kVec * tid;
        const int64_t i = it.start + base + kVec * tid;
        if (cnt >= kVec) {
            const f4 gv = G::load4(g, i), ev = E::load4(err, i);
            f4 pv = {0.0f, 0.0f, 0.0f, 0.0f};
            if (LAMB) pv = ld4(p, i);
#pragma unroll
            for (int k = 0; k < kVec; ++k) {
                const double x = compensate<CLIP>(gv[k], ev[k], clip);
                acc = fma(x, x, acc);
                if (LAMB) accw = fma(static_cast<double>(pv[k]), static_cast<double>(pv[k]), accw);
                if (DIAG) acce = fma(static_cast<double>(ev[k]), static_cast<double>(ev[k]), acce);
            }
        } else {
            #pragma unroll
            for (int k = 0; k < kVec; ++k) {
                if (k >= cnt) continue;
                const float e = E::load1(err, i + k);
                const double x = compensate<CLIP>(G::load1(g, i + k), e, clip);
                acc = fma(x, x, acc);
                if (LAMB) accw = fma(static_cast<double>(p[i + k]), static_cast<double>(p[i + k]), accw);
                if (DIAG) acce = fma(static_cast<double>(e), static_cast<double>(e), acce);
            }
        }
    }
    const double s = block_sum(acc, lds);
    if (tid == 0) pd.partials[blk] = s;
    if (LAMB) {
        const double sw = block_sum(accw, lds);
        if (tid == 0) pd.partials_w[blk] = sw;
    }
    if (DIAG) {
        const double se = block_sum(acce, lds);
        if (tid == 0) pd.partials_e[blk] = se;
    }
}

// ------------------------------------------------------------------------------------------------
// compressed step, pass 2: scale, sign bits, error, m, p in one streaming pass
// (LAMB: no update of p; the block's sum of u^2 for the layer's ||u|| instead)
// ------------------------------------------------------------------------------------------------

template <class G, class E, bool CLIP, bool EMA, bool SIGNS, bool NONFIN, bool LAMB, bool SR>
__global__ __launch_bounds__(kBlock) void k_compress(PlanDev pd, const typename G::T* __restrict__ g,
                                                     typename E::T* __restrict__ err, float* __restrict__ m,
                                                     const float* __restrict__ v, float* __restrict__ p,
                                                     uint32_t* __restrict__ words, float* __restrict__ scales,
                                                     int8_t* __restrict__ signs,
                                                     unsigned long long* __restrict__ nonfinite,
                                                     CompressParams cp)
{
    __shared__ double lds[kBlock / 64];
    const int blk = pd.item0 + static_cast<int>(blockIdx.x);
    const Item it = pd.items[blk];
    const int tid = threadIdx.x;
    constexpr int U = OB_P2_UNROLL;
    f4 gv[U], ev[U], mv[U], vv[U], pv[U];
    auto load_group = [&](int b) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = it.start + b + u * kTile + kVec * tid;
            gv[u] = G::template load4<OB_NT_P2>(g, i);
            ev[u] = E::template load4<OB_NT_P2>(err, i);
            mv[u] = ld4<OB_NT_P2>(m, i);
            vv[u] = ld4<OB_NT_P2>(v, i);
            if (!LAMB) pv[u] = ld4<OB_NT_P2>(p, i);
        }
    };
    // the chunk's scale, reduced while the block's first group of tiles is in flight
    const float scale = chunk_scale_overlapped(pd, it.chunk, lds, U * kTile <= it.len, [&] { load_group(0); });
    if (tid == 0 && blk == pd.chunk_first[it.chunk]) scales[it.chunk] = scale;

    uint32_t nf = 0, plus = 0;
    double usq = 0.0;
    int base = 0;
    for (; base + U * kTile <= it.len; base += U * kTile) {
        if (base > 0) load_group(base);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = it.start + base + u * kTile + kVec * tid;
            const u4 rw = SR ? philox_block(cp.sr_seed, cp.sr_step, i) : u4{};
            uint32_t nib = 0;
#pragma unroll
            for (int k = 0; k < kVec; ++k) {
                const float x = compensate<CLIP>(gv[u][k], ev[u][k], cp.clip);
                float e = ev[u][k], mm = mv[u][k], pp = LAMB ? 0.0f : pv[u][k];
                nib |= compress_elem<EMA, LAMB>(x, e, mm, vv[u][k], pp, usq, scale, cp) << k;
                e = SR ? E::rounded_sr(e, rw.x[k] >> 16) : E::rounded(e);
                ev[u][k] = e;
                mv[u][k] = mm;
                if (!LAMB) pv[u][k] = pp;
                if (NONFIN) nf += __builtin_isfinite(e) ? 0u : 1u;
            }
            E::template store4<OB_NT_ST>(err, i, ev[u]);
            st4<OB_NT_ST>(m, i, mv[u]);
            if (!LAMB) st4<OB_NT_ST>(p, i, pv[u]);
            if (SIGNS) {
                uint32_t* sp = reinterpret_cast<uint32_t*>(signs + i);
                if (OB_NT_BITS)
                    __builtin_nontemporal_store(signs4(nib), sp);
                else
                    *sp = signs4(nib);
            }
            store_word<OB_NT_BITS>(words, i, nib, true);
            plus += __builtin_popcount(nib);
        }
    }
    for (; base < it.len; base += kTile) {
        const int rem = it.len - base;
        const int cnt = rem - kVec * tid;
        const int64_t i = it.start + base + kVec * tid;
        const u4 rw = (SR && cnt > 0) ? philox_block(cp.sr_seed, cp.sr_step, i) : u4{};
        uint32_t nib = 0;
        if (cnt >= kVec) {
            const f4 gv = G::load4(g, i), vv = ld4(v, i);
            f4 ev = E::load4(err, i), mv = ld4(m, i), pv = {0.0f, 0.0f, 0.0f, 0.0f};
            if (!LAMB) pv = ld4(p, i);
#pragma unroll
            for (int k = 0; k < kVec; ++k) {
                const float x = compensate<CLIP>(gv[k], ev[k], cp.clip);
                float e = ev[k], mm = mv[k], pp = pv[k];
                nib |= compress_elem<EMA, LAMB>(x, e, mm, vv[k], pp, usq, scale, cp) << k;
                e = SR ? E::rounded_sr(e, rw.x[k] >> 16) : E::rounded(e);
                ev[k] = e;
                mv[k] = mm;
                pv[k] = pp;
                if (NONFIN) nf += __builtin_isfinite(e) ? 0u : 1u;
            }
            E::store4(err, i, ev);
            st4(m, i, mv);
            if (!LAMB) st4(p, i, pv);
            if (SIGNS) *reinterpret_cast<uint32_t*>(signs + i) = signs4(nib);
        } else if (cnt > 0) {
            #pragma unroll
            for (int k = 0; k < kVec; ++k) {
                if (k >= cnt) continue;
                float e = E::load1(err, i + k), mm = m[i + k], pp = LAMB ? 0.0f : p[i + k];
                const float x = compensate<CLIP>(G::load1(g, i + k), e, cp.clip);
                const uint32_t b = compress_elem<EMA, LAMB>(x, e, mm, v[i + k], pp, usq, scale, cp);
                nib |= b << k;
                e = SR ? E::rounded_sr(e, rw.x[k] >> 16) : E::rounded(e);
                E::store1(err, i + k, e);
                m[i + k] = mm;
                if (!LAMB) p[i + k] = pp;
                if (SIGNS) signs[i + k] = b ? int8_t(1) : int8_t(-1);
                if (NONFIN) nf += __builtin_isfinite(e) ? 0u : 1u;
            }
        }
        store_word<OB_NT_BITS>(words, i, nib, 32 * (tid >> 3) < rem);
        plus += __builtin_popcount(nib);
    }
    if (pd.partials_b != nullptr) {   // diagnostics: +1 signs of the block (nib holds valid elements only)
        __shared__ uint32_t ldsb[kBlock / 64];
        const uint32_t t = block_sum_u32(plus, ldsb);
        if (tid == 0) pd.partials_b[blk] = t;
    }
    if (NONFIN) {
        __shared__ uint32_t ldsu[kBlock / 64];
        const uint32_t t = block_sum_u32(nf, ldsu);
        if (tid == 0 && t) atomicAdd(nonfinite, static_cast<unsigned long long>(t));
    }
    if (LAMB) {
        const double su = block_sum(usq, lds);
        if (tid == 0) pd.partials_u[blk] = su;
    }
}

// ------------------------------------------------------------------------------------------------
// the worker's half of a compressed step before the exchange (more than one worker): pass 2 without
// m, v and p -- scale, sign bits and the error from the worker's own g_hat
// ------------------------------------------------------------------------------------------------

template <class G, class E, bool CLIP, bool EMA, bool SR>
__global__ __launch_bounds__(kBlock) void k_worker_compress(PlanDev pd, const typename G::T* __restrict__ g,
                                                            typename E::T* __restrict__ err,
                                                            uint32_t* __restrict__ words, float* __restrict__ scales,
                                                            int8_t* __restrict__ signs,
                                                            unsigned long long* __restrict__ nonfinite,
                                                            CompressParams cp)
{
    __shared__ double lds[kBlock / 64];
    const int blk = pd.item0 + static_cast<int>(blockIdx.x);
    const Item it = pd.items[blk];
    const int tid = threadIdx.x;
    constexpr int U = OB_P2_UNROLL;
    f4 gv[U], ev[U];
    auto load_group = [&](int b) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = it.start + b + u * kTile + kVec * tid;
            gv[u] = G::template load4<OB_NT_P2>(g, i);
            ev[u] = E::template load4<OB_NT_P2>(err, i);
        }
    };
    // the chunk's scale, reduced while the block's first group of tiles is in flight
    const float scale = chunk_scale_overlapped(pd, it.chunk, lds, U * kTile <= it.len, [&] { load_group(0); });
    if (tid == 0 && blk == pd.chunk_first[it.chunk]) scales[it.chunk] = scale;
    uint32_t nf = 0;
    int base = 0;
    for (; base + U * kTile <= it.len; base += U * kTile) {
        if (base > 0) load_group(base);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = it.start + base + u * kTile + kVec * tid;
            const u4 rw = SR ? philox_block(cp.sr_seed, cp.sr_step, i) : u4{};
            uint32_t nib = 0;
#pragma unroll
            for (int k = 0; k < kVec; ++k) {
                const float x = compensate<CLIP>(gv[u][k], ev[u][k], cp.clip);
                float e = ev[u][k];
                nib |= error_elem<EMA>(x, e, scale, cp) << k;
                e = SR ? E::rounded_sr(e, rw.x[k] >> 16) : E::rounded(e);
                ev[u][k] = e;
                nf += __builtin_isfinite(e) ? 0u : 1u;
            }
            E::template store4<OB_NT_ST>(err, i, ev[u]);
            if (signs) {
                uint32_t* sp = reinterpret_cast<uint32_t*>(signs + i);
                if (OB_NT_BITS)
                    __builtin_nontemporal_store(signs4(nib), sp);
                else
                    *sp = signs4(nib);
            }
            store_word<OB_NT_BITS>(words, i, nib, true);
        }
    }
    for (; base < it.len; base += kTile) {
        const int rem = it.len - base;
        const int cnt = rem - kVec * tid;
        const int64_t i = it.start + base + kVec * tid;
        const u4 rw = (SR && cnt > 0) ? philox_block(cp.sr_seed, cp.sr_step, i) : u4{};
        uint32_t nib = 0;
        #pragma unroll
        for (int k = 0; k < kVec; ++k) {
            if (k >= cnt) continue;
            float e = E::load1(err, i + k);
            const float x = compensate<CLIP>(G::load1(g, i + k), e, cp.clip);
            const uint32_t b = error_elem<EMA>(x, e, scale, cp);
            nib |= b << k;
            e = SR ? E::rounded_sr(e, rw.x[k] >> 16) : E::rounded(e);
            E::store1(err, i + k, e);
            if (signs) signs[i + k] = b ? int8_t(1) : int8_t(-1);
            nf += __builtin_isfinite(e) ? 0u : 1u;
        }
        store_word<OB_NT_BITS>(words, i, nib, 32 * (tid >> 3) < rem);
    }
    if (nonfinite) {
        __shared__ uint32_t ldsu[kBlock / 64];
        const uint32_t t = block_sum_u32(nf, ldsu);
        if (tid == 0 && t) atomicAdd(nonfinite, static_cast<unsigned long long>(t));
    }
}

}  // namespace

// ------------------------------------------------------------------------------------------------
// launchers
// ------------------------------------------------------------------------------------------------

namespace {
template <class G, class E>
void sumsq_dispatch(int sel, bool nt, dim3 grid, dim3 block, hipStream_t s, const PlanDev& pd,
                    const typename G::T* g, const typename E::T* err, float clip, const float* p)
{
#define OB_CASE(k, CL, LA, DG)                                                                              \
    case k:                                                                                                  \
        if (nt)                                                                                              \
            hipLaunchKernelGGL((k_chunk_sumsq<G, E, CL, LA, DG, true>), grid, block, 0, s, pd, g, err, clip, p);  \
        else                                                                                                 \
            hipLaunchKernelGGL((k_chunk_sumsq<G, E, CL, LA, DG, false>), grid, block, 0, s, pd, g, err, clip, p); \
        break;
    switch (sel) {
        OB_CASE(0, false, false, false)
        OB_CASE(1, true, false, false)
        OB_CASE(2, false, true, false)
        OB_CASE(3, true, true, false)
        OB_CASE(4, false, false, true)
        OB_CASE(5, true, false, true)
        OB_CASE(6, false, true, true)
        OB_CASE(7, true, true, true)
    }
#undef OB_CASE
}
}  // namespace

template <int EF>
hipError_t launch_chunk_sumsq(const PlanDev& pd, const void* g, int g_bf16, const void* err_v, float clip,
                              const float* lamb_p, int nontemporal, hipStream_t s)
{
    using E = typename ErrOf<EF>::type;
    auto err = static_cast<const typename E::T*>(err_v);
    const dim3 grid(static_cast<unsigned>(pd.n_items)), block(kBlock);
    const int sel = (clip > 0.0f ? 1 : 0) | (lamb_p ? 2 : 0) | (pd.partials_e ? 4 : 0);
    if (g_bf16)
        sumsq_dispatch<GradBF16, E>(sel, nontemporal != 0, grid, block, s, pd, static_cast<const uint16_t*>(g), err,
                                    clip, lamb_p);
    else
        sumsq_dispatch<GradF32, E>(sel, nontemporal != 0, grid, block, s, pd, static_cast<const float*>(g), err,
                                   clip, lamb_p);
    return hipGetLastError();
}

namespace {
template <class G, class E, bool CLIP, bool EMA, bool LAMB, bool SR>
void compress_dispatch_sr(const PlanDev& pd, const typename G::T* g, typename E::T* err, float* m,
                          const float* v, float* p, uint32_t* words, float* scales, int8_t* signs,
                          unsigned long long* nonfinite, const CompressParams& cp, hipStream_t s)
{
    const dim3 grid(static_cast<unsigned>(pd.n_items)), block(kBlock);
    const int sel = (signs ? 1 : 0) | (nonfinite ? 2 : 0);
    switch (sel) {
    case 0:
        hipLaunchKernelGGL((k_compress<G, E, CLIP, EMA, false, false, LAMB, SR>), grid, block, 0, s, pd, g, err,
                           m, v, p, words, scales, signs, nonfinite, cp);
        break;
    case 1:
        hipLaunchKernelGGL((k_compress<G, E, CLIP, EMA, true, false, LAMB, SR>), grid, block, 0, s, pd, g, err,
                           m, v, p, words, scales, signs, nonfinite, cp);
        break;
    case 2:
        hipLaunchKernelGGL((k_compress<G, E, CLIP, EMA, false, true, LAMB, SR>), grid, block, 0, s, pd, g, err,
                           m, v, p, words, scales, signs, nonfinite, cp);
        break;
    default:
        hipLaunchKernelGGL((k_compress<G, E, CLIP, EMA, true, true, LAMB, SR>), grid, block, 0, s, pd, g, err,
                           m, v, p, words, scales, signs, nonfinite, cp);
        break;
    }
}

// stochastic rounding exists for the 16-bit formats only (the host rejects it for fp32 buffers)
template <class G, class E, bool CLIP, bool EMA, bool LAMB>
void compress_dispatch(const PlanDev& pd, const typename G::T* g, typename E::T* err, float* m, const float* v,
                       float* p, uint32_t* words, float* scales, int8_t* signs,
                       unsigned long long* nonfinite, const CompressParams& cp, hipStream_t s)
{
    if constexpr (!std::is_same<E, ErrF32>::value) {
        if (cp.stochastic) {
            compress_dispatch_sr<G, E, CLIP, EMA, LAMB, true>(pd, g, err, m, v, p, words, scales, signs,
                                                              nonfinite, cp, s);
            return;
        }
    }
    compress_dispatch_sr<G, E, CLIP, EMA, LAMB, false>(pd, g, err, m, v, p, words, scales, signs, nonfinite,
                                                       cp, s);
}

template <class G, class E>
void compress_dispatch_g(const PlanDev& pd, const typename G::T* g, typename E::T* err, float* m, const float* v,
                         float* p, uint32_t* words, float* scales, int8_t* signs,
                         unsigned long long* nonfinite, int ema, int lamb, const CompressParams& cp,
                         hipStream_t s)
{
    const int sel = (cp.clip > 0.0f ? 1 : 0) | (ema ? 2 : 0) | (lamb ? 4 : 0);
#define OB_CASE(k, CL, EM, LA)                                                                              \
    case k:                                                                                                  \
        compress_dispatch<G, E, CL, EM, LA>(pd, g, err, m, v, p, words, scales, signs, nonfinite, cp, s); \
        break;
    switch (sel) {
        OB_CASE(0, false, false, false)
        OB_CASE(1, true, false, false)
        OB_CASE(2, false, true, false)
        OB_CASE(3, true, true, false)
        OB_CASE(4, false, false, true)
        OB_CASE(5, true, false, true)
        OB_CASE(6, false, true, true)
        OB_CASE(7, true, true, true)
    }
#undef OB_CASE
}
}  // namespace

template <int EF>
hipError_t launch_compress(const PlanDev& pd, const void* g, int g_bf16, void* err_v, float* m, const float* v,
                           float* p, uint32_t* words, float* scales, int8_t* signs,
                           unsigned long long* nonfinite, int ema, int lamb, const CompressParams& cp,
                           hipStream_t s)
{
    using E = typename ErrOf<EF>::type;
    auto err = static_cast<typename E::T*>(err_v);
    if (g_bf16)
        compress_dispatch_g<GradBF16, E>(pd, static_cast<const uint16_t*>(g), err, m, v, p, words, scales,
                                         signs, nonfinite, ema, lamb, cp, s);
    else
        compress_dispatch_g<GradF32, E>(pd, static_cast<const float*>(g), err, m, v, p, words, scales, signs,
                                        nonfinite, ema, lamb, cp, s);
    return hipGetLastError();
}

namespace {
template <class G, class E, bool CLIP, bool EMA>
void worker_dispatch(const PlanDev& pd, const typename G::T* g, typename E::T* err, uint32_t* words,
                     float* scales, int8_t* signs, unsigned long long* nonfinite, const CompressParams& cp,
                     hipStream_t s)
{
    const dim3 grid(static_cast<unsigned>(pd.n_items)), block(kBlock);
    if constexpr (!std::is_same<E, ErrF32>::value) {
        if (cp.stochastic) {
            hipLaunchKernelGGL((k_worker_compress<G, E, CLIP, EMA, true>), grid, block, 0, s, pd, g, err, words,
                               scales, signs, nonfinite, cp);
            return;
        }
    }
    hipLaunchKernelGGL((k_worker_compress<G, E, CLIP, EMA, false>), grid, block, 0, s, pd, g, err, words, scales,
                       signs, nonfinite, cp);
}

template <class G, class E>
void worker_dispatch_g(const PlanDev& pd, const typename G::T* g, typename E::T* err, uint32_t* words,
                       float* scales, int8_t* signs, unsigned long long* nonfinite, int ema,
                       const CompressParams& cp, hipStream_t s)
{
    const int sel = (cp.clip > 0.0f ? 1 : 0) | (ema ? 2 : 0);
    switch (sel) {
    case 0: worker_dispatch<G, E, false, false>(pd, g, err, words, scales, signs, nonfinite, cp, s); break;
    case 1: worker_dispatch<G, E, true, false>(pd, g, err, words, scales, signs, nonfinite, cp, s); break;
    case 2: worker_dispatch<G, E, false, true>(pd, g, err, words, scales, signs, nonfinite, cp, s); break;
    default: worker_dispatch<G, E, true, true>(pd, g, err, words, scales, signs, nonfinite, cp, s); break;
    }
}
}  // namespace

template <int EF>
hipError_t launch_worker_compress(const PlanDev& pd, const void* g, int g_bf16, void* err_v, uint32_t* words,
                                  float* scales, int8_t* signs, unsigned long long* nonfinite, int ema,
                                  const CompressParams& cp, hipStream_t s)
{
    using E = typename ErrOf<EF>::type;
    auto err = static_cast<typename E::T*>(err_v);
    if (g_bf16)
        worker_dispatch_g<GradBF16, E>(pd, static_cast<const uint16_t*>(g), err, words, scales, signs, nonfinite,
                                       ema, cp, s);
    else
        worker_dispatch_g<GradF32, E>(pd, static_cast<const float*>(g), err, words, scales, signs, nonfinite, ema,
                                      cp, s);
    return hipGetLastError();
}

// the error format this translation unit is compiled for
template hipError_t launch_chunk_sumsq<OB_ERR_FMT>(const PlanDev&, const void*, int, const void*, float,
                                                   const float*, int, hipStream_t);
template hipError_t launch_compress<OB_ERR_FMT>(const PlanDev&, const void*, int, void*, float*, const float*,
                                                float*, uint32_t*, float*, int8_t*, unsigned long long*, int,
                                                int, const CompressParams&, hipStream_t);
template hipError_t launch_worker_compress<OB_ERR_FMT>(const PlanDev&, const void*, int, void*, uint32_t*, float*,
                                                       int8_t*, unsigned long long*, int, const CompressParams&,
                                                       hipStream_t);

}  // namespace ob

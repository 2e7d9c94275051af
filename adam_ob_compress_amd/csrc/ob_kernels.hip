// ob_kernels.hip -- HIP kernels of the 1-bit Adam step for gfx950 (MI355X) other than the compressed
// step (which is in ob_compress.hip): the dense Adam step, the server half of the compressed
// allreduce, unpack + dequantize, and plain pack.
//
// Pages cited (title and section):
//   [P2] "DeepSpeed Communication Compression and Hiding": "baseline" section (Adam moments),
//        "1-bit Adam: warmup, frozen variance, error feedback" (dequantize, compressed_allreduce),
//        "0/1 Adam" (refresh step = dense step), "1-bit LAMB: also protect the layer-wise trust
//        ratio" (r = ||w|| / ||u|| per layer, w -= lr * r * u).
//
// Design (memory bound, no dense contraction, so no MFMA): every per-element kernel walks work
// blocks ("items") of one chunk each; a block of 256 threads = four wave64s; each lane owns 4
// consecutive elements per 1024-element tile, so each fp32 array moves as one 16-byte access per
// lane.  Server pass 2 reduces the chunk's pass-1 partials in a fixed order at its start, as the
// compressed step does.  All fp32 arithmetic is plain IEEE (no fast-math, denormals kept).
#include "ob_device.h"

namespace ob {
namespace {

// ------------------------------------------------------------------------------------------------
// dense Adam step ([P2] baseline section; warmup / 0-1 Adam refresh)
// ------------------------------------------------------------------------------------------------

// Each line in double from fp32 operands, rounded once when stored; p uses the stored m and v.
// LAMB: p is left alone; the direction u = mh / (sqrt(vh) + eps) (double, not stored) adds u^2 to usq
// and p^2 goes to wsq, for the layer's trust ratio.
template <bool BC, bool LAMB>
__device__ __forceinline__ void dense_elem(float g, float& mm, float& vv, float& pp, double& wsq, double& usq,
                                           const DenseParams& dp)
{
    const double gd = static_cast<double>(g);
    mm = static_cast<float>(dp.beta1 * static_cast<double>(mm) + dp.one_m_beta1 * gd);
    vv = static_cast<float>(dp.beta2 * static_cast<double>(vv) + dp.one_m_beta2 * (gd * gd));
    double mh = static_cast<double>(mm), vh = static_cast<double>(vv);
    if (BC) {
        mh = mh / dp.bc1;
        vh = vh / dp.bc2;
    }
    const double u = mh / (sqrt(vh) + dp.eps);
    if (LAMB) {
        wsq = fma(static_cast<double>(pp), static_cast<double>(pp), wsq);
        usq = fma(u, u, usq);
    } else {
        pp = static_cast<float>(static_cast<double>(pp) - dp.lr * u);
    }
}

template <class G, bool BC, bool LAMB>
__global__ __launch_bounds__(kBlock) void k_dense(PlanDev pd, const typename G::T* __restrict__ g,
                                                  float* __restrict__ m, float* __restrict__ v,
                                                  float* __restrict__ p, DenseParams dp)
{
    const Item it = pd.items[blockIdx.x];
    const int tid = threadIdx.x;
    double wsq = 0.0, usq = 0.0;
    constexpr int U = 2;
    int base = 0;
    for (; base + U * kTile <= it.len; base += U * kTile) {
        f4 gv[U], mv[U], vv[U], pv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = it.start + base + u * kTile + kVec * tid;
            gv[u] = G::template load4<OB_NT_DENSE>(g, i);
            mv[u] = ld4<OB_NT_DENSE>(m, i);
            vv[u] = ld4<OB_NT_DENSE>(v, i);
            pv[u] = ld4<OB_NT_DENSE>(p, i);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = it.start + base + u * kTile + kVec * tid;
#pragma unroll
            for (int k = 0; k < kVec; ++k) {
                float mm = mv[u][k], vq = vv[u][k], pp = pv[u][k];
                dense_elem<BC, LAMB>(gv[u][k], mm, vq, pp, wsq, usq, dp);
                mv[u][k] = mm;
                vv[u][k] = vq;
                pv[u][k] = pp;
            }
            st4<OB_NT_DENSE>(m, i, mv[u]);
            st4<OB_NT_DENSE>(v, i, vv[u]);
            if (!LAMB) st4<OB_NT_DENSE>(p, i, pv[u]);
        }
    }
    for (; base < it.len; base += kTile) {
        const int cnt = it.len - base - kVec * tid;
        const int64_t i = it.start + base + kVec * tid;
        if (cnt >= kVec) {
            const f4 gv = G::load4(g, i);
            f4 mv = ld4(m, i), vv = ld4(v, i), pv = ld4(p, i);
#pragma unroll
            for (int k = 0; k < kVec; ++k) {
                float mm = mv[k], vq = vv[k], pp = pv[k];
                dense_elem<BC, LAMB>(gv[k], mm, vq, pp, wsq, usq, dp);
                mv[k] = mm;
                vv[k] = vq;
                pv[k] = pp;
            }
            st4(m, i, mv);
            st4(v, i, vv);
            if (!LAMB) st4(p, i, pv);
        } else {
            #pragma unroll
            for (int k = 0; k < kVec; ++k) {
                if (k >= cnt) continue;
                float mm = m[i + k], vq = v[i + k], pp = p[i + k];
                dense_elem<BC, LAMB>(G::load1(g, i + k), mm, vq, pp, wsq, usq, dp);
                m[i + k] = mm;
                v[i + k] = vq;
                if (!LAMB) p[i + k] = pp;
            }
        }
    }
    if (LAMB) {
        __shared__ double lds[kBlock / 64];
        const double sw = block_sum(wsq, lds);
        const double su = block_sum(usq, lds);
        if (tid == 0) {
            pd.partials_w[blockIdx.x] = sw;
            pd.partials_u[blockIdx.x] = su;
        }
    }
}

// ------------------------------------------------------------------------------------------------
// LAMB ([P2] "1-bit LAMB"): the layer's trust ratio from the per-block sums, then the update
// ------------------------------------------------------------------------------------------------

// One block per chunk: S_c = the chunk's pass-1 partials added in the fixed order chunk_scale uses
// (for plans whose chunks have so many partials that every pass-2 block adding them all would cost
// more than this launch).
__global__ __launch_bounds__(kBlock) void k_chunk_sums(PlanDev pd, double* __restrict__ sums)
{
    __shared__ double lds[kBlock / 64];
    const int c = blockIdx.x;
    double s = 0.0;
    for (int i = pd.p1_first[c] + static_cast<int>(threadIdx.x); i < pd.p1_first[c + 1]; i += kBlock)
        s += pd.partials[i];
    s = block_sum(s, lds);
    if (threadIdx.x == 0) sums[c] = s;
}

// One block per layer (chunk): r = ||w|| / ||u||, the chunk's partial sums added in a fixed order;
// r = 1 when either sum is 0 (the ratio is undefined there; NaN and Inf propagate).
__global__ __launch_bounds__(kBlock) void k_trust_ratio(PlanDev pd, float* __restrict__ ratios)
{
    __shared__ double lds[kBlock / 64];
    const int c = blockIdx.x;
    const int tid = threadIdx.x;
    double sw = 0.0, su = 0.0;
    for (int i = pd.w_first[c] + tid; i < pd.w_first[c + 1]; i += kBlock) sw += pd.partials_w[i];
    for (int i = pd.u_first[c] + tid; i < pd.u_first[c + 1]; i += kBlock) su += pd.partials_u[i];
    sw = block_sum(sw, lds);
    su = block_sum(su, lds);
    if (tid == 0) ratios[c] = (sw == 0.0 || su == 0.0) ? 1.0f : static_cast<float>(sqrt(sw) / sqrt(su));
}

// ------------------------------------------------------------------------------------------------
// diagnostics ([P1] sec. 6.2 and 8): one block per chunk adds its blocks' partial results in a fixed
// order: the sum of squares of the error buffer the step read, and the number of +1 signs
// ------------------------------------------------------------------------------------------------

__global__ __launch_bounds__(kBlock) void k_diag_reduce(PlanDev pd, double* __restrict__ err_sumsq,
                                                        unsigned long long* __restrict__ plus_count)
{
    __shared__ double lds[kBlock / 64];
    const int c = blockIdx.x;
    const int tid = threadIdx.x;
    double se = 0.0;
    unsigned long long pc = 0;
    for (int i = pd.p1_first[c] + tid; i < pd.p1_first[c + 1]; i += kBlock) se += pd.partials_e[i];
    for (int i = pd.chunk_first[c] + tid; i < pd.chunk_first[c + 1]; i += kBlock) pc += pd.partials_b[i];
    se = block_sum(se, lds);
    // the counts are integers below 2^53, exact in double whatever the order
    const double pcs = block_sum(static_cast<double>(pc), lds);
    if (tid == 0) {
        err_sumsq[c] = se;
        plus_count[c] = static_cast<unsigned long long>(pcs);
    }
}

// p -= lr * (r * u), u = mh / (sqrt(vh) + eps) from the stored m and v, in double, rounded once.
template <bool BC>
__device__ __forceinline__ float lamb_elem(float mm, float vv, float pp, double r, const LambParams& lp)
{
    double mh = static_cast<double>(mm), vh = static_cast<double>(vv);
    if (BC) {
        mh = mh / lp.bc1;
        vh = vh / lp.bc2;
    }
    const double u = mh / (sqrt(vh) + lp.eps);
    return static_cast<float>(static_cast<double>(pp) - lp.lr * (r * u));
}

template <bool BC>
__global__ __launch_bounds__(kBlock) void k_lamb_apply(PlanDev pd, const float* __restrict__ m,
                                                       const float* __restrict__ v, float* __restrict__ p,
                                                       const float* __restrict__ ratios, LambParams lp)
{
    const Item it = pd.items[blockIdx.x];
    const int tid = threadIdx.x;
    const double r = static_cast<double>(ratios[it.chunk]);
    constexpr int U = 2;
    int base = 0;
    for (; base + U * kTile <= it.len; base += U * kTile) {
        f4 mv[U], vv[U], pv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = it.start + base + u * kTile + kVec * tid;
            mv[u] = ld4<OB_NT_DENSE>(m, i);
            vv[u] = ld4<OB_NT_DENSE>(v, i);
            pv[u] = ld4<OB_NT_DENSE>(p, i);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = it.start + base + u * kTile + kVec * tid;
#pragma unroll
            for (int k = 0; k < kVec; ++k) pv[u][k] = lamb_elem<BC>(mv[u][k], vv[u][k], pv[u][k], r, lp);
            st4<OB_NT_DENSE>(p, i, pv[u]);
        }
    }
    for (; base < it.len; base += kTile) {
        const int cnt = it.len - base - kVec * tid;
        const int64_t i = it.start + base + kVec * tid;
        if (cnt >= kVec) {
            const f4 mv = ld4(m, i), vv = ld4(v, i);
            f4 pv = ld4(p, i);
#pragma unroll
            for (int k = 0; k < kVec; ++k) pv[k] = lamb_elem<BC>(mv[k], vv[k], pv[k], r, lp);
            st4(p, i, pv);
        } else {
            #pragma unroll
            for (int k = 0; k < kVec; ++k) {
                if (k >= cnt) continue;
                p[i + k] = lamb_elem<BC>(m[i + k], v[i + k], p[i + k], r, lp);
            }
        }
    }
}

// ------------------------------------------------------------------------------------------------
// server half of compressed_allreduce ([P2] 1-bit Adam)
// ------------------------------------------------------------------------------------------------

// Averages of the 4 elements i..i+3 (one nibble of one word) over W workers: exact double sum of
// +-s in ascending worker order, one division by W, one rounding to fp32.
// Workers are taken kWorkerBatch at a time: the batch's word loads are all issued before the sums
// use them, so the memory latency is paid once per batch, not once per worker.  The additions stay
// in ascending worker order.
constexpr int kWorkerBatch = 8;

__device__ __forceinline__ f4 server_avg4(int W, const uint32_t* __restrict__ ww, int64_t nw,
                                          const float* __restrict__ ws, int K, int c, int64_t i)
{
    double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
    const int64_t wi = i >> 5;
    const int sh = static_cast<int>(i & 31);
    for (int w0 = 0; w0 < W; w0 += kWorkerBatch) {
        uint32_t bits[kWorkerBatch];
        double s[kWorkerBatch];
#pragma unroll
        for (int j = 0; j < kWorkerBatch; ++j) {
            const int w = w0 + j < W ? w0 + j : W - 1;  // in-range index; surplus lanes of the batch unused
            bits[j] = ww[static_cast<int64_t>(w) * nw + wi] >> sh;
            s[j] = static_cast<double>(ws[static_cast<int64_t>(w) * K + c]);
        }
        // past the last worker the batch adds +0.0, an exact no-op (the sums start at +0 and an IEEE
        // sum is never -0 unless both terms are), so the loop has no branch the loads must wait for
#pragma unroll
        for (int j = 0; j < kWorkerBatch; ++j) {
            const double sj = w0 + j < W ? s[j] : 0.0;
            a0 += (bits[j] & 1u) ? sj : -sj;
            a1 += (bits[j] & 2u) ? sj : -sj;
            a2 += (bits[j] & 4u) ? sj : -sj;
            a3 += (bits[j] & 8u) ? sj : -sj;
        }
    }
    f4 r;
    if ((W & (W - 1)) == 0) {
        // W a power of two: 1/W is exact, so the product equals the IEEE quotient
        const double rw = 1.0 / static_cast<double>(W);
        r.x = static_cast<float>(a0 * rw);
        r.y = static_cast<float>(a1 * rw);
        r.z = static_cast<float>(a2 * rw);
        r.w = static_cast<float>(a3 * rw);
    } else {
        const double dw = static_cast<double>(W);
        r.x = static_cast<float>(a0 / dw);
        r.y = static_cast<float>(a1 / dw);
        r.z = static_cast<float>(a2 / dw);
        r.w = static_cast<float>(a3 / dw);
    }
    return r;
}

// Sign patterns of the 4 elements of a lane, one byte each: byte k holds bit k of worker w's nibble
// at bit w.  Input: the 8 workers' nibbles of the lane packed as bits 4w+k; the 32-bit index is
// rotated right by two index bits (4w+k -> 8k+w) with four delta swaps.
__device__ __forceinline__ uint32_t delta_swap(uint32_t x, int d, uint32_t mask)
{
    const uint32_t t = ((x >> d) ^ x) & mask;
    return x ^ t ^ (t << d);
}

// 8x8 transpose of nibbles across each group of 8 lanes: on entry lane j holds the 8 nibbles
// M[j][0..7] (nibble q at bits 4q..4q+3), on exit M[0..7][j] (M[w][j] at bits 4w..4w+3).  Three
// butterfly stages; the stage of distance d swaps lane-index bit d with nibble-index bit d: the
// lane with that bit clear keeps its low nibbles and takes its partner's low nibbles as its high
// ones, the other lane the reverse.  DPP moves, no LDS; all lanes must be active.
__device__ __forceinline__ uint32_t nib_transpose8(uint32_t x)
{
    const int j = threadIdx.x & 7;
    uint32_t y;
    y = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0xB1, 0xF, 0xF, false));  // lane j^1
    x = (j & 1) ? ((x & 0xF0F0F0F0u) | ((y & 0xF0F0F0F0u) >> 4)) : ((x & 0x0F0F0F0Fu) | ((y & 0x0F0F0F0Fu) << 4));
    y = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x4E, 0xF, 0xF, false));  // lane j^2
    x = (j & 2) ? ((x & 0xFF00FF00u) | ((y & 0xFF00FF00u) >> 8)) : ((x & 0x00FF00FFu) | ((y & 0x00FF00FFu) << 8));
    // lane j^4: row_shl:4 (lane l reads lane l+4) for j < 4, row_shr:4 (lane l-4) for j >= 4
    const uint32_t up = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x104, 0xF, 0xF, false));
    const uint32_t dn = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x114, 0xF, 0xF, false));
    x = (j & 4) ? ((x & 0xFFFF0000u) | (dn >> 16)) : ((x & 0x0000FFFFu) | (up << 16));
    return x;
}

__device__ __forceinline__ uint32_t patterns_of(uint32_t x)
{
    x = delta_swap(x, 3, 0x0A0A0A0Au);   // index bits 0 <-> 2
    x = delta_swap(x, 6, 0x00CC00CCu);   // index bits 1 <-> 3
    x = delta_swap(x, 12, 0x0000F0F0u);  // index bits 2 <-> 4
    x = delta_swap(x, 8, 0x0000FF00u);   // index bits 3 <-> 4
    return x;
}

// The server average of an element depends only on its W sign bits and the chunk's W scales.  For
// W <= 8 each block tabulates all 2^W averages of its chunk in LDS, each computed exactly as
// server_avg4 does (double sum in ascending worker order, one division, one rounding), and looks
// them up; for larger W it sums per element.
template <bool APPLY>
__global__ __launch_bounds__(kBlock) void k_server(PlanDev pd, int W, const uint32_t* __restrict__ ww,
                                                   int64_t nw, const float* __restrict__ ws,
                                                   float* __restrict__ e, uint32_t* __restrict__ words,
                                                   float* __restrict__ scales)
{
    __shared__ double lds[kBlock / 64];
    __shared__ float table[1 << kWorkerBatch];
    const Item it = pd.items[blockIdx.x];
    const int tid = threadIdx.x;
    const int c = it.chunk;
    const bool tabulate = W <= kWorkerBatch;
    constexpr bool NTS = (!APPLY && OB_NT_SRV) || (APPLY && OB_NT_SRV2);
    constexpr bool NTW = (!APPLY && OB_NT_SRV_WORDS) || (APPLY && OB_NT_SRV2);
    constexpr int U = APPLY ? OB_SRV2_UNROLL : OB_SRV_UNROLL;
    // lane j of each 8-lane group loads worker j's word of the group's 32 elements (worker index
    // clamped to W-1; the surplus nibbles are masked off after the transpose)
    const int wc = (tid & 7) < W ? (tid & 7) : W - 1;
    const uint32_t* __restrict__ wrow = ww + static_cast<int64_t>(wc) * nw;
    auto load_word = [&](int64_t i) -> uint32_t {
        const uint32_t* wp = wrow + (i >> 5);
        return NTW ? __builtin_nontemporal_load(wp) : *wp;
    };
    f4 grp_e[U];
    uint32_t grp_w[U];
    auto load_group = [&](int b) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = it.start + b + u * kTile + kVec * tid;
            grp_e[u] = ld4<NTS>(e, i);
            grp_w[u] = tabulate ? load_word(i) : 0u;
        }
    };
    // Prologue, ordered so that its latency overlaps the first tiles' loads: the chunk's worker scales
    // (pass 2: and the chunk's pass-1 partials) are loaded first, then the block's first group of
    // tiles; the table of averages (pass 2: and the scale) is formed while the tiles are in flight.
    // The table adds +-s_w in ascending w and the scale adds the chunk's partials in chunk_scale's
    // order, so every block of a chunk forms the same bits.
    float sc[kWorkerBatch];
#pragma unroll
    for (int w = 0; w < kWorkerBatch; ++w) sc[w] = (tabulate && w < W) ? ws[static_cast<int64_t>(w) * pd.K + c] : 0.0f;
    double part = 0.0;
    if (APPLY) {
        const int f0 = pd.p1_first[c], f1 = pd.p1_first[c + 1];
        for (int j = f0 + tid; j < f1; j += kBlock) part += pd.partials[j];
    }
    if (U * kTile <= it.len) load_group(0);
    if (tabulate) {
        const bool pow2 = (W & (W - 1)) == 0;
        for (int pat = tid; pat < (1 << W); pat += kBlock) {
            double a = 0.0;
#pragma unroll
            for (int w = 0; w < kWorkerBatch; ++w) {
                if (w >= W) break;
                const double s = static_cast<double>(sc[w]);
                a += ((pat >> w) & 1) ? s : -s;
            }
            table[pat] = static_cast<float>(pow2 ? a * (1.0 / static_cast<double>(W)) : a / static_cast<double>(W));
        }
    }
    float scale = 0.0f;
    if (APPLY) {
        // block_sum's barriers also publish the table
        const double s = block_sum(part, lds);
        const int64_t nc = pd.chunk_off[c + 1] - pd.chunk_off[c];
        scale = static_cast<float>(sqrt(s / static_cast<double>(nc)));
        if (tid == 0 && static_cast<int>(blockIdx.x) == pd.chunk_first[c]) scales[c] = scale;
    } else if (tabulate) {
        __syncthreads();
    }
    double acc = 0.0;
    // One tile's worth: given the error and (W <= 8) the lane's worker word, form x = avg + e, then
    // the sum of squares (pass 1) or the new error and sign nibble (pass 2).
    auto tile = [&](int64_t i, int cnt, f4 ev, uint32_t wd) -> uint32_t {
        uint32_t pats = 0;
        if (tabulate) {
            // the transpose hands every lane its own nibble of all workers' words
            wd = nib_transpose8(wd);
            if (W < kWorkerBatch) wd &= (1u << (4 * W)) - 1u;
            pats = patterns_of(wd);
        }
        uint32_t nib = 0;
        if (cnt <= 0) return nib;
        f4 avg;
        if (tabulate) {
#pragma unroll
            for (int k = 0; k < kVec; ++k) avg[k] = table[(pats >> (8 * k)) & 0xFFu];
        } else {
            avg = server_avg4(W, ww, nw, ws, pd.K, c, i);
        }
        if (cnt >= kVec) {
            f4 x;
#pragma unroll
            for (int k = 0; k < kVec; ++k) x[k] = avg[k] + ev[k];
            if (APPLY) {
#pragma unroll
                for (int k = 0; k < kVec; ++k) {
                    const bool b = x[k] >= 0.0f;
                    ev[k] = x[k] - (b ? scale : -scale);
                    nib |= (b ? 1u : 0u) << k;
                }
                st4<OB_NT_SRV2>(e, i, ev);
            } else {
#pragma unroll
                for (int k = 0; k < kVec; ++k) acc = fma(static_cast<double>(x[k]), static_cast<double>(x[k]), acc);
            }
        } else {
#pragma unroll
            for (int k = 0; k < kVec; ++k) {
                if (k >= cnt) continue;
                const float x = avg[k] + e[i + k];
                if (APPLY) {
                    const bool b = x >= 0.0f;
                    e[i + k] = x - (b ? scale : -scale);
                    nib |= (b ? 1u : 0u) << k;
                } else {
                    acc = fma(static_cast<double>(x), static_cast<double>(x), acc);
                }
            }
        }
        return nib;
    };
    // whole tiles, U in flight: all their loads are issued before any is used (the first
    // group's in the prologue)
    int base = 0;
    for (; base + U * kTile <= it.len; base += U * kTile) {
        if (base > 0) load_group(base);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = it.start + base + u * kTile + kVec * tid;
            const uint32_t nib = tile(i, kVec, grp_e[u], grp_w[u]);
            if (APPLY) store_word<OB_NT_SRV2>(words, i, nib, true);
        }
    }
    // the rest, one (possibly ragged) tile at a time
    for (; base < it.len; base += kTile) {
        const int rem = it.len - base;
        const int cnt = rem - kVec * tid;
        const int64_t i = it.start + base + kVec * tid;
        const bool group_valid = 32 * (tid >> 3) < rem;   // the word of this lane's 8-lane group exists
        f4 ev = {0.0f, 0.0f, 0.0f, 0.0f};
        if (cnt >= kVec) ev = ld4<NTS>(e, i);
        const uint32_t wd = (tabulate && group_valid) ? load_word(i) : 0u;
        const uint32_t nib = tile(i, cnt, ev, wd);
        if (APPLY) store_word<OB_NT_SRV2>(words, i, nib, group_valid);
    }
    if (!APPLY) {
        const double s = block_sum(acc, lds);
        if (tid == 0) pd.partials[blockIdx.x] = s;
    }
}

// Server pass 1 with whole-line word loads (W <= 8; chunk offsets multiples of 128 elements and word
// rows 16-byte aligned, which the host checks before choosing it).  A wave takes 1024 consecutive
// elements at a time (a "wave tile"): its error values as four 1 KiB runs, 16 bytes per lane, and the
// W workers' 32 words of the tile with one 16-byte load per lane -- lanes 8r..8r+7 read worker r's
// 128 bytes, one whole line per row, so a word-load instruction touches only whole lines that no
// other wave reads.  The words go through a 1 KiB LDS stage of the wave and come back as the 8 words
// of each lane's 32-element group (one per worker); the lane's nibble of each, packed, is the layout
// k_server's transpose produces, and from there the averages come from the same table, built by the
// same code, so x = avg + e is bit for bit pass 2's.  A chunk's last block may end with a partial
// wave tile; its elements are taken one at a time.
__global__ __launch_bounds__(kBlock) void k_server_sumsq_lines(PlanDev pd, int W, const uint32_t* __restrict__ ww,
                                                               int64_t nw, const float* __restrict__ ws,
                                                               const float* __restrict__ e)
{
    typedef unsigned int w4 __attribute__((ext_vector_type(4)));
    __shared__ double lds[kBlock / 64];
    __shared__ float table[1 << kWorkerBatch];
    __shared__ w4 stage[kBlock / 64][64];
    constexpr bool NTS = OB_NT_SRV, NTW = OB_NT_SRV_WORDS;
    constexpr int U = OB_SRV_LINES_UNROLL;
    const Item it = pd.items[blockIdx.x];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int c = it.chunk;
    const int row = lane >> 3;                        // the worker row this lane loads
    const bool loads = row < W;
    const uint32_t* __restrict__ wrow = ww + static_cast<int64_t>(loads ? row : 0) * nw + 4 * (lane & 7);
    const int ntiles = it.len >> 10;                  // whole wave tiles of the block
    f4 ev[U][kVec];
    w4 wv[U];
    auto load_group = [&](int t0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = t0 + 4 * u;
            if (t < ntiles) {
                const int64_t base = it.start + (static_cast<int64_t>(t) << 10);
#pragma unroll
                for (int k = 0; k < kVec; ++k) ev[u][k] = ld4<NTS>(e, base + 256 * k + kVec * lane);
                wv[u] = loads ? ldv<NTW>(reinterpret_cast<const w4*>(wrow + (base >> 5))) : w4{0u, 0u, 0u, 0u};
            }
        }
    };
    // the chunk's worker scales, then the first group of loads, then the table (as k_server's prologue)
    float sc[kWorkerBatch];
#pragma unroll
    for (int w = 0; w < kWorkerBatch; ++w) sc[w] = w < W ? ws[static_cast<int64_t>(w) * pd.K + c] : 0.0f;
    load_group(wave);
    {
        const bool pow2 = (W & (W - 1)) == 0;
        for (int pat = tid; pat < (1 << W); pat += kBlock) {
            double a = 0.0;
#pragma unroll
            for (int w = 0; w < kWorkerBatch; ++w) {
                if (w >= W) break;
                const double s = static_cast<double>(sc[w]);
                a += ((pat >> w) & 1) ? s : -s;
            }
            table[pat] = static_cast<float>(pow2 ? a * (1.0 / static_cast<double>(W)) : a / static_cast<double>(W));
        }
    }
    __syncthreads();
    const uint32_t keep = W < kWorkerBatch ? (1u << (4 * W)) - 1u : 0xFFFFFFFFu;
    const int sh = 4 * (lane & 7);
    double acc = 0.0;
    for (int t0 = wave; t0 < ntiles; t0 += 4 * U) {
        if (t0 > wave) load_group(t0);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (t0 + 4 * u >= ntiles) break;
            stage[wave][lane] = wv[u];
            __builtin_amdgcn_wave_barrier();
            const uint32_t* st = reinterpret_cast<const uint32_t*>(&stage[wave][0]);
#pragma unroll
            for (int k = 0; k < kVec; ++k) {
                // this lane's 4 elements of run k lie in word 8k + lane/8 of every row
                const int wi = 8 * k + (lane >> 3);
                uint32_t wd = 0;
#pragma unroll
                for (int r = 0; r < kWorkerBatch; ++r) wd |= ((st[32 * r + wi] >> sh) & 0xFu) << (4 * r);
                const uint32_t pats = patterns_of(wd & keep);
#pragma unroll
                for (int q = 0; q < kVec; ++q) {
                    const float x = table[(pats >> (8 * q)) & 0xFFu] + ev[u][k][q];
                    acc = fma(static_cast<double>(x), static_cast<double>(x), acc);
                }
            }
            __builtin_amdgcn_wave_barrier();
        }
    }
    // a partial wave tile at the end of a chunk's last block: one element at a time
    for (int j = (ntiles << 10) + tid; j < it.len; j += kBlock) {
        const int64_t i = it.start + j;
        uint32_t pat = 0;
        for (int w = 0; w < W; ++w) pat |= ((ww[static_cast<int64_t>(w) * nw + (i >> 5)] >> (i & 31)) & 1u) << w;
        const float x = table[pat] + e[i];
        acc = fma(static_cast<double>(x), static_cast<double>(x), acc);
    }
    const double s = block_sum(acc, lds);
    if (tid == 0) pd.partials[blockIdx.x] = s;
}

// ------------------------------------------------------------------------------------------------
// unpack + dequantize, and plain pack
// ------------------------------------------------------------------------------------------------

__global__ __launch_bounds__(kBlock) void k_unpack(const Item* __restrict__ items, int64_t n,
                                                   const uint32_t* __restrict__ words,
                                                   const float* __restrict__ scales, float* __restrict__ out)
{
    int64_t start;
    int len;
    float s = 1.0f;
    if (items != nullptr) {
        const Item it = items[blockIdx.x];
        start = it.start;
        len = it.len;
        s = scales[it.chunk];
    } else {
        start = static_cast<int64_t>(blockIdx.x) * kPlainItem;
        len = static_cast<int>(min(static_cast<int64_t>(kPlainItem), n - start));
    }
    const int tid = threadIdx.x;
    auto values = [&](uint32_t bits) {
        f4 r;
#pragma unroll
        for (int k = 0; k < kVec; ++k) r[k] = ((bits >> k) & 1u) ? s : -s;
        return r;
    };
    // whole tiles, OB_UNPACK_UNROLL in flight: the word loads are issued before the stores
    constexpr int U = OB_UNPACK_UNROLL;
    int base = 0;
    for (; base + U * kTile <= len; base += U * kTile) {
        uint32_t bits[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = start + base + u * kTile + kVec * tid;
            bits[u] = words[i >> 5] >> (i & 31);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = start + base + u * kTile + kVec * tid;
            st4<OB_NT_UNPACK>(out, i, values(bits[u]));
        }
    }
    for (; base < len; base += kTile) {
        const int cnt = len - base - kVec * tid;
        const int64_t i = start + base + kVec * tid;
        if (cnt <= 0) continue;
        const f4 r = values(words[i >> 5] >> (i & 31));
        if (cnt >= kVec) {
            st4<OB_NT_UNPACK>(out, i, r);
        } else {
            #pragma unroll
            for (int k = 0; k < kVec; ++k)
                if (k < cnt) out[i + k] = r[k];
        }
    }
}

template <class G>
__global__ __launch_bounds__(kBlock) void k_pack(const typename G::T* __restrict__ x, int64_t n,
                                                 uint32_t* __restrict__ words)
{
    const int64_t start = static_cast<int64_t>(blockIdx.x) * kPlainItem;
    const int len = static_cast<int>(min(static_cast<int64_t>(kPlainItem), n - start));
    const int tid = threadIdx.x;
    for (int base = 0; base < len; base += kTile) {
        const int rem = len - base;
        const int cnt = rem - kVec * tid;
        const int64_t i = start + base + kVec * tid;
        uint32_t nib = 0;
        if (cnt >= kVec) {
            const f4 xv = G::load4(x, i);
#pragma unroll
            for (int k = 0; k < kVec; ++k) nib |= (xv[k] >= 0.0f ? 1u : 0u) << k;
        } else {
            #pragma unroll
            for (int k = 0; k < kVec; ++k)
                if (k < cnt) nib |= (G::load1(x, i + k) >= 0.0f ? 1u : 0u) << k;
        }
        store_word<false>(words, i, nib, 32 * (tid >> 3) < rem);
    }
}

}  // namespace

// ------------------------------------------------------------------------------------------------
// launchers
// ------------------------------------------------------------------------------------------------

hipError_t launch_dense(const PlanDev& pd, const void* g, int g_bf16, float* m, float* v, float* p,
                        int lamb, const DenseParams& dp, hipStream_t s)
{
    const dim3 grid(static_cast<unsigned>(pd.n_items)), block(kBlock);
    const int sel = (dp.bias_correction ? 1 : 0) | (lamb ? 2 : 0);
#define OB_DENSE(G, T)                                                                                   \
    {                                                                                                    \
        auto gp = static_cast<const T*>(g);                                                              \
        switch (sel) {                                                                                   \
        case 0: hipLaunchKernelGGL((k_dense<G, false, false>), grid, block, 0, s, pd, gp, m, v, p, dp); break; \
        case 1: hipLaunchKernelGGL((k_dense<G, true, false>), grid, block, 0, s, pd, gp, m, v, p, dp); break;  \
        case 2: hipLaunchKernelGGL((k_dense<G, false, true>), grid, block, 0, s, pd, gp, m, v, p, dp); break;  \
        default: hipLaunchKernelGGL((k_dense<G, true, true>), grid, block, 0, s, pd, gp, m, v, p, dp); break;  \
        }                                                                                                \
    }
    if (g_bf16)
        OB_DENSE(GradBF16, uint16_t)
    else
        OB_DENSE(GradF32, float)
#undef OB_DENSE
    return hipGetLastError();
}

hipError_t launch_diag_reduce(const PlanDev& pd, double* err_sumsq, unsigned long long* plus_count,
                              hipStream_t s)
{
    hipLaunchKernelGGL(k_diag_reduce, dim3(static_cast<unsigned>(pd.K)), dim3(kBlock), 0, s, pd, err_sumsq,
                       plus_count);
    return hipGetLastError();
}

hipError_t launch_chunk_sums(const PlanDev& pd, double* sums, hipStream_t s)
{
    hipLaunchKernelGGL(k_chunk_sums, dim3(static_cast<unsigned>(pd.K)), dim3(kBlock), 0, s, pd, sums);
    return hipGetLastError();
}
// ------------------------------------------------------------------------------------------------
// the worker's half of a compressed step after the exchange (more than one worker): g_hat from the
// exchanged words and per-chunk scales, then m and the frozen-v update (LAMB: m, and the block's sums
// of p^2 and u^2 for the layer's trust ratio; p is updated after the ratios)
// ------------------------------------------------------------------------------------------------

template <bool LAMB>
__device__ __forceinline__ void worker_elem(float gh, float& mm, float vv, float& pp, double& sw, double& su,
                                            const CompressParams& cp)
{
    if (!LAMB) {
        update_elem(gh, mm, vv, pp, cp);
        return;
    }
    mm = static_cast<float>(cp.beta1 * static_cast<double>(mm) + cp.one_m_beta1 * static_cast<double>(gh));
    const double u = static_cast<double>(mm) / (sqrt(static_cast<double>(vv)) + cp.eps);
    su = fma(u, u, su);
    sw = fma(static_cast<double>(pp), static_cast<double>(pp), sw);
}

template <bool LAMB>
__global__ __launch_bounds__(kBlock) void k_worker_update(PlanDev pd, const uint32_t* __restrict__ words,
                                                          const float* __restrict__ scales, float* __restrict__ m,
                                                          const float* __restrict__ v, float* __restrict__ p,
                                                          CompressParams cp)
{
    __shared__ double lds[kBlock / 64];
    const Item it = pd.items[blockIdx.x];
    const int tid = threadIdx.x;
    const float s = scales[it.chunk];
    constexpr int U = OB_P2_UNROLL;
    double sw = 0.0, su = 0.0;
    int base = 0;
    for (; base + U * kTile <= it.len; base += U * kTile) {
        f4 mv[U], vv[U], pv[U];
        uint32_t wv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = it.start + base + u * kTile + kVec * tid;
            wv[u] = words[i >> 5];
            mv[u] = ld4<OB_NT_P2>(m, i);
            vv[u] = ld4<OB_NT_P2>(v, i);
            pv[u] = ld4<OB_NT_P2>(p, i);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = it.start + base + u * kTile + kVec * tid;
            const uint32_t nib = wv[u] >> (static_cast<uint32_t>(i) & 31u);
#pragma unroll
            for (int k = 0; k < kVec; ++k) {
                float mm = mv[u][k], pp = pv[u][k];
                worker_elem<LAMB>((nib >> k) & 1u ? s : -s, mm, vv[u][k], pp, sw, su, cp);
                mv[u][k] = mm;
                pv[u][k] = pp;
            }
            st4<OB_NT_ST>(m, i, mv[u]);
            if (!LAMB) st4<OB_NT_ST>(p, i, pv[u]);
        }
    }
    for (; base < it.len; base += kTile) {
        const int cnt = it.len - base - kVec * tid;
        const int64_t i = it.start + base + kVec * tid;
        if (cnt <= 0) continue;
        const uint32_t nib = words[i >> 5] >> (static_cast<uint32_t>(i) & 31u);
        if (cnt >= kVec) {
            f4 mv = ld4(m, i), pv = ld4(p, i);
            const f4 vv = ld4(v, i);
#pragma unroll
            for (int k = 0; k < kVec; ++k) {
                float mm = mv[k], pp = pv[k];
                worker_elem<LAMB>((nib >> k) & 1u ? s : -s, mm, vv[k], pp, sw, su, cp);
                mv[k] = mm;
                pv[k] = pp;
            }
            st4(m, i, mv);
            if (!LAMB) st4(p, i, pv);
        } else {
            #pragma unroll
            for (int k = 0; k < kVec; ++k) {
                if (k >= cnt) continue;
                float mm = m[i + k], pp = p[i + k];
                worker_elem<LAMB>((nib >> k) & 1u ? s : -s, mm, v[i + k], pp, sw, su, cp);
                m[i + k] = mm;
                if (!LAMB) p[i + k] = pp;
            }
        }
    }
    if (LAMB) {
        const double tw = block_sum(sw, lds);
        const double tu = block_sum(su, lds);
        if (tid == 0) {
            pd.partials_w[blockIdx.x] = tw;
            pd.partials_u[blockIdx.x] = tu;
        }
    }
}

hipError_t launch_worker_update(const PlanDev& pd, const uint32_t* words, const float* scales, float* m,
                                const float* v, float* p, int lamb, const CompressParams& cp, hipStream_t s)
{
    const dim3 grid(static_cast<unsigned>(pd.n_items)), block(kBlock);
    if (lamb)
        hipLaunchKernelGGL(k_worker_update<true>, grid, block, 0, s, pd, words, scales, m, v, p, cp);
    else
        hipLaunchKernelGGL(k_worker_update<false>, grid, block, 0, s, pd, words, scales, m, v, p, cp);
    return hipGetLastError();
}

hipError_t launch_trust_ratio(const PlanDev& pd, float* ratios, hipStream_t s)
{
    hipLaunchKernelGGL(k_trust_ratio, dim3(static_cast<unsigned>(pd.K)), dim3(kBlock), 0, s, pd, ratios);
    return hipGetLastError();
}

hipError_t launch_lamb_apply(const PlanDev& pd, const float* m, const float* v, float* p, const float* ratios,
                             int bias_correction, const LambParams& lp, hipStream_t s)
{
    const dim3 grid(static_cast<unsigned>(pd.n_items)), block(kBlock);
    if (bias_correction)
        hipLaunchKernelGGL((k_lamb_apply<true>), grid, block, 0, s, pd, m, v, p, ratios, lp);
    else
        hipLaunchKernelGGL((k_lamb_apply<false>), grid, block, 0, s, pd, m, v, p, ratios, lp);
    return hipGetLastError();
}

hipError_t launch_server_sumsq(const PlanDev& pd, int W, const uint32_t* ww, const float* ws,
                               const float* e, bool lines_ok, hipStream_t s)
{
    const dim3 grid(static_cast<unsigned>(pd.n_items)), block(kBlock);
    const int64_t nw = (pd.n + 31) / 32;
    // whole-line word loads need 16-byte aligned word rows and blocks starting at multiples of 128
    // elements (lines_ok: the plan's chunk offsets are multiples of 128)
    if (OB_SRV_LINES && W <= kWorkerBatch && lines_ok && nw % 4 == 0 && reinterpret_cast<uintptr_t>(ww) % 16 == 0) {
        hipLaunchKernelGGL(k_server_sumsq_lines, grid, block, 0, s, pd, W, ww, nw, ws, e);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((k_server<false>), grid, block, 0, s, pd, W, ww, nw, ws, const_cast<float*>(e),
                       static_cast<uint32_t*>(nullptr), static_cast<float*>(nullptr));
    return hipGetLastError();
}

hipError_t launch_server_apply(const PlanDev& pd, int W, const uint32_t* ww, const float* ws,
                               float* e, uint32_t* words, float* scales, hipStream_t s)
{
    const dim3 grid(static_cast<unsigned>(pd.n_items)), block(kBlock);
    const int64_t nw = (pd.n + 31) / 32;
    hipLaunchKernelGGL((k_server<true>), grid, block, 0, s, pd, W, ww, nw, ws, e, words, scales);
    return hipGetLastError();
}

hipError_t launch_unpack(const PlanDev* pd, const uint32_t* words, int64_t n, const float* scales,
                         float* out, hipStream_t s)
{
    const int64_t blocks = pd ? pd->n_items : (n + kPlainItem - 1) / kPlainItem;
    const dim3 grid(static_cast<unsigned>(blocks)), block(kBlock);
    hipLaunchKernelGGL(k_unpack, grid, block, 0, s, pd ? pd->items : nullptr, n, words, scales, out);
    return hipGetLastError();
}

hipError_t launch_pack(const void* x, int x_bf16, int64_t n, uint32_t* words, hipStream_t s)
{
    const int64_t blocks = (n + kPlainItem - 1) / kPlainItem;
    const dim3 grid(static_cast<unsigned>(blocks)), block(kBlock);
    if (x_bf16)
        hipLaunchKernelGGL((k_pack<GradBF16>), grid, block, 0, s, static_cast<const uint16_t*>(x), n, words);
    else
        hipLaunchKernelGGL((k_pack<GradF32>), grid, block, 0, s, static_cast<const float*>(x), n, words);
    return hipGetLastError();
}

}  // namespace ob

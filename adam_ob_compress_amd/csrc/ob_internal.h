// ob_internal.h -- shared between the host runtime (ob_api.cpp) and the kernels (ob_kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ob_tables.h"

namespace ob {

// Launch geometry of every per-element kernel: 256 threads (four 64-wide waves), each lane owning
// 4 consecutive elements per tile, so one tile is 1024 consecutive elements and one 16-byte access
// per lane per fp32 array.
constexpr int kBlock = 256;
constexpr int kVec = 4;
constexpr int kTile = kBlock * kVec;
// elements per block of the plan-less pack and unpack (their grid is n / kPlainItem blocks, so n is at
// most INT32_MAX * kPlainItem)
constexpr int kPlainItem = 16 * kTile;

// Device-side view of a plan for one launch.  Pass-1 kernels (sums of squares) and pass-2 kernels
// (everything that needs a chunk's scale, and the dense step) use different block tables: pass 1
// takes large blocks so that a chunk has few partial sums, pass 2 small blocks; a pass-2 block
// forms its chunk's scale from the pass-1 partials.
struct PlanDev {
    const Item* items;          // [n_items] blocks of this launch
    const int32_t* chunk_first; // [K + 1]: blocks of chunk c in `items` are [chunk_first[c], chunk_first[c+1])
    const int32_t* p1_first;    // [K + 1]: the same for the pass-1 table (indexes `partials`)
    const int64_t* chunk_off;   // [K + 1]: element offsets
    double* partials;           // [pass-1 blocks]: per-block sum of squares (workspace)
    // LAMB (layer = chunk): per-block sums of p^2 and of u^2, and the chunk_first arrays of the tables
    // whose blocks wrote them
    double* partials_w;
    const int32_t* w_first;
    double* partials_u;
    const int32_t* u_first;
    // diagnostics (nullptr = off): per pass-1 block, the sum of squares of the error buffer read;
    // per pass-2 block, the number of +1 signs
    double* partials_e;
    uint32_t* partials_b;
    int64_t n;
    int64_t n_items;            // blocks of this launch: items [item0, item0 + n_items)
    int32_t K;
    // index in `items` of this launch's first block; its per-block results go to the same index of the
    // partials arrays.  Non-zero only for the chunk-group launches of the compressed step's two passes
    // (k_chunk_sumsq, k_compress, k_worker_compress); every other kernel takes 0.
    int32_t item0;
};

struct CompressParams {
    double lr, beta1, one_m_beta1, eps, ef_beta, one_m_ef_beta;
    float clip;
    int stochastic;          // 16-bit error buffers: stochastic rounding with (sr_seed, sr_step)
    uint64_t sr_seed, sr_step;
};

struct DenseParams {
    double lr, beta1, one_m_beta1, beta2, one_m_beta2, eps, bc1, bc2;
    int bias_correction;
};

// LAMB update: p -= lr * r_c * (m / bc1) / (sqrt(v / bc2) + eps)
struct LambParams {
    double lr, eps, bc1, bc2;
};

// Compressed-step launchers for error-buffer format EF (0 fp32, 1 bf16, 2 fp16); ob_compress.hip,
// built once per format, instantiates each.
// lamb_p != nullptr: also the per-block sum of p^2 (LAMB), into pd.partials_w.  nontemporal != 0:
// nontemporal loads (a launch over all chunks at once); 0: ordinary loads, which leave the lines in the
// last-level cache for the pass 2 that follows on the same chunk group.
template <int EF>
hipError_t launch_chunk_sumsq(const PlanDev& pd, const void* g, int g_bf16, const void* err, float clip,
                              const float* lamb_p, int nontemporal, hipStream_t s);
// lamb != 0: no parameter update; the per-block sum of u^2 goes to pd.partials_u (p is not touched).
template <int EF>
hipError_t launch_compress(const PlanDev& pd, const void* g, int g_bf16, void* err, float* m, const float* v,
                           float* p, uint32_t* words, float* scales, int8_t* signs,
                           unsigned long long* nonfinite, int ema, int lamb, const CompressParams& cp,
                           hipStream_t s);
// The worker's step split at the exchange: pass 2 without m, v, p (scale, bits, error from the worker's
// own g_hat), and the update from exchanged words and scales (m, p).
template <int EF>
hipError_t launch_worker_compress(const PlanDev& pd, const void* g, int g_bf16, void* err, uint32_t* words,
                                  float* scales, int8_t* signs, unsigned long long* nonfinite, int ema,
                                  const CompressParams& cp, hipStream_t s);
// lamb != 0: m only, plus per-block sums of p^2 and u^2 into pd.partials_w / partials_u (this table).
hipError_t launch_worker_update(const PlanDev& pd, const uint32_t* words, const float* scales, float* m,
                                const float* v, float* p, int lamb, const CompressParams& cp, hipStream_t s);
// lamb != 0: moments only, plus per-block sums of p^2 and u^2 into pd.partials_w / partials_u.
hipError_t launch_dense(const PlanDev& pd, const void* g, int g_bf16, float* m, float* v, float* p,
                        int lamb, const DenseParams& dp, hipStream_t s);
// One block per chunk: the diagnostics of the chunk from partials_e (pass-1 table, p1_first) and
// partials_b (this launch's pass-2 table, chunk_first).
hipError_t launch_diag_reduce(const PlanDev& pd, double* err_sumsq, unsigned long long* plus_count,
                              hipStream_t s);
// One block per chunk: the chunk's pass-1 partials (p1_first ranges) added in a fixed order into
// sums[c].  A pass-2 view whose p1_first is the identity 0..K and whose partials are `sums` then forms
// the same scale from one partial per chunk.
hipError_t launch_chunk_sums(const PlanDev& pd, double* sums, hipStream_t s);
// One block per chunk: r_c from the chunk's partials_w / partials_u.
hipError_t launch_trust_ratio(const PlanDev& pd, float* ratios, hipStream_t s);
hipError_t launch_lamb_apply(const PlanDev& pd, const float* m, const float* v, float* p, const float* ratios,
                             int bias_correction, const LambParams& lp, hipStream_t s);
// lines_ok: every block of pd starts at a multiple of 128 elements (the whole-line variant of pass 1
// may then be used when the word rows are 16-byte aligned and W <= 8)
hipError_t launch_server_sumsq(const PlanDev& pd, int W, const uint32_t* ww, const float* ws,
                               const float* e, bool lines_ok, hipStream_t s);
hipError_t launch_server_apply(const PlanDev& pd, int W, const uint32_t* ww, const float* ws,
                               float* e, uint32_t* words, float* scales, hipStream_t s);
hipError_t launch_unpack(const PlanDev* pd, const uint32_t* words, int64_t n, const float* scales,
                         float* out, hipStream_t s);
hipError_t launch_pack(const void* x, int x_bf16, int64_t n, uint32_t* words, hipStream_t s);

// ---- the no-allocation compressed step (ob_noalloc.hip) ----
// Bytes of the static device buffer that holds its block tables and per-block sums.
constexpr int64_t kNoallocScratchBytes = int64_t(64) << 20;
// This device's address of that buffer (the device must be current), looked up on the first call on
// each device and kept; nullptr if the lookup failed.
void* noalloc_scratch(int device);
// The block tables of uniform chunks (chunk c = [c*chunk, min((c+1)*chunk, n)), K chunks), for two
// block sizes (pass 1: be1, pass 2: be2), written into device memory by one kernel: items1/first1 and
// items2/first2 as ob_plan_create builds them on the host, chunk offsets, and (ident != nullptr) the
// identity table 0..K.  nbf1 / nbf2: blocks of a chunk other than the last.
struct UniformTables {
    Item* items1;
    int32_t* first1;
    Item* items2;
    int32_t* first2;
    int64_t* off;
    int32_t* ident;
    int64_t n, chunk, be1, be2, n1, n2;
    int32_t K, nbf1, nbf2;
};
hipError_t launch_uniform_tables(const UniformTables& t, hipStream_t s);

}  // namespace ob

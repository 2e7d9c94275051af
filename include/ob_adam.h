/*
 * ob_adam.h -- C ABI of the 1-bit Adam step on one AMD MI355X (gfx950).
 *
 * The library (libobadam.so) runs every step of the optimizer in hand-written HIP kernels.  All data
 * pointers are DEVICE pointers owned by the caller; every call is asynchronous on the caller's
 * `stream` and returns once its kernels are enqueued.  No torch types cross this boundary.
 *
 * Pages cited (title and section):
 *   [P1] "1bit Adam" tutorial (intelliparadigm.com article 2150495): sec. 2.1 quantization and error
 *        compensation, sec. 2.2 momentum on the compressed gradient, sec. 3.1 per-parameter state,
 *        sec. 3.2 compress routine (clip, NaN check, int8 signs), sec. 4.2 packing into one buffer.
 *   [P2] "DeepSpeed Communication Compression and Hiding": section "baseline: why Adam is hard to
 *        compress" (Adam moments), section "1-bit Adam: warmup, frozen variance, error feedback"
 *        (the two-phase step and compressed_allreduce), section "0/1 Adam" (variance refresh),
 *        section "1-bit LAMB: also protect the layer-wise trust ratio".
 *   [P3] gradient-compression survey (bmjup.com post 14450): Q&A on the memory cost of error
 *        feedback (the error term kept in a 16-bit format such as FP16).
 *
 * Definitions used by every call
 *   - Elements are a flat index 0..n-1 over one contiguous buffer per state array (the parameters
 *     packed into one block, [P1] sec. 4.2).  n may exceed 2^32.
 *   - A plan splits 0..n-1 into K chunks; every chunk has its own fp32 scale.  Chunk c spans
 *     [o_c, o_{c+1}).  Interior chunk boundaries must be multiples of 64.
 *   - sign(x) = +1 iff x >= 0.0f (so +0 and -0 give +1, NaN gives -1).
 *   - Packed signs: bit j of uint32 word w is 1 iff sign(x[32w + j]) = +1; ceil(n/32) words; bits
 *     for indices >= n are 0.  The packing ignores chunk boundaries.
 *   - scale_c = ||x_c||_2 / sqrt(n_c), with ||x_c||^2 accumulated in double and sqrt(S/n_c) taken in
 *     double, then rounded to fp32.  g_hat = +scale_c or -scale_c by the sign.
 *
 * Alignment: fp32 state and fp32 gradient pointers 16 bytes; bf16 gradient and 16-bit error buffer
 * 8 bytes; words, scales and int8 signs 4 bytes; the non-finite counter 8 bytes.  (torch allocations
 * are 256-byte aligned.)
 *
 * Errors: arguments are validated on the host before anything is enqueued, and a failed check
 * returns a status without touching the GPU: OB_ERR_ARG (null required pointer, bad size, bad chunk
 * table, W < 1, n differs from the plan), OB_ERR_ALIGN (pointer or chunk-boundary alignment),
 * OB_ERR_DTYPE (unknown dtype).  A failed launch returns OB_ERR_HIP; faults during execution surface
 * at the caller's next synchronisation.  OB_ERR_OOM: an allocation failed (a plan's device memory, or
 * host memory for its tables or for timing records).  n = 0 is a no-op.
 * No C++ exception crosses the ABI and nothing aborts.  NaN and Inf propagate per IEEE.
 *
 * Threads and streams: distinct plans are independent.  A plan holds a small workspace (one double
 * per work block), so one plan must not be used by two calls that may run concurrently on the GPU;
 * calls on one stream are ordered and therefore safe.
 */
#ifndef OB_ADAM_H
#define OB_ADAM_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    OB_OK = 0,
    OB_ERR_ARG = 1,
    OB_ERR_ALIGN = 2,
    OB_ERR_DTYPE = 3,
    OB_ERR_HIP = 4,
    OB_ERR_OOM = 5,
    OB_ERR_SIZE = 6     /* ob_adam_compress_step_noalloc: the problem needs more than its static buffer */
} ob_status;

/* Element types.  Gradients and packed inputs: OB_F32 or OB_BF16.  The error buffer of the compressed
 * step may also be OB_F16 (IEEE binary16). */
typedef enum { OB_F32 = 0, OB_BF16 = 1, OB_F16 = 2 } ob_dtype;

/* Error feedback rule: PLAIN replaces the error with x - g_hat ([P2] 1-bit Adam pseudo-code);
 * EMA keeps ef_beta*err + (1-ef_beta)*(x - g_hat) ([P1] sec. 2.1). */
typedef enum { OB_EF_PLAIN = 0, OB_EF_EMA = 1 } ob_ef_mode;

/* How a new error is stored in a 16-bit error buffer: to nearest, ties to even, or stochastically
 * (round up with probability equal to the fraction of the quantum; 16 random bits per element from
 * Philox4x32-10 at counter (i >> 2, step) with key sr_seed; see ob_adam_compress_step). */
typedef enum { OB_ROUND_NEAREST = 0, OB_ROUND_STOCHASTIC = 1 } ob_rounding;

/* Hyperparameters, fp32 as in the per-parameter state of [P1] sec. 3.1. */
typedef struct {
    float lr;
    float beta1;
    float beta2;            /* dense step only */
    float eps;
    float clip;             /* compressed step: clamp g to [-clip, clip] before adding the error
                               ([P1] sec. 3.2); <= 0 disables; NaN passes through */
    int32_t ef_mode;        /* ob_ef_mode */
    float ef_beta;          /* EMA coefficient ([P1] sec. 2.1 uses beta1 = 0.9) */
    int32_t bias_correction;/* dense step only: divide m, v by 1 - beta^step (textbook Adam);
                               the pages' step has none, so 0 is the default */
    int64_t step;           /* dense step with bias_correction: t >= 1; compressed step with
                               stochastic rounding: the random stream (use a new value every step) */
    int32_t err_rounding;   /* ob_rounding; compressed steps with a 16-bit error buffer only */
    int32_t reserved;       /* 0 */
    uint64_t sr_seed;       /* stochastic rounding: the generator's key, with step */
} ob_hparams;

typedef struct ob_plan_s* ob_plan;

/* Create a plan for n elements on the current HIP device.
 *   chunk_offsets == NULL: uniform chunks of chunk_size elements (the last one ends at n);
 *                          chunk_size > 0 and, when n > chunk_size, a multiple of 64.
 *   chunk_offsets != NULL: n_chunks + 1 host int64 offsets, 0 = o_0 < o_1 < ... < o_K = n, interior
 *                          offsets multiples of 64 (one chunk per parameter tensor).
 * The plan owns its device tables and workspace (hipMalloc here, hipFree in ob_plan_destroy);
 * *out is set to NULL on failure. */
ob_status ob_plan_create(int64_t n, int64_t chunk_size, const int64_t* chunk_offsets,
                         int64_t n_chunks, ob_plan* out);
ob_status ob_plan_destroy(ob_plan plan);
int64_t ob_plan_num_elements(ob_plan plan);   /* -1 for a NULL plan */
int64_t ob_plan_num_chunks(ob_plan plan);     /* -1 for a NULL plan */
int64_t ob_plan_num_blocks(ob_plan plan);     /* work blocks = grid size of the per-element kernels */
int64_t ob_plan_block_elems(ob_plan plan);    /* elements per work block (except chunk tails) */
/* Chunk groups of the compressed step (ob_adam_compress_step, ob_adam_worker_compress): the step runs
 * its two kernels group by group, each group being consecutive chunks whose bytes read by the first
 * kernel (g and err) stay within a budget sized to the GPU's last-level cache (320 MB; the environment
 * variable OB_GROUP_BYTES, read when the plan is created, overrides it and 0 turns grouping off), so
 * that the second kernel re-reads them from that cache.  A chunk above the budget is a group of its
 * own; plans whose chunks need a per-chunk sums launch (more than 4096 first-kernel blocks in a chunk)
 * are one group, and so is 1-bit LAMB (lamb != 0: ob_lamb_compress_step, whose first kernel also reads
 * p).  Returns the number of groups, i.e. the launches of each of the two kernels per step; -1 for a
 * NULL plan or an invalid dtype. */
int64_t ob_plan_num_groups(ob_plan plan, ob_dtype g_dtype, ob_dtype err_dtype, int32_t lamb);

/* Dense Adam step ([P2] baseline section; the step used before freeze_step in [P2] 1-bit Adam and for
 * the variance refresh of [P2] 0/1 Adam):
 *   m = beta1*m + (1-beta1)*g;  v = beta2*v + (1-beta2)*g^2;
 *   p -= lr * mh / (sqrt(vh) + eps)   with mh = m, vh = v, or m/(1-beta1^t), v/(1-beta2^t) when
 *   hp->bias_correction.  The error buffer is not touched.
 * g: n elements of `g_dtype` (read only); m, v, p: fp32[n], updated in place. */
ob_status ob_adam_warmup_step(ob_plan plan, const void* g, ob_dtype g_dtype, float* m, float* v,
                              float* p, const ob_hparams* hp, hipStream_t stream);

/* Compressed step ([P2] 1-bit Adam, compressed branch with W = 1; [P1] sec. 2.1-2.2, 3.2):
 *   g' = clip(widen(g));  x = g' + err (fp32);  words = pack(sign(x));  scales_c per chunk;
 *   g_hat = +-scale_c;  err = x - g_hat (PLAIN) or ef_beta*err + (1-ef_beta)*(x - g_hat) (EMA);
 *   m = beta1*m + (1-beta1)*g_hat;  p -= lr * m / (sqrt(v) + eps)  (v frozen, read only).
 * Runs two kernels: a per-chunk sum of squares, then one fused streaming pass, one pair of launches
 * per chunk group (ob_plan_num_groups; the results do not depend on the grouping).
 * g: n elements (read only); err: n elements of err_dtype, in place; m, p: fp32[n] in place;
 * v: fp32[n] read only; words_out: uint32[ceil(n/32)]; scales_out: fp32[K];
 * err_dtype ([P3] Q&A on error-feedback memory): OB_F32, or OB_BF16 / OB_F16 -- the stored error is
 *   widened exactly when read, and the new error, computed in fp32 as above, is rounded to the format
 *   (nearest, ties to even; beyond the largest finite value, +-Inf) when stored.  With
 *   hp->err_rounding = OB_ROUND_STOCHASTIC it is stored as lo or hi = lo + q (lo its truncation toward
 *   zero, q the format's quantum there), hi iff r*q < (|e| - lo)*65536 with r the element's 16
 *   random bits: the high half of output word i & 3 of Philox4x32-10 (Salmon et al., SC 2011) at the
 *   128-bit counter (i >> 2, hp->step) under the 64-bit key hp->sr_seed (32-bit words, low first).
 *   OB_ERR_ARG for an fp32 error buffer;
 * signs_out (optional, NULL = off): int8[n] of +1/-1 ([P1] sec. 3.2);
 * nonfinite_out (optional, NULL = off): device uint64 counter to which the number of non-finite
 * STORED new error elements is added ([P1] sec. 3.2 NaN check; the caller zeroes it), so an fp16
 * overflow is counted.
 * Outputs must not alias inputs. */
ob_status ob_adam_compress_step(ob_plan plan, const void* g, ob_dtype g_dtype, void* err, ob_dtype err_dtype,
                                float* m, const float* v, float* p, uint32_t* words_out, float* scales_out,
                                int8_t* signs_out, uint64_t* nonfinite_out, const ob_hparams* hp,
                                hipStream_t stream);

/* ---- 1-bit LAMB ([P2] section "1-bit LAMB: also protect the layer-wise trust ratio") ----
 * LAMB scales the Adam direction of each layer by the trust ratio r = ||w|| / ||u|| and updates
 * w -= lr * r * u; in 1-bit LAMB the direction is built from the reconstructed (compressed) gradient.
 * Here a layer is a chunk of the plan (create the plan with one chunk per parameter tensor):
 *   u_i = mh_i / (sqrt(vh_i) + eps)      (double, not stored; mh = m, vh = v unless bias-corrected)
 *   r_c = ||p_c|| / ||u_c||               (p before the update; sums of squares in double, rounded
 *                                         once to fp32; r_c = 1 when either norm is 0, NaN/Inf propagate)
 *   p_i -= lr * r_c * u_i                 (double, rounded once)
 * No weight decay and no clamp of r.  ratios_out: fp32[K], the ratio each layer used.
 * Each call runs 4 kernels (compressed) or 3 (dense): the passes below, one block per layer for the
 * ratios, and the update. */

/* Compressed 1-bit LAMB step: exactly ob_adam_compress_step's compensate / quantize / pack / error /
 * momentum (same arguments and outputs), then the trust ratio on the new m and the frozen v, and the
 * update of p. */
ob_status ob_lamb_compress_step(ob_plan plan, const void* g, ob_dtype g_dtype, void* err, ob_dtype err_dtype,
                                float* m, const float* v, float* p, uint32_t* words_out, float* scales_out,
                                float* ratios_out, int8_t* signs_out, uint64_t* nonfinite_out,
                                const ob_hparams* hp, hipStream_t stream);

/* Dense LAMB step (the warmup of 1-bit LAMB): m and v as in ob_adam_warmup_step (bias correction by
 * hp->bias_correction / hp->step), then the trust ratio and the update of p. */
ob_status ob_lamb_warmup_step(ob_plan plan, const void* g, ob_dtype g_dtype, float* m, float* v, float* p,
                              float* ratios_out, const ob_hparams* hp, hipStream_t stream);

/* Server half of compressed_allreduce ([P2] 1-bit Adam) on this GPU's share of n elements:
 *   avg_i = (sum_{w<W} (bit_w(i) ? s_{w,c} : -s_{w,c})) / W, summed in double in ascending w and
 *           rounded once to fp32;
 *   x = avg + server_err;  words_out = pack(sign(x));  scales_out per chunk of x;
 *   server_err = x - g_hat (plain error feedback kept by the server).
 * worker_words: W rows of ceil(n/32) uint32 (row w starts at w*ceil(n/32)); pad bits are ignored;
 * worker_scales: W rows of K fp32; server_err: fp32[n] in place; words_out: uint32[ceil(n/32)];
 * scales_out: fp32[K].  1 <= W <= 1024. */
ob_status ob_server_reduce(ob_plan plan, int32_t W, const uint32_t* worker_words,
                           const float* worker_scales, float* server_err, uint32_t* words_out,
                           float* scales_out, hipStream_t stream);

/* ---- the worker's compressed step split at the exchange (more than one worker; [P2] "1-bit Adam:
 * warmup, frozen variance, error feedback", compressed branch: the quantize line runs before
 * compressed_allreduce, the dequantize, momentum and update lines after it) ----
 * ob_adam_worker_compress: ob_adam_compress_step up to the packed signs, scales and error: the error
 *   uses the worker's own g_hat; m, v and p are not touched.  Arguments, layout and errors as there.
 * ob_adam_worker_update: g_hat_i = bit(i) ? scales[c] : -scales[c] from the exchanged words
 *   (uint32[ceil(n/32)], pad bits ignored) and scales (fp32[K]), e.g. the output of ob_server_reduce
 *   gathered back; then m = beta1*m + (1-beta1)*g_hat and p -= lr * m / (sqrt(v) + eps), m and p in
 *   place, v read only (hp: lr, beta1, eps).
 * With one worker and a zero server error the exchange returns the worker's own words and scales, and
 * the two calls give bit for bit the results of ob_adam_compress_step.
 * ob_lamb_worker_update ([P2] "1-bit LAMB"): the same g_hat and m, then the layer-wise trust ratio on
 *   the reconstructed direction and the update, as in ob_lamb_compress_step (ratios_out: fp32[K]).
 *   Its sums of p^2 and u^2 are grouped by other blocks than the fused step's, so a ratio may differ
 *   from that step's in the last bit. */
ob_status ob_adam_worker_compress(ob_plan plan, const void* g, ob_dtype g_dtype, void* err, ob_dtype err_dtype,
                                  uint32_t* words_out, float* scales_out, int8_t* signs_out,
                                  uint64_t* nonfinite_out, const ob_hparams* hp, hipStream_t stream);
ob_status ob_adam_worker_update(ob_plan plan, const uint32_t* words, const float* scales, float* m,
                                const float* v, float* p, const ob_hparams* hp, hipStream_t stream);
ob_status ob_lamb_worker_update(ob_plan plan, const uint32_t* words, const float* scales, float* m,
                                const float* v, float* p, float* ratios_out, const ob_hparams* hp,
                                hipStream_t stream);

/* Pack signs of x (OB_F32 or OB_BF16, n elements) into ceil(n/32) words ([P2] one_bit_quantize, sign part).
 * n at most (2^31 - 1) * 16384 (one block per 16384 elements); OB_ERR_ARG beyond. */
ob_status ob_pack(const void* x, ob_dtype x_dtype, int64_t n, uint32_t* words_out, hipStream_t stream);

/* Unpack + dequantize ([P2] dequantize): out_i = bit(i) ? s_c : -s_c, s_c = scales[c] for the plan's
 * chunk c of i; with scales == NULL, s = 1 and plan may be NULL.  With scales, plan is required and n
 * must equal the plan's n.  out: fp32[n].  Without a plan's tables (scales == NULL) n is at most
 * (2^31 - 1) * 16384, as for ob_pack. */
ob_status ob_unpack(ob_plan plan, const uint32_t* words, int64_t n, const float* scales, float* out,
                    hipStream_t stream);

const char* ob_status_str(ob_status s);

/* ---- the compressed step without any allocation ----
 * For callers that cannot allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  ob_adam_compress_step for uniform chunks of chunk_size elements
 * (the last chunk ends at n; chunk_size > 0 and, when n > chunk_size, a multiple of 64 -- the chunking
 * of ob_plan_create with chunk_offsets == NULL), without a plan.  Arguments, layouts, outputs and
 * errors otherwise as ob_adam_compress_step; the results are bit for bit those of
 * ob_adam_compress_step with a plan of the same n and chunk_size.
 * It calls no hipMalloc, hipFree or other allocating routine.  Its block tables and per-block sums of
 * squares live in a static device buffer of OB_NOALLOC_SCRATCH_BYTES that the library holds on every
 * GPU it runs on until the process ends; the first call on a device looks up that device's copy.
 * Each call rewrites the tables it needs (one small kernel ahead of the two passes), so consecutive
 * calls may change n and chunk_size.  The two passes run by chunk groups as in ob_adam_compress_step
 * (groups of equal numbers of chunks within the same budget, OB_GROUP_BYTES read on every call).  All calls on one GPU share its buffer: calls that may overlap on
 * one GPU (other streams, other host threads) race and must not be issued; calls on one stream are
 * ordered.  Space needed: 24 bytes per first-pass block, 16 per 4096-element block of the fused pass,
 * 16 per chunk (plus 12 per chunk for chunks of more than 4096 first-pass blocks), each region rounded
 * up to 256 bytes -- with chunks of 2^24 elements about 1.3e10 elements fit.  A larger problem returns
 * OB_ERR_SIZE before any HIP call.  No diagnostics and no timing (those belong to a plan). */
#define OB_NOALLOC_SCRATCH_BYTES (64ll << 20)
ob_status ob_adam_compress_step_noalloc(int64_t n, int64_t chunk_size, const void* g, ob_dtype g_dtype,
                                        void* err, ob_dtype err_dtype, float* m, const float* v, float* p,
                                        uint32_t* words_out, float* scales_out, int8_t* signs_out,
                                        uint64_t* nonfinite_out, const ob_hparams* hp, hipStream_t stream);

/* ---- kernel timing (measurement support) ----
 * With timing on, every call made with this plan records hipEvents around each kernel it launches, on
 * the call's stream: a pair per launch, except that the launches a compressed step makes one after the
 * other for its chunk groups share them (each starts at the event that ended the one before), one
 * event per launch.  ob_plan_read_timing waits for the recorded events and returns the summed
 * milliseconds and launch count of one kernel kind since timing was switched on.  The events are
 * created with hipEventDisableSystemFence: they measure time only and order no memory. */
typedef enum {
    OB_KERNEL_CHUNK_SUMSQ = 0,     /* compressed step (Adam or LAMB), pass 1 */
    OB_KERNEL_COMPRESS = 1,        /* compressed step (Adam or LAMB), pass 2 (fused streaming pass) */
    OB_KERNEL_DENSE = 2,           /* dense step (Adam, or the moments pass of dense LAMB) */
    OB_KERNEL_SERVER_SUMSQ = 3,    /* server reduce, pass 1 */
    OB_KERNEL_SERVER_APPLY = 4,    /* server reduce, pass 2 */
    OB_KERNEL_UNPACK = 5,
    OB_KERNEL_TRUST_RATIO = 6,     /* LAMB: per-layer ratios */
    OB_KERNEL_LAMB_APPLY = 7,      /* LAMB: parameter update */
    OB_KERNEL_DIAG = 8,            /* diagnostics: per-chunk totals */
    OB_KERNEL_SCALE = 9,           /* per-chunk sums of squares formed before pass 2 (plans with a
                                      chunk of more than 4096 pass-1 blocks) */
    OB_KERNEL_WORKER_COMPRESS = 10,/* worker compress, pass 2 (pass 1 is OB_KERNEL_CHUNK_SUMSQ) */
    OB_KERNEL_WORKER_UPDATE = 11,  /* worker update */
    OB_KERNEL_COUNT = 12
} ob_kernel;

ob_status ob_plan_set_timing(ob_plan plan, int32_t enable);
ob_status ob_plan_read_timing(ob_plan plan, int32_t kernel, double* total_ms, int64_t* launches);

/* ---- diagnostics ([P1] sec. 6.2: warn when a parameter's error-buffer L2 norm is below 1e-6;
 * [P1] sec. 8: monitor that norm and the quantization rate) ----
 * With both pointers set (device arrays of K elements, 8-byte aligned), every later compressed step
 * with this plan (ob_adam_compress_step or ob_lamb_compress_step) also writes, per chunk c:
 *   err_sumsq_out[c]  = sum of squares (double) of the error buffer as that step read it, i.e. the
 *                       error left by the previous step; sqrt gives the L2 norm;
 *   plus_count_out[c] = number of elements of the chunk whose sign bit is +1 (the bit balance).
 * The first pass accumulates the first, the fused pass the second, and a one-block-per-chunk kernel
 * writes both.  The first call that enables them allocates two workspaces for the plan.  Both NULL
 * switches them off; exactly one NULL is OB_ERR_ARG. */
ob_status ob_plan_set_diagnostics(ob_plan plan, double* err_sumsq_out, uint64_t* plus_count_out);

#ifdef __cplusplus
}
#endif

#endif /* OB_ADAM_H */

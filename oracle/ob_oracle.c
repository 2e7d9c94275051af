/*
 * ob_oracle.c -- CPU oracle for the 1-bit Adam optimizer step.
 *
 * TEST INFRASTRUCTURE ONLY.  Plain, single-threaded, slow and meant to be checked by eye against
 * the pages.  Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of bench.py may load or
 * call it.  The HIP library never links, includes or executes anything from this folder, and this
 * file takes no code, header, table or constant from that library.
 *
 * Pages (cited by title and section; no line numbers):
 *   [P1] "1bit Adam" tutorial (intelliparadigm.com, article 2150495):
 *        sec. 2.1 (sign quantization, error computation, EMA error compensation),
 *        sec. 2.2 (first moment driven by the compressed gradient),
 *        sec. 3.1 (per-parameter state: error buffer, momentum, variance, beta1/beta2/eps),
 *        sec. 3.2 (compress routine; clipping at +/-5 before quantizing, NaN check after the error
 *                  update, int8 storage of the signs),
 *        sec. 5.1 (BERT-base table: 3.12% communication volume => one bit per fp32 element).
 *   [P2] "DeepSpeed Communication Compression and Hiding" (shaojiemike.top):
 *        section "baseline: why Adam is hard to compress" (the Adam moment equations),
 *        section "1-bit Adam: warmup, frozen variance, error feedback" (the two-phase pseudo-code),
 *        section "0/1 Adam" (periodic variance refresh alternating with 1-bit steps).
 *   [P3] gradient-compression survey (bmjup.com post 14450), section on the core principle
 *        (plain error feedback: the residual of the compressor is added to the next gradient).
 *
 * Readings taken where the pages leave a step open (each is listed with its reason in the design
 * notes of the repository):
 *   R1 scale: one fp32 scale per chunk, scale_c = ||x_c||_2 / sqrt(n_c).  ||x||^2 is summed in
 *      double in ascending index order; sqrt(S / n_c) is taken in double and rounded once to fp32.
 *   R2 sign(x) = +1 iff x >= 0.0f (IEEE ordered compare): +0 and -0 give +1, NaN gives -1.
 *   R3 packing: bit j of uint32 word w is the sign bit of flat element 32*w + j (1 <=> +1), bits of
 *      indices >= n are 0; the packing ignores chunk boundaries.
 *   R4 precision: every tensor the method keeps or hands on (compensated x, g_hat, error, m, v, p,
 *      scales) is fp32, as the state of [P1] sec. 3.1 and the in-place fp32 compensation of
 *      [P1] sec. 3.2 are.  Each formula of the pages is evaluated here in double from its fp32
 *      operands and rounded once to fp32 when its tensor is written.  bf16 gradients are widened
 *      exactly to fp32 first.
 *   R5 the update uses the new m (and in the dense step the new v).
 *   R6 the error in plain mode is replaced (x - g_hat) as in [P2]/[P3]; in EMA mode ([P1] sec. 2.1)
 *      it is ef_beta*err_old + (1-ef_beta)*delta with delta = fl32(x - g_hat), g_hat scaled.
 *   R7 clipping ([P1] sec. 3.2) clamps the widened gradient elementwise to [-clip, clip] before the
 *      error is added; clip <= 0 means off; NaN passes through.
 *   R8 the NaN check of [P1] sec. 3.2 counts non-finite new-error elements; it changes nothing.
 *   R9 server: avg_i = sum_w (+/- s_{w,c}) / W, summed in double over w = 0..W-1 and rounded once
 *      to fp32; x = fl32(avg + e_srv); then the same scale/pack/plain error as the worker.
 *   R15 error storage ([P3] Q&A on the memory cost of error feedback, which suggests keeping the
 *      fp32 error term in a 16-bit format such as FP16): the error buffer may be held as fp32, bf16
 *      or fp16.  A stored value is widened exactly when read; the new error is computed in fp32 as
 *      in R4/R6 and then rounded to the storage format to nearest, ties to even (IEEE 754's default
 *      rounding), overflowing to +-Inf.  The R8 check counts non-finite STORED values, so an fp16
 *      overflow is reported.
 *   R18 stochastic rounding of a 16-bit error buffer (optional; the nearest-even store of R15 is the
 *      default): the new fp32 error e is stored as lo or hi, the two format values around |e| (lo
 *      toward zero, hi = lo + one quantum q), choosing hi iff r * q < (|e| - lo) * 65536, where r is a
 *      16-bit random integer; so hi comes with probability (|e| - lo)/q (to 1/65536).  Values of the
 *      format, +-0, NaN and +-Inf are stored unchanged; a hi beyond the largest finite value is Inf.
 *      r for flat element i: the high 16 bits of output word i & 3 of Philox4x32-10 (Salmon, Moraes,
 *      Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011) at the 128-bit counter
 *      (i >> 2, step) -- 32-bit words lo(i >> 2), hi(i >> 2), lo(step), hi(step) -- under the 64-bit
 *      key seed -- words lo(seed), hi(seed): a counter-based generator, so every element's bits are
 *      a function of (seed, step, i) alone, and four consecutive elements share one output block.
 *   R16 1-bit LAMB ([P2] section "1-bit LAMB: also protect the layer-wise trust ratio"): a layer is a
 *      chunk (one chunk per parameter tensor).  The direction is u_i = m_i / (sqrt(v_i) + eps) with
 *      the new m (compressed step: v frozen, m driven by g_hat as in R5/R6; dense step: the new m and
 *      v, divided by 1 - beta^t when bias correction is on), evaluated in double and not stored.
 *      S_w = sum p_i^2 over the layer's parameters before the update and S_u = sum u_i^2, both in
 *      double in ascending index order; r = fl32(sqrt(S_w) / sqrt(S_u)), and r = 1 when S_w == 0 or
 *      S_u == 0 (the ratio is undefined there, and a zero-initialised layer must still move);
 *      p_i = fl32(p_i - lr * (r * u_i)) in double.  No weight decay and no clamp of r: the pages
 *      give neither.
 *   R17 diagnostics ([P1] sec. 6.2: the L2 norm of each parameter's error buffer, warned about below
 *      1e-6; [P1] sec. 8: monitor that norm and the quantization rate): per chunk, the sum of squares
 *      of the stored error buffer as the step reads it (double, ascending index; its square root is
 *      the norm) and the number of elements whose sign bit is +1 in the step's packed words (the
 *      bit balance; the ideal share for a zero-mean gradient is one half).
 *   R19 the worker's compressed step split at the exchange ([P2] compressed branch: the quantize
 *      line runs before compressed_allreduce, the dequantize, momentum and update lines after it).
 *      (a) worker compress: compensate, per-chunk scale, pack, and the new error from the worker's
 *      OWN g_hat (R10), stored as in R15/R18; m and p are not touched.  (b) worker update: g_hat
 *      from the words and scales the exchange returns (the server's), then m and the frozen-v
 *      update exactly as in the fused step.  With one worker and a zero server error the exchange
 *      returns the worker's own words and scales, and (a) then (b) is the fused step.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_OK 0
#define OR_ERR_ARG 1
#define OR_ERR_OOM 5

/* ---------- element helpers ---------- */

/* bf16 -> fp32 is exact: the bf16 bits are the high half of the fp32 bits. */
static float bf16_bits_to_float(uint16_t b)
{
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static float load_grad(const void* g, int g_is_bf16, int64_t i)
{
    if (g_is_bf16)
        return bf16_bits_to_float(((const uint16_t*)g)[i]);
    return ((const float*)g)[i];
}

/* ---------- R15: storage formats of the error buffer ---------- */

#define OR_FMT_F32 0
#define OR_FMT_BF16 1
#define OR_FMT_F16 2

/* Nearest value of a binary floating-point format with `prec` significand bits (the implicit bit
 * included), smallest normal exponent emin and largest finite value maxf, ties to even; a result
 * beyond maxf becomes +-Inf.  x is an fp32 value, so every step below is exact in double. */
static double round_to_format(double x, int prec, int emin, double maxf)
{
    if (isnan(x) || isinf(x)) return x;
    double a = fabs(x);
    int e;
    frexp(a, &e);                 /* a in [2^(e-1), 2^e) */
    int E = e - 1;
    if (a == 0.0 || E < emin) E = emin;   /* subnormals: the quantum of the lowest normal binade */
    double q = ldexp(1.0, E - (prec - 1));
    double r = nearbyint(a / q) * q;      /* default rounding mode: nearest, ties to even */
    if (r > maxf) r = INFINITY;
    return copysign(r, x);
}

/* R18: the format value next to |x| toward zero, and its quantum (x an fp32 value, finite). */
static double truncate_to_format(double a, int prec, int emin, double* quantum)
{
    int e;
    frexp(a, &e);
    int E = e - 1;
    if (a == 0.0 || E < emin) E = emin;
    double q = ldexp(1.0, E - (prec - 1));
    *quantum = q;
    return floor(a / q) * q;
}

/* R18: stochastic rounding of x to the format with the 16-bit random integer r. */
static double stochastic_round(double x, int prec, int emin, double maxf, uint32_t r)
{
    if (isnan(x) || isinf(x)) return x;
    double a = fabs(x), q;
    double lo = truncate_to_format(a, prec, emin, &q);
    double v = lo;
    if (lo != a && (double)r * q < (a - lo) * 65536.0) v = lo + q;
    if (v > maxf) v = INFINITY;
    return copysign(v, x);
}

/* Philox4x32-10: ten rounds of the Philox S-box on a 4 x 32-bit counter with a 2 x 32-bit key, the
 * key bumped by the Weyl constants between rounds (SC 2011 paper cited with R18). */
void or_philox4x32(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3], k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += W0;
            k1 += W1;
        }
        uint64_t p0 = (uint64_t)M0 * c0, p1 = (uint64_t)M1 * c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0, n1 = lo1, n2 = hi0 ^ c3 ^ k1, n3 = lo0;
        c0 = n0;
        c1 = n1;
        c2 = n2;
        c3 = n3;
    }
    out[0] = c0;
    out[1] = c1;
    out[2] = c2;
    out[3] = c3;
}

/* R18: the 16 random bits of flat element i. */
static uint32_t sr_bits(uint64_t seed, uint64_t step, int64_t i)
{
    uint64_t blk = (uint64_t)i >> 2;
    uint32_t ctr[4] = {(uint32_t)blk, (uint32_t)(blk >> 32), (uint32_t)step, (uint32_t)(step >> 32)};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)}, out[4];
    or_philox4x32(ctr, key, out);
    return out[i & 3] >> 16;
}

#define BF16_MAXF ((2.0 - ldexp(1.0, -7)) * ldexp(1.0, 127))
#define F16_MAXF 65504.0

/* bf16 bits of a value of the bf16 format: bf16 values are fp32 values whose low 16 bits are 0. */
static uint16_t bf16_bits_of(double r)
{
    if (isnan(r)) return (uint16_t)(signbit(r) ? 0xFFC0u : 0x7FC0u);
    float f = (float)r;           /* exact */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/* fp16 (IEEE binary16) bits of a value of the fp16 format: 1 sign, 5 exponent (bias 15), 10 bits. */
static uint16_t f16_bits_of(double r)
{
    uint16_t s = signbit(r) ? 0x8000u : 0u;
    if (isnan(r)) return (uint16_t)(s | 0x7E00u);
    if (isinf(r)) return (uint16_t)(s | 0x7C00u);
    double a = fabs(r);
    if (a < ldexp(1.0, -14)) return (uint16_t)(s | (uint16_t)ldexp(a, 24));   /* zero, subnormal */
    int e;
    frexp(a, &e);
    int E = e - 1;
    return (uint16_t)(s | (uint16_t)((E + 15) << 10) | (uint16_t)(ldexp(a, 10 - E) - 1024.0));
}

static float f16_bits_to_float(uint16_t h)
{
    int ex = (h >> 10) & 0x1F, mant = h & 0x3FF;
    double v;
    if (ex == 0x1F)
        v = mant ? NAN : INFINITY;
    else if (ex == 0)
        v = ldexp((double)mant, -24);
    else
        v = ldexp((double)(mant + 1024), ex - 25);
    return (float)((h & 0x8000u) ? -v : v);
}

/* R2: the sign decision, made on the fp32 compensated value. */
static int sign_bit(float x)
{
    return x >= 0.0f ? 1 : 0;
}

/* Element i of an error buffer in format fmt, widened exactly to fp32. */
static float load_err(const void* buf, int fmt, int64_t i)
{
    if (fmt == OR_FMT_BF16) return bf16_bits_to_float(((const uint16_t*)buf)[i]);
    if (fmt == OR_FMT_F16) return f16_bits_to_float(((const uint16_t*)buf)[i]);
    return ((const float*)buf)[i];
}

/* R18: store e (fp32) as element i of a 16-bit error buffer, stochastically rounded with r. */
static float store_err_sr(void* buf, int fmt, int64_t i, float e, uint32_t r)
{
    if (fmt == OR_FMT_BF16) {
        uint16_t b = bf16_bits_of(stochastic_round(e, 8, -126, BF16_MAXF, r));
        ((uint16_t*)buf)[i] = b;
        return bf16_bits_to_float(b);
    }
    uint16_t h = f16_bits_of(stochastic_round(e, 11, -14, F16_MAXF, r));
    ((uint16_t*)buf)[i] = h;
    return f16_bits_to_float(h);
}

/* Store e (fp32) as element i of an error buffer in format fmt; returns the stored value, widened. */
static float store_err(void* buf, int fmt, int64_t i, float e)
{
    if (fmt == OR_FMT_BF16) {
        uint16_t b = bf16_bits_of(round_to_format(e, 8, -126, BF16_MAXF));
        ((uint16_t*)buf)[i] = b;
        return bf16_bits_to_float(b);
    }
    if (fmt == OR_FMT_F16) {
        uint16_t h = f16_bits_of(round_to_format(e, 11, -14, F16_MAXF));
        ((uint16_t*)buf)[i] = h;
        return f16_bits_to_float(h);
    }
    ((float*)buf)[i] = e;
    return e;
}

/* Narrow n fp32 values to a 16-bit error format (bits out), or widen bits back: exposed so the
 * conversions can be checked on their own. */
int or_to_format(const float* x, int64_t n, int fmt, uint16_t* bits)
{
    if (n < 0 || (fmt != OR_FMT_BF16 && fmt != OR_FMT_F16)) return 1;
    for (int64_t i = 0; i < n; ++i) store_err(bits, fmt, i, x[i]);
    return 0;
}

/* R18 on its own: x[k] stored as flat element index0 + k of a 16-bit buffer with (seed, step). */
int or_to_format_sr(const float* x, int64_t n, int fmt, uint64_t seed, uint64_t step, int64_t index0,
                    uint16_t* bits)
{
    if (n < 0 || (fmt != OR_FMT_BF16 && fmt != OR_FMT_F16)) return 1;
    for (int64_t k = 0; k < n; ++k) {
        uint16_t tmp[1];
        store_err_sr(tmp, fmt, 0, x[k], sr_bits(seed, step, index0 + k));
        bits[k] = tmp[0];
    }
    return 0;
}

int or_from_format(const uint16_t* bits, int64_t n, int fmt, float* out)
{
    if (n < 0 || (fmt != OR_FMT_BF16 && fmt != OR_FMT_F16)) return 1;
    for (int64_t i = 0; i < n; ++i) out[i] = load_err(bits, fmt, i);
    return 0;
}

static int check_offsets(int64_t n, int64_t K, const int64_t* off)
{
    if (n < 0 || K < 0 || off == NULL) return 0;
    if (n == 0) return K == 0 || (K >= 0 && off[0] == 0);
    if (K < 1 || off[0] != 0 || off[K] != n) return 0;
    for (int64_t c = 0; c < K; ++c)
        if (off[c + 1] <= off[c]) return 0;
    return 1;
}

/* ---------- R1: per-chunk scale ---------- */

double or_chunk_sumsq(const float* x, int64_t begin, int64_t end)
{
    double s = 0.0;
    for (int64_t i = begin; i < end; ++i)
        s += (double)x[i] * (double)x[i];
    return s;
}

float or_chunk_scale(const float* x, int64_t begin, int64_t end)
{
    double s = or_chunk_sumsq(x, begin, end);
    return (float)sqrt(s / (double)(end - begin));
}

/* ---------- R3: packing and unpacking ---------- */

int or_pack(const void* x, int x_is_bf16, int64_t n, uint32_t* words)
{
    if (n < 0 || (n > 0 && (x == NULL || words == NULL))) return OR_ERR_ARG;
    int64_t nw = (n + 31) / 32;
    for (int64_t w = 0; w < nw; ++w) words[w] = 0u;
    for (int64_t i = 0; i < n; ++i)
        if (sign_bit(load_grad(x, x_is_bf16, i)))
            words[i / 32] |= (uint32_t)1u << (i % 32);
    return OR_OK;
}

static int word_bit(const uint32_t* words, int64_t i)
{
    return (int)((words[i / 32] >> (i % 32)) & 1u);
}

/* out_i = +s_c or -s_c by the bit of i; s_c = 1 when scales == NULL.  [P2] 1-bit Adam: dequantize. */
int or_unpack(const uint32_t* words, int64_t n, int64_t K, const int64_t* off, const float* scales,
              float* out)
{
    if (n < 0 || (n > 0 && (words == NULL || out == NULL))) return OR_ERR_ARG;
    if (scales != NULL) {
        if (!check_offsets(n, K, off)) return OR_ERR_ARG;
        for (int64_t c = 0; c < K; ++c)
            for (int64_t i = off[c]; i < off[c + 1]; ++i)
                out[i] = word_bit(words, i) ? scales[c] : -scales[c];
    } else {
        for (int64_t i = 0; i < n; ++i)
            out[i] = word_bit(words, i) ? 1.0f : -1.0f;
    }
    return OR_OK;
}

/* ---------- compressed step ([P2] 1-bit Adam, compressed branch; [P1] sec. 2.1, 2.2, 3.2) ---------- */

/* The compressed step; adam_update = 0 stops before the parameter update (1-bit LAMB, R16). */
static int compress_core(int64_t n, int64_t K, const int64_t* off,
                         const void* g, int g_is_bf16,
                         void* err_store, int err_fmt, float* m, const float* v, float* p,
                         uint32_t* words, float* scales, int8_t* signs, int64_t* nonfinite,
                         float lr, float beta1, float eps, float clip, int ef_mode, float ef_beta,
                         int adam_update, int stochastic, uint64_t sr_seed, uint64_t sr_step,
                         int64_t sr_index0)
{
    if (stochastic && err_fmt == OR_FMT_F32) return OR_ERR_ARG;
    if (!check_offsets(n, K, off)) return OR_ERR_ARG;
    if (err_fmt != OR_FMT_F32 && err_fmt != OR_FMT_BF16 && err_fmt != OR_FMT_F16) return OR_ERR_ARG;
    if (n == 0) return OR_OK;
    if (!g || !err_store || !m || !v || !p || !words || !scales) return OR_ERR_ARG;

    float* x = (float*)calloc((size_t)n, sizeof(float));
    float* err = (float*)calloc((size_t)n, sizeof(float));
    if (x == NULL || err == NULL) {
        free(x);
        free(err);
        return OR_ERR_OOM;
    }
    /* R15: the error as fp32 (exact widening of the stored values). */
    for (int64_t i = 0; i < n; ++i) err[i] = load_err(err_store, err_fmt, i);

    /* x: the gradient (clipped, R7) plus the stored error, kept as an fp32 value (R4). */
    for (int64_t i = 0; i < n; ++i) {
        double gi = (double)load_grad(g, g_is_bf16, i);
        if (clip > 0.0f) {
            double c = (double)clip;
            if (gi > c)
                gi = c;
            else if (gi < -c)
                gi = -c;
        }
        x[i] = (float)(gi + (double)err[i]);
    }

    /* R1: one scale per chunk of x; R2/R3: the sign bits of x, packed over the flat index. */
    for (int64_t c = 0; c < K; ++c)
        scales[c] = or_chunk_scale(x, off[c], off[c + 1]);
    or_pack(x, 0, n, words);

    const double b1 = (double)beta1;
    const double eb = (double)ef_beta;
    for (int64_t c = 0; c < K; ++c) {
        for (int64_t i = off[c]; i < off[c + 1]; ++i) {
            int b = sign_bit(x[i]);
            /* the chunk's scale carrying the element's sign: the value the bit stands for. */
            float gh = b ? scales[c] : -scales[c];
            /* R6: what the bit failed to carry, x less that value; plain feedback keeps it, the EMA
             * rule of [P1] sec. 2.1 blends it with the previous error by ef_beta. */
            float delta = (float)((double)x[i] - (double)gh);
            float e_new;
            if (ef_mode == 1)
                e_new = (float)(eb * (double)err[i] + (1.0 - eb) * (double)delta);
            else
                e_new = delta;
            err[i] = e_new;
            /* R5: the first moment moves toward the quantized value, not the raw gradient
             * ([P1] sec. 2.2; [P2] compressed branch). */
            m[i] = (float)(b1 * (double)m[i] + (1.0 - b1) * (double)gh);
            /* the parameter step divides the new first moment by the root of the frozen second
             * moment (plus eps); v is only read ([P2] compressed branch). */
            if (adam_update)
                p[i] = (float)((double)p[i] -
                               (double)lr * ((double)m[i] / (sqrt((double)v[i]) + (double)eps)));
            if (signs != NULL) signs[i] = (int8_t)(b ? 1 : -1);
        }
    }
    /* R15 (R18 when stochastic): store the new error in its format; R8: count non-finite stored values. */
    for (int64_t i = 0; i < n; ++i) {
        float stored = stochastic ? store_err_sr(err_store, err_fmt, i, err[i],
                                                 sr_bits(sr_seed, sr_step, sr_index0 + i))
                                  : store_err(err_store, err_fmt, i, err[i]);
        if (nonfinite != NULL && !isfinite(stored)) *nonfinite += 1;
    }
    free(x);
    free(err);
    return OR_OK;
}

int or_compress_step(int64_t n, int64_t K, const int64_t* off,
                     const void* g, int g_is_bf16,
                     void* err_store, int err_fmt, float* m, const float* v, float* p,
                     uint32_t* words, float* scales, int8_t* signs, int64_t* nonfinite,
                     float lr, float beta1, float eps, float clip, int ef_mode, float ef_beta)
{
    return compress_core(n, K, off, g, g_is_bf16, err_store, err_fmt, m, v, p, words, scales, signs,
                         nonfinite, lr, beta1, eps, clip, ef_mode, ef_beta, 1, 0, 0, 0, 0);
}


/* ---------- R17: per-chunk diagnostics of a compressed step ([P1] sec. 6.2 and 8) ----------
 * err_store: the error buffer as the step read it (before the step); words: the step's packed signs. */
int or_diagnostics(int64_t n, int64_t K, const int64_t* off, const void* err_store, int err_fmt,
                   const uint32_t* words, double* err_sumsq, int64_t* plus_count)
{
    if (!check_offsets(n, K, off)) return OR_ERR_ARG;
    if (err_fmt != OR_FMT_F32 && err_fmt != OR_FMT_BF16 && err_fmt != OR_FMT_F16) return OR_ERR_ARG;
    for (int64_t c = 0; c < K; ++c) {
        double s = 0.0;
        int64_t plus = 0;
        for (int64_t i = off[c]; i < off[c + 1]; ++i) {
            double e = (double)load_err(err_store, err_fmt, i);
            s += e * e;
            plus += word_bit(words, i);
        }
        err_sumsq[c] = s;
        plus_count[c] = plus;
    }
    return OR_OK;
}

/* ---------- dense Adam step (warmup before freeze_step, and the 0/1 Adam refresh) ----------
 * [P2] baseline section: m = b1 m + (1-b1) g, v = b2 v + (1-b2) g^2; update as in the 1-bit Adam
 * pseudo-code with the new m and v.  bias_correction != 0 divides m and v by (1 - b^t), t = step
 * (textbook Adam); the pages' pseudo-code has no bias correction, so it is off by default.
 * The error buffer is not touched. */
/* The dense step; adam_update = 0 stops after the moments (1-bit LAMB warmup, R16). */
static int warmup_core(int64_t n, const void* g, int g_is_bf16, float* m, float* v, float* p,
                       float lr, float beta1, float beta2, float eps, int bias_correction, int64_t step,
                       int adam_update)
{
    if (n < 0) return OR_ERR_ARG;
    if (n == 0) return OR_OK;
    if (!g || !m || !v || !p) return OR_ERR_ARG;
    if (bias_correction && step < 1) return OR_ERR_ARG;
    const double b1 = (double)beta1, b2 = (double)beta2;
    double bc1 = 1.0, bc2 = 1.0;
    if (bias_correction) {
        bc1 = 1.0 - pow(b1, (double)step);
        bc2 = 1.0 - pow(b2, (double)step);
    }
    for (int64_t i = 0; i < n; ++i) {
        double gi = (double)load_grad(g, g_is_bf16, i);
        m[i] = (float)(b1 * (double)m[i] + (1.0 - b1) * gi);
        v[i] = (float)(b2 * (double)v[i] + (1.0 - b2) * (gi * gi));
        double mh = (double)m[i] / bc1;
        double vh = (double)v[i] / bc2;
        if (adam_update)
            p[i] = (float)((double)p[i] - (double)lr * (mh / (sqrt(vh) + (double)eps)));
    }
    return OR_OK;
}

int or_warmup_step(int64_t n, const void* g, int g_is_bf16, float* m, float* v, float* p,
                   float lr, float beta1, float beta2, float eps, int bias_correction, int64_t step)
{
    return warmup_core(n, g, g_is_bf16, m, v, p, lr, beta1, beta2, eps, bias_correction, step, 1);
}

/* ---------- 1-bit LAMB ([P2] section "1-bit LAMB"; reading R16) ---------- */

/* Per layer (chunk) c: trust ratio r_c = ||w_c|| / ||u_c|| of the parameters before the update and
 * the direction u_i = (m_i / bc1) / (sqrt(v_i / bc2) + eps); then p_i -= lr * r_c * u_i. */
static void lamb_update(int64_t K, const int64_t* off, const float* m, const float* v, float* p,
                        float* ratios, float lr, float eps, double bc1, double bc2)
{
    for (int64_t c = 0; c < K; ++c) {
        double sw = 0.0, su = 0.0;
        for (int64_t i = off[c]; i < off[c + 1]; ++i) {
            double u = ((double)m[i] / bc1) / (sqrt((double)v[i] / bc2) + (double)eps);
            sw += (double)p[i] * (double)p[i];
            su += u * u;
        }
        float r = (sw == 0.0 || su == 0.0) ? 1.0f : (float)(sqrt(sw) / sqrt(su));
        ratios[c] = r;
        for (int64_t i = off[c]; i < off[c + 1]; ++i) {
            double u = ((double)m[i] / bc1) / (sqrt((double)v[i] / bc2) + (double)eps);
            p[i] = (float)((double)p[i] - (double)lr * ((double)r * u));
        }
    }
}

/* Compressed 1-bit LAMB step: the compressed step's compensate / quantize / error / momentum on the
 * reconstructed direction, then the layer-wise trust ratio and the update (v frozen). */
int or_lamb_compress_step(int64_t n, int64_t K, const int64_t* off,
                          const void* g, int g_is_bf16,
                          void* err_store, int err_fmt, float* m, const float* v, float* p,
                          uint32_t* words, float* scales, float* ratios, int8_t* signs,
                          int64_t* nonfinite, float lr, float beta1, float eps, float clip,
                          int ef_mode, float ef_beta)
{
    if (n > 0 && ratios == NULL) return OR_ERR_ARG;
    int rc = compress_core(n, K, off, g, g_is_bf16, err_store, err_fmt, m, v, p, words, scales, signs,
                           nonfinite, lr, beta1, eps, clip, ef_mode, ef_beta, 0, 0, 0, 0, 0);
    if (rc != OR_OK || n == 0) return rc;
    lamb_update(K, off, m, v, p, ratios, lr, eps, 1.0, 1.0);
    return OR_OK;
}

/* Dense LAMB step (the warmup of 1-bit LAMB): Adam moments, then the trust ratio and update. */
int or_lamb_warmup_step(int64_t n, int64_t K, const int64_t* off, const void* g, int g_is_bf16,
                        float* m, float* v, float* p, float* ratios, float lr, float beta1, float beta2,
                        float eps, int bias_correction, int64_t step)
{
    if (!check_offsets(n, K, off)) return OR_ERR_ARG;
    if (n > 0 && ratios == NULL) return OR_ERR_ARG;
    int rc = warmup_core(n, g, g_is_bf16, m, v, p, lr, beta1, beta2, eps, bias_correction, step, 0);
    if (rc != OR_OK || n == 0) return rc;
    double bc1 = 1.0, bc2 = 1.0;
    if (bias_correction) {
        bc1 = 1.0 - pow((double)beta1, (double)step);
        bc2 = 1.0 - pow((double)beta2, (double)step);
    }
    lamb_update(K, off, m, v, p, ratios, lr, eps, bc1, bc2);
    return OR_OK;
}

/* The compressed step with the new error stochastically rounded into a 16-bit buffer (R18).  The arrays
 * hold flat elements sr_index0 .. sr_index0 + n - 1 of the buffer (the random bits follow the flat
 * index). */
int or_compress_step_sr(int64_t n, int64_t K, const int64_t* off,
                        const void* g, int g_is_bf16,
                        void* err_store, int err_fmt, float* m, const float* v, float* p,
                        uint32_t* words, float* scales, int8_t* signs, int64_t* nonfinite,
                        float lr, float beta1, float eps, float clip, int ef_mode, float ef_beta,
                        int lamb, float* ratios, uint64_t sr_seed, uint64_t sr_step, int64_t sr_index0)
{
    if (lamb && n > 0 && ratios == NULL) return OR_ERR_ARG;
    int rc = compress_core(n, K, off, g, g_is_bf16, err_store, err_fmt, m, v, p, words, scales, signs,
                           nonfinite, lr, beta1, eps, clip, ef_mode, ef_beta, !lamb, 1, sr_seed, sr_step,
                           sr_index0);
    if (rc != OR_OK || n == 0 || !lamb) return rc;
    lamb_update(K, off, m, v, p, ratios, lr, eps, 1.0, 1.0);
    return OR_OK;
}

/* ---------- R19: the worker's step split at the exchange ---------- */

/* (a) compensate, scale, pack, error with the worker's own g_hat; m, v, p are not part of it. */
int or_worker_compress(int64_t n, int64_t K, const int64_t* off, const void* g, int g_is_bf16,
                       void* err_store, int err_fmt, uint32_t* words, float* scales, int8_t* signs,
                       int64_t* nonfinite, float clip, int ef_mode, float ef_beta,
                       int stochastic, uint64_t sr_seed, uint64_t sr_step, int64_t sr_index0)
{
    if (stochastic && err_fmt == OR_FMT_F32) return OR_ERR_ARG;
    if (!check_offsets(n, K, off)) return OR_ERR_ARG;
    if (err_fmt != OR_FMT_F32 && err_fmt != OR_FMT_BF16 && err_fmt != OR_FMT_F16) return OR_ERR_ARG;
    if (n == 0) return OR_OK;
    if (!g || !err_store || !words || !scales) return OR_ERR_ARG;
    float* x = (float*)calloc((size_t)n, sizeof(float));
    float* err = (float*)calloc((size_t)n, sizeof(float));
    if (x == NULL || err == NULL) {
        free(x);
        free(err);
        return OR_ERR_OOM;
    }
    for (int64_t i = 0; i < n; ++i) err[i] = load_err(err_store, err_fmt, i);
    /* x: the gradient (clipped, R7) plus the stored error, an fp32 value (R4) */
    for (int64_t i = 0; i < n; ++i) {
        double gi = (double)load_grad(g, g_is_bf16, i);
        if (clip > 0.0f) {
            double c = (double)clip;
            if (gi > c)
                gi = c;
            else if (gi < -c)
                gi = -c;
        }
        x[i] = (float)(gi + (double)err[i]);
    }
    /* R1 scales and R2/R3 sign bits of x */
    for (int64_t c = 0; c < K; ++c) scales[c] = or_chunk_scale(x, off[c], off[c + 1]);
    or_pack(x, 0, n, words);
    /* R6 with the value the worker's own bits stand for (R10), plain or EMA */
    const double eb = (double)ef_beta;
    for (int64_t c = 0; c < K; ++c) {
        for (int64_t i = off[c]; i < off[c + 1]; ++i) {
            int b = sign_bit(x[i]);
            float gh = b ? scales[c] : -scales[c];
            float delta = (float)((double)x[i] - (double)gh);
            err[i] = ef_mode == 1 ? (float)(eb * (double)err[i] + (1.0 - eb) * (double)delta) : delta;
            if (signs != NULL) signs[i] = (int8_t)(b ? 1 : -1);
        }
    }
    for (int64_t i = 0; i < n; ++i) {
        float stored = stochastic ? store_err_sr(err_store, err_fmt, i, err[i],
                                                 sr_bits(sr_seed, sr_step, sr_index0 + i))
                                  : store_err(err_store, err_fmt, i, err[i]);
        if (nonfinite != NULL && !isfinite(stored)) *nonfinite += 1;
    }
    free(x);
    free(err);
    return OR_OK;
}

/* (b) the values the exchanged words and scales stand for, then m and the frozen-v update. */
int or_worker_update(int64_t n, int64_t K, const int64_t* off, const uint32_t* words, const float* scales,
                     float* m, const float* v, float* p, float lr, float beta1, float eps)
{
    if (!check_offsets(n, K, off)) return OR_ERR_ARG;
    if (n == 0) return OR_OK;
    if (!words || !scales || !m || !v || !p) return OR_ERR_ARG;
    const double b1 = (double)beta1;
    for (int64_t c = 0; c < K; ++c) {
        for (int64_t i = off[c]; i < off[c + 1]; ++i) {
            float ghat = word_bit(words, i) ? scales[c] : -scales[c];
            m[i] = (float)(b1 * (double)m[i] + (1.0 - b1) * (double)ghat);
            p[i] = (float)((double)p[i] - (double)lr * ((double)m[i] / (sqrt((double)v[i]) + (double)eps)));
        }
    }
    return OR_OK;
}

/* (b) for 1-bit LAMB (R16): g_hat from the exchanged words and scales, m on it, then the layer-wise
 * trust ratio on the reconstructed direction and the update (v frozen). */
int or_lamb_worker_update(int64_t n, int64_t K, const int64_t* off, const uint32_t* words, const float* scales,
                          float* m, const float* v, float* p, float* ratios, float lr, float beta1, float eps)
{
    if (!check_offsets(n, K, off)) return OR_ERR_ARG;
    if (n == 0) return OR_OK;
    if (!words || !scales || !m || !v || !p || !ratios) return OR_ERR_ARG;
    const double b1 = (double)beta1;
    for (int64_t c = 0; c < K; ++c) {
        for (int64_t i = off[c]; i < off[c + 1]; ++i) {
            float gl = word_bit(words, i) ? scales[c] : -scales[c];
            m[i] = (float)(b1 * (double)m[i] + (1.0 - b1) * (double)gl);
        }
    }
    lamb_update(K, off, m, v, p, ratios, lr, eps, 1.0, 1.0);
    return OR_OK;
}

/* ---------- server half of the compressed allreduce on one GPU's share ([P2] compressed_allreduce) ----
 * worker_words: W rows of ceil(n/32) words; worker_scales: W rows of K scales.  R9. */
int or_server_reduce(int64_t n, int64_t K, const int64_t* off, int W,
                     const uint32_t* worker_words, const float* worker_scales,
                     float* server_err, uint32_t* words_out, float* scales_out)
{
    if (!check_offsets(n, K, off) || W < 1) return OR_ERR_ARG;
    if (n == 0) return OR_OK;
    if (!worker_words || !worker_scales || !server_err || !words_out || !scales_out) return OR_ERR_ARG;
    const int64_t nw = (n + 31) / 32;
    float* x = (float*)calloc((size_t)n, sizeof(float));
    if (x == NULL) return OR_ERR_OOM;

    for (int64_t c = 0; c < K; ++c) {
        for (int64_t i = off[c]; i < off[c + 1]; ++i) {
            double a = 0.0;
            for (int w = 0; w < W; ++w) {
                double s = (double)worker_scales[(int64_t)w * K + c];
                a += word_bit(worker_words + (int64_t)w * nw, i) ? s : -s;
            }
            float avg = (float)(a / (double)W);
            x[i] = (float)((double)avg + (double)server_err[i]);
        }
    }
    for (int64_t c = 0; c < K; ++c)
        scales_out[c] = or_chunk_scale(x, off[c], off[c + 1]);
    or_pack(x, 0, n, words_out);
    for (int64_t c = 0; c < K; ++c) {
        for (int64_t i = off[c]; i < off[c + 1]; ++i) {
            float gh = sign_bit(x[i]) ? scales_out[c] : -scales_out[c];
            server_err[i] = (float)((double)x[i] - (double)gh);
        }
    }
    free(x);
    return OR_OK;
}

/* Per-element server average alone (for checking the exact-average reading R9 by itself). */
int or_server_average(int64_t n, int64_t K, const int64_t* off, int W,
                      const uint32_t* worker_words, const float* worker_scales, float* avg_out)
{
    if (!check_offsets(n, K, off) || W < 1) return OR_ERR_ARG;
    const int64_t nw = (n + 31) / 32;
    for (int64_t c = 0; c < K; ++c) {
        for (int64_t i = off[c]; i < off[c + 1]; ++i) {
            double a = 0.0;
            for (int w = 0; w < W; ++w) {
                double s = (double)worker_scales[(int64_t)w * K + c];
                a += word_bit(worker_words + (int64_t)w * nw, i) ? s : -s;
            }
            avg_out[i] = (float)(a / (double)W);
        }
    }
    return OR_OK;
}

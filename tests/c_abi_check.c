/*
 * c_abi_check.c -- drives libobadam.so through its C ABI from plain C: device buffers from the HIP
 * runtime, no Python and no torch.  Runs two hand-derived worked examples (exact dyadic values, so
 * every output is compared for equality) and a few error paths, and prints "c_abi_check ok".
 *
 * Worked examples (derivations in tests/golden/worked_examples.json):
 *   compressed step, one chunk of 4 ("DeepSpeed Communication Compression and Hiding", section
 *     "1-bit Adam: warmup, frozen variance, error feedback", compressed branch): x = g = [3,-4,0,12],
 *     scale = sqrt(169/4) = 6.5, word 0b1101, err = x - g_hat, m = 0.5 m + 0.5 g_hat,
 *     p -= 0.5 m / (sqrt(v) + 1);
 *   dense step (same page, section "baseline: why Adam is hard to compress"): m = 0.5 g,
 *     v = 0.25 g^2, p = 1 - 0.5 m / sqrt(v);
 *   server reduce, two workers (same page, 1-bit Adam, compressed_allreduce): words 0b0011 and
 *     0b0101 with scales 0.5 and 1.5 average to [1, -0.5, 0.5, -1]; plus the server error
 *     [1, 0.5, -2.5, 0] gives x = [2, 0, -2, -1], scale sqrt(9/4) = 1.5, word 0b0011 and the new
 *     server error x - g_hat = [0.5, -1.5, -0.5, 0.5]; its unpack is [1.5, 1.5, -1.5, -1.5];
 *   pack (the sign part of one_bit_quantize; bit j of word w is element 32w + j, 1 for +1, and
 *     sign(+-0) = +1, sign(NaN) = -1): [1, -1, 0, -0] -> 13 (fp32 and bf16 input),
 *     [NaN, Inf, -Inf, -1e-45] -> 2, 33 elements of -1 with x[32] = 1 -> [0, 1], 64 elements of 1
 *     with x[0] = x[31] = x[63] = -1 -> [0x7FFFFFFE, 0x7FFFFFFF].
 */
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "ob_adam.h"

#define CHECK_HIP(x)                                                                  \
    do {                                                                              \
        hipError_t e_ = (x);                                                          \
        if (e_ != hipSuccess) {                                                       \
            fprintf(stderr, "HIP error %d at line %d\n", (int)e_, __LINE__);          \
            return 1;                                                                 \
        }                                                                             \
    } while (0)
#define CHECK_OB(x)                                                                   \
    do {                                                                              \
        ob_status s_ = (x);                                                           \
        if (s_ != OB_OK) {                                                            \
            fprintf(stderr, "ob error %s at line %d\n", ob_status_str(s_), __LINE__); \
            return 1;                                                                 \
        }                                                                             \
    } while (0)

static int same(const char* what, const float* got, const float* want, int n)
{
    for (int i = 0; i < n; ++i)
        if (got[i] != want[i]) {
            fprintf(stderr, "%s[%d] = %.9g, expected %.9g\n", what, i, got[i], want[i]);
            return 0;
        }
    return 1;
}

int main(void)
{
    enum { N = 4 };
    float *g, *err, *m, *v, *p, *scales, *out;
    uint32_t* words;
    int8_t* signs;
    CHECK_HIP(hipSetDevice(0));
    CHECK_HIP(hipMalloc((void**)&g, N * sizeof(float)));
    CHECK_HIP(hipMalloc((void**)&err, N * sizeof(float)));
    CHECK_HIP(hipMalloc((void**)&m, N * sizeof(float)));
    CHECK_HIP(hipMalloc((void**)&v, N * sizeof(float)));
    CHECK_HIP(hipMalloc((void**)&p, N * sizeof(float)));
    CHECK_HIP(hipMalloc((void**)&out, N * sizeof(float)));
    CHECK_HIP(hipMalloc((void**)&scales, sizeof(float)));
    CHECK_HIP(hipMalloc((void**)&words, sizeof(uint32_t)));
    CHECK_HIP(hipMalloc((void**)&signs, N));

    ob_plan plan = NULL;
    CHECK_OB(ob_plan_create(N, N, NULL, 0, &plan));
    if (ob_plan_num_chunks(plan) != 1 || ob_plan_num_elements(plan) != N) return 1;

    /* compressed step */
    const float g0[N] = {3, -4, 0, 12}, z[N] = {0, 0, 0, 0}, m0[N] = {1, 1, -1, 0}, v0[N] = {9, 9, 49, 1},
                p0[N] = {0, 1, 2, 3};
    CHECK_HIP(hipMemcpy(g, g0, sizeof g0, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(err, z, sizeof z, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(m, m0, sizeof m0, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(v, v0, sizeof v0, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(p, p0, sizeof p0, hipMemcpyHostToDevice));
    ob_hparams hp;
    memset(&hp, 0, sizeof hp);
    hp.lr = 0.5f;
    hp.beta1 = 0.5f;
    hp.beta2 = 0.999f;
    hp.eps = 1.0f;
    hp.ef_mode = OB_EF_PLAIN;
    CHECK_OB(ob_adam_compress_step(plan, g, OB_F32, err, OB_F32, m, v, p, words, scales, signs, NULL, &hp,
                                   NULL));
    CHECK_HIP(hipDeviceSynchronize());
    float he[N], hm[N], hv[N], hpp[N], hs, ho[N];
    uint32_t hw;
    int8_t hsg[N];
    CHECK_HIP(hipMemcpy(he, err, sizeof he, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(hm, m, sizeof hm, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(hv, v, sizeof hv, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(hpp, p, sizeof hpp, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(&hs, scales, sizeof hs, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(&hw, words, sizeof hw, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(hsg, signs, sizeof hsg, hipMemcpyDeviceToHost));
    const float want_e[N] = {-3.5f, 2.5f, -6.5f, 5.5f}, want_m[N] = {3.75f, -2.75f, 2.75f, 3.25f},
                want_p[N] = {-0.46875f, 1.34375f, 1.828125f, 2.1875f};
    const int8_t want_s[N] = {1, -1, 1, 1};
    if (hw != 13u || hs != 6.5f || memcmp(hsg, want_s, N) != 0) {
        fprintf(stderr, "word %u scale %.9g\n", hw, hs);
        return 1;
    }
    if (!same("err", he, want_e, N) || !same("m", hm, want_m, N) || !same("p", hpp, want_p, N) ||
        !same("v", hv, v0, N))
        return 1;

    /* unpack of the step's words with its scale */
    CHECK_OB(ob_unpack(plan, words, N, scales, out, NULL));
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_HIP(hipMemcpy(ho, out, sizeof ho, hipMemcpyDeviceToHost));
    const float want_o[N] = {6.5f, -6.5f, 6.5f, 6.5f};
    if (!same("unpack", ho, want_o, N)) return 1;

    /* the same step split at the exchange, with one worker: the same results */
    CHECK_HIP(hipMemcpy(err, z, sizeof z, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(m, m0, sizeof m0, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(p, p0, sizeof p0, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemset(words, 0, sizeof(uint32_t)));
    CHECK_HIP(hipMemset(scales, 0, sizeof(float)));
    CHECK_OB(ob_adam_worker_compress(plan, g, OB_F32, err, OB_F32, words, scales, signs, NULL, &hp, NULL));
    CHECK_OB(ob_adam_worker_update(plan, words, scales, m, v, p, &hp, NULL));
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_HIP(hipMemcpy(he, err, sizeof he, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(hm, m, sizeof hm, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(hpp, p, sizeof hpp, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(&hs, scales, sizeof hs, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(&hw, words, sizeof hw, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(hsg, signs, sizeof hsg, hipMemcpyDeviceToHost));
    if (hw != 13u || hs != 6.5f || memcmp(hsg, want_s, N) != 0) {
        fprintf(stderr, "split: word %u scale %.9g\n", hw, hs);
        return 1;
    }
    if (!same("split err", he, want_e, N) || !same("split m", hm, want_m, N) || !same("split p", hpp, want_p, N))
        return 1;

    /* dense step */
    const float gd[N] = {2, -2, 0.5f, -4}, ones[N] = {1, 1, 1, 1};
    CHECK_HIP(hipMemcpy(g, gd, sizeof gd, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(m, z, sizeof z, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(v, z, sizeof z, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(p, ones, sizeof ones, hipMemcpyHostToDevice));
    hp.beta2 = 0.75f;
    hp.eps = 0.0f;
    CHECK_OB(ob_adam_warmup_step(plan, g, OB_F32, m, v, p, &hp, NULL));
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_HIP(hipMemcpy(hm, m, sizeof hm, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(hv, v, sizeof hv, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(hpp, p, sizeof hpp, hipMemcpyDeviceToHost));
    const float dm[N] = {1, -1, 0.25f, -2}, dv[N] = {1, 1, 0.0625f, 4}, dp[N] = {0.5f, 1.5f, 0.5f, 1.5f};
    if (!same("dense m", hm, dm, N) || !same("dense v", hv, dv, N) || !same("dense p", hpp, dp, N)) return 1;

    /* server reduce over two workers, then the unpack of its words and scale */
    {
        uint32_t *ww, *wo;
        float *wsc, *esrv, *so, *uo;
        const uint32_t hww[2] = {3u, 5u};
        const float hws[2] = {0.5f, 1.5f}, he0[N] = {1.0f, 0.5f, -2.5f, 0.0f};
        CHECK_HIP(hipMalloc((void**)&ww, sizeof hww));
        CHECK_HIP(hipMalloc((void**)&wsc, sizeof hws));
        CHECK_HIP(hipMalloc((void**)&esrv, sizeof he0));
        CHECK_HIP(hipMalloc((void**)&wo, sizeof(uint32_t)));
        CHECK_HIP(hipMalloc((void**)&so, sizeof(float)));
        CHECK_HIP(hipMalloc((void**)&uo, N * sizeof(float)));
        CHECK_HIP(hipMemcpy(ww, hww, sizeof hww, hipMemcpyHostToDevice));
        CHECK_HIP(hipMemcpy(wsc, hws, sizeof hws, hipMemcpyHostToDevice));
        CHECK_HIP(hipMemcpy(esrv, he0, sizeof he0, hipMemcpyHostToDevice));
        CHECK_OB(ob_server_reduce(plan, 2, ww, wsc, esrv, wo, so, NULL));
        CHECK_OB(ob_unpack(plan, wo, N, so, uo, NULL));
        CHECK_HIP(hipDeviceSynchronize());
        uint32_t hwo;
        float hso, heo[N], huo[N];
        CHECK_HIP(hipMemcpy(&hwo, wo, sizeof hwo, hipMemcpyDeviceToHost));
        CHECK_HIP(hipMemcpy(&hso, so, sizeof hso, hipMemcpyDeviceToHost));
        CHECK_HIP(hipMemcpy(heo, esrv, sizeof heo, hipMemcpyDeviceToHost));
        CHECK_HIP(hipMemcpy(huo, uo, sizeof huo, hipMemcpyDeviceToHost));
        const float want_se[N] = {0.5f, -1.5f, -0.5f, 0.5f}, want_uo[N] = {1.5f, 1.5f, -1.5f, -1.5f};
        if (hwo != 3u || hso != 1.5f) {
            fprintf(stderr, "server: word %u scale %.9g\n", hwo, hso);
            return 1;
        }
        if (!same("server err", heo, want_se, N) || !same("server unpack", huo, want_uo, N)) return 1;
        if (ob_server_reduce(plan, 0, ww, wsc, esrv, wo, so, NULL) != OB_ERR_ARG) return 1;   /* W = 0 */
        hipFree(ww);
        hipFree(wsc);
        hipFree(esrv);
        hipFree(wo);
        hipFree(so);
        hipFree(uo);
    }

    /* pack: fp32 and bf16 inputs, zeros, NaN, Inf, a negative denormal, a 33- and a 64-element case */
    {
        enum { M = 64 };
        float* x;
        uint16_t* xb;
        uint32_t* pw;
        CHECK_HIP(hipMalloc((void**)&x, M * sizeof(float)));
        CHECK_HIP(hipMalloc((void**)&xb, M * sizeof(uint16_t)));
        CHECK_HIP(hipMalloc((void**)&pw, 2 * sizeof(uint32_t)));
        float hx[M];
        uint32_t hpw[2];
        const float c1[4] = {1.0f, -1.0f, 0.0f, -0.0f}, c2[4] = {NAN, INFINITY, -INFINITY, -1e-45f};
        const uint16_t c1b[4] = {0x3F80u, 0xBF80u, 0x0000u, 0x8000u};
        CHECK_HIP(hipMemcpy(x, c1, sizeof c1, hipMemcpyHostToDevice));
        CHECK_OB(ob_pack(x, OB_F32, 4, pw, NULL));
        CHECK_HIP(hipMemcpy(hpw, pw, sizeof(uint32_t), hipMemcpyDeviceToHost));
        if (hpw[0] != 13u) return fprintf(stderr, "pack [1,-1,0,-0] = %u\n", hpw[0]), 1;
        CHECK_HIP(hipMemcpy(xb, c1b, sizeof c1b, hipMemcpyHostToDevice));
        CHECK_OB(ob_pack(xb, OB_BF16, 4, pw, NULL));
        CHECK_HIP(hipMemcpy(hpw, pw, sizeof(uint32_t), hipMemcpyDeviceToHost));
        if (hpw[0] != 13u) return fprintf(stderr, "pack bf16 [1,-1,0,-0] = %u\n", hpw[0]), 1;
        CHECK_HIP(hipMemcpy(x, c2, sizeof c2, hipMemcpyHostToDevice));
        CHECK_OB(ob_pack(x, OB_F32, 4, pw, NULL));
        CHECK_HIP(hipMemcpy(hpw, pw, sizeof(uint32_t), hipMemcpyDeviceToHost));
        if (hpw[0] != 2u) return fprintf(stderr, "pack [NaN,Inf,-Inf,-1e-45] = %u\n", hpw[0]), 1;
        for (int i = 0; i < 33; ++i) hx[i] = -1.0f;
        hx[32] = 1.0f;
        CHECK_HIP(hipMemcpy(x, hx, 33 * sizeof(float), hipMemcpyHostToDevice));
        CHECK_OB(ob_pack(x, OB_F32, 33, pw, NULL));
        CHECK_HIP(hipMemcpy(hpw, pw, 2 * sizeof(uint32_t), hipMemcpyDeviceToHost));
        if (hpw[0] != 0u || hpw[1] != 1u) return fprintf(stderr, "pack n=33: %u %u\n", hpw[0], hpw[1]), 1;
        for (int i = 0; i < M; ++i) hx[i] = 1.0f;
        hx[0] = hx[31] = hx[63] = -1.0f;
        CHECK_HIP(hipMemcpy(x, hx, sizeof hx, hipMemcpyHostToDevice));
        CHECK_OB(ob_pack(x, OB_F32, M, pw, NULL));
        CHECK_HIP(hipMemcpy(hpw, pw, 2 * sizeof(uint32_t), hipMemcpyDeviceToHost));
        if (hpw[0] != 0x7FFFFFFEu || hpw[1] != 0x7FFFFFFFu)
            return fprintf(stderr, "pack n=64: %08x %08x\n", hpw[0], hpw[1]), 1;
        if (ob_pack(x, (ob_dtype)5, 4, pw, NULL) != OB_ERR_DTYPE) return 1;
        if (ob_pack((const float*)((const char*)x + 4), OB_F32, 4, pw, NULL) != OB_ERR_ALIGN) return 1;
        hipFree(x);
        hipFree(xb);
        hipFree(pw);
    }

    /* error paths: rejected on the host, nothing enqueued */
    if (ob_adam_compress_step(NULL, g, OB_F32, err, OB_F32, m, v, p, words, scales, NULL, NULL, &hp, NULL) !=
        OB_ERR_ARG)
        return 1;
    if (ob_adam_compress_step(plan, g, OB_F32, err, (ob_dtype)7, m, v, p, words, scales, NULL, NULL, &hp,
                              NULL) != OB_ERR_DTYPE)
        return 1;
    if (ob_adam_compress_step(plan, g, OB_F32, err, OB_F32, (float*)((char*)m + 4), v, p, words, scales, NULL,
                              NULL, &hp, NULL) != OB_ERR_ALIGN)
        return 1;
    if (strcmp(ob_status_str(OB_ERR_ALIGN), "misaligned pointer or chunk boundary") != 0) return 1;

    CHECK_OB(ob_plan_destroy(plan));
    hipFree(g);
    hipFree(err);
    hipFree(m);
    hipFree(v);
    hipFree(p);
    hipFree(out);
    hipFree(scales);
    hipFree(words);
    hipFree(signs);
    printf("c_abi_check ok\n");
    return 0;
}

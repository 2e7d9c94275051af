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
 *     v = 0.25 g^2, p = 1 - 0.5 m / sqrt(v).
 */
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

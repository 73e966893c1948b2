/* Host-side driver for a sanitizer build of the C ABI (api.hip built with
 * AddressSanitizer and UndefinedBehaviorSanitizer on the host side). It calls
 * only the entry points that never reach the GPU: plan creation with valid,
 * invalid and tuned arguments, query, describe (into short and long
 * buffers), the dispatch table, the workspace and packed-filter queries, the
 * string functions, argument errors of run/train_run/layout/bn_fold that are
 * rejected before any launch, and destroy. Exit status 0 when every call
 * returned what is expected; the sanitizers abort on the first memory or
 * undefined-behaviour error. */
#include <stdio.h>
#include <string.h>

#include "tg_conv_bn_silu.h"

static int failures = 0;
#define EXPECT(cond)                                                   \
    do {                                                               \
        if (!(cond)) {                                                 \
            fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                \
        }                                                              \
    } while (0)

static const int shapes[][9] = {
    {32, 56, 56, 64, 256, 1, 1, 1, 0}, {32, 28, 28, 128, 128, 3, 3, 1, 1},
    {64, 224, 224, 3, 16, 3, 3, 2, 1}, {64, 224, 224, 3, 24, 3, 3, 2, 1},
    {16, 56, 56, 64, 64, 7, 7, 1, 3},  {1, 16, 16, 3, 8, 3, 3, 1, 1},
    {2, 9, 9, 8, 1, 3, 3, 1, 1},       {1, 1, 1, 8, 16, 3, 3, 1, 1},
    {3, 17, 13, 16, 33, 3, 3, 3, 2},   {1, 6, 6, 16, 320, 1, 1, 1, 0},
    {1, 9, 10, 256, 96, 5, 5, 1, 2},   {2, 8, 9, 3, 5, 2, 3, 2, 1},
};

int main(void) {
    const int nshapes = (int)(sizeof(shapes) / sizeof(shapes[0]));
    const tg_kernel kernels[] = {TG_KERNEL_AUTO, TG_KERNEL_SCALAR, TG_KERNEL_TILED,
                                 TG_KERNEL_IGEMM, TG_KERNEL_AUTO | TG_UNFUSED,
                                 TG_KERNEL_AUTO | TG_SPLIT};
    char buf[512], tiny[7];
    for (int i = 0; i < nshapes; ++i) {
        const int *s = shapes[i];
        for (int dt = 0; dt < 2; ++dt)
            for (int k = 0; k < 6; ++k) {
                tg_conv_bn_silu_plan *p = NULL;
                tg_status st = tg_conv_bn_silu_create(&p, s[0], s[1], s[2], s[3], s[4], s[5],
                                                      s[6], s[7], s[8], (tg_dtype)dt, kernels[k]);
                if (st != TG_OK) {
                    EXPECT(p == NULL);
                    continue;
                }
                int P = 0, Q = 0;
                tg_kernel chosen;
                size_t ws = 0, tws = 0, pk = 0;
                EXPECT(tg_conv_bn_silu_query(p, &P, &Q, &chosen, &ws) == TG_OK);
                EXPECT(P >= 1 && Q >= 1);
                EXPECT(tg_conv_bn_silu_describe(p, buf, sizeof(buf)) == TG_OK);
                EXPECT(strlen(buf) < sizeof(buf));
                EXPECT(tg_conv_bn_silu_describe(p, tiny, sizeof(tiny)) == TG_OK);
                EXPECT(strlen(tiny) == sizeof(tiny) - 1);
                EXPECT(tg_conv_bn_silu_train_workspace(p, &tws) == TG_OK && tws > 0);
                st = tg_conv_bn_silu_packed_filter_bytes(p, &pk);
                EXPECT(st == TG_OK || (st == TG_ERR_UNSUPPORTED && pk == 0));
                EXPECT(strlen(tg_kernel_name(chosen)) > 0);
                /* Argument errors: rejected before any launch. */
                EXPECT(tg_conv_bn_silu_run(p, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) ==
                       TG_ERR_INVALID_ARGUMENT);
                EXPECT(tg_conv_bn_silu_train_run(p, NULL, NULL, NULL, NULL, 1e-5f, 0.1f, NULL,
                                                 NULL, NULL, NULL, NULL, NULL, 0,
                                                 NULL) == TG_ERR_INVALID_ARGUMENT);
                EXPECT(tg_conv_bn_silu_destroy(p) == TG_OK);
            }
        tg_kernel ch;
        EXPECT(tg_dispatch_choose(s[0], s[1], s[2], s[3], s[4], s[5], s[6], s[7], s[8], TG_F16,
                                  TG_DISPATCH_PAGES, &ch) == TG_OK);
    }
    /* Tuning text: good, bad, and every key. */
    const char *good[] = {NULL, "", "cu=2,cu_pd=1", "cu=0", "igemm_rw=0,patch_cfg=3",
                          "stem=0,tm_pipe=0,tm_rows=4", "stream=8,xdma=2,nt=0",
                          "igemm_patch=0,dma_cfg=5", "igemm_cfg=1", "rw_nf=8,rw_cs=2,rw_ncw=4",
                          "rw_wg_per_cu=2", "stem=2,stem_rows=3", "tiled_mfma=0",
                          "tm_wg_per_cu=2"};
    const char *bad[] = {"bogus=1", "cu", "cu=", "cu=x", "cu=2,", "=3", "cu=99999999",
                         "cu=2,,cu_pd=1", "cu_pd=9", " cu=2"};
    for (size_t i = 0; i < sizeof(good) / sizeof(good[0]); ++i)
        for (int j = 0; j < nshapes; ++j) {
            const int *s = shapes[j];
            tg_conv_bn_silu_plan *p = NULL;
            tg_status st = tg_conv_bn_silu_create_tuned(&p, s[0], s[1], s[2], s[3], s[4], s[5],
                                                        s[6], s[7], s[8], TG_F16, TG_KERNEL_AUTO,
                                                        TG_ACT_SILU, TG_F16, good[i]);
            EXPECT(st == TG_OK || st == TG_ERR_UNSUPPORTED);
            if (st == TG_OK) {
                EXPECT(tg_conv_bn_silu_describe(p, buf, sizeof(buf)) == TG_OK);
                tg_conv_bn_silu_destroy(p);
            }
        }
    for (size_t i = 0; i < sizeof(bad) / sizeof(bad[0]); ++i) {
        tg_conv_bn_silu_plan *p = (tg_conv_bn_silu_plan *)1;
        EXPECT(tg_conv_bn_silu_create_tuned(&p, 1, 8, 8, 64, 64, 1, 1, 1, 0, TG_F16,
                                            TG_KERNEL_AUTO, TG_ACT_SILU, TG_F16,
                                            bad[i]) == TG_ERR_INVALID_ARGUMENT);
        EXPECT(p == NULL);
    }
    /* Invalid and oversized shapes. */
    tg_conv_bn_silu_plan *p = NULL;
    EXPECT(tg_conv_bn_silu_create(&p, 0, 8, 8, 3, 4, 3, 3, 1, 1, TG_F16, TG_KERNEL_AUTO) ==
           TG_ERR_INVALID_ARGUMENT);
    EXPECT(tg_conv_bn_silu_create(&p, 2048, 1024, 1024, 1, 1, 1, 1, 1, 0, TG_F16,
                                  TG_KERNEL_AUTO) == TG_ERR_UNSUPPORTED);
    EXPECT(tg_conv_bn_silu_create(NULL, 1, 8, 8, 3, 4, 3, 3, 1, 1, TG_F16, TG_KERNEL_AUTO) ==
           TG_ERR_INVALID_ARGUMENT);
    EXPECT(tg_conv_bn_silu_destroy(NULL) == TG_OK);
    EXPECT(tg_bn_fold(NULL, NULL, NULL, NULL, 1e-5f, 4, NULL, NULL, NULL) ==
           TG_ERR_INVALID_ARGUMENT);
    EXPECT(tg_nchw_to_nhwc(NULL, NULL, 1, 1, 1, 1, TG_F16, NULL) == TG_ERR_INVALID_ARGUMENT);
    for (int s = -1; s < 8; ++s) EXPECT(strlen(tg_status_string((tg_status)s)) > 0);
    for (int k = 0; k < 0x400; ++k) EXPECT(tg_kernel_name((tg_kernel)k) != NULL);
    printf("abi_driver: %d failures\n", failures);
    return failures == 0 ? 0 : 1;
}

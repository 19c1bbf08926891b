/* Host logic of libswiglu under AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_sanitize.py builds the library with the sanitizers on its host
 * code): every size query and the planners behind them over all dtypes,
 * paths and a spread of shapes up to the limits, and every entry point with
 * arguments that each validation branch rejects.  No call here passes
 * validation, so nothing reaches a HIP launch and the program needs no GPU.
 * Prints "abi_sanitize ok" when every result meets the header's contract. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "swiglu.h"

static int failures = 0;
#define CHECK(c)                                                              \
    do {                                                                      \
        if (!(c)) {                                                           \
            if (failures++ < 20)                                              \
                fprintf(stderr, "line %d: check failed: %s\n", __LINE__, #c); \
        }                                                                     \
    } while (0)

#define MAX_M ((int64_t)1 << 18)
#define MAX_DIM ((int64_t)1 << 20)

int main(void)
{
    static const int64_t Ms[] = {0, 1, 2, 3, 4, 5, 8, 9, 16, 17, 32, 33, 48, 64, 65, 80, 128,
                                 129, 256, 300, 1024, 2048, 4096, 32768, MAX_M, MAX_M + 1, -1};
    static const int64_t dims[] = {8, 16, 24, 64, 72, 128, 136, 1000, 1024, 4096, 8192, 14336,
                                   29568, MAX_DIM, MAX_DIM + 8, 0, -8, 12};
    static const int dtypes[] = {SWIGLU_F32, SWIGLU_BF16, SWIGLU_BF16_FP8W, SWIGLU_BF16_MXFP4W,
                                 7, -1};
    static const int paths[] = {SWIGLU_PATH_AUTO, SWIGLU_PATH_SKINNY, SWIGLU_PATH_WIDE,
                                SWIGLU_PATH_WIDE_PHASED, SWIGLU_PATH_FUSED_DOWN, 9};
    const int nM = sizeof Ms / sizeof Ms[0], nD = sizeof dims / sizeof dims[0];
    const int nT = sizeof dtypes / sizeof dtypes[0], nP = sizeof paths / sizeof paths[0];
    long queries = 0;

    for (int t = 0; t < nT; ++t) {
        const int dt = dtypes[t];
        const int known = dt >= SWIGLU_F32 && dt <= SWIGLU_BF16_MXFP4W;
        for (int i = 0; i < nD; ++i) {
            for (int j = 0; j < nD; ++j) {
                const int64_t d = dims[i], dff = dims[j];
                const int ve = dt == SWIGLU_F32 ? 4 : 8;   /* 16-byte activation vectors */
                const int dims_ok = known && d > 0 && dff > 0 && d <= MAX_DIM && dff <= MAX_DIM &&
                                    d % ve == 0 && dff % ve == 0;
                const size_t pb = swiglu_packed_bytes(d, dff, dt);
                const size_t pdb = swiglu_down_packed_bytes(d, dff, dt);
                /* two matrices of d x dff at the storage width, at least */
                const double wbytes = dt == SWIGLU_F32 ? 4 : dt == SWIGLU_BF16 ? 2
                                      : dt == SWIGLU_BF16_FP8W ? 1 : 0.5;
                CHECK(dims_ok ? pb >= 2 * wbytes * (double)d * (double)dff : pb == 0);
                CHECK(dims_ok ? pdb >= wbytes * (double)d * (double)dff : pdb == 0);
                for (int m = 0; m < nM; ++m) {
                    const int64_t M = Ms[m];
                    const int ok = dims_ok && M >= 0 && M <= MAX_M;
                    const int sel = swiglu_select_path(M, d, dff, dt);
                    CHECK(ok ? (sel == SWIGLU_PATH_SKINNY || sel == SWIGLU_PATH_WIDE) : sel < 0);
                    if (ok && dt != SWIGLU_BF16)
                        CHECK(sel == SWIGLU_PATH_SKINNY);
                    if (ok && M <= 64)
                        CHECK(sel == SWIGLU_PATH_SKINNY);
                    for (int p = 0; p < nP; ++p) {
                        const int path = paths[p];
                        for (int down = 0; down <= 1; ++down) {
                            const size_t w =
                                swiglu_workspace_bytes_ex(M, d, dff, dt, down, path);
                            CHECK(w % 256 == 0);
                            if (!ok || M == 0 || path == 9)
                                CHECK(w == 0);
                            /* the MLP keeps h in the workspace: never empty */
                            if (ok && M > 0 && down && path == SWIGLU_PATH_AUTO)
                                CHECK(w >= (size_t)M * (size_t)dff);
                            ++queries;
                        }
                        const size_t b = mlp_block_workspace_bytes_ex(M, d, dff, dt, path);
                        const size_t mw = swiglu_workspace_bytes_ex(M, d, dff, dt, 1, path);
                        CHECK(b % 256 == 0 && b >= mw);
                        ++queries;
                    }
                    CHECK(swiglu_workspace_bytes(M, d, dff, dt, 0) ==
                          swiglu_workspace_bytes_ex(M, d, dff, dt, 0, SWIGLU_PATH_AUTO));
                    CHECK(mlp_block_workspace_bytes(M, d, dff, dt) ==
                          mlp_block_workspace_bytes_ex(M, d, dff, dt, SWIGLU_PATH_AUTO));
                }
            }
        }
    }

    /* every entry point, rejected by each kind of check before any launch */
    void *fake = (void *)(uintptr_t)0x10000000u;   /* aligned, never dereferenced */
    void *odd = (char *)fake + 8;
    swiglu_graph_t g = NULL;
    for (int s = -8; s <= 2; ++s)
        CHECK(swiglu_status_string(s) != NULL && strlen(swiglu_status_string(s)) > 0);
    CHECK(swiglu_pack_weights(NULL, fake, fake, 64, 64, SWIGLU_BF16, NULL) ==
          SWIGLU_ERR_INVALID_ARG);
    CHECK(swiglu_pack_weights(fake, odd, fake, 64, 64, SWIGLU_BF16, NULL) ==
          SWIGLU_ERR_MISALIGNED);
    CHECK(swiglu_pack_weights(fake, fake, fake, 64, 64, 7, NULL) == SWIGLU_ERR_UNSUPPORTED);
    CHECK(swiglu_pack_down(fake, NULL, 64, 64, SWIGLU_BF16, NULL) == SWIGLU_ERR_INVALID_ARG);
    CHECK(swiglu_pack_down(odd, fake, 64, 64, SWIGLU_BF16, NULL) == SWIGLU_ERR_MISALIGNED);
    CHECK(swiglu_pack_down(fake, fake, 64, MAX_DIM + 8, SWIGLU_BF16, NULL) ==
          SWIGLU_ERR_UNSUPPORTED);
    CHECK(swiglu_up(fake, NULL, fake, 4, 64, 64, SWIGLU_BF16, NULL, 0, NULL) ==
          SWIGLU_ERR_INVALID_ARG);
    CHECK(swiglu_up(fake, fake, fake, 4, 64, 64, SWIGLU_BF16, odd, 1 << 20, NULL) ==
          SWIGLU_ERR_MISALIGNED);
    CHECK(swiglu_up(fake, fake, fake, MAX_M + 1, 64, 64, SWIGLU_BF16, NULL, 0, NULL) ==
          SWIGLU_ERR_UNSUPPORTED);
    CHECK(swiglu_up(fake, fake, fake, 4, 60, 64, SWIGLU_BF16, NULL, 0, NULL) ==
          SWIGLU_ERR_UNSUPPORTED);
    CHECK(swiglu_up_ex(fake, fake, fake, 4, 64, 64, SWIGLU_BF16, NULL, 0, NULL, 9) ==
          SWIGLU_ERR_UNSUPPORTED);
    CHECK(swiglu_up_ex(fake, fake, fake, 4, 64, 64, SWIGLU_BF16_FP8W, NULL, 0, NULL,
                       SWIGLU_PATH_WIDE_PHASED) == SWIGLU_ERR_UNSUPPORTED);
    CHECK(swiglu_up_ex(fake, fake, fake, 4, 64, 64, SWIGLU_BF16, NULL, 0, NULL,
                       SWIGLU_PATH_FUSED_DOWN) == SWIGLU_ERR_UNSUPPORTED);
    CHECK(swiglu_up_noalloc(NULL, fake, fake, 4, 64, 64, SWIGLU_BF16, NULL) ==
          SWIGLU_ERR_INVALID_ARG);
    CHECK(swiglu_up_noalloc(fake, fake, odd, 4, 64, 64, SWIGLU_BF16, NULL) ==
          SWIGLU_ERR_MISALIGNED);
    CHECK(swiglu_up_noalloc(fake, fake, fake, 4, 64, 64, -1, NULL) == SWIGLU_ERR_UNSUPPORTED);
    CHECK(swiglu_up_noalloc(fake, fake, fake, 0, 64, 64, SWIGLU_BF16, NULL) == SWIGLU_OK);
    CHECK(mlp_forward(fake, fake, fake, fake, 4, 64, 64, SWIGLU_BF16, NULL, 0, NULL) ==
          SWIGLU_ERR_INVALID_ARG);
    CHECK(mlp_forward(fake, fake, odd, fake, 4, 64, 64, SWIGLU_BF16, fake, 1 << 20, NULL) ==
          SWIGLU_ERR_MISALIGNED);
    CHECK(mlp_forward(fake, fake, fake, fake, 4, 64, 64, SWIGLU_BF16, fake, 256, NULL) ==
          SWIGLU_ERR_WORKSPACE);
    CHECK(mlp_forward_ex(fake, fake, fake, fake, 4, 64, 64, SWIGLU_F32, fake, 1 << 20, NULL,
                         SWIGLU_PATH_FUSED_DOWN) == SWIGLU_ERR_UNSUPPORTED);
    CHECK(mlp_forward_ex(fake, fake, fake, fake, 0, 64, 64, SWIGLU_BF16, NULL, 0, NULL,
                         SWIGLU_PATH_WIDE) == SWIGLU_OK);
    const float bad_eps[] = {-1.0f, 1.0f / 0.0f, 0.0f / 0.0f};
    for (int i = 0; i < 3; ++i)
        CHECK(mlp_block_forward(fake, fake, bad_eps[i], fake, fake, NULL, fake, 4, 64, 64,
                                SWIGLU_BF16, fake, 1 << 20, NULL) == SWIGLU_ERR_INVALID_ARG);
    CHECK(mlp_block_forward(fake, fake, 1e-6f, fake, fake, (char *)fake + 1, fake, 4, 64, 64,
                            SWIGLU_BF16, fake, 1 << 20, NULL) == SWIGLU_ERR_MISALIGNED);
    CHECK(mlp_block_forward(fake, fake, 1e-6f, fake, fake, NULL, fake, 4, 64, 64, SWIGLU_BF16,
                            fake, 256, NULL) == SWIGLU_ERR_WORKSPACE);
    CHECK(mlp_block_forward_ex(fake, fake, 1e-6f, fake, fake, NULL, fake, 4, 64, 64,
                               SWIGLU_BF16_MXFP4W, fake, 1 << 20, NULL, SWIGLU_PATH_WIDE) ==
          SWIGLU_ERR_UNSUPPORTED);
    CHECK(swiglu_up_graph_create(fake, fake, fake, 4, 64, 64, SWIGLU_BF16, NULL, 0,
                                 SWIGLU_PATH_AUTO, NULL) == SWIGLU_ERR_INVALID_ARG);
    CHECK(swiglu_up_graph_create(odd, fake, fake, 4, 64, 64, SWIGLU_BF16, NULL, 0,
                                 SWIGLU_PATH_AUTO, &g) == SWIGLU_ERR_MISALIGNED && g == NULL);
    CHECK(mlp_forward_graph_create(fake, fake, fake, fake, 4, 64, 64, SWIGLU_BF16, fake, 256,
                                   SWIGLU_PATH_AUTO, &g) == SWIGLU_ERR_WORKSPACE && g == NULL);
    CHECK(mlp_block_graph_create(fake, fake, -1.0f, fake, fake, NULL, fake, 4, 64, 64,
                                 SWIGLU_BF16, fake, 1 << 20, SWIGLU_PATH_AUTO, &g) ==
              SWIGLU_ERR_INVALID_ARG && g == NULL);
    CHECK(swiglu_graph_launch(NULL, NULL) == SWIGLU_ERR_INVALID_ARG);
    CHECK(swiglu_graph_destroy(NULL) == SWIGLU_OK);

    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("abi_sanitize ok (%ld size queries)\n", queries);
    return 0;
}

/* Plain C99 user of include/swiglu.h: checks that the header compiles as C
 * and that the library rejects bad arguments before touching the GPU (so
 * this runs on a machine without one).  Exit status 0 on success. */
#include <stdio.h>
#include <stdint.h>
#include <string.h>

#include "swiglu.h"

#define CHECK(cond)                                                   \
    do {                                                              \
        if (!(cond)) {                                                \
            fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__,    \
                    __LINE__, #cond);                                 \
            return 1;                                                 \
        }                                                             \
    } while (0)

int main(void)
{
    void *fake = (void *)(uintptr_t)0x10000000u;   /* aligned, never dereferenced */
    char *odd = (char *)fake + 4;
    swiglu_graph_t g = NULL;

    CHECK(swiglu_version() == 1);
    CHECK(strcmp(swiglu_status_string(SWIGLU_OK), "ok") == 0);
    CHECK(swiglu_packed_bytes(4096, 14336, SWIGLU_BF16) == (size_t)2 * 4096 * 14336 * 2);
    CHECK(swiglu_packed_bytes(4096, 14336, SWIGLU_BF16_FP8W) ==
          (size_t)4096 * 14336 * 2 + 896 * 32 * 4);
    CHECK(swiglu_select_path(1, 4096, 14336, SWIGLU_BF16) == SWIGLU_PATH_SKINNY);
    CHECK(swiglu_select_path(4096, 4096, 14336, SWIGLU_BF16) == SWIGLU_PATH_WIDE);
    CHECK(swiglu_up(fake, fake, fake, -1, 64, 64, SWIGLU_BF16, NULL, 0, NULL) ==
          SWIGLU_ERR_INVALID_ARG);
    CHECK(swiglu_up(odd, fake, fake, 4, 64, 64, SWIGLU_BF16, NULL, 0, NULL) ==
          SWIGLU_ERR_MISALIGNED);
    CHECK(swiglu_up_ex(fake, fake, fake, 4, 64, 64, SWIGLU_F32, NULL, 0, NULL,
                       SWIGLU_PATH_WIDE) == SWIGLU_ERR_UNSUPPORTED);
    CHECK(mlp_forward(fake, fake, fake, fake, 4, 64, 64, SWIGLU_BF16, NULL, 0, NULL) ==
          SWIGLU_ERR_INVALID_ARG);
    CHECK(mlp_block_forward(fake, fake, -1.0f, fake, fake, NULL, fake, 4, 64, 64, SWIGLU_BF16,
                            fake, 1 << 20, NULL) == SWIGLU_ERR_INVALID_ARG);
    CHECK(swiglu_up(NULL, NULL, NULL, 0, 64, 64, SWIGLU_BF16, NULL, 0, NULL) == SWIGLU_OK);
    CHECK(swiglu_up_graph_create(fake, fake, fake, -1, 64, 64, SWIGLU_BF16, NULL, 0,
                                 SWIGLU_PATH_AUTO, &g) == SWIGLU_ERR_INVALID_ARG);
    CHECK(g == NULL);
    CHECK(mlp_block_graph_create(fake, fake, -1.0f, fake, fake, NULL, fake, 4, 64, 64, SWIGLU_BF16,
                                 fake, 1 << 20, SWIGLU_PATH_AUTO, &g) == SWIGLU_ERR_INVALID_ARG);
    CHECK(swiglu_graph_launch(NULL, NULL) == SWIGLU_ERR_INVALID_ARG);
    CHECK(swiglu_graph_destroy(NULL) == SWIGLU_OK);
    puts("abi_check ok");
    return 0;
}

/* The C ABI used from plain C99: include/fa.h compiles as C, libfa.so links,
 * and every entry point answers argument errors on the host (no device
 * memory is touched: validation precedes any launch).  Built and run by
 * tests/test_abi.py; exit status 0 when every check holds. */
#include <stdio.h>
#include <stdint.h>
#include "fa.h"

#define CHECK(cond)                                                  \
    do {                                                             \
        if (!(cond)) {                                               \
            fprintf(stderr, "check failed, line %d: %s\n", __LINE__, #cond); \
            return 1;                                                \
        }                                                            \
    } while (0)

int main(void) {
    /* a non-NULL, 256-byte aligned address that is never dereferenced */
    void* P = (void*)(uintptr_t)0x100000;
    int32_t br = 0, bc = 0;
    fa_opts o = {0};
    o.struct_size = sizeof(fa_opts);

    CHECK(fa_abi_version() == FA_ABI_VERSION);
    CHECK(fa_tile_shape(128, FA_BF16, 0, 4096, 1, &br, &bc) == FA_OK && br > 0 && bc > 0 && 128 % br == 0 && 128 % bc == 0);
    CHECK(fa_tile_shape(96, FA_BF16, 0, 4096, 1, &br, &bc) == FA_ERR_HEAD_DIM);
    CHECK(fa_status_string(FA_ERR_SHAPE) != NULL);

    /* forward / backward: NULL pointer, bad head dim, bad dropout, bad opts size */
    CHECK(fa_fwd(NULL, P, P, P, (float*)P, 1, 2, 256, 64, FA_BF16, 0.125f, 0, 0.0f, 0, NULL, NULL, P, 1 << 20,
                 NULL) == FA_ERR_NULL);
    CHECK(fa_fwd(P, P, P, P, (float*)P, 1, 2, 256, 80, FA_BF16, 0.125f, 0, 0.0f, 0, NULL, NULL, P, 1 << 20,
                 NULL) == FA_ERR_HEAD_DIM);
    CHECK(fa_fwd(P, P, P, P, (float*)P, 1, 2, 256, 64, FA_F16, 0.125f, 0, 1.5f, 0, NULL, NULL, NULL, 0,
                 NULL) == FA_ERR_DROPOUT);
    o.struct_size = 3;
    CHECK(fa_fwd(P, P, P, P, (float*)P, 1, 2, 256, 64, FA_F16, 0.125f, 0, 0.0f, 0, NULL, &o, NULL, 0,
                 NULL) == FA_ERR_OPTS);
    o.struct_size = sizeof(fa_opts);
    CHECK(fa_fwd_workspace_bytes(1, 2, 256, 64, FA_BF16) > 0 && fa_fwd_workspace_bytes(1, 2, 256, 64, FA_F16) == 0);
    CHECK(fa_bwd(P, P, P, P, P, (const float*)P, P, P, P, 0, 2, 256, 64, FA_BF16, 0.125f, 0, 0.0f, 0, NULL, &o,
                 P, 1 << 20, NULL) == FA_ERR_SHAPE);
    CHECK(fa_bwd_workspace_bytes(1, 2, 256, 64) >= 2 * 256 * sizeof(float));

    /* decode, key/value-outer forward, keep mask */
    CHECK(fa_decode(P, P, P, P, (float*)P, 1, 4, 3, 1, 100, 64, FA_BF16, 0.125f, 0, NULL, NULL, P, 1 << 20,
                    NULL) == FA_ERR_SHAPE);
    CHECK(fa_decode(P, P, P, P, (float*)P, 1, 4, 2, 1, 100, 64, FA_F32, 0.125f, 0, NULL, NULL, P, 1 << 20,
                    NULL) == FA_ERR_DTYPE);
    CHECK(fa_decode_workspace_bytes(1, 4, 2, 1, 100, 64) > 0);
    CHECK(fa_fwd_kv_outer(P, P, P, P, (float*)P, 1, 2, 300, 64, FA_BF16, 0.125f, 0, 32, 0, NULL, P, 1 << 24,
                          NULL) == FA_ERR_OPTS);
    CHECK(fa_fwd_kv_outer_workspace_bytes(1, 2, 300, 64) > 0);
    CHECK(fa_dropout_keep_mask(1, 0, -0.5f, 1, 1, 16, (uint8_t*)P, NULL) == FA_ERR_DROPOUT);
    printf("c abi ok: version %d, forward tile %d x %d\n", fa_abi_version(), br, bc);
    return 0;
}

/*
 * A plain C11 client of libkvarn.so: include/kvarn.h compiles as C, the library
 * links and loads without Python, and the host-side entry points and argument
 * checks behave as the header documents.  It makes no call that would reach the
 * GPU: every compute call below is rejected during argument validation (or is an
 * empty batch), so the program runs on a machine without one.
 */
#include "kvarn.h"

#include <stdio.h>
#include <string.h>

static int failures = 0;

#define CHECK(cond)                                                 \
    do {                                                            \
        if (!(cond)) {                                              \
            fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond); \
            ++failures;                                             \
        }                                                           \
    } while (0)

int main(void) {
    /* stand-in device addresses: validation never dereferences them */
    const void *a = (const void *)(uintptr_t)0x10000, *mis = (const void *)(uintptr_t)0x10008;
    void *out = (void *)(uintptr_t)0x20000;
    const int32_t *counts = (const int32_t *)(uintptr_t)0x30000;

    CHECK(kvarn_format_version() == KVARN_FORMAT_VERSION);
    CHECK(kvarn_tile_bytes(2) == 4608 && kvarn_tile_bytes(4) == 8704 && kvarn_tile_bytes(3) == 0);

    int bk = 0, bv = 0, g = 0;
    const int st = kvarn_parse_preset("kvarn_k4v2_g128", &bk, &bv, &g);
    CHECK(st == KVARN_OK && bk == 4 && bv == 2 && g == 128);
    CHECK(kvarn_parse_preset("kvarn_k4v2_g64", &bk, &bv, &g) == KVARN_EUNSUPPORTED);
    CHECK(kvarn_parse_preset("kivi", &bk, &bv, &g) == KVARN_EINVAL);

    const int codes[] = {KVARN_OK, KVARN_EINVAL, KVARN_EUNSUPPORTED, KVARN_EALIGN, KVARN_EWORKSPACE, KVARN_EHIP};
    for (size_t i = 0; i < sizeof codes / sizeof codes[0]; ++i) {
        const char *s = kvarn_status_string(codes[i]);
        CHECK(s != NULL && strlen(s) > 0);
    }

    /* quantise: one bf16 K tile, dense layout */
    CHECK(kvarn_quantize_tiles(NULL, KVARN_BF16, 1, 16384, 128, NULL, 2, KVARN_AXIS_K, 8, out, NULL, 0, NULL) ==
          KVARN_EINVAL);
    CHECK(kvarn_quantize_tiles(a, KVARN_BF16, 1, 16384, 128, NULL, 3, KVARN_AXIS_K, 8, out, NULL, 0, NULL) ==
          KVARN_EUNSUPPORTED);
    CHECK(kvarn_quantize_tiles(mis, KVARN_BF16, 1, 16384, 128, NULL, 2, KVARN_AXIS_K, 8, out, NULL, 0, NULL) ==
          KVARN_EALIGN);
    CHECK(kvarn_quantize_tiles(a, KVARN_BF16, 0, 16384, 128, NULL, 2, KVARN_AXIS_K, 8, out, NULL, 0, NULL) ==
          KVARN_OK);

    /* dequantise */
    CHECK(kvarn_dequantize_tiles(a, NULL, 1, 2, KVARN_AXIS_V, out, 7, 16384, 128, NULL, 0, NULL) == KVARN_EINVAL);
    CHECK(kvarn_dequantize_tiles(a, NULL, 0, 2, KVARN_AXIS_V, out, KVARN_F16, 16384, 128, NULL, 0, NULL) == KVARN_OK);

    /* decode attention: 2 sequences, 8 query heads on 2 KV heads, 4 tiles each */
    const size_t ws = kvarn_decode_attn_workspace_bytes(2, 8, 2, 4);
    CHECK(ws > 0);
    CHECK(kvarn_decode_attn(a, a, a, NULL, counts, 10, 2, 8, 2, 4, 2, 2, 0.088f, out, out, ws - 1, 0, NULL) ==
          KVARN_EWORKSPACE);
    CHECK(kvarn_decode_attn(a, a, a, NULL, counts, 10, 2, 6, 4, 4, 2, 2, 0.088f, out, out, ws, 0, NULL) ==
          KVARN_EINVAL);
    CHECK(kvarn_decode_attn(a, a, a, NULL, counts, 10, 0, 8, 2, 4, 2, 2, 0.088f, out, out, ws, 0, NULL) == KVARN_OK);
    CHECK(kvarn_decode_attn_windows(a, a, a, NULL, counts, 10, 2, 8, 2, 4, 2, 2, 0.088f, a, NULL, 128, NULL, NULL,
                                    NULL, 0, out, out, ws, 0, NULL) == KVARN_EINVAL);

    if (failures) return 1;
    printf("ok\n");
    return 0;
}

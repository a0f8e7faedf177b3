/* A plain C99 consumer of include/nvfp4.h: checks that the header is valid C and that a C program can
 * link the library and call its entry points.  Without a GPU every call stops at the device check (or
 * earlier, at argument validation), so nothing is launched and no memory is touched. */
#include <stdio.h>
#include <string.h>

#include "nvfp4.h"

static int expect(const char* what, nvfp4_status got, nvfp4_status want) {
    if (got != want) {
        fprintf(stderr, "%s: status %d, expected %d (%s)\n", what, (int)got, (int)want, nvfp4_last_error());
        return 1;
    }
    return 0;
}

int main(void) {
    int bad = 0;
    static unsigned char fake[1 << 16];           /* never dereferenced: every call below stops first */
    void* p = (void*)(((size_t)fake + 255) & ~(size_t)255);
    float* g = (float*)p;
    nvfp4_weight_desc d;
    nvfp4_epilogue ep;
    const int64_t rows[2] = {32, 48};
    const nvfp4_status no_dev = nvfp4_device_check();

    if (nvfp4_abi_version() != NVFP4_ABI_VERSION) { fprintf(stderr, "abi version\n"); bad = 1; }
    if (nvfp4_quantize_workspace_bytes(16, 5120) == 0) { fprintf(stderr, "workspace query\n"); bad = 1; }
    if (nvfp4_packed_weight_bytes(2, rows, 256) == 0) { fprintf(stderr, "packed size query\n"); bad = 1; }

    /* argument validation comes before the device check */
    bad |= expect("quantize K % 16", nvfp4_quantize(p, NVFP4_IN_BF16, 4, 24, 24, p, p, g, NVFP4_G_GIVEN, NULL, 0,
                                                    NULL), NVFP4_ERR_SHAPE);
    bad |= expect("quantize_t rows % 16", nvfp4_quantize_t(p, NVFP4_IN_F32, 24, 8, 8, p, p, g, NVFP4_G_GIVEN, NULL,
                                                           0, NULL), NVFP4_ERR_SHAPE);
    bad |= expect("rht signs", nvfp4_quantize_rht(p, NVFP4_IN_F32, 16, 64, 64, 1u << 16, p, p, g, NVFP4_G_GIVEN,
                                                  NULL, 0, NULL), NVFP4_ERR_INVALID_ARG);
    bad |= expect("kv scale NULL", nvfp4_kv_quantize_fp8(p, NVFP4_IN_BF16, 4, 8, 8, p, NULL, NVFP4_G_GIVEN, NULL,
                                                         0, NULL), NVFP4_ERR_INVALID_ARG);
    memset(&d, 0, sizeof d);
    memset(&ep, 0, sizeof ep);
    ep.y_dtype = 7;
    bad |= expect("gemm_ex bad descriptor", nvfp4_gemm_ex(16, p, p, g, &d, &ep, p, 64, NULL, 0, NULL),
                  NVFP4_ERR_INVALID_ARG);

    /* well-formed calls reach the device check */
    if (no_dev == NVFP4_ERR_NO_DEVICE) {
        bad |= expect("quantize", nvfp4_quantize(p, NVFP4_IN_BF16, 4, 64, 64, p, p, g, NVFP4_G_GIVEN, NULL, 0, NULL),
                      NVFP4_ERR_NO_DEVICE);
        bad |= expect("quantize_both", nvfp4_quantize_both(p, NVFP4_IN_BF16, 32, 48, 48, p, p, p, p, g,
                                                           NVFP4_G_GIVEN, NULL, 0, NULL), NVFP4_ERR_NO_DEVICE);
        bad |= expect("kv", nvfp4_kv_quantize_fp8(p, NVFP4_IN_F32, 3, 5, 5, p, g, NVFP4_G_GIVEN, NULL, 0, NULL),
                      NVFP4_ERR_NO_DEVICE);
    }
    if (!bad) printf("c abi consumer ok (%s)\n", no_dev == NVFP4_OK ? "gpu visible" : "no gpu");
    return bad;
}

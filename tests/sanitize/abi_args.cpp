// Argument checking of the C ABI (include/moe.h) under the host address and
// undefined-behaviour sanitizers: every call below fails an argument check
// (or is the T = 0 no-op) and must return its status code before any HIP
// call, without a sanitizer report.  Built and run by
// tests/test_sanitizers.py on the CPU; no call reaches a device.
#include <stdint.h>
#include <stdio.h>

#include "moe.h"

static int failures = 0;

static void expect(int got, int want, const char *what)
{
    if (got != want) {
        fprintf(stderr, "%s: got %d, want %d\n", what, got, want);
        ++failures;
    }
}

int main()
{
    char buf[256] __attribute__((aligned(256)));
    void *p = buf;                                  // never dereferenced on these paths
    void *odd = buf + 8;
    const float *fp = (const float *)p;
    const uint8_t *up = (const uint8_t *)p;
    moe_dims_t good = {64, 256, 8, 512, 1e-6f};
    moe_dims_t bad_d = {64, 200, 8, 512, 1e-6f};
    moe_dims_t bad_eps = {64, 256, 8, 512, -1.0f};
    moe_dims_t zero = {0, 256, 8, 512, 1e-6f};
    moe_dims_t big = {4096, 8192, 256, 2048, 1e-6f};

    expect(moe_layer_forward(nullptr, p, fp, up, up, fp, fp, 2, p, p, 1 << 30, nullptr, nullptr),
           MOE_ERR_NULL, "dims NULL");
    expect(moe_layer_forward(&good, nullptr, fp, up, up, fp, fp, 2, p, p, 1 << 30, nullptr, nullptr),
           MOE_ERR_NULL, "x NULL");
    expect(moe_layer_forward(&good, p, fp, up, up, fp, fp, 2, p, nullptr, 1 << 30, nullptr, nullptr),
           MOE_ERR_NULL, "workspace NULL");
    expect(moe_layer_forward(&bad_d, p, fp, up, up, fp, fp, 2, p, p, 1 << 30, nullptr, nullptr),
           MOE_ERR_SHAPE, "d = 200");
    expect(moe_layer_forward(&bad_eps, p, fp, up, up, fp, fp, 2, p, p, 1 << 30, nullptr, nullptr),
           MOE_ERR_SHAPE, "eps < 0");
    expect(moe_layer_forward(&good, p, fp, up, up, fp, fp, 9, p, p, 1 << 30, nullptr, nullptr),
           MOE_ERR_SHAPE, "k > E");
    expect(moe_layer_forward(&good, odd, fp, up, up, fp, fp, 2, p, p, 1 << 30, nullptr, nullptr),
           MOE_ERR_ALIGN, "x misaligned");
    expect(moe_layer_forward(&good, p, fp, up, up, fp, fp, 2, p, p, 1024, nullptr, nullptr),
           MOE_ERR_WORKSPACE, "workspace small");
    expect(moe_layer_forward(&zero, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 2, nullptr,
                             nullptr, 0, nullptr, nullptr),
           MOE_OK, "T = 0");
    expect(moe_layer_forward_noalloc(&big, p, fp, up, up, fp, fp, 8, p, nullptr, nullptr),
           MOE_ERR_SCRATCH, "noalloc too big");
    expect(moe_layer_forward_noalloc(&good, p, fp, up, up, fp, fp, 2, nullptr, nullptr, nullptr),
           MOE_ERR_NULL, "noalloc s_out NULL");
    expect(moe_layer_workspace_size(&bad_d, 2) == 0, 1, "workspace size of a bad shape");
    expect(moe_layer_workspace_size(&good, 2) > 0, 1, "workspace size");
    expect(moe_pack_weights(&bad_d, up, up, (uint8_t *)p, (uint8_t *)p, nullptr), MOE_ERR_SHAPE, "pack d");
    expect(moe_dequant_mxfp4(up, up, 4, 48, p, nullptr), MOE_ERR_SHAPE, "dequant K");
    moe_latent_dims_t lbad = {64, 500, 256, 8, 256, 1e-6f};
    expect(moe_latent_forward(&lbad, p, fp, p, up, up, p, fp, fp, 2, p, p, 1 << 30, nullptr, nullptr),
           MOE_ERR_SHAPE, "latent D");
    expect(moe_block_forward(&good, p, nullptr, fp, up, up, fp, fp, fp, 2, p, p, 1 << 30, nullptr, nullptr),
           MOE_ERR_NULL, "block gamma NULL");
    expect(moe_layer_forward_nvfp4(&good, p, fp, up, up, nullptr, fp, fp, 2, p, p, 1 << 30, nullptr, nullptr),
           MOE_ERR_NULL, "nvfp4 gscale NULL");
    for (int code = -8; code <= 1; ++code)
        if (!moe_status_string(code)) ++failures;
    printf("abi argument checks: %d failure(s)\n", failures);
    return failures ? 1 : 0;
}

/* A plain C99 client of libgdr.so, built and run by tests/test_abi.py with gcc on the host.
 * It checks that include/gdr.h is a C header (no C++ needed), that the library links and
 * that the host-side checks answer as documented.  No call here passes validation, so
 * nothing reaches the GPU. */
#include <stdio.h>
#include <string.h>

#include "gdr.h"

static int fails = 0;
#define CHECK(cond)                                              \
    do {                                                         \
        if (!(cond)) {                                           \
            fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__); \
            ++fails;                                             \
        }                                                        \
    } while (0)

int main(void) {
    CHECK(gdr_abi_version() == GDR_ABI_VERSION);
    CHECK(strcmp(gdr_status_str(GDR_OK), "ok") == 0);

    gdr_dims d;
    memset(&d, 0, sizeof d); /* flags = 0: fp32 g */
    d.B = 1; d.T = 4097; d.HK = 16; d.HV = 32; d.dk = 128; d.dv = 128; d.chunk = 64;
    d.qkv_dtype = GDR_BF16;
    /* 65 chunk records of 65 KiB per (batch, head) */
    CHECK(gdr_chunk_prefill_workspace_bytes(&d) == (size_t)32 * 65 * 65 * 1024);

    /* null pointers and bad shapes are refused on the host */
    float dummy[4] __attribute__((aligned(16)));
    CHECK(gdr_chunk_prefill(&d, NULL, dummy, dummy, dummy, dummy, NULL, dummy, NULL, NULL, 0, NULL) == GDR_ERR_NULL);
    d.T = 1;
    d.dk = 48;
    CHECK(gdr_decode_step(&d, dummy, dummy, dummy, dummy, dummy, NULL, dummy, NULL, NULL) == GDR_ERR_UNSUPPORTED);
    d.dk = 128;
    d.flags = GDR_G_BF16;
    d.qkv_dtype = GDR_F32;
    CHECK(gdr_decode_step(&d, dummy, dummy, dummy, dummy, dummy, NULL, dummy, NULL, NULL) == GDR_ERR_UNSUPPORTED);
    d.flags = 0;
    d.HK = 3;
    CHECK(gdr_fused_recurrent(&d, dummy, dummy, dummy, dummy, dummy, NULL, dummy, NULL, NULL) == GDR_ERR_SHAPE);

    if (fails) return 1;
    printf("c abi ok\n");
    return 0;
}

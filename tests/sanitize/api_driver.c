/* Drives the host entry points of libgdr (gdr_api.cpp, built with the kernel launchers
 * stubbed out) under AddressSanitizer and UndefinedBehaviorSanitizer: every validation path
 * -- null pointers, shapes, sizes past 2^31, flags, alignment, aliasing, workspace sizes,
 * packed batches -- on fake device addresses, which no call dereferences.  Built and run on
 * the host by tests/test_sanitizers.py. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "gdr.h"

static int fails = 0;
#define CHECK(cond)                                                                     \
    do {                                                                                \
        if (!(cond)) {                                                                  \
            fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__);          \
            ++fails;                                                                    \
        }                                                                               \
    } while (0)

#define P(i) ((void*)(uintptr_t)((1ull << 40) + (uint64_t)(i) * (1ull << 32)))

static gdr_dims dims(int B, int T, int HK, int HV, int dk, int dv, int C, int flags) {
    gdr_dims d;
    memset(&d, 0, sizeof d);
    d.B = B; d.T = T; d.HK = HK; d.HV = HV; d.dk = dk; d.dv = dv; d.chunk = C;
    d.qkv_dtype = GDR_BF16; d.flags = flags;
    return d;
}

static int prefill(const gdr_dims* d, size_t ws) {
    return gdr_chunk_prefill(d, P(0), P(1), P(2), P(3), P(4), P(5), P(6), P(7), P(8), ws, NULL);
}

int main(void) {
    /* sizes, every supported combination and a few unsupported ones */
    const int hd[] = {16, 32, 64, 128, 256};
    const int cs[] = {8, 16, 32, 64};
    for (unsigned a = 0; a < 5; ++a)
        for (unsigned b = 0; b < 5; ++b)
            for (unsigned c = 0; c < 4; ++c) {
                gdr_dims d = dims(3, 1000, 2, 4, hd[a], hd[b], cs[c], 0);
                size_t n = gdr_chunk_prefill_workspace_bytes(&d);
                size_t nv = gdr_chunk_prefill_varlen_workspace_bytes(&d);
                int ok = hd[a] >= 32 && hd[a] <= 128 && hd[b] >= 32 && hd[b] <= 128 && cs[c] >= 16;
                CHECK((n != 0) == ok && (nv != 0) == ok);
                if (ok) {
                    CHECK(prefill(&d, n - 1) == GDR_ERR_WORKSPACE);
                    CHECK(prefill(&d, n) == GDR_ERR_HIP);
                }
            }
    /* overflowing and invalid shapes */
    gdr_dims big = dims(1 << 20, 1 << 20, 16, 32, 128, 128, 64, 0);
    CHECK(prefill(&big, (size_t)-1) == GDR_ERR_SHAPE);
    gdr_dims neg = dims(-1, 5, 1, 1, 32, 32, 16, 0);
    CHECK(gdr_chunk_prefill_workspace_bytes(&neg) == 0 && prefill(&neg, 1 << 20) == GDR_ERR_SHAPE);
    gdr_dims huge_t = dims(1, 0x7fffffff, 1, 1, 128, 128, 64, 0);
    {   /* refused on the host: past the 31-bit offsets, or (fake pointers 4 GiB apart) aliased */
        int r = prefill(&huge_t, (size_t)-1);
        CHECK(r == GDR_ERR_SHAPE || r == GDR_ERR_ALIAS);
    }
    CHECK(gdr_chunk_prefill(NULL, P(0), P(1), P(2), P(3), P(4), NULL, P(6), NULL, P(8), 0, NULL) == GDR_ERR_NULL);
    /* flags */
    for (int f = -1; f < 0x80; ++f) {
        gdr_dims d = dims(2, 5, 2, 4, 64, 32, 16, f);
        int r = gdr_decode_step(&d, P(0), P(1), P(2), P(3), P(4), P(5), P(6), P(5), NULL);
        CHECK(r == GDR_ERR_SHAPE || r == GDR_ERR_UNSUPPORTED);
        d.T = 1;
        r = gdr_decode_step(&d, P(0), P(1), P(2), P(3), P(4), P(5), P(6), P(5), NULL);
        CHECK(r == GDR_ERR_HIP || r == GDR_ERR_UNSUPPORTED);
        r = gdr_fused_recurrent(&d, P(0), P(1), P(2), P(3), P(4), P(5), P(6), P(5), NULL);
        CHECK(r == GDR_ERR_HIP || r == GDR_ERR_UNSUPPORTED);
    }
    /* alignment and aliasing */
    gdr_dims d = dims(2, 5, 2, 4, 64, 32, 16, 0);
    size_t n = gdr_chunk_prefill_workspace_bytes(&d);
    CHECK(gdr_chunk_prefill(&d, (void*)((char*)P(0) + 8), P(1), P(2), P(3), P(4), P(5), P(6), P(7), P(8), n, NULL) == GDR_ERR_ALIGN);
    CHECK(gdr_chunk_prefill(&d, P(0), P(1), P(2), P(3), P(4), P(5), P(0), P(7), P(8), n, NULL) == GDR_ERR_ALIAS);
    CHECK(gdr_chunk_prefill(&d, P(0), P(1), P(2), P(3), P(4), P(5), P(6), (float*)((char*)P(5) + 16), P(8), n, NULL) == GDR_ERR_ALIAS);
    CHECK(gdr_chunk_prefill(&d, P(0), P(1), P(2), P(3), P(4), P(5), P(6), P(5), P(8), n, NULL) == GDR_ERR_HIP);
    CHECK(gdr_chunk_prefill(&d, P(0), P(1), P(2), P(3), P(4), P(5), P(6), P(7), P(0), n, NULL) == GDR_ERR_ALIAS);
    /* packed batches */
    for (int N = 1; N <= 4097; N += 1024) {
        gdr_dims v = dims(N, 5000, 2, 4, 128, 128, 64, 0);
        size_t nv = gdr_chunk_prefill_varlen_workspace_bytes(&v);
        int r = gdr_chunk_prefill_varlen(&v, P(9), P(0), P(1), P(2), P(3), P(4), P(5), P(6), P(7), P(8), nv, NULL);
        CHECK(N <= GDR_VARLEN_MAX_SEQS ? r == GDR_ERR_HIP : (r == GDR_ERR_SHAPE && nv == 0));
        r = gdr_fused_recurrent_varlen(&v, P(9), P(0), P(1), P(2), P(3), P(4), P(5), P(6), P(7), NULL);
        CHECK(N <= GDR_VARLEN_MAX_SEQS ? r == GDR_ERR_HIP : r == GDR_ERR_SHAPE);
    }
    gdr_dims v = dims(3, 50, 2, 4, 64, 64, 32, GDR_G_PER_KEY_HEAD | GDR_PREP_SPLIT);
    size_t nv = gdr_chunk_prefill_varlen_workspace_bytes(&v);
    CHECK(gdr_chunk_prefill_varlen(&v, NULL, P(0), P(1), P(2), P(3), P(4), P(5), P(6), P(7), P(8), nv, NULL) == GDR_ERR_NULL);
    CHECK(gdr_chunk_prefill_varlen(&v, P(9), P(0), P(1), P(2), P(3), P(4), P(5), P(6), P(7), P(8), nv - 4, NULL) == GDR_ERR_WORKSPACE);
    CHECK(gdr_chunk_prefill_varlen(&v, P(9), P(0), P(1), P(2), P(3), P(4), P(5), P(9), P(7), P(8), nv, NULL) == GDR_ERR_ALIAS);
    CHECK(gdr_chunk_prefill_varlen(&v, P(9), P(0), P(1), P(2), P(3), P(4), P(5), P(6), P(7), P(8), nv, NULL) == GDR_ERR_HIP);
    /* the allocation-free entry point: within the scratch it reaches the runtime, past it refuses */
    gdr_dims s = dims(1, 1984, 16, 32, 128, 128, 64, 0);
    CHECK(gdr_chunk_prefill_noalloc(&s, P(0), P(1), P(2), P(3), P(4), P(5), P(6), P(7), NULL) == GDR_ERR_HIP);
    s.T = 1985;
    CHECK(gdr_chunk_prefill_noalloc(&s, P(0), P(1), P(2), P(3), P(4), P(5), P(6), P(7), NULL) == GDR_ERR_SCRATCH);
    for (int st = -2; st < 12; ++st) CHECK(gdr_status_str(st) != NULL);
    if (fails) return 1;
    printf("api sanitize ok\n");
    return 0;
}

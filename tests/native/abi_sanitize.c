/*
 * Host-side argument validation of libssd under AddressSanitizer and
 * UndefinedBehaviorSanitizer.  Built from the library's sources compiled for
 * the host only (no device code, no GPU needed), linked with this driver; run
 * by tests/test_sanitizers.py.  Every call made here is one that validation
 * rejects or that returns before any launch, so no device memory is touched:
 * the pointers are fake, far-apart device addresses that are never
 * dereferenced.  Sizes near the limits exercise the overflow guards of the
 * size arithmetic, which UBSan would flag if they wrapped.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "ssd.h"

static int failures = 0;

#define EXPECT(call, want)                                                                \
    do {                                                                                  \
        int got_ = (int)(call);                                                           \
        if (got_ != (int)(want)) {                                                        \
            fprintf(stderr, "%s:%d: %s returned %d, expected %d\n", __FILE__, __LINE__,  \
                    #call, got_, (int)(want));                                            \
            ++failures;                                                                   \
        }                                                                                 \
    } while (0)

/* fake device addresses: 256-byte aligned, 64 MiB apart */
static void* fake(int k) { return (void*)(uintptr_t)(0x100000000ull + (uint64_t)k * (64ull << 20)); }
static void* off(void* p, size_t bytes) { return (void*)((uintptr_t)p + bytes); }

static ssd_dims dims(int64_t b, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G, int64_t Q) {
    ssd_dims d = {b, L, H, P, N, G, Q};
    return d;
}

static ssd_status scan(const ssd_dims* d, ssd_dtype io, void* x, void* y, float lo, float hi,
                       void* ws, size_t ws_bytes, float* init, float* fin) {
    return ssd_chunk_scan_fwd(d, io, x, fake(1), NULL, 1, lo, hi, fake(2), fake(3), fake(4), NULL,
                              init, NULL, y, fin, ws, ws_bytes, NULL);
}

static void check_queries(void) {
    const int64_t big = (int64_t)1 << 40;
    ssd_dims d = dims(1, 8192, 64, 64, 128, 8, 128);
    if (ssd_chunk_scan_workspace_bytes(&d, SSD_BF16) == 0) ++failures;
    if (ssd_chunk_scan_segments(&d, SSD_BF16) != 4) ++failures;
    /* sizes whose products overflow 64 bits are rejected, not wrapped */
    d = dims(big, big, 64, 64, 128, 8, 128);
    EXPECT(ssd_chunk_scan_workspace_bytes(&d, SSD_BF16), 0);
    EXPECT(ssd_chunk_scan_segments(&d, SSD_BF16), 0);
    EXPECT(ssd_chunk_scan_cached_workspace_bytes(&d, SSD_BF16), 0);
    EXPECT(ssd_chunk_scan_varlen_workspace_bytes(&d, SSD_BF16), 0);
    EXPECT(ssd_chunk_scan_bwd_workspace_bytes(&d, SSD_BF16), 0);
    d = dims(INT64_MAX, 1, 1, 64, 128, 1, 128);
    EXPECT(ssd_chunk_scan_workspace_bytes(&d, SSD_BF16), 0);
    d = dims(1, INT64_MAX, 1, 64, 128, 1, 128);
    EXPECT(ssd_chunk_scan_workspace_bytes(&d, SSD_BF16), 0);
    EXPECT(ssd_chunk_scan_bwd_workspace_bytes(&d, SSD_BF16), 0);
    d = dims(-1, 128, 8, 64, 128, 1, 128);
    EXPECT(ssd_chunk_scan_workspace_bytes(&d, SSD_BF16), 0);
    EXPECT(ssd_chunk_scan_workspace_bytes(NULL, SSD_BF16), 0);
    d = dims(1, 128, 8, 64, 128, 1, 128);
    EXPECT(ssd_chunk_scan_workspace_bytes(&d, (ssd_dtype)7), 0);
    EXPECT(ssd_decode_emulated_workspace_bytes(&d, SSD_BF16) > 0, 1);
    EXPECT(ssd_chunk_scan_supported(SSD_BF16, 64, 128, 128), 1);
    EXPECT(ssd_chunk_scan_supported(SSD_BF16, 48, 128, 128), 0);
    EXPECT(ssd_chunk_scan_supported((ssd_dtype)-3, 64, 128, 128), 0);
    for (int s = -2; s < 12; ++s)
        if (ssd_status_string(s) == NULL) ++failures;
    EXPECT(ssd_abi_version(), SSD_ABI_VERSION);
}

static void check_scan(void) {
    const size_t ws_bytes = (size_t)1 << 30;
    ssd_dims d = dims(1, 1024, 4, 16, 16, 1, 64);
    EXPECT(scan(NULL, SSD_F32, fake(5), fake(6), 0.f, INFINITY, fake(7), ws_bytes, NULL, NULL),
           SSD_ERR_NULL_ARG);
    EXPECT(scan(&d, (ssd_dtype)7, fake(5), fake(6), 0.f, INFINITY, fake(7), ws_bytes, NULL, NULL),
           SSD_ERR_BAD_DTYPE);
    ssd_dims bad = dims(1, 256, 6, 16, 16, 4, 64);
    EXPECT(scan(&bad, SSD_F32, fake(5), fake(6), 0.f, INFINITY, fake(7), ws_bytes, NULL, NULL),
           SSD_ERR_BAD_SHAPE);
    bad = dims(1, 256, 4, 16, 16, 1, 0);
    EXPECT(scan(&bad, SSD_F32, fake(5), fake(6), 0.f, INFINITY, fake(7), ws_bytes, NULL, NULL),
           SSD_ERR_BAD_SHAPE);
    bad = dims(INT64_MAX, INT64_MAX, 4, 16, 16, 1, 64);
    EXPECT(scan(&bad, SSD_F32, fake(5), fake(6), 0.f, INFINITY, fake(7), ws_bytes, NULL, NULL),
           SSD_ERR_BAD_SHAPE);
    bad = dims(1, 256, INT64_MAX, 16, 16, 1, 64);
    EXPECT(scan(&bad, SSD_F32, fake(5), fake(6), 0.f, INFINITY, fake(7), ws_bytes, NULL, NULL),
           SSD_ERR_BAD_SHAPE);
    bad = dims(1, 256, 4, 24, 16, 1, 64);
    EXPECT(scan(&bad, SSD_F32, fake(5), fake(6), 0.f, INFINITY, fake(7), ws_bytes, NULL, NULL),
           SSD_ERR_UNSUPPORTED);
    EXPECT(scan(&d, SSD_F32, NULL, fake(6), 0.f, INFINITY, fake(7), ws_bytes, NULL, NULL),
           SSD_ERR_NULL_ARG);
    EXPECT(scan(&d, SSD_F32, fake(5), fake(6), 0.f, INFINITY, NULL, ws_bytes, NULL, NULL),
           SSD_ERR_WORKSPACE);
    EXPECT(scan(&d, SSD_F32, fake(5), fake(6), 0.f, INFINITY, fake(7), 16, NULL, NULL),
           SSD_ERR_WORKSPACE);
    EXPECT(scan(&d, SSD_F32, fake(5), fake(6), 0.f, INFINITY, off(fake(7), 16), ws_bytes, NULL,
                NULL),
           SSD_ERR_WORKSPACE);
    EXPECT(scan(&d, SSD_F32, fake(5), fake(6), 1.f, 0.5f, fake(7), ws_bytes, NULL, NULL),
           SSD_ERR_BAD_ARG);
    EXPECT(scan(&d, SSD_F32, fake(5), fake(6), NAN, INFINITY, fake(7), ws_bytes, NULL, NULL),
           SSD_ERR_BAD_ARG);
    EXPECT(scan(&d, SSD_F32, off(fake(5), 4), fake(6), 0.f, INFINITY, fake(7), ws_bytes, NULL,
                NULL),
           SSD_ERR_BAD_ARG);
    EXPECT(scan(&d, SSD_F32, fake(5), off(fake(5), 1024), 0.f, INFINITY, fake(7), ws_bytes, NULL,
                NULL),
           SSD_ERR_ALIAS);
    EXPECT(scan(&d, SSD_F32, fake(5), fake(6), 0.f, INFINITY, fake(7), ws_bytes, fake(8),
                (float*)off(fake(8), 256)),
           SSD_ERR_ALIAS);
    EXPECT(scan(&d, SSD_F32, fake(5), fake(7), 0.f, INFINITY, fake(7), ws_bytes, NULL, NULL),
           SSD_ERR_ALIAS);
    ssd_dims empty = dims(0, 256, 4, 16, 16, 1, 64);
    EXPECT(scan(&empty, SSD_F32, NULL, NULL, 0.f, INFINITY, fake(7), ws_bytes, NULL, NULL),
           SSD_OK);
    EXPECT(ssd_chunk_scan_fwd_noalloc(&bad, SSD_F32, fake(5), fake(1), NULL, 1, 0.f, INFINITY,
                                      fake(2), fake(3), fake(4), NULL, NULL, NULL, fake(6), NULL,
                                      NULL),
           SSD_ERR_UNSUPPORTED);
    ssd_dims huge = dims(64, 1 << 20, 64, 64, 128, 8, 128);
    EXPECT(ssd_chunk_scan_fwd_noalloc(&huge, SSD_BF16, fake(5), fake(1), NULL, 1, 0.f, INFINITY,
                                      fake(2), fake(3), fake(4), NULL, NULL, NULL, fake(6), NULL,
                                      NULL),
           SSD_ERR_TOO_LARGE);
}

static void check_cached_and_varlen(void) {
    ssd_dims d = dims(2, 300, 8, 64, 128, 2, 128);
    const size_t ws = (size_t)1 << 23;
    EXPECT(ssd_chunk_scan_fwd_cached(&d, SSD_BF16, fake(1), fake(2), NULL, 1, 0.f, INFINITY,
                                     fake(3), fake(4), fake(5), NULL, NULL, fake(6), 16, NULL, 1,
                                     0, fake(8), fake(9), ws, NULL),
           SSD_ERR_NULL_ARG);
    EXPECT(ssd_chunk_scan_fwd_cached(&d, SSD_BF16, fake(1), fake(2), NULL, 1, 0.f, INFINITY,
                                     fake(3), fake(4), fake(5), NULL, NULL, fake(6), -1, fake(7),
                                     1, 0, fake(8), fake(9), ws, NULL),
           SSD_ERR_BAD_SHAPE);
    EXPECT(ssd_chunk_scan_fwd_cached(&d, SSD_BF16, fake(1), fake(2), NULL, 1, 0.f, INFINITY,
                                     fake(3), fake(4), fake(5), NULL, NULL, fake(6), INT64_MAX,
                                     fake(7), 1, 0, fake(8), fake(9), ws, NULL),
           SSD_ERR_BAD_SHAPE);
    EXPECT(ssd_chunk_scan_fwd_cached(&d, SSD_BF16, fake(1), fake(2), NULL, 1, 0.f, INFINITY,
                                     fake(3), fake(4), fake(5), NULL, NULL, fake(6), 16, fake(7),
                                     1, 0, off(fake(6), 4096), fake(9), ws, NULL),
           SSD_ERR_ALIAS);
    EXPECT(ssd_chunk_scan_fwd_cached(&d, SSD_BF16, fake(1), fake(2), NULL, 1, 0.f, INFINITY,
                                     fake(3), fake(4), fake(5), NULL, NULL, fake(6), 16, fake(7),
                                     1, 0, fake(8), NULL, ws, NULL),
           SSD_ERR_WORKSPACE);

    d = dims(4, 128, 64, 64, 128, 8, 128);
    EXPECT(ssd_decode_emulated(&d, SSD_BF16, fake(1), fake(2), NULL, 1, 0.f, INFINITY, fake(3),
                               fake(4), fake(5), NULL, fake(6), fake(7), fake(8), fake(9),
                               fake(10), 8, fake(11), NULL, fake(12), fake(13), (size_t)1 << 26,
                               NULL),
           SSD_ERR_NULL_ARG);
    ssd_dims two_chunks = dims(4, 256, 64, 64, 128, 8, 128);
    EXPECT(ssd_decode_emulated(&two_chunks, SSD_BF16, fake(1), fake(2), NULL, 1, 0.f, INFINITY,
                               fake(3), fake(4), fake(5), NULL, fake(6), fake(7), fake(8),
                               fake(9), fake(10), 8, fake(11), fake(14), fake(12), fake(13),
                               (size_t)1 << 26, NULL),
           SSD_ERR_BAD_SHAPE);

    d = dims(3, 300, 8, 64, 128, 2, 128);
    EXPECT(ssd_chunk_scan_fwd_varlen(&d, -1, SSD_BF16, fake(1), fake(2), NULL, 1, 0.f, INFINITY,
                                     fake(3), fake(4), fake(5), NULL, fake(6), fake(7), 16,
                                     fake(8), 1, 0, fake(9), fake(10), (size_t)1 << 26, NULL),
           SSD_ERR_BAD_SHAPE);
    EXPECT(ssd_chunk_scan_fwd_varlen(&d, INT64_MAX, SSD_BF16, fake(1), fake(2), NULL, 1, 0.f,
                                     INFINITY, fake(3), fake(4), fake(5), NULL, fake(6), fake(7),
                                     16, fake(8), 1, 0, fake(9), fake(10), (size_t)1 << 26, NULL),
           SSD_ERR_BAD_SHAPE);
    EXPECT(ssd_chunk_scan_fwd_varlen(&d, 500, SSD_BF16, fake(1), fake(2), NULL, 1, 0.f, INFINITY,
                                     fake(3), fake(4), fake(5), NULL, NULL, fake(7), 16, fake(8),
                                     1, 0, fake(9), fake(10), (size_t)1 << 26, NULL),
           SSD_ERR_NULL_ARG);
}

static void check_bwd_and_mixer(void) {
    ssd_dims d = dims(1, 256, 4, 64, 128, 1, 128);
    const size_t ws = (size_t)1 << 28;
    EXPECT(ssd_chunk_scan_bwd(&d, SSD_BF16, fake(1), fake(2), NULL, 1, 0.f, INFINITY, fake(3),
                              fake(4), fake(5), NULL, NULL, NULL, NULL, NULL, fake(7), fake(8),
                              fake(9), fake(10), fake(11), NULL, NULL, NULL, fake(12), ws, NULL),
           SSD_ERR_NULL_ARG);
    EXPECT(ssd_chunk_scan_bwd(&d, SSD_BF16, fake(1), fake(2), NULL, 1, 0.f, INFINITY, fake(3),
                              fake(4), fake(5), NULL, NULL, NULL, fake(6), NULL, off(fake(1), 4096),
                              fake(8), fake(9), fake(10), fake(11), NULL, NULL, NULL, fake(12), ws,
                              NULL),
           SSD_ERR_ALIAS);
    EXPECT(ssd_chunk_scan_bwd(&d, SSD_F32, fake(1), fake(2), NULL, 1, 0.f, INFINITY, fake(3),
                              fake(4), fake(5), NULL, NULL, NULL, fake(6), NULL, fake(7), fake(8),
                              fake(9), fake(10), fake(11), NULL, NULL, NULL, fake(12), ws, NULL),
           SSD_ERR_UNSUPPORTED);

    EXPECT(ssd_conv1d_fwd(1, 64, 128, 64, 32, SSD_BF16, fake(1), fake(2), 3, NULL, NULL, NULL,
                          fake(3), fake(4), fake(5), NULL, NULL),
           SSD_ERR_UNSUPPORTED);
    EXPECT(ssd_conv1d_fwd(1, 64, 100, 64, 32, SSD_BF16, fake(1), fake(2), 4, NULL, NULL, NULL,
                          fake(3), fake(4), fake(5), NULL, NULL),
           SSD_ERR_BAD_SHAPE);
    EXPECT(ssd_conv1d_fwd(INT64_MAX, INT64_MAX, 128, 64, 32, SSD_BF16, fake(1), fake(2), 4, NULL,
                          NULL, NULL, fake(3), fake(4), fake(5), NULL, NULL),
           SSD_ERR_BAD_SHAPE);
    EXPECT(ssd_conv1d_update(2, 128, 64, 32, SSD_BF16, fake(1), fake(2), 4, NULL, NULL, fake(3),
                             fake(4), fake(5), NULL),
           SSD_ERR_NULL_ARG);
    EXPECT(ssd_conv1d_update_cached(2, -1, 128, 64, 32, SSD_BF16, fake(1), fake(2), 4, NULL,
                                    fake(3), fake(6), fake(4), fake(5), fake(7), NULL),
           SSD_ERR_BAD_SHAPE);
    EXPECT(ssd_gated_rmsnorm(8, 1024, 512, SSD_BF16, fake(1), fake(2), fake(3), -1.f, fake(4),
                             NULL),
           SSD_ERR_BAD_ARG);
    EXPECT(ssd_gated_rmsnorm(INT64_MAX, INT64_MAX, 512, SSD_BF16, fake(1), fake(2), fake(3), 1e-6f,
                             fake(4), NULL),
           SSD_ERR_BAD_SHAPE);

    EXPECT(ssd_state_update(2, 4, 16, 48, 1, SSD_F32, fake(1), fake(2), fake(3), NULL, 1, 0.f,
                            INFINITY, fake(4), fake(5), fake(6), NULL, fake(7), NULL),
           SSD_ERR_UNSUPPORTED);
    EXPECT(ssd_state_update(2, 4, 16, 16, 1, SSD_F32, fake(1), fake(2), fake(3), NULL, 1, 0.f,
                            INFINITY, fake(4), fake(5), fake(6), NULL, off(fake(1), 64), NULL),
           SSD_ERR_ALIAS);
    EXPECT(ssd_state_update(INT64_MAX, INT64_MAX, 16, 16, 1, SSD_F32, fake(1), fake(2), fake(3),
                            NULL, 1, 0.f, INFINITY, fake(4), fake(5), fake(6), NULL, fake(7), NULL),
           SSD_ERR_BAD_SHAPE);
    EXPECT(ssd_state_update_cached(2, (int64_t)1 << 30, 1 << 16, 1 << 10, 16, 1, SSD_F32, fake(1),
                                   fake(8), fake(2), fake(3), NULL, 1, 0.f, INFINITY, fake(4),
                                   fake(5), fake(6), NULL, fake(7), NULL),
           SSD_ERR_BAD_SHAPE);
}

static void check_seq_idx(void) {
    const int32_t ok[10] = {0, 0, 1, 1, 5, 2, 2, 2, 3, 3};
    const int32_t bad[10] = {0, 0, 1, 1, 5, 2, 2, 2, 1, 3};
    EXPECT(ssd_check_seq_idx_host(ok, 2, 5), SSD_OK);
    EXPECT(ssd_check_seq_idx_host(bad, 2, 5), SSD_ERR_BAD_SEQ_IDX);
    EXPECT(ssd_check_seq_idx_host(NULL, 2, 5), SSD_ERR_NULL_ARG);
    EXPECT(ssd_check_seq_idx_host(NULL, 0, 5), SSD_OK);
    EXPECT(ssd_check_seq_idx_host(ok, -1, 5), SSD_ERR_BAD_SHAPE);
    EXPECT(ssd_check_seq_idx_host(ok, INT64_MAX, INT64_MAX), SSD_ERR_BAD_SHAPE);
    /* the exact extent: a heap buffer of b * L entries, read to its last */
    int32_t* h = (int32_t*)malloc(3 * 7 * sizeof(int32_t));
    for (int i = 0; i < 21; ++i) h[i] = i % 7;
    EXPECT(ssd_check_seq_idx_host(h, 3, 7), SSD_OK);
    h[20] = 0;
    EXPECT(ssd_check_seq_idx_host(h, 3, 7), SSD_ERR_BAD_SEQ_IDX);
    free(h);
}

int main(void) {
    check_queries();
    check_scan();
    check_cached_and_varlen();
    check_bwd_and_mixer();
    check_seq_idx();
    if (failures) {
        fprintf(stderr, "abi sanitize: %d failures\n", failures);
        return 1;
    }
    printf("abi sanitize: ok\n");
    return 0;
}

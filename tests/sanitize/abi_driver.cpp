// Host sanitizer run of the C ABI (test infrastructure): the library's host code built with
// AddressSanitizer and UndefinedBehaviorSanitizer, driven through every entry point's
// argument validation, the size and chunk helpers at the edges of int64, and the empty
// problems.  Every call here returns before any HIP call, so no GPU is needed.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "mosaic.h"

static int failures = 0;
#define EXPECT(cond)                                                         \
    do {                                                                     \
        if (!(cond)) {                                                       \
            fprintf(stderr, "abi driver: %s failed at line %d\n", #cond, __LINE__); \
            ++failures;                                                      \
        }                                                                    \
    } while (0)

int main()
{
    char *A16 = (char *)(uintptr_t)(1 << 20), *A8 = A16 + 8;   // never dereferenced
    const int64_t big = INT64_MAX, neg = -1;
    // helpers at the edges
    for (int64_t M : {neg, (int64_t)0, (int64_t)1, (int64_t)29491, big})
        for (int64_t C : {neg, (int64_t)0, (int64_t)1, (int64_t)4096, big}) {
            const int64_t k = mosaic_num_chunks(M, C);
            EXPECT(k >= 0);
            (void)mosaic_logits_argmax_lse_workspace_bytes(M, C, 126464);
            (void)mosaic_logits_argmax_lse_workspace_bytes(M, C, big);
            (void)mosaic_logits_fp8_workspace_bytes(M, C, 4096);
            (void)mosaic_logits_fp8_workspace_bytes(M, C, big);
        }
    int64_t bytes = 0, cr = 0, nc = 0;
    EXPECT(mosaic_logits_bytes(big, big, MOSAIC_BF16, &bytes) == MOSAIC_ERR_INVALID_ARG);
    EXPECT(mosaic_logits_bytes(16 * 2048, 126464, MOSAIC_BF16, &bytes) == MOSAIC_OK && bytes == 8287944704LL);
    EXPECT(mosaic_lazy_chunk_rows(big, big, MOSAIC_F32, big, &cr, &nc) == MOSAIC_ERR_UNSUPPORTED ||
           cr > 0);
    EXPECT(mosaic_lazy_chunk_rows((int64_t)1 << 40, (int64_t)1 << 30, MOSAIC_BF16, (int64_t)1 << 62, &cr, &nc) ==
           MOSAIC_OK);
    EXPECT(mosaic_mask_compact_workspace_bytes(big) == 0);
    for (int v : {-1, 0, 3, 99})
        EXPECT(mosaic_logits_variant(100, 1000, 256, (mosaic_dtype_t)v, MOSAIC_BF16) >= -1);
    EXPECT(mosaic_status_string((mosaic_status_t)42) != nullptr);
    // compaction validation
    EXPECT(mosaic_mask_compact((int32_t *)A16, -1, 0, (int32_t *)A16, (int32_t *)A16, nullptr, 0, nullptr) == 1);
    EXPECT(mosaic_mask_compact((int32_t *)A16, big, 0, (int32_t *)A16, (int32_t *)A16, nullptr, 0, nullptr) == 2);
    EXPECT(mosaic_mask_compact((int32_t *)A16, 10, 0, (int32_t *)A16, (int32_t *)A16, nullptr, 64, nullptr) == 1);
    EXPECT(mosaic_mask_compact_flags(nullptr, 10, (int32_t *)A16, (int32_t *)A16, nullptr, 0, nullptr) == 1);
    EXPECT(mosaic_mask_compact_batched((int32_t *)A16, 10, (int32_t *)A16, 0, 0, (int32_t *)A16, (int32_t *)A16,
                                       nullptr, 0, nullptr) == 1);
    // logits validation, including products that overflow int64
    const void *H = A16, *W = A16;
    const int32_t *idx = (const int32_t *)A16;
    EXPECT(mosaic_masked_logits(H, 100, 64, idx, big, W, big, A16, 0, MOSAIC_BF16, MOSAIC_BF16, nullptr) == 1);
    EXPECT(mosaic_masked_logits(H, big, big, idx, 10, W, 10, A16, 0, MOSAIC_BF16, MOSAIC_BF16, nullptr) == 1);
    EXPECT(mosaic_masked_logits(H, 100, 64, idx, 10, W, 10, A8, 0, MOSAIC_BF16, MOSAIC_BF16, nullptr) == 1);
    EXPECT(mosaic_masked_logits(H, 100, 12, idx, 10, W, 10, A16, 0, MOSAIC_BF16, MOSAIC_BF16, nullptr) == 2);
    EXPECT(mosaic_masked_logits(H, 100, 64, idx, 0, W, 10, nullptr, 0, MOSAIC_BF16, MOSAIC_BF16, nullptr) == 0);
    EXPECT(mosaic_masked_logits(H, (int64_t)1 << 31, 64, idx, 10, W, 10, A16, 0, MOSAIC_BF16, MOSAIC_BF16,
                                nullptr) == 2);
    // the device-count entry point: validation only (the count is never read on the host)
    const int32_t *cnt = (const int32_t *)A16;
    EXPECT(mosaic_masked_logits_device_count(H, 100, 64, idx, cnt, big, W, big, A16, MOSAIC_BF16, MOSAIC_BF16,
                                             nullptr) == 1);
    EXPECT(mosaic_masked_logits_device_count(H, 100, 96, idx, cnt, 10, W, 10, A16, MOSAIC_BF16, MOSAIC_BF16,
                                             nullptr) == 2);
    EXPECT(mosaic_masked_logits_device_count(H, 100, 64, idx, nullptr, 10, W, 10, A16, MOSAIC_BF16, MOSAIC_BF16,
                                             nullptr) == 1);
    EXPECT(mosaic_masked_logits_device_count(H, 100, 64, idx, cnt, 0, W, 10, nullptr, MOSAIC_BF16, MOSAIC_BF16,
                                             nullptr) == 0);
    EXPECT(mosaic_masked_logits_device_count(H, 100, 64, idx, cnt, (int64_t)1 << 31, W, 10, A16, MOSAIC_BF16,
                                             MOSAIC_BF16, nullptr) == 2);
    EXPECT(mosaic_masked_logits_device_count(H, 100, 64, idx, cnt, 10, W, 10, A16, (mosaic_dtype_t)7, MOSAIC_BF16,
                                             nullptr) == 1);
    float *f = (float *)A16;
    int32_t *ia = (int32_t *)A16;
    EXPECT(mosaic_masked_logits_argmax_lse_device_count(H, 100, 64, idx, cnt, 10, W, 50, nullptr, MOSAIC_BF16,
                                                        MOSAIC_BF16, f, ia, f, A16, 16, nullptr) == 1);   // short
    EXPECT(mosaic_masked_logits_argmax_lse_device_count(H, 100, 64, idx, nullptr, 10, W, 50, nullptr, MOSAIC_BF16,
                                                        MOSAIC_BF16, f, ia, f, A16, 1 << 20, nullptr) == 1);
    EXPECT(mosaic_masked_logits_argmax_lse_device_count(H, 100, 96, idx, cnt, 10, W, 50, nullptr, MOSAIC_BF16,
                                                        MOSAIC_BF16, f, ia, f, A16, 1 << 20, nullptr) == 2);
    EXPECT(mosaic_masked_logits_argmax_lse_device_count(H, 100, 64, idx, cnt, big, W, big, nullptr, MOSAIC_BF16,
                                                        MOSAIC_BF16, f, ia, f, A16, big, nullptr) == 1);   // overflow
    EXPECT(mosaic_masked_logits_argmax_lse(H, 100, 64, idx, 10, W, 50, nullptr, 0, MOSAIC_BF16, MOSAIC_BF16, f, ia,
                                           f, A16, 10, nullptr) == 1);   // workspace short
    EXPECT(mosaic_masked_logits_argmax_lse(H, 100, 64, idx, big, W, big, nullptr, big, MOSAIC_BF16, MOSAIC_BF16, f,
                                           ia, f, A16, big, nullptr) != 0);
    EXPECT(mosaic_masked_logits_argmax_lse_noalloc(H, 40000, 4096, idx, 6000, W, 126464, nullptr, 0, MOSAIC_BF16,
                                                   MOSAIC_BF16, f, ia, f, nullptr) == 2);   // beyond the array
    EXPECT(mosaic_masked_logits_argmax_lse_noalloc(H, 100, 64, idx, 0, W, 50, nullptr, 0, MOSAIC_BF16, MOSAIC_BF16,
                                                   nullptr, nullptr, nullptr, nullptr) == 0);
    const int64_t big8 = big / 8 * 8;   // a multiple of 8 whose products overflow
    EXPECT(mosaic_quantize_rows_fp8(H, big, big8, MOSAIC_BF16, nullptr, 10, (uint8_t *)A16, f, nullptr) == 1);
    EXPECT(mosaic_quantize_rows_fp8(H, big, big, MOSAIC_BF16, nullptr, 10, (uint8_t *)A16, f, nullptr) == 2);
    EXPECT(mosaic_masked_logits_fp8(H, 100, 128, idx, 10, (const uint8_t *)A16, f, 50, A16, 0, MOSAIC_BF16, A16,
                                    10, nullptr) == 1);   // workspace short
    EXPECT(mosaic_masked_logits_fp8(H, 100, 128, idx, big, (const uint8_t *)A16, f, big, A16, big, MOSAIC_BF16, A16,
                                    big, nullptr) == 1);
    if (failures)
        return 1;
    printf("abi sanitizer driver ok\n");
    return 0;
}

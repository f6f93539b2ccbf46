// Internal launchers of the HIP kernels (not part of the public C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mosaic {

// flag[0] = 1 if some idx[i] (i < M) is outside [0, L), else 0 (clears flag first).
hipError_t launch_idx_range_check(const int32_t *idx, int64_t M, int64_t L, int32_t *flag, hipStream_t stream);

hipError_t launch_mask_compact(const int32_t *tokens, int64_t L, int32_t mask_id, int32_t *idx,
                               int32_t *count, hipStream_t stream);
hipError_t launch_mask_compact_flags(const uint8_t *flags, int64_t L, int32_t *idx, int32_t *count,
                                     hipStream_t stream);
hipError_t launch_mask_compact_batched(const int32_t *tokens, int64_t L, const int32_t *seq_offsets,
                                       int32_t nseq, int32_t mask_id, int32_t *idx,
                                       int32_t *idx_offsets, hipStream_t stream);

// Kernel variants of the logits GEMM.  The numbers are stable identifiers (reported by
// mosaic_logits_variant and accepted by MOSAIC_TUNE); gaps are retired experiment forms.
enum LogitsVariant : int {
    kVariantF32 = 0,               // fp32 inputs: LDS-tiled FMA kernel
    kVariantBf16Simple = 2,        // bf16 inputs, any d % 8 == 0: LDS-tiled FMA kernel
    kVariantBf16PersistK32 = 11,   // bf16, d % 32 == 0: persistent 256 x 256, 4 waves, BK 32, 4 stages
    kVariantBf16W8K64S2 = 12,      // bf16, d % 64 == 0: 256 x 256, 8 waves, BK 64 (the bf16 -> fp32 default)
    kVariantBf16DeferS4I8 = 16,    // bf16 -> bf16, d % 64 == 0: persistent 8-wave, 32 x 32 x 16 MFMA,
                                   // half the stores deferred over 4 K steps (comparison form)
    kVariantBf16M16S1 = 19,        // bf16 -> bf16, d % 64 == 0: persistent 8-wave, 16 x 16 x 32 MFMA,
                                   // every wave requests K tiles
    kVariantBf16LowMShared = 20,   // bf16, d % 64 == 0, M <= 64: W streaming with a workgroup-shared H tile
    kVariantBf16M16Dma4 = 21,      // bf16 -> bf16, d % 64 == 0: as 19, K tiles requested by one wave per
                                   // SIMD
    kVariantBf16M16Dma4W3 = 22,    // as 21 with a third W stage (the bf16-output default)
};

// Default number of row tiles that share the W slabs of one XCD (tile order).
constexpr int kDefaultGroupM = 8;



// Whether a chunk of `rows` rows over V vocabulary rows fits the variant's launch grid.
bool gather_gemm_grid_fits(int variant, int64_t rows, int64_t V);

// One chunk: out[i, v] for i < rows, v < V, out row stride ldo elements.
hipError_t launch_gather_gemm(int variant, const void *H, const int32_t *idx, int64_t rows,
                              const void *W, int64_t V, int64_t d, void *out, int64_t ldo,
                              bool out_bf16, int group_m, hipStream_t stream);

// One launch whose row count is read by the kernel from device memory: rows =
// clamp(*rows_dev, 0, max_rows) (bf16 -> bf16, d % 64 == 0; the default persistent form,
// its grid sized for max_rows).
hipError_t launch_gather_gemm_device_rows(const void *H, const int32_t *idx, const int32_t *rows_dev,
                                          int64_t max_rows, const void *W, int64_t V, int64_t d, void *out,
                                          int64_t ldo, int group_m, hipStream_t stream);

// One chunk of the per-row consumer (bf16 in, d % 64 == 0): the persistent kernel
// reduces every (row, 256-entry vocabulary tile) to a partial in pmax / parg / psum
// ([ceil(V/256)][rows] each) and, when `out` is not null, also stores the bf16 logits;
// a finish kernel combines the partials into row_max / row_argmax / row_lse.  With rows_dev,
// both kernels take clamp(*rows_dev, 0, rows) rows from device memory (rows is then the
// capacity: the grids and the partials' row stride).  m16 selects
// the 16 x 16 x 32 MFMA form of the kernel (else 32 x 32 x 16); the two give the same
// logits, maxima and argmax, and exp sums added in different orders.
hipError_t launch_logits_argmax_lse(const void *H, const int32_t *idx, int64_t rows, const void *W, int64_t V,
                                    int64_t d, void *out, int64_t ldo, float *pmax, int32_t *parg, float *psum,
                                    float *row_max, int32_t *row_argmax, float *row_lse, int group_m,
                                    bool m16, hipStream_t stream, const int32_t *rows_dev = nullptr);

// FP8 LM head.  Quantize `rows` rows of X ([*, d], bf16 or fp32, d % 8 == 0; row r is
// source row row_idx[r], or r when row_idx is null) to E4M3 codes q ([rows, d]) and
// fp32 row scales.
hipError_t launch_quantize_rows_e4m3(const void *X, bool in_bf16, int64_t d, const int32_t *row_idx, int64_t rows,
                                     uint8_t *q, float *scale, hipStream_t stream);

// out[i, v] (bf16) = (sum_k Hq[i, k] Wq[v, k]) * hs[i] * ws[v] for i < rows, v < V;
// d % 128 == 0; nwaves 4 or 8: the comparison forms with every wave requesting K tiles,
// anything else: the default (eight waves, four requesting, three W stages).  All three
// give the same bits.
hipError_t launch_gemm_fp8(const uint8_t *Hq, const float *hs, int64_t rows, const uint8_t *Wq, const float *ws,
                           int64_t V, int64_t d, void *out, int64_t ldo, int group_m, int nwaves, hipStream_t stream);

// The same logits for rows <= 64 (d % 128 == 0): a W-streaming kernel, bit-identical to
// launch_gemm_fp8.
hipError_t launch_gemm_fp8_lowm(const uint8_t *Hq, const float *hs, int64_t rows, const uint8_t *Wq, const float *ws,
                                int64_t V, int64_t d, void *out, int64_t ldo, hipStream_t stream);

}  // namespace mosaic

/* Host sanitizer run of the CPU oracle (test infrastructure): every oracle entry point on
 * tiny inputs, edge cases included (empty sequences, rows at both ends, chunk tails), so
 * that AddressSanitizer and UndefinedBehaviorSanitizer see each loop and index.  Values
 * are pinned elsewhere; this only asserts counts that are fixed by construction. */
#include <assert.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int64_t oracle_mask_compact(const int32_t *tokens, int64_t L, int32_t mask_id, int32_t *idx);
int64_t oracle_mask_compact_flags(const uint8_t *flags, int64_t L, int32_t *idx);
int64_t oracle_mask_compact_batched(const int32_t *tokens, const int32_t *seq_offsets, int32_t nseq,
                                    int32_t mask_id, int32_t *idx, int32_t *idx_offsets);
int64_t oracle_num_chunks(int64_t M, int64_t C);
void oracle_chunk_range(int64_t M, int64_t C, int64_t k, int64_t *r0, int64_t *r1);
int oracle_lazy_chunk_rows(int64_t M, int64_t V, int64_t esize, int64_t budget, int64_t *chunk_rows,
                           int64_t *num_chunks);
int oracle_masked_logits_bf16(const uint16_t *H, int64_t L, int64_t d, const int32_t *idx, int64_t M,
                              const uint16_t *W, int64_t V, const int64_t *rows, int64_t nrows, double *out);
int oracle_masked_logits_f32(const float *H, int64_t L, int64_t d, const int32_t *idx, int64_t M,
                             const float *W, int64_t V, const int64_t *rows, int64_t nrows, double *out);
int oracle_masked_logits_chunked_bf16(const uint16_t *H, int64_t L, int64_t d, const int32_t *idx, int64_t M,
                                      const uint16_t *W, int64_t V, int64_t C, double *out);
int oracle_masked_logits_argmax_lse_bf16(const uint16_t *H, int64_t L, int64_t d, const int32_t *idx, int64_t M,
                                         const uint16_t *W, int64_t V, const int64_t *rows, int64_t nrows,
                                         double *row_max, int64_t *row_argmax, double *row_lse);
double oracle_e4m3_value(uint8_t c);
uint8_t oracle_e4m3_encode(float x);
int oracle_quantize_rows_e4m3(const void *X, int64_t nsrc, int64_t d, int in_bf16, const int32_t *row_idx,
                              int64_t rows, uint8_t *q, float *scale);
int oracle_logits_fp8(const uint8_t *qh, const float *scale_h, int64_t M, const uint8_t *qw, const float *scale_w,
                      int64_t V, int64_t d, const int64_t *rows, int64_t nrows, double *out);
int64_t oracle_logits_bytes(int64_t rows, int64_t V, int64_t esize);

static uint16_t bf16_of(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    return (uint16_t)(u >> 16);
}

int main(void)
{
    enum { L = 37, D = 24, V = 19 };
    int32_t tokens[L], idx[L], off[5];
    uint8_t flags[L];
    int32_t seq[5] = {0, 0, 10, 30, L};                       /* an empty sequence first */
    for (int p = 0; p < L; ++p) {
        tokens[p] = (p % 3 == 0 || p == L - 1) ? 7 : p % 5;
        flags[p] = (uint8_t)(tokens[p] == 7);
    }
    int64_t want = 0;
    for (int p = 0; p < L; ++p)
        want += tokens[p] == 7;
    int64_t M = oracle_mask_compact(tokens, L, 7, idx);
    assert(M == want && idx[0] == 0 && idx[M - 1] == L - 1);
    assert(oracle_mask_compact(tokens, 0, 7, idx) == 0);
    assert(oracle_mask_compact_flags(flags, L, idx) == M);
    assert(oracle_mask_compact_batched(tokens, seq, 4, 7, idx, off) == M && off[4] == M && off[1] == 0);
    for (int64_t C = -1; C <= M + 1; ++C) {
        int64_t K = oracle_num_chunks(M, C), r0, r1, rows = 0;
        for (int64_t k = 0; k < K; ++k) {
            oracle_chunk_range(M, C, k, &r0, &r1);
            rows += r1 - r0;
        }
        assert(rows == M);
    }
    int64_t cr, nc;
    assert(oracle_lazy_chunk_rows(M, V, 2, 5 * V * 2, &cr, &nc) == 0 && nc == 3);
    assert(oracle_logits_bytes(16, 126464, 2) * 2048 == 8287944704LL);

    uint16_t Hb[L * D], Wb[V * D];
    float Hf[L * D], Wf[V * D];
    for (int i = 0; i < L * D; ++i) {
        Hf[i] = (float)((i * 7919) % 13) / 4.0f - 1.5f;
        Hb[i] = bf16_of(Hf[i]);
    }
    for (int i = 0; i < V * D; ++i) {
        Wf[i] = (float)((i * 104729) % 11) / 8.0f - 0.625f;
        Wb[i] = bf16_of(Wf[i]);
    }
    oracle_mask_compact(tokens, L, 7, idx);
    double *out = malloc(sizeof(double) * M * V), *out2 = malloc(sizeof(double) * M * V);
    double rmax[L], rlse[L];
    int64_t rarg[L], rows[L];
    for (int64_t i = 0; i < M; ++i)
        rows[i] = i;
    const int64_t bad_row = M;
    assert(oracle_masked_logits_bf16(Hb, L, D, idx, M, Wb, V, &bad_row, 1, out) == -1);
    assert(oracle_masked_logits_bf16(Hb, L, D, idx, M, Wb, V, rows, M, out) == 0);
    assert(oracle_masked_logits_f32(Hf, L, D, idx, M, Wf, V, rows, M, out2) == 0);
    for (int64_t C = 0; C <= M + 1; ++C) {
        assert(oracle_masked_logits_chunked_bf16(Hb, L, D, idx, M, Wb, V, C, out2) == 0);
        assert(memcmp(out, out2, sizeof(double) * M * V) == 0);
    }
    assert(oracle_masked_logits_argmax_lse_bf16(Hb, L, D, idx, M, Wb, V, rows, M, rmax, rarg, rlse) == 0);
    for (int64_t i = 0; i < M; ++i)
        assert(rarg[i] >= 0 && rarg[i] < V && rlse[i] >= rmax[i]);

    for (int c = 0; c < 256; ++c) {
        const double v = oracle_e4m3_value((uint8_t)c);
        if (!isnan(v))
            assert(oracle_e4m3_encode((float)v) == (uint8_t)c || v == 0.0);
    }
    uint8_t qh[L * D], qw[V * D];
    float sh[L], sw[V];
    assert(oracle_quantize_rows_e4m3(Hb, L, D, 1, idx, M, qh, sh) == 0);
    assert(oracle_quantize_rows_e4m3(Wf, V, D, 0, NULL, V, qw, sw) == 0);
    assert(oracle_logits_fp8(qh, sh, M, qw, sw, V, D, rows, M, out) == 0);
    free(out);
    free(out2);
    printf("oracle sanitizer driver ok: M=%lld\n", (long long)M);
    return 0;
}

/*
 * CPU oracle for the mask-only logits path -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
 * load this library.  The product path (the HIP library and its binding) never
 * links, loads or calls it.  It shares no code, header or table with the HIP path.
 *
 * What it computes is the plain definition of each step, written out:
 *
 *  (1) compaction -- the list of masked positions in ascending order.  The pages
 *      take "the mask indices" as an input of the fused kernel ("Mosaic: Unlocking
 *      Long-Context Inference for Diffusion LLMs via Global Memory" review, 核心组件
 *      1. Mask-only Logits Kernel; "扩散大语言模型内存优化：Mosaic系统突破与实践",
 *      §2.2 indirect addressing through the mask index).  Ascending order is the
 *      reading taken where the pages are silent.
 *
 *  (2) chunk partition -- dLLM-Serve's logit budget ("扩散大语言模型内存优化：从理论
 *      到系统设计", §3.2.2): when the number of rows that need logits exceeds
 *      max_num_logits, rows are processed in consecutive micro-batches of at most
 *      max_num_logits rows and the results are concatenated in order.
 *
 *  (3) logits -- the LM head applied to the masked rows only: row i of the output is
 *      H[idx[i], :] . W^T (Mosaic review, 核心观察 #2: only masked tokens are sampled,
 *      so logits are computed for them alone; the Mosaic abstract states that the
 *      system preserves exact model outputs, so these rows equal the dense logits'
 *      rows).  Each element is an fp64 sum over k in ascending order of exact fp64
 *      products (bf16 and fp32 inputs convert to fp64 exactly; products of two bf16
 *      or two fp32 values are exact in fp64).  No bias, scale or softcap: the pages
 *      name only the lm_head projection.
 *
 *  (2b) lazy chunk choice -- Mosaic's lazy chunking applied to the logits operator
 *      ("扩散大语言模型内存优化：Mosaic系统突破与实践", §2.3; Mosaic review, 核心组件 3):
 *      chunking is off unless the memory available for the logits is too small, and
 *      then the smallest number of chunks that fits is used.  The oracle searches k =
 *      1, 2, ... and stops at the first k whose largest chunk, ceil(M / k) rows, fits
 *      the byte budget; the chunks are then ceil(M / k) rows each (the last shorter).
 *
 *  (5) FP8 LM head -- "扩散大语言模型内存优化：从理论到系统设计", §5 names combining the
 *      logits micro-batching with FP8 quantization as a next step, without a scheme.
 *      The plainest reading: OCP FP8 E4M3 codes (4 exponent bits, bias 7, 3 mantissa
 *      bits, largest finite value 448, subnormals 2^-9 apart) with one fp32 scale per
 *      row of W and per masked row of H.  A row x is quantized as
 *          amax = max_k |x_k|, scale = amax / 448, q_k = RNE_e4m3(x_k * (448 / amax))
 *      with each fp32 operation rounded to nearest even (a zero row gives zero codes
 *      and scale 0).  The logits are the exact dot product of the decoded codes times
 *      both row scales: out[i, v] = (sum_k q_h[i][k] q_w[v][k]) * scale_h[i] * scale_w[v],
 *      in fp64 (products of E4M3 values are exact, and 4096-term sums of them fit in
 *      the 53-bit significand).
 *
 *  (4) per-row consumer -- what the sampler reads from a masked row's logits z[v]:
 *      the largest logit, the first vocabulary index that attains it (greedy
 *      decoding), and log(sum_v exp z[v]), from which the softmax confidence of any
 *      token follows.  The pages say only that the masked tokens' logits are sampled
 *      (Mosaic review, 核心观察 #2) and that a micro-batch's logits can be freed as
 *      soon as they are consumed ("扩散大语言模型内存优化：从理论到系统设计", §3.2.3);
 *      they do not define the sampler, so these three reductions are the plainest
 *      reading.  The logits are (3)'s fp64 values; the log-sum-exp subtracts the
 *      maximum before exponentiating (the textbook stable form) and uses libm exp/log.
 *
 * Parallelism: OpenMP over output elements (rows for (4)).  It does not change any
 * arithmetic; every element is still one ascending-k fp64 sum.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- (1) compaction */

/* idx[0..M) = ascending p in [0, L) with tokens[p] == mask_id.  Returns M. */
int64_t oracle_mask_compact(const int32_t *tokens, int64_t L, int32_t mask_id, int32_t *idx)
{
    int64_t m = 0;
    for (int64_t p = 0; p < L; ++p)
        if (tokens[p] == mask_id)
            idx[m++] = (int32_t)p;
    return m;
}

/* Same, with a flag array: position p is masked when flags[p] != 0. */
int64_t oracle_mask_compact_flags(const uint8_t *flags, int64_t L, int32_t *idx)
{
    int64_t m = 0;
    for (int64_t p = 0; p < L; ++p)
        if (flags[p] != 0)
            idx[m++] = (int32_t)p;
    return m;
}

/* Ragged batch over concatenated sequences: sequence s owns positions
 * [seq_offsets[s], seq_offsets[s+1]).  idx holds global positions, sequence by
 * sequence; idx_offsets[s] is where sequence s starts in idx, idx_offsets[nseq] = M. */
int64_t oracle_mask_compact_batched(const int32_t *tokens, const int32_t *seq_offsets, int32_t nseq,
                                    int32_t mask_id, int32_t *idx, int32_t *idx_offsets)
{
    int64_t m = 0;
    for (int32_t s = 0; s < nseq; ++s) {
        idx_offsets[s] = (int32_t)m;
        for (int64_t p = seq_offsets[s]; p < seq_offsets[s + 1]; ++p)
            if (tokens[p] == mask_id)
                idx[m++] = (int32_t)p;
    }
    idx_offsets[nseq] = (int32_t)m;
    return m;
}

/* ---------------------------------------------------------- (2) chunk partition */

/* Number of micro-batches for M rows with at most C rows each.  C <= 0 means no
 * limit.  M <= C is a single call of the LM head; M == 0 is no work. */
int64_t oracle_num_chunks(int64_t M, int64_t C)
{
    if (M <= 0)
        return 0;
    if (C <= 0 || M <= C)
        return 1;
    return (M + C - 1) / C;
}

/* Rows [*r0, *r1) of chunk k: consecutive slices of C rows, the last one shorter. */
void oracle_chunk_range(int64_t M, int64_t C, int64_t k, int64_t *r0, int64_t *r1)
{
    if (C <= 0 || M <= C) {
        *r0 = 0;
        *r1 = M;
        return;
    }
    *r0 = k * C;
    *r1 = (k + 1) * C < M ? (k + 1) * C : M;
}

/* (2b) Lazy chunk choice for M rows of V entries of esize bytes under a budget of
 * `budget` bytes for the logits buffer.  Sets *chunk_rows (0 = no chunking) and
 * *num_chunks.  Returns 0, or -1 when one row does not fit (V * esize > budget) or an
 * argument is negative. */
int oracle_lazy_chunk_rows(int64_t M, int64_t V, int64_t esize, int64_t budget, int64_t *chunk_rows,
                           int64_t *num_chunks)
{
    if (M < 0 || V < 0 || esize <= 0 || budget < 0)
        return -1;
    if (M == 0) {
        *chunk_rows = 0;
        *num_chunks = 0;
        return 0;
    }
    for (int64_t k = 1; k <= M; ++k) {
        const int64_t rows = (M + k - 1) / k;            /* the largest chunk */
        /* rows * V * esize <= budget, without overflow */
        const int fits = V == 0 || (rows <= budget / esize / V && rows * V * esize <= budget);
        if (fits) {
            *chunk_rows = (k == 1) ? 0 : rows;
            *num_chunks = k;
            return 0;
        }
    }
    return -1;
}

/* ------------------------------------------------------------------ (3) logits */

/* bfloat16 is the upper half of an IEEE-754 binary32: widen exactly. */
static double bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double lm_head_dot_bf16(const uint16_t *h_row, const uint16_t *w_row, int64_t d)
{
    double acc = 0.0;
    for (int64_t k = 0; k < d; ++k)
        acc += bf16_value(h_row[k]) * bf16_value(w_row[k]);
    return acc;
}

static double lm_head_dot_f32(const float *h_row, const float *w_row, int64_t d)
{
    double acc = 0.0;
    for (int64_t k = 0; k < d; ++k)
        acc += (double)h_row[k] * (double)w_row[k];
    return acc;
}

/* out[r][v] = logits of output row rows[r] (an index into idx[0..M)) against every
 * vocabulary row v < V:  sum_k H[idx[rows[r]]][k] * W[v][k].  H is [L, d] and W is
 * [V, d], both row-major bfloat16 bit patterns.  out is [nrows][V] fp64.
 * Returns 0, or -1 when an index is out of range. */
int oracle_masked_logits_bf16(const uint16_t *H, int64_t L, int64_t d, const int32_t *idx, int64_t M,
                              const uint16_t *W, int64_t V, const int64_t *rows, int64_t nrows,
                              double *out)
{
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= M || idx[rows[r]] < 0 || idx[rows[r]] >= L)
            return -1;
    int64_t total = nrows * V;
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < total; ++e) {
        int64_t r = e / V, v = e % V;
        const uint16_t *h_row = H + (int64_t)idx[rows[r]] * d;
        out[e] = lm_head_dot_bf16(h_row, W + v * d, d);
    }
    return 0;
}

int oracle_masked_logits_f32(const float *H, int64_t L, int64_t d, const int32_t *idx, int64_t M,
                             const float *W, int64_t V, const int64_t *rows, int64_t nrows,
                             double *out)
{
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= M || idx[rows[r]] < 0 || idx[rows[r]] >= L)
            return -1;
    int64_t total = nrows * V;
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < total; ++e) {
        int64_t r = e / V, v = e % V;
        const float *h_row = H + (int64_t)idx[rows[r]] * d;
        out[e] = lm_head_dot_f32(h_row, W + v * d, d);
    }
    return 0;
}

/* The chunked logits operator as dLLM-Serve's micro-batching describes it: run the
 * LM head on each slice of at most C rows and concatenate the slices in order.
 * out is [M][V] fp64. */
int oracle_masked_logits_chunked_bf16(const uint16_t *H, int64_t L, int64_t d, const int32_t *idx,
                                      int64_t M, const uint16_t *W, int64_t V, int64_t C, double *out)
{
    for (int64_t i = 0; i < M; ++i)
        if (idx[i] < 0 || idx[i] >= L)
            return -1;
    int64_t K = oracle_num_chunks(M, C);
    for (int64_t k = 0; k < K; ++k) {
        int64_t r0, r1;
        oracle_chunk_range(M, C, k, &r0, &r1);
        /* LM head over the slice idx[r0..r1); its rows land at rows r0.. of out. */
        int64_t total = (r1 - r0) * V;
        double *chunk_out = out + r0 * V;
#pragma omp parallel for schedule(static)
        for (int64_t e = 0; e < total; ++e) {
            int64_t r = r0 + e / V, v = e % V;
            chunk_out[e] = lm_head_dot_bf16(H + (int64_t)idx[r] * d, W + v * d, d);
        }
    }
    return 0;
}

/* ------------------------------------------------------- (4) per-row consumer */

/* For each output row rows[r] (an index into idx[0..M)): its logits z[v] = (3) for
 * v < V, then
 *   row_max[r]    = max_v z[v]
 *   row_argmax[r] = the smallest v with z[v] == row_max[r]
 *   row_lse[r]    = row_max[r] + log(sum_v exp(z[v] - row_max[r])).
 * bf16 H and W as in (3).  V must be >= 1.  Returns 0, -1 for an index out of range,
 * -2 when V < 1 or a row buffer cannot be allocated. */
int oracle_masked_logits_argmax_lse_bf16(const uint16_t *H, int64_t L, int64_t d, const int32_t *idx,
                                         int64_t M, const uint16_t *W, int64_t V, const int64_t *rows,
                                         int64_t nrows, double *row_max, int64_t *row_argmax,
                                         double *row_lse)
{
    if (V < 1)
        return -2;
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= M || idx[rows[r]] < 0 || idx[rows[r]] >= L)
            return -1;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        double *z = (double *)malloc((size_t)V * sizeof(double));
        if (!z) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        const uint16_t *h_row = H + (int64_t)idx[rows[r]] * d;
        for (int64_t v = 0; v < V; ++v)
            z[v] = lm_head_dot_bf16(h_row, W + v * d, d);
        double m = z[0];
        int64_t am = 0;
        for (int64_t v = 1; v < V; ++v)
            if (z[v] > m) {
                m = z[v];
                am = v;
            }
        double s = 0.0;
        for (int64_t v = 0; v < V; ++v)
            s += exp(z[v] - m);
        row_max[r] = m;
        row_argmax[r] = am;
        row_lse[r] = m + log(s);
        free(z);
    }
    return failed ? -2 : 0;
}

/* ----------------------------------------------------------- (5) FP8 LM head */

/* Value of an OCP FP8 E4M3 code: sign bit 7, exponent bits 6..3 (bias 7), mantissa
 * bits 2..0; exponent 0 is subnormal (m/8 * 2^-6); exponent 15 with mantissa 7 is NaN. */
double oracle_e4m3_value(uint8_t c)
{
    const double sgn = (c & 0x80) ? -1.0 : 1.0;
    const int e = (c >> 3) & 0xF, m = c & 7;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        return sgn * ldexp((double)m / 8.0, -6);
    return sgn * ldexp(1.0 + (double)m / 8.0, e - 7);
}

/* Nearest E4M3 code to x (ties to the code with an even mantissa), saturating at
 * +-448; NaN gives the NaN code.  The finite non-negative codes 0x00..0x7E are
 * increasing in value, so the nearest one is found by bisection for the first code
 * not below |x| and a comparison with the code before it. */
uint8_t oracle_e4m3_encode(float x)
{
    if (isnan(x))
        return 0x7F;
    const uint8_t sgn = signbit(x) ? 0x80 : 0x00;
    const double a = fabs((double)x);
    if (a >= 448.0)
        return (uint8_t)(sgn | 0x7E);
    int lo = 0, hi = 0x7E;           /* value(hi) >= a */
    while (lo < hi) {
        const int mid = (lo + hi) / 2;
        if (oracle_e4m3_value((uint8_t)mid) < a)
            lo = mid + 1;
        else
            hi = mid;
    }
    int best = lo;
    if (lo > 0) {
        const double up = oracle_e4m3_value((uint8_t)lo) - a;
        const double down = a - oracle_e4m3_value((uint8_t)(lo - 1));
        if (down < up || (down == up && ((lo - 1) & 1) == 0))
            best = lo - 1;
    }
    return (uint8_t)(sgn | best);
}

static float row_value(const void *X, int in_bf16, int64_t off)
{
    if (in_bf16) {
        uint32_t u = (uint32_t)((const uint16_t *)X)[off] << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return f;
    }
    return ((const float *)X)[off];
}

/* Quantize `rows` rows of X ([*, d], bf16 when in_bf16 else fp32) to E4M3 codes q
 * ([rows, d]) and fp32 scales.  Row r is source row row_idx[r] (or r when row_idx is
 * NULL).  Returns 0, or -1 for a source row outside [0, nsrc). */
int oracle_quantize_rows_e4m3(const void *X, int64_t nsrc, int64_t d, int in_bf16, const int32_t *row_idx,
                              int64_t rows, uint8_t *q, float *scale)
{
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t src = row_idx ? (int64_t)row_idx[r] : r;
        if (src < 0 || src >= nsrc)
            return -1;
    }
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t src = row_idx ? (int64_t)row_idx[r] : r;
        float amax = 0.0f;
        for (int64_t k = 0; k < d; ++k) {
            const float a = fabsf(row_value(X, in_bf16, src * d + k));
            if (a > amax)
                amax = a;
        }
        if (amax == 0.0f) {
            memset(q + r * d, 0, (size_t)d);
            scale[r] = 0.0f;
            continue;
        }
        const volatile float inv = 448.0f / amax;    /* one fp32 division, rounded */
        scale[r] = amax / 448.0f;
        for (int64_t k = 0; k < d; ++k) {
            const volatile float y = row_value(X, in_bf16, src * d + k) * inv;   /* fp32 product */
            q[r * d + k] = oracle_e4m3_encode(y);
        }
    }
    return 0;
}

/* out[r][v] = (sum_k value(qh[rows[r]][k]) * value(qw[v][k])) * scale_h[rows[r]] * scale_w[v]
 * for the quantized rows qh ([M, d]) and qw ([V, d]); fp64, ascending k.  Returns 0,
 * or -1 for a row outside [0, M). */
int oracle_logits_fp8(const uint8_t *qh, const float *scale_h, int64_t M, const uint8_t *qw,
                      const float *scale_w, int64_t V, int64_t d, const int64_t *rows, int64_t nrows,
                      double *out)
{
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= M)
            return -1;
    double lut[256];
    for (int c = 0; c < 256; ++c)
        lut[c] = oracle_e4m3_value((uint8_t)c);
    const int64_t total = nrows * V;
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < total; ++e) {
        const int64_t r = e / V, v = e % V;
        const uint8_t *a = qh + rows[r] * d, *b = qw + v * d;
        double acc = 0.0;
        for (int64_t k = 0; k < d; ++k)
            acc += lut[a[k]] * lut[b[k]];
        out[e] = acc * (double)scale_h[rows[r]] * (double)scale_w[v];
    }
    return 0;
}

/* Number of OpenMP threads the logits loops run on (1 when built without OpenMP). */
#ifdef _OPENMP
#include <omp.h>
int oracle_num_threads(void) { return omp_get_max_threads(); }
/* Threads of the later parallel loops of the calling thread (n >= 1). */
void oracle_set_num_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
#else
int oracle_num_threads(void) { return 1; }
void oracle_set_num_threads(int n) { (void)n; }
#endif

/* Bytes of a logits tensor of `rows` rows over a vocabulary of V entries with
 * `esize`-byte elements: rows * V * esize ("扩散大语言模型内存优化：从理论到系统设计",
 * §2.2, where the dense [B, L, V] logits of a batch are sized this way).  Returns -1
 * on overflow of a signed 64-bit count. */
int64_t oracle_logits_bytes(int64_t rows, int64_t V, int64_t esize)
{
    if (rows < 0 || V < 0 || esize <= 0)
        return -1;
    if (rows != 0 && V > INT64_MAX / rows)
        return -1;
    int64_t n = rows * V;
    if (n != 0 && esize > INT64_MAX / n)
        return -1;
    return n * esize;
}

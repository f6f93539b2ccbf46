/*
 * mosaic.h -- C ABI of the mask-only logits hot path on AMD Instinct MI355X (gfx950).
 *
 * The path has three steps, each an entry point below:
 *
 *   1. compaction   mask (token ids or flags) -> ascending list idx[M] of masked rows;
 *   2. logits       logits[M, V] = H[idx, :] . W^T, a gather fused into the GEMM: the
 *                   masked rows are read from the full hidden states through idx and
 *                   no gathered copy of H is ever written;
 *   3. chunking     step 2 in consecutive row slices of at most max_num_logits rows.
 *
 * Sources (web pages on Mosaic, a diffusion-LLM memory system):
 *   [MR]  "Mosaic: Unlocking Long-Context Inference for Diffusion LLMs via Global
 *         Memory" (paper review, xllm-io.github.io), 核心观察 #2 (logits over unmasked
 *         tokens are wasted work; only masked tokens are sampled) and 核心组件
 *         "1. Mask-only Logits Kernel" (the kernel takes all tokens' hidden states and
 *         the mask indices, tiles the work over the compute units, addresses rows
 *         indirectly through the indices, needs no intermediate buffer, runs as one
 *         launch).
 *   [MP]  "扩散大语言模型内存优化：Mosaic系统突破与实践" (jsqmd.com), §2.2 (gather-GEMM
 *         fusion: indirect addressing through the mask index into the original hidden
 *         states; tiles over compute units; on-chip staging, no global temporary).
 *   [DS]  "扩散大语言模型内存优化：从理论到系统设计" (cnnetsun.cn), §3.2.2 (when more
 *         rows need logits than max_num_logits, process them in micro-batches of at most
 *         max_num_logits rows and concatenate the results in order) and §2.2 (the
 *         logits tensor of a batch is rows x V elements).
 *   [MA]  Mosaic abstract (zhuanzhiai.com): the system preserves exact model outputs,
 *         i.e. the mask-only rows equal the dense logits' rows.
 *
 * Conventions shared by every entry point
 *   - Every array pointer is a DEVICE pointer owned by the caller.  The library never
 *     allocates, frees or synchronises (the MOSAIC_CHECK_IDX=1 debug mode below
 *     excepted); all work is enqueued on `stream` (a hipStream_t passed as void*,
 *     NULL = the null stream) and is asynchronous.
 *   - Every function returns a status and prints nothing.  All argument validation
 *     happens before anything is enqueued; on INVALID_ARG or UNSUPPORTED no output
 *     is touched.  MOSAIC_ERR_DEVICE means a launch failed (earlier chunks of a
 *     chunked call may already be written; rerunning the call rewrites them).
 *   - Calls on different streams are independent; the library holds no state.
 *   - Sizes are int64_t; positions and row ids are int32_t (so L < 2^31).
 */
#ifndef MOSAIC_H
#define MOSAIC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* In C++ the enums take int as their fixed underlying type, so that every int a C caller
 * passes is a valid value (out-of-range codes are then rejected, not undefined). */
#ifdef __cplusplus
#define MOSAIC_INT_ENUM : int
#else
#define MOSAIC_INT_ENUM
#endif

typedef enum MOSAIC_INT_ENUM {
    MOSAIC_OK = 0,
    MOSAIC_ERR_INVALID_ARG = 1,   /* null pointer, negative size, misalignment, overflow */
    MOSAIC_ERR_UNSUPPORTED = 2,   /* valid but not supported: dtype pair, d not a multiple of 8 */
    MOSAIC_ERR_DEVICE = 3         /* a HIP launch failed */
} mosaic_status_t;

typedef enum MOSAIC_INT_ENUM {
    MOSAIC_F32 = 0,               /* IEEE binary32 */
    MOSAIC_BF16 = 1               /* bfloat16 (upper half of binary32) */
} mosaic_dtype_t;

/* Human-readable name of a status code (static string, never NULL). */
const char *mosaic_status_string(mosaic_status_t s);

/* ---------------------------------------------------------------- compaction --- */

/* Workspace bytes the three compaction calls need for L positions ([MR] 核心组件 1
 * and [MP] §2.2 take the mask indices as the kernel's input; building them needs no
 * intermediate buffer in this design).  Always 0: each workgroup counts the masked
 * positions before its own segment itself, so no cross-workgroup state exists.  The
 * calls take a workspace anyway so that a caller written against this query keeps
 * working if a later design needs one. */
size_t mosaic_mask_compact_workspace_bytes(int64_t L);

/* Step 1 for one sequence ([MR] 核心组件 1 takes "the mask indices" as an input; [MP]
 * §2.2 addresses rows through them).
 *   tokens     int32[L]  token ids; position p is masked when tokens[p] == mask_id.
 *   idx        int32[L]  capacity L; on return idx[0..M) = the masked positions in
 *                        ascending order (entries from M on are left untouched).
 *   count      int32[1]  on return M.
 *   workspace  device memory of at least mosaic_mask_compact_workspace_bytes(L) bytes
 *              (0 today: NULL with workspace_bytes 0 is the usual call); owned by the
 *              caller, untouched.
 * L == 0 writes count = 0.  L >= 2^31 -> UNSUPPORTED.  Null tokens/idx with L > 0,
 * null count, L < 0, workspace_bytes below the query's value, or a NULL workspace
 * with workspace_bytes > 0 -> INVALID_ARG.  One launch of at most 64 workgroups. */
mosaic_status_t mosaic_mask_compact(const int32_t *tokens, int64_t L, int32_t mask_id,
                                    int32_t *idx, int32_t *count,
                                    void *workspace, size_t workspace_bytes, void *stream);

/* Same as mosaic_mask_compact with a flag array: position p is masked when
 * flags[p] != 0.  flags is uint8[L]. */
mosaic_status_t mosaic_mask_compact_flags(const uint8_t *flags, int64_t L,
                                          int32_t *idx, int32_t *count,
                                          void *workspace, size_t workspace_bytes, void *stream);

/* Step 1 for a ragged batch of nseq sequences concatenated into tokens[L].
 *   seq_offsets  int32[nseq+1]  sequence s owns positions [seq_offsets[s], seq_offsets[s+1]);
 *                               the caller guarantees seq_offsets[0] = 0, nondecreasing,
 *                               seq_offsets[nseq] = L (not checked on the device).
 *   idx          int32[L]       on return the masked GLOBAL positions, sequence by
 *                               sequence, ascending within each (so ascending overall).
 *   idx_offsets  int32[nseq+1]  on return CSR offsets: sequence s's masked rows are
 *                               idx[idx_offsets[s] .. idx_offsets[s+1]); idx_offsets[nseq] = M.
 *   workspace    as for mosaic_mask_compact.
 * nseq <= 0 -> INVALID_ARG.  Two launches (compaction, then the CSR offsets). */
mosaic_status_t mosaic_mask_compact_batched(const int32_t *tokens, int64_t L,
                                            const int32_t *seq_offsets, int32_t nseq,
                                            int32_t mask_id, int32_t *idx, int32_t *idx_offsets,
                                            void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------- logits --- */

/* Steps 2 and 3: out[i, v] = sum_k H[idx[i], k] * W[v, k] for i < M, v < V
 * ([MR] 核心观察 #2 and 核心组件 1; [MP] §2.2), computed in row chunks of at most
 * chunk_rows rows, one kernel launch per chunk, written in order ([DS] §3.2.2).
 *   H      [L, d] row-major, in_dtype   final hidden states of ALL L positions.
 *   idx    int32[M]                     rows of H to use, each in [0, L); any order,
 *                                       repeats allowed.  Out-of-range values are a
 *                                       contract violation (undefined behaviour), unless
 *                                       the environment has MOSAIC_CHECK_IDX=1: then
 *                                       every logits entry point first checks idx on the
 *                                       device, waits for the answer (synchronous) and
 *                                       returns INVALID_ARG, enqueuing no compute and
 *                                       touching no output, if a value is out of range.
 *                                       This debug mode breaks two conventions above on
 *                                       purpose: it allocates a 4-byte flag once per
 *                                       (device, stream) pair, kept until the process
 *                                       ends, and it synchronises the stream.  Checked
 *                                       calls on different streams use different flags;
 *                                       checked calls that overlap on one stream from
 *                                       several host threads are not supported.
 *   W      [V, d] row-major, in_dtype   LM-head weight (K-contiguous rows).
 *   out    [M, V] row-major, out_dtype  row i holds the logits of position idx[i].
 *   chunk_rows  max_num_logits: <= 0 or >= M runs one chunk; otherwise
 *               ceil(M / chunk_rows) chunks [k*C, min(M, (k+1)*C)).  Every chunk
 *               runs the kernel variant chosen for C rows, except a last chunk of at
 *               most 64 rows, which may take the low-M streaming kernel.  All variants
 *               that one (d, dtype pair) can select add each output's products in the
 *               same order, so the output is bit-identical for every chunk_rows value.
 * Dtype pairs (in -> out): F32->F32, BF16->BF16, BF16->F32.  Products are
 * accumulated in fp32 (bf16 MFMA with fp32 accumulators; fp32 FMA for F32 inputs);
 * bf16 outputs are rounded to nearest even.
 * Requirements: d % 8 == 0 (BF16) or d % 4 == 0 (F32), else UNSUPPORTED; H, W and
 * out 16-byte aligned, else INVALID_ARG; M * V * esize must fit in int64.
 * M == 0 or V == 0: MOSAIC_OK and nothing is enqueued (pointers may be NULL).
 * Streaming use ([DS] §3.2.3, free each micro-batch early): call once per chunk with
 * idx + k*C, M = rows of chunk k, chunk_rows = 0 and a reused [C, V] buffer. */
mosaic_status_t mosaic_masked_logits(const void *H, int64_t L, int64_t d,
                                     const int32_t *idx, int64_t M,
                                     const void *W, int64_t V,
                                     void *out, int64_t chunk_rows,
                                     mosaic_dtype_t in_dtype, mosaic_dtype_t out_dtype,
                                     void *stream);

/* Steps 2 and 3 with the row count read on the device ([MR] 核心组件 1; [MP] §2.2):
 * as mosaic_masked_logits in one chunk, with M = min(max(*count, 0), max_rows) read by
 * the kernel when it starts.  count is an int32 in device memory written earlier on the
 * same stream, for example mosaic_mask_compact's count, so the host neither reads it back
 * nor waits: the compaction and the logits can be enqueued back to back (and captured in
 * a graph).  A denoising loop whose masked set only shrinks can size out once, from the
 * first step's count, and pass that as max_rows afterwards.
 *   idx       int32[max_rows]      rows of H, as in mosaic_masked_logits; only the
 *                                  first M are read.
 *   count     int32* (device)      the number of rows.  Negative values count as 0,
 *                                  values above max_rows as max_rows: nothing waits for
 *                                  the value, so no error can be reported for it.
 *   max_rows  capacity of idx and out in rows; the launch is sized for it.
 *   out       [max_rows, V]        rows < M get the logits; rows >= M are not written.
 * Supported: BF16 -> BF16 with d % 64 == 0 (the persistent kernel of the default path,
 * bit-identical to mosaic_masked_logits), else UNSUPPORTED.  Other requirements and
 * argument errors as for mosaic_masked_logits; count must be 4-byte aligned.
 * max_rows == 0 or V == 0: MOSAIC_OK and nothing is enqueued.  The MOSAIC_CHECK_IDX debug
 * check is not made here (it needs M on the host). */
mosaic_status_t mosaic_masked_logits_device_count(const void *H, int64_t L, int64_t d,
                                                  const int32_t *idx, const int32_t *count,
                                                  int64_t max_rows, const void *W, int64_t V,
                                                  void *out, mosaic_dtype_t in_dtype,
                                                  mosaic_dtype_t out_dtype, void *stream);

/* ------------------------------------------------------- per-row consumer --- */

/* The sampler's view of each masked row, reduced inside the logits kernel so a row's
 * logits are consumed as they are produced ([MR] 核心观察 #2: only masked tokens are
 * sampled; [DS] §3.2.3: a micro-batch's logits can be freed once consumed).  The pages
 * do not define the sampler; these are the plainest per-row quantities it needs
 * (greedy choice and softmax confidence).  For i < M, with z_v the fp32 logit of row i
 * (the accumulator of mosaic_masked_logits, before any bf16 rounding):
 *   row_max[i]    = max_v z_v
 *   row_argmax[i] = the smallest v with z_v == row_max[i]
 *   row_lse[i]    = row_max[i] + log(sum_v exp(z_v - row_max[i]))   (fp32)
 * softmax(z)_v = exp(z_v - row_lse[i]); the greedy token's confidence is
 * exp(row_max[i] - row_lse[i]).
 *   H, idx, W, M, chunk_rows   as for mosaic_masked_logits; in_dtype must be BF16 and
 *                              d % 64 == 0 (else UNSUPPORTED).
 *   out        NULL: the logits are never stored (no [M, V] buffer at all), or an
 *              [M, V] row-major BF16 buffer (out_dtype BF16, else UNSUPPORTED) that
 *              receives the same bits mosaic_masked_logits would write.
 *   row_max    float[M], row_argmax int32[M], row_lse float[M]: device, 4-byte aligned.
 *   workspace  device scratch of at least
 *              mosaic_logits_argmax_lse_workspace_bytes(M, chunk_rows, V) bytes,
 *              16-byte aligned; owned by the caller; its contents on entry do not
 *              matter and on return are undefined.
 * Results are deterministic and do not depend on chunk_rows.  M == 0: MOSAIC_OK and
 * nothing is enqueued.  V == 0 with M > 0, a NULL required pointer, misalignment or a
 * short workspace: INVALID_ARG; nothing is enqueued and no output is touched. */
mosaic_status_t mosaic_masked_logits_argmax_lse(const void *H, int64_t L, int64_t d,
                                                const int32_t *idx, int64_t M,
                                                const void *W, int64_t V,
                                                void *out, int64_t chunk_rows,
                                                mosaic_dtype_t in_dtype, mosaic_dtype_t out_dtype,
                                                float *row_max, int32_t *row_argmax, float *row_lse,
                                                void *workspace, int64_t workspace_bytes,
                                                void *stream);

/* The per-row consumer with the row count read on the device, as
 * mosaic_masked_logits_device_count is to mosaic_masked_logits: one chunk, M =
 * min(max(*count, 0), max_rows) read by the kernels when they start, so a sampling step
 * (compaction, then the per-row reductions) needs no read-back and no host wait.
 *   count      int32* (device); values outside [0, max_rows] are clamped (no error can be
 *              reported: nothing waits for the value).
 *   max_rows   capacity of idx, out (if given), row_max, row_argmax and row_lse in rows.
 *   workspace  at least mosaic_logits_argmax_lse_workspace_bytes(max_rows, 0, V) bytes.
 * Rows >= M of out, row_max, row_argmax and row_lse are not written.  Other arguments,
 * requirements and errors as for mosaic_masked_logits_argmax_lse (count 4-byte aligned);
 * max_rows == 0: MOSAIC_OK, nothing enqueued.  The MOSAIC_CHECK_IDX check is not made. */
mosaic_status_t mosaic_masked_logits_argmax_lse_device_count(const void *H, int64_t L, int64_t d,
                                                             const int32_t *idx, const int32_t *count,
                                                             int64_t max_rows, const void *W, int64_t V,
                                                             void *out, mosaic_dtype_t in_dtype,
                                                             mosaic_dtype_t out_dtype, float *row_max,
                                                             int32_t *row_argmax, float *row_lse,
                                                             void *workspace, int64_t workspace_bytes,
                                                             void *stream);

/* Size of the library-owned device array behind mosaic_masked_logits_argmax_lse_noalloc
 * (32 MiB; each device that runs the call holds one until the process ends). */
#define MOSAIC_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): mosaic_masked_logits_argmax_lse with
 * no workspace argument and no allocation of any kind.  The per-row partials of a chunk
 * go to a library-owned device array of MOSAIC_NOALLOC_SCRATCH_BYTES bytes per device.
 *   Arguments, results and errors as for mosaic_masked_logits_argmax_lse, except:
 *   - a call whose chunks need more than the array,
 *     mosaic_logits_argmax_lse_workspace_bytes(M, chunk_rows, V) > MOSAIC_NOALLOC_SCRATCH_BYTES
 *     (about 5,600 rows per chunk at V = 126464), returns MOSAIC_ERR_UNSUPPORTED and
 *     enqueues nothing: pass a smaller chunk_rows;
 *   - the MOSAIC_CHECK_IDX debug check is not made (it would allocate and synchronise);
 *   - every call on one device shares the array, so calls that overlap in time on one
 *     device (on different streams, or from several host threads) race and their results
 *     are undefined: serialise them.  Calls in order on one stream are safe. */
mosaic_status_t mosaic_masked_logits_argmax_lse_noalloc(const void *H, int64_t L, int64_t d,
                                                        const int32_t *idx, int64_t M,
                                                        const void *W, int64_t V,
                                                        void *out, int64_t chunk_rows,
                                                        mosaic_dtype_t in_dtype, mosaic_dtype_t out_dtype,
                                                        float *row_max, int32_t *row_argmax, float *row_lse,
                                                        void *stream);

/* Workspace bytes of mosaic_masked_logits_argmax_lse for M rows in chunks of
 * chunk_rows over V vocabulary entries: 12 * ceil(V / 256) * C, with C the rows of the
 * largest chunk (three 4-byte partials per row and 256-entry tile; one chunk's partials
 * are live at a time), 0 for M == 0, or -1 on a negative size or int64 overflow. */
int64_t mosaic_logits_argmax_lse_workspace_bytes(int64_t M, int64_t chunk_rows, int64_t V);

/* ---------------------------------------------------------- FP8 LM head --- */

/* FP8 form of the logits step ([DS] §5 names combining the logits micro-batching with
 * FP8 quantization as a next step; the scheme below is this library's reading).  Codes
 * are OCP FP8 E4M3 (bias 7, 3 mantissa bits, largest finite value 448) with one fp32
 * scale per row:  amax = max_k |x_k|,  scale = amax / 448,  q_k = RNE(x_k * (448/amax)),
 * each fp32 operation rounded to nearest even; a zero row gives zero codes and scale 0.
 *
 * mosaic_quantize_rows_fp8: rows r < rows of X ([nsrc, d], in_dtype BF16 or F32,
 * row-major, 16-byte aligned) -- source row row_idx[r] (device int32, values in
 * [0, nsrc); a caller contract) or r when row_idx is NULL -- to q ([rows, d] uint8,
 * 16-byte aligned) and scale (float[rows]).  Used once for W.  d % 8 == 0, else
 * UNSUPPORTED.  rows == 0 or d == 0: OK, nothing enqueued. */
mosaic_status_t mosaic_quantize_rows_fp8(const void *X, int64_t nsrc, int64_t d, mosaic_dtype_t in_dtype,
                                         const int32_t *row_idx, int64_t rows, uint8_t *q, float *scale,
                                         void *stream);

/* Workspace bytes of mosaic_masked_logits_fp8 for M rows in chunks of chunk_rows:
 * C * d rounded up to 16, plus 4 * C, with C the rows of the largest chunk; 0 for
 * M == 0; -1 on a negative size or overflow. */
int64_t mosaic_logits_fp8_workspace_bytes(int64_t M, int64_t chunk_rows, int64_t d);

/* out[i, v] = (sum_k q_h[i][k] * Wq[v][k]) * scale_h[i] * w_scale[v], rounded to bf16, for
 * i < M, v < V, where q_h[i], scale_h[i] quantize row H[idx[i]] as above.  Each chunk
 * quantizes its rows into `workspace` (gathered through idx; H itself is not copied),
 * then runs one fp8 MFMA GEMM (fp32 accumulation) launch.
 *   H        [L, d] bf16 row-major, 16-byte aligned;  idx int32[M] in [0, L).
 *   Wq       [V, d] E4M3 codes and w_scale float[V] (16-byte aligned), from
 *            mosaic_quantize_rows_fp8 on W.
 *   out      [M, V] bf16 (out_dtype must be BF16), 16-byte aligned.
 *   chunk_rows, stream: as for mosaic_masked_logits.
 *   workspace >= mosaic_logits_fp8_workspace_bytes(M, chunk_rows, d) bytes; 16-byte
 *            aligned; contents undefined on return.
 * d % 128 == 0 (else UNSUPPORTED).  M == 0 or V == 0: OK, nothing enqueued.  Results
 * do not depend on chunk_rows. */
mosaic_status_t mosaic_masked_logits_fp8(const void *H, int64_t L, int64_t d, const int32_t *idx, int64_t M,
                                         const uint8_t *Wq, const float *w_scale, int64_t V, void *out,
                                         int64_t chunk_rows, mosaic_dtype_t out_dtype, void *workspace,
                                         int64_t workspace_bytes, void *stream);

/* ------------------------------------------------------------ host helpers --- */

/* Number of chunks a call of mosaic_masked_logits makes for M rows ([DS] §3.2.2):
 * 0 for M <= 0, 1 for chunk_rows <= 0 or chunk_rows >= M, else ceil(M / chunk_rows). */
int64_t mosaic_num_chunks(int64_t M, int64_t chunk_rows);

/* Lazy chunk choice for the logits operator ([MP] §2.3; [MR] 核心组件 3): chunking is
 * off while the whole [M, V] buffer of out_dtype fits budget_bytes (*chunk_rows = 0,
 * *num_chunks = 1); otherwise *num_chunks = k, the smallest k whose largest chunk,
 * ceil(M / k) rows, fits, and *chunk_rows = ceil(M / k), so that passing it to
 * mosaic_masked_logits makes exactly k balanced chunks.  M == 0 gives (0, 0).
 * UNSUPPORTED when one row does not fit (V * esize > budget_bytes); INVALID_ARG on a
 * negative size, an unknown dtype or a NULL output pointer. */
mosaic_status_t mosaic_lazy_chunk_rows(int64_t M, int64_t V, mosaic_dtype_t out_dtype,
                                      int64_t budget_bytes, int64_t *chunk_rows,
                                      int64_t *num_chunks);

/* Bytes of a logits tensor of `rows` rows over V vocabulary entries of dtype `dt`
 * ([DS] §2.2): rows * V * esize, written to *bytes.  INVALID_ARG on a negative size,
 * an unknown dtype, a NULL `bytes` or overflow of int64. */
mosaic_status_t mosaic_logits_bytes(int64_t rows, int64_t V, mosaic_dtype_t dt, int64_t *bytes);

/* Which kernel variant mosaic_masked_logits runs for one launch (one chunk) of M
 * rows of this dtype pair (a stable small integer, for tests and profiles), or -1 if
 * unsupported. */
int mosaic_logits_variant(int64_t M, int64_t V, int64_t d, mosaic_dtype_t in_dtype,
                          mosaic_dtype_t out_dtype);

/* ---------------------------------------------------------------- debugging --- */

/* The library reads two debug variables from the environment once per process, at the
 * first call that needs them: MOSAIC_CHECK_IDX (see mosaic_masked_logits) and
 * MOSAIC_TUNE (forces a kernel variant or tile grouping, for tests and sweeps).  This
 * call reads them again; calls already running keep the values they started with. */
void mosaic_debug_reload_env(void);

#ifdef __cplusplus
}
#endif

#endif /* MOSAIC_H */

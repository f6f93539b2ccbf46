// C ABI of the mask-only logits path (declared in include/mosaic.h): argument
// validation, kernel-variant choice and the row-chunk driver.
//
// The chunk driver follows dLLM-Serve's logit budget ("扩散大语言模型内存优化：从理论到
// 系统设计", §3.2.2): when more rows need logits than max_num_logits, the rows are
// processed in consecutive micro-batches of at most max_num_logits rows whose outputs
// land, in order, in consecutive row ranges of `out`.  Each chunk is one launch of the
// fused gather-GEMM, which reads its rows of H through its slice of idx.
//
// Validation happens entirely on the host, before any HIP call, so a rejected call
// touches neither the device nor `out`.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <map>
#include <mutex>
#include <utility>

#include "../../include/mosaic.h"
#include "launch.h"

namespace {

constexpr int64_t kMaxPos = 0x7fffffffLL;   // positions and rows are int32

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// ceil(a / b) for a >= 0, b > 0, without the overflow of (a + b - 1) / b near INT64_MAX.
int64_t ceil_div(int64_t a, int64_t b) { return a / b + (a % b != 0); }

int64_t esize_of(mosaic_dtype_t t) { return t == MOSAIC_F32 ? 4 : (t == MOSAIC_BF16 ? 2 : 0); }

// M * V * esize without int64 overflow; -1 on overflow.
int64_t checked_bytes(int64_t rows, int64_t V, int64_t esize)
{
    if (rows < 0 || V < 0 || esize <= 0)
        return -1;
    if (rows != 0 && V > INT64_MAX / rows)
        return -1;
    const int64_t n = rows * V;
    if (n != 0 && esize > INT64_MAX / n)
        return -1;
    return n * esize;
}

// Debug/tuning override, read from the environment once per process (the first call
// that needs it) and again on mosaic_debug_reload_env():
// MOSAIC_TUNE="variant=<n>,group_m=<g>,waves=<w>,fp8lowm=0" (waves=4 or 8: the FP8 GEMM's
// comparison forms with every wave requesting K tiles, one or two waves per SIMD; default:
// eight waves, four requesting, three W stages; fp8lowm=0: FP8 chunks of at most 64 rows
// also take the tiled FP8 kernel).
// A forced variant that cannot run the call's shape is ignored.  For the fused consumer,
// variant=16 selects its 32 x 32 x 16 MFMA form (default: 16 x 16 x 32).
struct Tune {
    int variant = -1;
    int group_m = 0;
    int waves = 0;   // FP8 GEMM form: 0 = default, 4 or 8 = comparison forms
    bool fp8_lowm = true;   // FP8 chunks of at most 64 rows take the W-streaming kernel
    bool check_idx = false;   // MOSAIC_CHECK_IDX=1
};

Tune parse_env()
{
    Tune t;
    const char *c = getenv("MOSAIC_CHECK_IDX");
    t.check_idx = c && c[0] == '1';
    const char *e = getenv("MOSAIC_TUNE");
    if (!e)
        return t;
    const char *p;
    if ((p = strstr(e, "variant=")))
        t.variant = atoi(p + 8);
    if ((p = strstr(e, "group_m=")))
        t.group_m = atoi(p + 8);
    if ((p = strstr(e, "waves=")) && (atoi(p + 6) == 4 || atoi(p + 6) == 8))
        t.waves = atoi(p + 6);
    if ((p = strstr(e, "fp8lowm=")) && atoi(p + 8) == 0)
        t.fp8_lowm = false;
    return t;
}

std::mutex g_env_mu;
Tune g_env;
bool g_env_read = false;

Tune read_tune()
{
    std::lock_guard<std::mutex> lk(g_env_mu);
    if (!g_env_read) {
        g_env = parse_env();
        g_env_read = true;
    }
    return g_env;
}

// Debug mode MOSAIC_CHECK_IDX=1 (read with MOSAIC_TUNE): before any compute is
// enqueued, check on the device that every idx[i] (i < M) lies in [0, L), and wait for
// the answer.  A 4-byte device flag is allocated on first use for each (device, stream)
// pair, so checked calls on different streams never share a flag.  Returns MOSAIC_OK
// (mode off, or all indices valid), MOSAIC_ERR_INVALID_ARG (an index out of range) or
// MOSAIC_ERR_DEVICE.
mosaic_status_t check_idx_if_asked(const int32_t *idx, int64_t M, int64_t L, hipStream_t stream)
{
    if (!read_tune().check_idx)
        return MOSAIC_OK;
    static std::mutex mu;
    static std::map<std::pair<int, hipStream_t>, int32_t *> flags;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return MOSAIC_ERR_DEVICE;
    int32_t *flag = nullptr;
    {
        std::lock_guard<std::mutex> lk(mu);
        const auto key = std::make_pair(dev, stream);
        auto it = flags.find(key);
        if (it == flags.end()) {
            if (hipMalloc((void **)&flag, sizeof(int32_t)) != hipSuccess)
                return MOSAIC_ERR_DEVICE;
            flags[key] = flag;
        } else {
            flag = it->second;
        }
    }
    int32_t host = 0;
    if (mosaic::launch_idx_range_check(idx, M, L, flag, stream) != hipSuccess ||
        hipMemcpyAsync(&host, flag, sizeof host, hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return MOSAIC_ERR_DEVICE;
    return host ? MOSAIC_ERR_INVALID_ARG : MOSAIC_OK;
}

bool variant_can_run(int v, int64_t M, int64_t d, mosaic_dtype_t in, mosaic_dtype_t out)
{
    const bool bf16_in = in == MOSAIC_BF16 && (out == MOSAIC_BF16 || out == MOSAIC_F32);
    // The tiled kernels address a 256-row W slab with 32-bit byte offsets.
    const bool small_d = d <= (1 << 22);
    switch (v) {
    case mosaic::kVariantF32: return in == MOSAIC_F32 && out == MOSAIC_F32 && d % 4 == 0;
    case mosaic::kVariantBf16Simple: return bf16_in && d % 8 == 0;
    case mosaic::kVariantBf16W8K64S2: return bf16_in && d % 64 == 0 && small_d;
    case mosaic::kVariantBf16DeferS4I8:
    case mosaic::kVariantBf16M16S1:
    case mosaic::kVariantBf16M16Dma4W3:
    case mosaic::kVariantBf16M16Dma4: return in == MOSAIC_BF16 && out == MOSAIC_BF16 && d % 64 == 0 && small_d;
    case mosaic::kVariantBf16PersistK32: return bf16_in && d % 32 == 0 && small_d;
    case mosaic::kVariantBf16LowMShared: return bf16_in && d % 64 == 0 && small_d && M <= 64;
    default: return false;
    }
}

int pick_variant(int64_t M, int64_t V, int64_t d, mosaic_dtype_t in, mosaic_dtype_t out)
{
    (void)V;
    const Tune t = read_tune();
    if (t.variant >= 0 && variant_can_run(t.variant, M, d, in, out))
        return t.variant;
    if (variant_can_run(mosaic::kVariantF32, M, d, in, out))
        return mosaic::kVariantF32;
    // Every bf16 variant below for one d accumulates each output in the same MFMA k
    // order, so the choice (made per launch from its row count) never changes a bit.
    if (variant_can_run(mosaic::kVariantBf16LowMShared, M, d, in, out))
        return mosaic::kVariantBf16LowMShared;
    if (variant_can_run(mosaic::kVariantBf16M16Dma4W3, M, d, in, out))
        return mosaic::kVariantBf16M16Dma4W3;
    if (variant_can_run(mosaic::kVariantBf16W8K64S2, M, d, in, out))
        return mosaic::kVariantBf16W8K64S2;
    if (variant_can_run(mosaic::kVariantBf16PersistK32, M, d, in, out))
        return mosaic::kVariantBf16PersistK32;
    if (variant_can_run(mosaic::kVariantBf16Simple, M, d, in, out))
        return mosaic::kVariantBf16Simple;
    return -1;
}

// Scratch of mosaic_masked_logits_argmax_lse_noalloc: the per-(row, vocabulary tile)
// partials of one chunk.  Each device the library runs on holds its own copy of this array
// until the process ends; host code uses the device address from hipGetSymbolAddress,
// taken once per device with that device current, never the array's name.
static __device__ __attribute__((aligned(256))) char scratch[MOSAIC_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
std::map<int, void *> g_scratch_ptr;

// The current device's address of `scratch` (looked up on the first call on a device).
mosaic_status_t noalloc_scratch(void **ptr)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return MOSAIC_ERR_DEVICE;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    auto it = g_scratch_ptr.find(dev);
    if (it == g_scratch_ptr.end()) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return MOSAIC_ERR_DEVICE;
        it = g_scratch_ptr.emplace(dev, p).first;
    }
    *ptr = it->second;
    return MOSAIC_OK;
}

}  // namespace

extern "C" {

void mosaic_debug_reload_env(void)
{
    std::lock_guard<std::mutex> lk(g_env_mu);
    g_env = parse_env();
    g_env_read = true;
}

const char *mosaic_status_string(mosaic_status_t s)
{
    switch (s) {
    case MOSAIC_OK: return "MOSAIC_OK";
    case MOSAIC_ERR_INVALID_ARG: return "MOSAIC_ERR_INVALID_ARG";
    case MOSAIC_ERR_UNSUPPORTED: return "MOSAIC_ERR_UNSUPPORTED";
    case MOSAIC_ERR_DEVICE: return "MOSAIC_ERR_DEVICE";
    }
    return "MOSAIC_ERR_UNKNOWN";
}

int64_t mosaic_num_chunks(int64_t M, int64_t chunk_rows)
{
    if (M <= 0)
        return 0;
    if (chunk_rows <= 0 || chunk_rows >= M)
        return 1;
    return ceil_div(M, chunk_rows);
}

mosaic_status_t mosaic_logits_bytes(int64_t rows, int64_t V, mosaic_dtype_t dt, int64_t *bytes)
{
    const int64_t es = esize_of(dt);
    if (!bytes || es == 0)
        return MOSAIC_ERR_INVALID_ARG;
    const int64_t n = checked_bytes(rows, V, es);
    if (n < 0)
        return MOSAIC_ERR_INVALID_ARG;
    *bytes = n;
    return MOSAIC_OK;
}

int mosaic_logits_variant(int64_t M, int64_t V, int64_t d, mosaic_dtype_t in_dtype, mosaic_dtype_t out_dtype)
{
    return pick_variant(M, V, d, in_dtype, out_dtype);
}

size_t mosaic_mask_compact_workspace_bytes(int64_t L)
{
    (void)L;   // each workgroup recounts the prefix before its segment: no shared state
    return 0;
}

// The workspace arguments of the compaction calls: enough bytes for the query, and a
// pointer wherever bytes are claimed.
static bool compact_workspace_ok(int64_t L, const void *workspace, size_t workspace_bytes)
{
    return workspace_bytes >= mosaic_mask_compact_workspace_bytes(L) && (workspace || workspace_bytes == 0);
}

mosaic_status_t mosaic_mask_compact(const int32_t *tokens, int64_t L, int32_t mask_id, int32_t *idx,
                                    int32_t *count, void *workspace, size_t workspace_bytes, void *stream)
{
    if (L < 0 || !count || (L > 0 && (!tokens || !idx)) || !compact_workspace_ok(L, workspace, workspace_bytes))
        return MOSAIC_ERR_INVALID_ARG;
    if (L > kMaxPos)
        return MOSAIC_ERR_UNSUPPORTED;
    return mosaic::launch_mask_compact(tokens, L, mask_id, idx, count, (hipStream_t)stream) == hipSuccess
               ? MOSAIC_OK
               : MOSAIC_ERR_DEVICE;
}

mosaic_status_t mosaic_mask_compact_flags(const uint8_t *flags, int64_t L, int32_t *idx, int32_t *count,
                                          void *workspace, size_t workspace_bytes, void *stream)
{
    if (L < 0 || !count || (L > 0 && (!flags || !idx)) || !compact_workspace_ok(L, workspace, workspace_bytes))
        return MOSAIC_ERR_INVALID_ARG;
    if (L > kMaxPos)
        return MOSAIC_ERR_UNSUPPORTED;
    return mosaic::launch_mask_compact_flags(flags, L, idx, count, (hipStream_t)stream) == hipSuccess
               ? MOSAIC_OK
               : MOSAIC_ERR_DEVICE;
}

mosaic_status_t mosaic_mask_compact_batched(const int32_t *tokens, int64_t L, const int32_t *seq_offsets,
                                            int32_t nseq, int32_t mask_id, int32_t *idx,
                                            int32_t *idx_offsets, void *workspace, size_t workspace_bytes,
                                            void *stream)
{
    if (L < 0 || nseq <= 0 || !seq_offsets || !idx_offsets || (L > 0 && (!tokens || !idx)) ||
        !compact_workspace_ok(L, workspace, workspace_bytes))
        return MOSAIC_ERR_INVALID_ARG;
    if (L > kMaxPos)
        return MOSAIC_ERR_UNSUPPORTED;
    return mosaic::launch_mask_compact_batched(tokens, L, seq_offsets, nseq, mask_id, idx, idx_offsets,
                                               (hipStream_t)stream) == hipSuccess
               ? MOSAIC_OK
               : MOSAIC_ERR_DEVICE;
}

mosaic_status_t mosaic_masked_logits(const void *H, int64_t L, int64_t d, const int32_t *idx, int64_t M,
                                     const void *W, int64_t V, void *out, int64_t chunk_rows,
                                     mosaic_dtype_t in_dtype, mosaic_dtype_t out_dtype, void *stream)
{
    if (M < 0 || V < 0 || L < 0 || d < 0)
        return MOSAIC_ERR_INVALID_ARG;
    const int64_t in_es = esize_of(in_dtype), out_es = esize_of(out_dtype);
    if (in_es == 0 || out_es == 0)
        return MOSAIC_ERR_INVALID_ARG;
    if (M == 0 || V == 0)
        return MOSAIC_OK;   // no rows or no vocabulary: nothing to compute
    if (!H || !W || !idx || !out || L == 0 || d == 0)
        return MOSAIC_ERR_INVALID_ARG;
    if (!aligned16(H) || !aligned16(W) || !aligned16(out) || ((uintptr_t)idx & 3u))
        return MOSAIC_ERR_INVALID_ARG;
    if (checked_bytes(M, V, out_es) < 0 || checked_bytes(L, d, in_es) < 0 || checked_bytes(V, d, in_es) < 0)
        return MOSAIC_ERR_INVALID_ARG;
    if (L > kMaxPos || V > kMaxPos || d > kMaxPos)
        return MOSAIC_ERR_UNSUPPORTED;
    // Row chunks ([k*C, min(M, (k+1)*C))), one launch each.  All chunks run the variant
    // chosen for C rows, except a last chunk small enough for the low-M streaming
    // kernel; all chunks are checked before the first launch.
    const int64_t K = mosaic_num_chunks(M, chunk_rows);
    const int64_t C = (K == 1) ? M : chunk_rows;
    const int64_t tail = M - (K - 1) * C;
    if (C > kMaxPos)
        return MOSAIC_ERR_UNSUPPORTED;
    const int v_full = pick_variant(C, V, d, in_dtype, out_dtype);
    int v_tail = pick_variant(tail, V, d, in_dtype, out_dtype);
    if (v_tail != mosaic::kVariantBf16LowMShared)
        v_tail = v_full;
    if (v_full < 0 || v_tail < 0 || !mosaic::gather_gemm_grid_fits(v_full, C, V) ||
        !mosaic::gather_gemm_grid_fits(v_tail, tail, V))
        return MOSAIC_ERR_UNSUPPORTED;
    const mosaic_status_t ck = check_idx_if_asked(idx, M, L, (hipStream_t)stream);
    if (ck != MOSAIC_OK)
        return ck;
    const bool out_bf16 = out_dtype == MOSAIC_BF16;
    const int group_m = read_tune().group_m;
    for (int64_t k = 0; k < K; ++k) {
        const int64_t r0 = k * C;
        const int64_t r1 = (r0 + C < M) ? r0 + C : M;
        const int variant = (r1 - r0 == C) ? v_full : v_tail;
        void *chunk_out = (char *)out + r0 * V * out_es;
        const hipError_t e = mosaic::launch_gather_gemm(variant, H, idx + r0, r1 - r0, W, V, d, chunk_out, V,
                                                        out_bf16, group_m, (hipStream_t)stream);
        if (e != hipSuccess)
            return MOSAIC_ERR_DEVICE;
    }
    return MOSAIC_OK;
}

mosaic_status_t mosaic_masked_logits_device_count(const void *H, int64_t L, int64_t d, const int32_t *idx,
                                                  const int32_t *count, int64_t max_rows, const void *W, int64_t V,
                                                  void *out, mosaic_dtype_t in_dtype, mosaic_dtype_t out_dtype,
                                                  void *stream)
{
    if (max_rows < 0 || V < 0 || L < 0 || d < 0)
        return MOSAIC_ERR_INVALID_ARG;
    const int64_t in_es = esize_of(in_dtype), out_es = esize_of(out_dtype);
    if (in_es == 0 || out_es == 0)
        return MOSAIC_ERR_INVALID_ARG;
    if (in_dtype != MOSAIC_BF16 || out_dtype != MOSAIC_BF16 || d % 64 != 0)
        return MOSAIC_ERR_UNSUPPORTED;
    if (max_rows == 0 || V == 0)
        return MOSAIC_OK;
    if (!H || !W || !idx || !count || !out || L == 0 || d == 0)
        return MOSAIC_ERR_INVALID_ARG;
    if (!aligned16(H) || !aligned16(W) || !aligned16(out) || ((uintptr_t)idx & 3u) || ((uintptr_t)count & 3u))
        return MOSAIC_ERR_INVALID_ARG;
    if (checked_bytes(max_rows, V, out_es) < 0 || checked_bytes(L, d, in_es) < 0 ||
        checked_bytes(V, d, in_es) < 0)
        return MOSAIC_ERR_INVALID_ARG;
    if (L > kMaxPos || V > kMaxPos || d > kMaxPos || max_rows > kMaxPos)
        return MOSAIC_ERR_UNSUPPORTED;
    if (!variant_can_run(mosaic::kVariantBf16M16Dma4W3, max_rows, d, in_dtype, out_dtype) ||
        !mosaic::gather_gemm_grid_fits(mosaic::kVariantBf16M16Dma4W3, max_rows, V))
        return MOSAIC_ERR_UNSUPPORTED;
    const hipError_t e = mosaic::launch_gather_gemm_device_rows(H, idx, count, max_rows, W, V, d, out, V,
                                                                read_tune().group_m, (hipStream_t)stream);
    return e == hipSuccess ? MOSAIC_OK : MOSAIC_ERR_DEVICE;
}

mosaic_status_t mosaic_lazy_chunk_rows(int64_t M, int64_t V, mosaic_dtype_t out_dtype, int64_t budget_bytes,
                                      int64_t *chunk_rows, int64_t *num_chunks)
{
    const int64_t es = esize_of(out_dtype);
    if (M < 0 || V < 0 || budget_bytes < 0 || es == 0 || !chunk_rows || !num_chunks)
        return MOSAIC_ERR_INVALID_ARG;
    if (M == 0) {
        *chunk_rows = 0;
        *num_chunks = 0;
        return MOSAIC_OK;
    }
    const int64_t all = checked_bytes(M, V, es);
    if (all >= 0 && all <= budget_bytes) {   // the whole buffer fits: chunking stays off
        *chunk_rows = 0;
        *num_chunks = 1;
        return MOSAIC_OK;
    }
    // rows that fit: r = floor(budget / (V * es)); the fewest chunks is ceil(M / r), and
    // balanced chunks of ceil(M / k) rows (<= r) give exactly k chunks in the driver
    const int64_t r = budget_bytes / es / V;
    if (r < 1)
        return MOSAIC_ERR_UNSUPPORTED;
    const int64_t k = ceil_div(M, r);
    *chunk_rows = ceil_div(M, k);
    *num_chunks = k;
    return MOSAIC_OK;
}

// Rows of the largest chunk of a call over M rows ([DS] §3.2.2): M when unchunked.
static int64_t largest_chunk_rows(int64_t M, int64_t chunk_rows)
{
    return mosaic_num_chunks(M, chunk_rows) <= 1 ? (M > 0 ? M : 0) : chunk_rows;
}

// The consumer's partials for launches of `rows` rows: 12 * ceil(V / 256) * rows bytes.
static int64_t argmax_lse_partials_bytes(int64_t rows, int64_t V)
{
    if (rows < 0 || V < 0)
        return -1;
    const int64_t ncol = ceil_div(V, 256);
    const int64_t n = checked_bytes(ncol, rows, 12);
    return n < 0 ? -1 : n;
}

int64_t mosaic_logits_argmax_lse_workspace_bytes(int64_t M, int64_t chunk_rows, int64_t V)
{
    if (M < 0 || V < 0)
        return -1;
    return argmax_lse_partials_bytes(largest_chunk_rows(M, chunk_rows), V);
}

// Shared body of the two consumer entry points.  noalloc: the partials go to this
// library's scratch array (workspace and workspace_bytes are ignored), and the idx debug
// check, which allocates and synchronises, is not made.
static mosaic_status_t argmax_lse_impl(const void *H, int64_t L, int64_t d, const int32_t *idx, int64_t M,
                                       const void *W, int64_t V, void *out, int64_t chunk_rows,
                                       mosaic_dtype_t in_dtype, mosaic_dtype_t out_dtype, float *row_max,
                                       int32_t *row_argmax, float *row_lse, void *workspace,
                                       int64_t workspace_bytes, bool noalloc, void *stream)
{
    if (M < 0 || V < 0 || L < 0 || d < 0)
        return MOSAIC_ERR_INVALID_ARG;
    if (esize_of(in_dtype) == 0 || (out && esize_of(out_dtype) == 0))
        return MOSAIC_ERR_INVALID_ARG;
    if (M == 0)
        return MOSAIC_OK;   // no rows: nothing to compute
    if (V == 0)
        return MOSAIC_ERR_INVALID_ARG;   // the maximum of an empty row does not exist
    if (in_dtype != MOSAIC_BF16 || (out && out_dtype != MOSAIC_BF16))
        return MOSAIC_ERR_UNSUPPORTED;
    if (d % 64 != 0 || d > (1 << 22))
        return MOSAIC_ERR_UNSUPPORTED;
    if (!H || !W || !idx || !row_max || !row_argmax || !row_lse || (!noalloc && !workspace) || L == 0 || d == 0)
        return MOSAIC_ERR_INVALID_ARG;
    if (!aligned16(H) || !aligned16(W) || (out && !aligned16(out)) || (!noalloc && !aligned16(workspace)) ||
        ((uintptr_t)idx & 3u) || ((uintptr_t)row_max & 3u) || ((uintptr_t)row_argmax & 3u) ||
        ((uintptr_t)row_lse & 3u))
        return MOSAIC_ERR_INVALID_ARG;
    if ((out && checked_bytes(M, V, 2) < 0) || checked_bytes(L, d, 2) < 0 || checked_bytes(V, d, 2) < 0)
        return MOSAIC_ERR_INVALID_ARG;
    if (L > kMaxPos || V > kMaxPos || d > kMaxPos)
        return MOSAIC_ERR_UNSUPPORTED;
    const int64_t K = mosaic_num_chunks(M, chunk_rows);
    const int64_t C = (K == 1) ? M : chunk_rows;
    if (C > kMaxPos || !mosaic::gather_gemm_grid_fits(mosaic::kVariantBf16DeferS4I8, C, V))
        return MOSAIC_ERR_UNSUPPORTED;
    const int64_t need = argmax_lse_partials_bytes(C, V);
    if (need < 0)
        return MOSAIC_ERR_INVALID_ARG;
    if (noalloc) {
        if (need > (int64_t)MOSAIC_NOALLOC_SCRATCH_BYTES)
            return MOSAIC_ERR_UNSUPPORTED;     // the partials of one chunk exceed the scratch array
        const mosaic_status_t sc = noalloc_scratch(&workspace);
        if (sc != MOSAIC_OK)
            return sc;
    } else if (workspace_bytes < need) {
        return MOSAIC_ERR_INVALID_ARG;
    }
    // workspace: pmax, parg, psum, each [ceil(V/256)][C] 4-byte words; every entry is written
    // by a chunk's GEMM launch before that chunk's finish kernel reads it, so nothing needs
    // clearing
    const int64_t plane = ceil_div(V, 256) * C;
    float *pmax = (float *)workspace;
    int32_t *parg = (int32_t *)(pmax + plane);
    float *psum = (float *)(parg + plane);
    if (!noalloc) {
        const mosaic_status_t ck = check_idx_if_asked(idx, M, L, (hipStream_t)stream);
        if (ck != MOSAIC_OK)
            return ck;
    }
    const Tune t = read_tune();
    const bool m16 = t.variant != mosaic::kVariantBf16DeferS4I8;   // 32 x 32 x 16 form on request
    for (int64_t k = 0; k < K; ++k) {
        const int64_t r0 = k * C;
        const int64_t r1 = (r0 + C < M) ? r0 + C : M;
        void *chunk_out = out ? (char *)out + r0 * V * 2 : nullptr;
        const hipError_t e = mosaic::launch_logits_argmax_lse(H, idx + r0, r1 - r0, W, V, d, chunk_out, V, pmax,
                                                              parg, psum, row_max + r0, row_argmax + r0,
                                                              row_lse + r0, t.group_m, m16, (hipStream_t)stream);
        if (e != hipSuccess)
            return MOSAIC_ERR_DEVICE;
    }
    return MOSAIC_OK;
}

mosaic_status_t mosaic_masked_logits_argmax_lse_device_count(const void *H, int64_t L, int64_t d, const int32_t *idx,
                                                             const int32_t *count, int64_t max_rows, const void *W,
                                                             int64_t V, void *out, mosaic_dtype_t in_dtype,
                                                             mosaic_dtype_t out_dtype, float *row_max,
                                                             int32_t *row_argmax, float *row_lse, void *workspace,
                                                             int64_t workspace_bytes, void *stream)
{
    if (max_rows < 0 || V < 0 || L < 0 || d < 0)
        return MOSAIC_ERR_INVALID_ARG;
    if (esize_of(in_dtype) == 0 || (out && esize_of(out_dtype) == 0))
        return MOSAIC_ERR_INVALID_ARG;
    if (max_rows == 0)
        return MOSAIC_OK;
    if (V == 0)
        return MOSAIC_ERR_INVALID_ARG;   // the maximum of an empty row does not exist
    if (in_dtype != MOSAIC_BF16 || (out && out_dtype != MOSAIC_BF16))
        return MOSAIC_ERR_UNSUPPORTED;
    if (d % 64 != 0 || d > (1 << 22))
        return MOSAIC_ERR_UNSUPPORTED;
    if (!H || !W || !idx || !count || !row_max || !row_argmax || !row_lse || !workspace || L == 0 || d == 0)
        return MOSAIC_ERR_INVALID_ARG;
    if (!aligned16(H) || !aligned16(W) || (out && !aligned16(out)) || !aligned16(workspace) ||
        ((uintptr_t)idx & 3u) || ((uintptr_t)count & 3u) || ((uintptr_t)row_max & 3u) ||
        ((uintptr_t)row_argmax & 3u) || ((uintptr_t)row_lse & 3u))
        return MOSAIC_ERR_INVALID_ARG;
    if ((out && checked_bytes(max_rows, V, 2) < 0) || checked_bytes(L, d, 2) < 0 || checked_bytes(V, d, 2) < 0)
        return MOSAIC_ERR_INVALID_ARG;
    if (L > kMaxPos || V > kMaxPos || d > kMaxPos || max_rows > kMaxPos ||
        !mosaic::gather_gemm_grid_fits(mosaic::kVariantBf16DeferS4I8, max_rows, V))
        return MOSAIC_ERR_UNSUPPORTED;
    const int64_t need = argmax_lse_partials_bytes(max_rows, V);
    if (need < 0 || workspace_bytes < need)
        return MOSAIC_ERR_INVALID_ARG;
    const int64_t plane = ceil_div(V, 256) * max_rows;
    float *pmax = (float *)workspace;
    int32_t *parg = (int32_t *)(pmax + plane);
    float *psum = (float *)(parg + plane);
    const Tune t = read_tune();
    const bool m16 = t.variant != mosaic::kVariantBf16DeferS4I8;
    const hipError_t e = mosaic::launch_logits_argmax_lse(H, idx, max_rows, W, V, d, out, V, pmax, parg, psum,
                                                          row_max, row_argmax, row_lse, t.group_m, m16,
                                                          (hipStream_t)stream, count);
    return e == hipSuccess ? MOSAIC_OK : MOSAIC_ERR_DEVICE;
}

mosaic_status_t mosaic_masked_logits_argmax_lse(const void *H, int64_t L, int64_t d, const int32_t *idx, int64_t M,
                                                const void *W, int64_t V, void *out, int64_t chunk_rows,
                                                mosaic_dtype_t in_dtype, mosaic_dtype_t out_dtype, float *row_max,
                                                int32_t *row_argmax, float *row_lse, void *workspace,
                                                int64_t workspace_bytes, void *stream)
{
    return argmax_lse_impl(H, L, d, idx, M, W, V, out, chunk_rows, in_dtype, out_dtype, row_max, row_argmax,
                           row_lse, workspace, workspace_bytes, false, stream);
}

mosaic_status_t mosaic_masked_logits_argmax_lse_noalloc(const void *H, int64_t L, int64_t d, const int32_t *idx,
                                                        int64_t M, const void *W, int64_t V, void *out,
                                                        int64_t chunk_rows, mosaic_dtype_t in_dtype,
                                                        mosaic_dtype_t out_dtype, float *row_max,
                                                        int32_t *row_argmax, float *row_lse, void *stream)
{
    return argmax_lse_impl(H, L, d, idx, M, W, V, out, chunk_rows, in_dtype, out_dtype, row_max, row_argmax,
                           row_lse, nullptr, 0, true, stream);
}

mosaic_status_t mosaic_quantize_rows_fp8(const void *X, int64_t nsrc, int64_t d, mosaic_dtype_t in_dtype,
                                         const int32_t *row_idx, int64_t rows, uint8_t *q, float *scale,
                                         void *stream)
{
    if (nsrc < 0 || d < 0 || rows < 0 || esize_of(in_dtype) == 0)
        return MOSAIC_ERR_INVALID_ARG;
    if (rows == 0 || d == 0)
        return MOSAIC_OK;
    if (d % 8 != 0)
        return MOSAIC_ERR_UNSUPPORTED;
    if (!X || !q || !scale || nsrc == 0 || (!row_idx && rows > nsrc))
        return MOSAIC_ERR_INVALID_ARG;
    if (!aligned16(X) || !aligned16(q) || ((uintptr_t)scale & 3u) || ((uintptr_t)row_idx & 3u))
        return MOSAIC_ERR_INVALID_ARG;
    if (checked_bytes(nsrc, d, esize_of(in_dtype)) < 0 || checked_bytes(rows, d, 1) < 0)
        return MOSAIC_ERR_INVALID_ARG;
    if (d > kMaxPos)
        return MOSAIC_ERR_UNSUPPORTED;
    return mosaic::launch_quantize_rows_e4m3(X, in_dtype == MOSAIC_BF16, d, row_idx, rows, q, scale,
                                             (hipStream_t)stream) == hipSuccess
               ? MOSAIC_OK
               : MOSAIC_ERR_DEVICE;
}

// The FP8 path's per-chunk buffer for launches of `rows` rows: codes [rows, d] (padded to
// 16 bytes), then the row scales.
static int64_t fp8_chunk_bytes(int64_t rows, int64_t d)
{
    const int64_t codes = checked_bytes(rows, d, 1);
    if (codes < 0 || rows < 0)
        return -1;
    if (codes > INT64_MAX - 15)
        return -1;
    const int64_t aligned = ceil_div(codes, 16) * 16;
    if (aligned > INT64_MAX - 4 * rows)
        return -1;
    return aligned + 4 * rows;
}

int64_t mosaic_logits_fp8_workspace_bytes(int64_t M, int64_t chunk_rows, int64_t d)
{
    if (M < 0 || d < 0)
        return -1;
    return fp8_chunk_bytes(largest_chunk_rows(M, chunk_rows), d);
}

mosaic_status_t mosaic_masked_logits_fp8(const void *H, int64_t L, int64_t d, const int32_t *idx, int64_t M,
                                         const uint8_t *Wq, const float *w_scale, int64_t V, void *out,
                                         int64_t chunk_rows, mosaic_dtype_t out_dtype, void *workspace,
                                         int64_t workspace_bytes, void *stream)
{
    if (M < 0 || V < 0 || L < 0 || d < 0 || esize_of(out_dtype) == 0)
        return MOSAIC_ERR_INVALID_ARG;
    if (M == 0 || V == 0)
        return MOSAIC_OK;
    if (out_dtype != MOSAIC_BF16 || d % 128 != 0 || d > (1 << 22))
        return MOSAIC_ERR_UNSUPPORTED;
    if (!H || !idx || !Wq || !w_scale || !out || !workspace || L == 0 || d == 0)
        return MOSAIC_ERR_INVALID_ARG;
    if (!aligned16(H) || !aligned16(Wq) || !aligned16(out) || !aligned16(workspace) || ((uintptr_t)idx & 3u) ||
        ((uintptr_t)w_scale & 15u))
        return MOSAIC_ERR_INVALID_ARG;
    if (checked_bytes(M, V, 2) < 0 || checked_bytes(L, d, 2) < 0 || checked_bytes(V, d, 1) < 0)
        return MOSAIC_ERR_INVALID_ARG;
    if (L > kMaxPos || V > kMaxPos || d > kMaxPos)
        return MOSAIC_ERR_UNSUPPORTED;
    const int64_t K = mosaic_num_chunks(M, chunk_rows);
    const int64_t C = (K == 1) ? M : chunk_rows;
    if (C > kMaxPos || ((C + 255) / 256) * ((V + 255) / 256) > 0x7fffffffLL)
        return MOSAIC_ERR_UNSUPPORTED;
    const int64_t need = fp8_chunk_bytes(C, d);
    if (need < 0 || workspace_bytes < need)
        return MOSAIC_ERR_INVALID_ARG;
    // workspace: the chunk's codes [C, d], then its row scales [C]
    uint8_t *hq = (uint8_t *)workspace;
    float *hs = (float *)(hq + (C * d + 15) / 16 * 16);
    const mosaic_status_t ck = check_idx_if_asked(idx, M, L, (hipStream_t)stream);
    if (ck != MOSAIC_OK)
        return ck;
    const Tune t = read_tune();
    for (int64_t k = 0; k < K; ++k) {
        const int64_t r0 = k * C;
        const int64_t r1 = (r0 + C < M) ? r0 + C : M;
        void *chunk_out = (char *)out + r0 * V * 2;
        const bool lowm = t.fp8_lowm && r1 - r0 <= 64;
        if (mosaic::launch_quantize_rows_e4m3(H, true, d, idx + r0, r1 - r0, hq, hs, (hipStream_t)stream) !=
                hipSuccess ||
            (lowm ? mosaic::launch_gemm_fp8_lowm(hq, hs, r1 - r0, Wq, w_scale, V, d, chunk_out, V, (hipStream_t)stream)
                  : mosaic::launch_gemm_fp8(hq, hs, r1 - r0, Wq, w_scale, V, d, chunk_out, V, t.group_m, t.waves,
                                            (hipStream_t)stream)) != hipSuccess)
            return MOSAIC_ERR_DEVICE;
    }
    return MOSAIC_OK;
}

}  // extern "C"

// Stream compaction of a mask into the ascending list of masked positions.
//
// The fused logits kernel reads the masked rows of the hidden states through a
// list of mask indices ("Mosaic: Unlocking Long-Context Inference for Diffusion
// LLMs via Global Memory" review, 核心组件 1. Mask-only Logits Kernel;
// "扩散大语言模型内存优化：Mosaic系统突破与实践", §2.2).  This kernel builds that
// list from token ids (or flags) on the device.
//
// Design (gfx950, wave64): the sequence is cut into G <= 64 segments, a multiple of
// the tile size each, one workgroup of 16 waves per segment.  A workgroup first counts
// the masked positions before its segment: it re-reads that prefix itself with 16-byte
// loads (the prefix is at most the whole input, 512 KiB for 2^17 positions, and comes
// from L2 and the Infinity Cache), so no cross-workgroup scan, flag protocol or
// workspace is needed, and the result does not depend on timing.  It then walks its
// segment in tiles of 16 x 64 x ITEMS positions.  Wave w owns a contiguous run of
// 64*ITEMS positions of the tile; for each group of 64 it takes a 64-bit ballot of
// "masked", so the rank of a lane among the masked lanes before it is mbcnt(ballot)
// and the wave's count is popcount(ballot).  The 16 wave counts are scanned through
// LDS, which gives every wave its output offset inside the tile; a running base
// carries the count across tiles.  Positions are therefore written in ascending order,
// and the result is unique (bit-identical to any correct compaction).  The last
// workgroup writes the total.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <stdint.h>

#include "launch.h"

namespace mosaic {
namespace {

constexpr int kWaves = 16;
constexpr int kThreads = kWaves * 64;
constexpr int kItems = 8;   // groups of 64 positions per wave per tile

__device__ __forceinline__ uint32_t rank_below(uint64_t mask)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

constexpr int64_t kTile = (int64_t)kThreads * kItems;   // positions per tile
constexpr int kMaxSegments = 64;

// Masked positions among [0, n) counted by this thread's share (n % 16 == 0).
template <typename T, bool kFlags>
__device__ __forceinline__ uint32_t count_prefix(const T *__restrict__ in, int64_t n, int32_t mask_id)
{
    uint32_t c = 0;
    const bool vec = ((uintptr_t)in & 15) == 0;
    if constexpr (kFlags) {
        if (vec) {
            const uint4 *v = (const uint4 *)in;
            const int64_t n16 = n / 16;
            auto nz = [](uint32_t w) {
                return (uint32_t)((w & 0xffu) != 0) + (uint32_t)((w & 0xff00u) != 0) +
                       (uint32_t)((w & 0xff0000u) != 0) + (uint32_t)((w & 0xff000000u) != 0);
            };
#pragma unroll 4
            for (int64_t i = threadIdx.x; i < n16; i += kThreads) {
                const uint4 x = v[i];
                c += nz(x.x) + nz(x.y) + nz(x.z) + nz(x.w);
            }
            return c;
        }
#pragma unroll 4
        for (int64_t p = threadIdx.x; p < n; p += kThreads)
            c += in[p] != 0;
    } else {
        if (vec) {
            const int4 *v = (const int4 *)in;
            const int64_t n4 = n / 4;
#pragma unroll 4
            for (int64_t i = threadIdx.x; i < n4; i += kThreads) {
                const int4 x = v[i];
                c += (uint32_t)(x.x == mask_id) + (uint32_t)(x.y == mask_id) + (uint32_t)(x.z == mask_id) +
                     (uint32_t)(x.w == mask_id);
            }
            return c;
        }
#pragma unroll 4
        for (int64_t p = threadIdx.x; p < n; p += kThreads)
            c += in[p] == mask_id;
    }
    return c;
}

template <typename T, bool kFlags>
__global__ __launch_bounds__(kThreads) void mask_compact_kernel(const T *__restrict__ in, int64_t L,
                                                                int32_t mask_id, int64_t seg,
                                                                int32_t *__restrict__ idx,
                                                                int32_t *__restrict__ count)
{
    __shared__ uint32_t wave_count[kWaves];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t s0 = (int64_t)blockIdx.x * seg;
    const int64_t s1 = s0 + seg < L ? s0 + seg : L;

    // masked positions before this segment: per-thread counts, summed over the wave and
    // then over the 16 waves
    uint32_t c = count_prefix<T, kFlags>(in, s0, mask_id);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        c += __shfl_xor(c, o, 64);
    if (lane == 0)
        wave_count[wave] = c;
    __syncthreads();
    uint32_t base = 0;   // masked positions before the current tile (same in every thread)
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
        base += wave_count[w];
    __syncthreads();     // wave_count is rewritten by the first tile

    for (int64_t t0 = s0; t0 < s1; t0 += kTile) {
        const int64_t w0 = t0 + (int64_t)wave * 64 * kItems;
        uint64_t masks[kItems];
        uint32_t wave_total = 0;
#pragma unroll
        for (int j = 0; j < kItems; ++j) {
            const int64_t p = w0 + j * 64 + lane;
            bool hit = false;
            if (p < s1) {
                if constexpr (kFlags)
                    hit = in[p] != 0;
                else
                    hit = in[p] == mask_id;
            }
            masks[j] = __ballot(hit);
            wave_total += (uint32_t)__popcll(masks[j]);
        }
        if (lane == 0)
            wave_count[wave] = wave_total;
        __syncthreads();
        uint32_t before = 0, tile_total = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const uint32_t cw = wave_count[w];
            before += (w < wave) ? cw : 0u;
            tile_total += cw;
        }
        __syncthreads();   // wave_count is rewritten by the next tile

        uint32_t off = base + before;
#pragma unroll
        for (int j = 0; j < kItems; ++j) {
            if ((masks[j] >> lane) & 1ull)
                idx[off + rank_below(masks[j])] = (int32_t)(w0 + j * 64 + lane);
            off += (uint32_t)__popcll(masks[j]);
        }
        base += tile_total;
    }
    if (blockIdx.x == gridDim.x - 1 && threadIdx.x == 0)
        *count = (int32_t)base;
}

// G segments of seg positions (a multiple of the tile), G <= kMaxSegments, G * seg >= L;
// at least one workgroup, so that an empty input still writes its count.
void segments(int64_t L, int64_t &seg, unsigned &G)
{
    const int64_t tiles = std::max<int64_t>(1, (L + kTile - 1) / kTile);
    const int64_t g = std::min<int64_t>(tiles, kMaxSegments);
    seg = (tiles + g - 1) / g * kTile;
    G = (unsigned)std::max<int64_t>(1, (L + seg - 1) / seg);
}

// idx_offsets[s] = number of masked positions before seq_offsets[s], found by binary
// search in the ascending global list (lower bound).  The last entry is the total.
__global__ __launch_bounds__(256) void csr_offsets_kernel(const int32_t *__restrict__ idx,
                                                          const int32_t *__restrict__ seq_offsets,
                                                          int32_t nseq, int32_t *__restrict__ idx_offsets)
{
    const int s = blockIdx.x * blockDim.x + threadIdx.x;
    if (s >= nseq)
        return;
    const int32_t M = idx_offsets[nseq];   // the compaction kernel left the total here
    const int32_t key = seq_offsets[s];
    int32_t lo = 0, hi = M;
    while (lo < hi) {
        const int32_t mid = lo + ((hi - lo) >> 1);
        if (idx[mid] < key)
            lo = mid + 1;
        else
            hi = mid;
    }
    idx_offsets[s] = lo;
}

// Index-list check (debug mode of the logits entry points): flag[0] is set to 1 when
// some idx[i], i < M, lies outside [0, L).  Only the lanes that find a bad index store,
// all the same value, so no atomic is needed.
__global__ __launch_bounds__(256) void idx_range_check_kernel(const int32_t *__restrict__ idx, int64_t M,
                                                              int64_t L, int32_t *__restrict__ flag)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < M; i += (int64_t)gridDim.x * 256) {
        const int32_t v = idx[i];
        if (v < 0 || (int64_t)v >= L)
            flag[0] = 1;
    }
}

__global__ void flag_clear_kernel(int32_t *__restrict__ flag)
{
    if (threadIdx.x == 0)
        flag[0] = 0;
}

}  // namespace

hipError_t launch_idx_range_check(const int32_t *idx, int64_t M, int64_t L, int32_t *flag, hipStream_t stream)
{
    hipLaunchKernelGGL(flag_clear_kernel, dim3(1), dim3(64), 0, stream, flag);
    if (M > 0) {
        const int64_t blocks = std::min<int64_t>((M + 255) / 256, 1024);
        hipLaunchKernelGGL(idx_range_check_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, idx, M, L, flag);
    }
    return hipGetLastError();
}

hipError_t launch_mask_compact(const int32_t *tokens, int64_t L, int32_t mask_id, int32_t *idx,
                               int32_t *count, hipStream_t stream)
{
    int64_t seg;
    unsigned G;
    segments(L, seg, G);
    hipLaunchKernelGGL((mask_compact_kernel<int32_t, false>), dim3(G), dim3(kThreads), 0, stream,
                       tokens, L, mask_id, seg, idx, count);
    return hipGetLastError();
}

hipError_t launch_mask_compact_flags(const uint8_t *flags, int64_t L, int32_t *idx, int32_t *count,
                                     hipStream_t stream)
{
    int64_t seg;
    unsigned G;
    segments(L, seg, G);
    hipLaunchKernelGGL((mask_compact_kernel<uint8_t, true>), dim3(G), dim3(kThreads), 0, stream,
                       flags, L, 0, seg, idx, count);
    return hipGetLastError();
}

hipError_t launch_mask_compact_batched(const int32_t *tokens, int64_t L, const int32_t *seq_offsets,
                                       int32_t nseq, int32_t mask_id, int32_t *idx,
                                       int32_t *idx_offsets, hipStream_t stream)
{
    // Ascending global positions are already grouped by sequence, so the batched list
    // is the flat compaction; its total goes to idx_offsets[nseq].
    int64_t seg;
    unsigned G;
    segments(L, seg, G);
    hipLaunchKernelGGL((mask_compact_kernel<int32_t, false>), dim3(G), dim3(kThreads), 0, stream,
                       tokens, L, mask_id, seg, idx, idx_offsets + nseq);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int blocks = (nseq + 255) / 256;
    hipLaunchKernelGGL(csr_offsets_kernel, dim3(blocks), dim3(256), 0, stream, idx, seq_offsets, nseq,
                       idx_offsets);
    return hipGetLastError();
}

}  // namespace mosaic

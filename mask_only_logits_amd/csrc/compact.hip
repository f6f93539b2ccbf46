// Stream compaction of a mask into the ascending list of masked positions.
//
// The fused logits kernel reads the masked rows of the hidden states through a
// list of mask indices ("Mosaic: Unlocking Long-Context Inference for Diffusion
// LLMs via Global Memory" review, 核心组件 1. Mask-only Logits Kernel;
// "扩散大语言模型内存优化：Mosaic系统突破与实践", §2.2).  This kernel builds that
// list from token ids (or flags) on the device.
//
// Design (gfx950, wave64): one workgroup of 16 waves walks the sequence in tiles of
// 16 x 64 x ITEMS positions.  Wave w owns a contiguous run of 64*ITEMS positions of
// the tile; for each group of 64 it takes a 64-bit ballot of "masked", so the rank
// of a lane among the masked lanes before it is mbcnt(ballot) and the wave's count is
// popcount(ballot).  The 16 wave counts are scanned through LDS, which gives every
// wave its output offset inside the tile; a running base carries the count across
// tiles.  Positions are therefore written in ascending order, and the result is
// unique (bit-identical to any correct compaction).  The whole input is read once
// with coalesced loads; at the sizes of a sequence (<= 2^17 positions, 512 KiB)
// a single workgroup finishes in a few microseconds, so no cross-workgroup scan
// (and no workspace) is needed.
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

template <typename T, bool kFlags>
__global__ __launch_bounds__(kThreads) void mask_compact_kernel(const T *__restrict__ in, int64_t L,
                                                                int32_t mask_id,
                                                                int32_t *__restrict__ idx,
                                                                int32_t *__restrict__ count)
{
    __shared__ uint32_t wave_count[kWaves];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    uint32_t base = 0;   // masked positions before the current tile (same in every thread)

    for (int64_t t0 = 0; t0 < L; t0 += (int64_t)kThreads * kItems) {
        const int64_t w0 = t0 + (int64_t)wave * 64 * kItems;
        uint64_t masks[kItems];
        uint32_t wave_total = 0;
#pragma unroll
        for (int j = 0; j < kItems; ++j) {
            const int64_t p = w0 + j * 64 + lane;
            bool hit = false;
            if (p < L) {
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
            const uint32_t c = wave_count[w];
            before += (w < wave) ? c : 0u;
            tile_total += c;
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
    if (threadIdx.x == 0)
        *count = (int32_t)base;
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
    hipLaunchKernelGGL((mask_compact_kernel<int32_t, false>), dim3(1), dim3(kThreads), 0, stream,
                       tokens, L, mask_id, idx, count);
    return hipGetLastError();
}

hipError_t launch_mask_compact_flags(const uint8_t *flags, int64_t L, int32_t *idx, int32_t *count,
                                     hipStream_t stream)
{
    hipLaunchKernelGGL((mask_compact_kernel<uint8_t, true>), dim3(1), dim3(kThreads), 0, stream,
                       flags, L, 0, idx, count);
    return hipGetLastError();
}

hipError_t launch_mask_compact_batched(const int32_t *tokens, int64_t L, const int32_t *seq_offsets,
                                       int32_t nseq, int32_t mask_id, int32_t *idx,
                                       int32_t *idx_offsets, hipStream_t stream)
{
    // Ascending global positions are already grouped by sequence, so the batched list
    // is the flat compaction; its total goes to idx_offsets[nseq].
    hipLaunchKernelGGL((mask_compact_kernel<int32_t, false>), dim3(1), dim3(kThreads), 0, stream,
                       tokens, L, mask_id, idx, idx_offsets + nseq);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int blocks = (nseq + 255) / 256;
    hipLaunchKernelGGL(csr_offsets_kernel, dim3(blocks), dim3(256), 0, stream, idx, seq_offsets, nseq,
                       idx_offsets);
    return hipGetLastError();
}

}  // namespace mosaic

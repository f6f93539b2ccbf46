// Epilogue helpers shared by the low-M streaming kernels (bf16 and FP8): a 32-row
// vocabulary block's results, held in registers and stored in bursts.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mosaic {
namespace lowm {

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// two floats to a pair of bf16 (round to nearest even)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    __bf16 a = static_cast<__bf16>(lo), b = static_cast<__bf16>(hi);
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// Vocabulary range of wave g of nw (g = nw gives the end, V): [bound(g), bound(g + 1)).
// Boundaries are g * V / nw rounded down to a multiple of 8 rows, so each lane's
// 4-entry store run starts 4-aligned and takes the vector store path.
__device__ __forceinline__ int range_bound(int64_t g, int64_t nw, int V)
{
    return g >= nw ? V : (int)(((g * V) / nw) & ~(int64_t)7);
}

// 32-row blocks of the longest range (at most ceil(V / nw) + 7 rows): every wave runs
// this many, padding blocks included.
__device__ __forceinline__ int range_blocks(int64_t nw, int V)
{
    return (int)(((V + nw - 1) / nw + 7 + 31) / 32);
}

// Low-M epilogue: store one finished 32-vocabulary-row block (AM x 32 masked rows) whose
// first vocabulary row is vb; rows >= `rows` and vocabulary rows >= v_hi are not stored.
// Lane (fr, hi) holds, in accumulators 4 gq .. 4 gq + 3 of block bm, vocabulary rows
// vb + 8 gq + 4 hi .. + 3 of masked row bm * 32 + fr.
template <int AM, bool OUT_BF16>
__device__ __forceinline__ void lowm_store_block(const f32x16_t (&res)[AM], int vb, int v_hi, int rows, int fr,
                                                 int hi, void *__restrict__ out, int64_t ldo)
{
#pragma unroll
    for (int bm = 0; bm < AM; ++bm) {
        const int row = bm * 32 + fr;
        if (row >= rows)
            continue;
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            const int v = vb + gq * 8 + hi * 4;
            const float x0 = res[bm][gq * 4 + 0], x1 = res[bm][gq * 4 + 1];
            const float x2 = res[bm][gq * 4 + 2], x3 = res[bm][gq * 4 + 3];
            // a vector store needs its address aligned to its size (8 or 16 bytes)
            const bool full = v + 3 < v_hi && (ldo & 3) == 0 && (v & 3) == 0;
            if constexpr (OUT_BF16) {
                __bf16 *o = (__bf16 *)out + (int64_t)row * ldo + v;
                if (full) {
                    uint2 p;
                    p.x = pack_bf16x2(x0, x1);
                    p.y = pack_bf16x2(x2, x3);
                    *(uint2 *)o = p;
                } else {
                    if (v + 0 < v_hi) o[0] = static_cast<__bf16>(x0);
                    if (v + 1 < v_hi) o[1] = static_cast<__bf16>(x1);
                    if (v + 2 < v_hi) o[2] = static_cast<__bf16>(x2);
                    if (v + 3 < v_hi) o[3] = static_cast<__bf16>(x3);
                }
            } else {
                float *o = (float *)out + (int64_t)row * ldo + v;
                if (full) {
                    *(f32x4_t *)o = f32x4_t{x0, x1, x2, x3};
                } else {
                    if (v + 0 < v_hi) o[0] = x0;
                    if (v + 1 < v_hi) o[1] = x1;
                    if (v + 2 < v_hi) o[2] = x2;
                    if (v + 3 < v_hi) o[3] = x3;
                }
            }
        }
    }
}

// Low-M block results are held in registers, NBK blocks at most, and stored in one burst
// when the wave's range ends or the registers are full.  Stores count in the same in-order
// vmcnt as the DMA loads, so a store issued in the K loop would make the next K tile's wait
// also wait for the store to be acknowledged by memory; holding the results keeps that
// wait out of the stream.  `held` is oldest first; block blk has just finished into acc.
template <int AM, int NBK, bool OUT_BF16>
__device__ __forceinline__ void lowm_block_done(f32x16_t (&held)[NBK][AM], f32x16_t (&acc)[AM], int blk,
                                                int nblocks, int v_lo, int v_hi, int rows, int fr, int hi,
                                                void *__restrict__ out, int64_t ldo)
{
#pragma unroll
    for (int i = 0; i + 1 < NBK; ++i)
#pragma unroll
        for (int bm = 0; bm < AM; ++bm)
            held[i][bm] = held[i + 1][bm];
#pragma unroll
    for (int bm = 0; bm < AM; ++bm) {
        held[NBK - 1][bm] = acc[bm];
#pragma unroll
        for (int e = 0; e < 16; ++e)
            acc[bm][e] = 0.0f;
    }
    const int n = blk % NBK + 1;   // blocks held since the last burst
    if (n == NBK || blk == nblocks - 1) {
#pragma unroll
        for (int i = 0; i < NBK; ++i)
            if (i >= NBK - n)
                lowm_store_block<AM, OUT_BF16>(held[i], v_lo + (blk - (NBK - 1 - i)) * 32, v_hi, rows, fr, hi, out,
                                               ldo);
    }
}

}  // namespace lowm
}  // namespace mosaic

// Fused gather-GEMM: logits[i, v] = sum_k H[idx[i], k] * W[v, k].
//
// What it computes follows the mask-only logits kernel of Mosaic ("Mosaic: Unlocking
// Long-Context Inference for Diffusion LLMs via Global Memory" review, 核心组件
// 1. Mask-only Logits Kernel; "扩散大语言模型内存优化：Mosaic系统突破与实践", §2.2):
// it takes the hidden states of every position plus the mask index list, reads the
// masked rows through the indices, splits the product into tiles spread over the
// compute units, stages operands on chip and writes no gathered copy of H.
//
// gfx950 design (bf16 path):
//  * Tile: 256 vocabulary rows x 256 masked rows per workgroup, K staged 64 deep
//    (128 bytes per row).  Four waves, each owning a 128 x 128 sub-tile as 4 x 4 blocks
//    of v_mfma_f32_32x32x16_bf16 (fp32 accumulators: 256 per lane).  W is the MFMA
//    A operand (vocabulary rows) and the gathered H rows are the B operand, so each
//    lane's accumulators hold four consecutive vocabulary entries of one masked row.
//  * Operands reach LDS with global_load_lds_dwordx4 (16 bytes per lane, written to
//    LDS without passing through VGPRs).  The gather is free: each lane's source
//    address is just H + idx[row] * d + k, and a 64-lane instruction fills 8 rows x
//    128 bytes of the tile.  Rows are stored as eight 16-byte chunks whose position is
//    XOR-swizzled by the row, so that the MFMA fragment reads (ds_read_b128, 16 rows
//    per phase at the same logical chunk) hit distinct banks.
//  * K pipeline: NSTAGE LDS buffers; tile kt+NSTAGE-1 is requested while tile kt is
//    multiplied, with explicit vmcnt waits and a bare s_barrier (no full fence).
//  * Block mapping: the hardware deals consecutive workgroups round-robin to the 8
//    XCDs.  Workgroup ids are renumbered so each XCD works on a contiguous range of
//    tiles, ordered so that groups of GROUP_M row-tiles share one W slab in that XCD's
//    L2.
//  * Bit-identity across chunks: every output element is one accumulation chain over
//    k = 0, 16, 32, ... in the same MFMA positions whatever the chunk, tile or row
//    position, so splitting the rows into chunks never changes a bit.
//
// fp32 path (small fp32 problems): an LDS-tiled FMA kernel, 64 x 64 outputs per
// workgroup, fp32 accumulation in ascending k.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#include "launch.h"

namespace mosaic {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt with only the vector-memory counter constrained (expcnt/lgkmcnt at max).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Workgroup barrier without the memory fence of __syncthreads(): the fence would wait
// for every outstanding global load, including the prefetches still in flight.
__device__ __forceinline__ void barrier_no_fence()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    // round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
    __bf16 a = static_cast<__bf16>(lo), b = static_cast<__bf16>(hi);
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// Logical 16-byte chunk c of tile row r sits at physical chunk c ^ swz(r).
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

template <int BV, int BM, int NSTAGE, bool OUT_BF16>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1))) void
gather_gemm_bf16_kernel(const __bf16 *__restrict__ H, const int32_t *__restrict__ idx, int32_t rows,
                        const __bf16 *__restrict__ W, int32_t V, int32_t d, void *__restrict__ out,
                        int64_t ldo, int32_t group_m)
{
    constexpr int BK = 64;                    // k per stage; d % 64 == 0 is required
    constexpr int ROW_BYTES = BK * 2;         // 128
    constexpr int W_TILE = BV * ROW_BYTES;
    constexpr int H_TILE = BM * ROW_BYTES;
    constexpr int STAGE = W_TILE + H_TILE;
    constexpr int WV = BV / 2, WM = BM / 2;   // wave sub-tile (2 x 2 waves)
    constexpr int AV = WV / 32, AM = WM / 32; // 32 x 32 MFMA blocks per wave
    constexpr int LW = BV / 32, LH = BM / 32; // DMA instructions per wave and K tile
    static_assert(AV >= 1 && AM >= 1, "tile too small");

    __shared__ __attribute__((aligned(1024))) char smem[NSTAGE * STAGE];

    const int nvt = (V + BV - 1) / BV;
    const int nmt = (rows + BM - 1) / BM;
    const int nblk = nvt * nmt;

    // XCD-aware renumbering: hardware block b runs on XCD b % 8.
    const int b = blockIdx.x;
    const int q = nblk >> 3, rem = nblk & 7, xcd = b & 7, slot = b >> 3;
    const int t = (xcd < rem ? xcd * (q + 1) : rem * (q + 1) + (xcd - rem) * q) + slot;
    // Grouped order: GROUP_M row tiles x all vocabulary tiles, row tiles fastest.
    const int per_group = group_m * nvt;
    const int g = t / per_group;
    const int first_m = g * group_m;
    const int gsz = min(nmt - first_m, group_m);
    const int local = t - g * per_group;
    const int mt = first_m + local % gsz;
    const int vt = local / gsz;
    const int v0 = vt * BV, m0 = mt * BM;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wv = wave & 1, wm = wave >> 1;

    // ---- DMA sources.  Lane i of DMA instruction j writes 16 bytes at LDS offset
    // j*1024 + i*16 of the tile: tile row j*8 + i/8, physical chunk i%8, which holds
    // logical chunk (i%8) ^ swz(row).  Rows past V or past `rows` re-read the last
    // valid row; their results are never stored.
    const char *wbase = (const char *)(W + (int64_t)v0 * d);
    uint32_t woff[LW];
#pragma unroll
    for (int j = 0; j < LW; ++j) {
        const int r = (wave * LW + j) * 8 + (lane >> 3);
        const int vr = min(v0 + r, V - 1) - v0;
        woff[j] = (uint32_t)vr * (uint32_t)d * 2u + (uint32_t)(((lane & 7) ^ swz(r)) * 16);
    }
    const char *hsrc[LH];
#pragma unroll
    for (int j = 0; j < LH; ++j) {
        const int r = (wave * LH + j) * 8 + (lane >> 3);
        const int m = min(m0 + r, rows - 1);
        hsrc[j] = (const char *)(H + (int64_t)idx[m] * d) + ((lane & 7) ^ swz(r)) * 16;
    }

    const int nk = d / BK;

    f32x16_t acc[AV][AM];
#pragma unroll
    for (int a = 0; a < AV; ++a)
#pragma unroll
        for (int bm = 0; bm < AM; ++bm)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[a][bm][e] = 0.0f;

    // Fragment reads: lane reads row (lane & 31) of a 32-row block, logical chunk
    // 2*s + (lane >> 5) for k sub-step s.  Because swz(row) depends on the lane only and
    // tile rows start at multiples of 128 bytes, the byte address for sub-step s is
    // the s = 0 address XOR 32*s.
    const int fr = lane & 31, hi = lane >> 5;
    const int lane_chunk = ((hi ^ swz(fr)) * 16);
    const int a_addr = (wv * WV + fr) * ROW_BYTES + lane_chunk;
    const int b_addr = W_TILE + (wm * WM + fr) * ROW_BYTES + lane_chunk;

    auto issue = [&](char *sb, int kt) {
        const int kb = kt * ROW_BYTES;
#pragma unroll
        for (int j = 0; j < LW; ++j)
            __builtin_amdgcn_global_load_lds((const void *)(wbase + kb + woff[j]),
                                             (lds_void_t *)(sb + (wave * LW + j) * 1024), 16, 0, 0);
#pragma unroll
        for (int j = 0; j < LH; ++j)
            __builtin_amdgcn_global_load_lds((const void *)(hsrc[j] + kb),
                                             (lds_void_t *)(sb + W_TILE + (wave * LH + j) * 1024), 16, 0, 0);
    };

    auto compute = [&](const char *sb) {
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
            bf16x8_t af[AV], bf[AM];
#pragma unroll
            for (int a = 0; a < AV; ++a)
                af[a] = *(const bf16x8_t *)(sb + ((a_addr + a * 32 * ROW_BYTES) ^ (32 * s)));
#pragma unroll
            for (int bm = 0; bm < AM; ++bm)
                bf[bm] = *(const bf16x8_t *)(sb + ((b_addr + bm * 32 * ROW_BYTES) ^ (32 * s)));
#pragma unroll
            for (int a = 0; a < AV; ++a)
#pragma unroll
                for (int bm = 0; bm < AM; ++bm)
                    acc[a][bm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a], bf[bm], acc[a][bm], 0, 0, 0);
        }
    };

    // One pipeline step on stage ST: wait for tile kt, let every wave pass (tile kt is
    // complete in LDS and the stage about to be refilled is no longer read), request
    // tile kt + NSTAGE - 1, multiply tile kt.
    auto step = [&](auto st_tag, int kt) {
        constexpr int ST = decltype(st_tag)::value;
        const int ahead = min(NSTAGE - 2, nk - 1 - kt);   // tiles requested after kt
        if constexpr (NSTAGE >= 4) {
            if (ahead >= 2) wait_vmcnt<2 * (LW + LH)>();
            else if (ahead == 1) wait_vmcnt<LW + LH>();
            else wait_vmcnt<0>();
        } else if constexpr (NSTAGE == 3) {
            if (ahead >= 1) wait_vmcnt<LW + LH>();
            else wait_vmcnt<0>();
        } else {
            wait_vmcnt<0>();
        }
        barrier_no_fence();
        if (kt + NSTAGE - 1 < nk)
            issue(smem + ((ST + NSTAGE - 1) % NSTAGE) * STAGE, kt + NSTAGE - 1);
        compute(smem + ST * STAGE);
    };

#pragma unroll
    for (int s = 0; s < NSTAGE - 1; ++s)
        if (s < nk)
            issue(smem + s * STAGE, s);

    int kt = 0;
    for (; kt + NSTAGE <= nk; kt += NSTAGE) {
        [&]<int... S>(std::integer_sequence<int, S...>) {
            (step(std::integral_constant<int, S>{}, kt + S), ...);
        }(std::make_integer_sequence<int, NSTAGE>{});
    }
    [&]<int... S>(std::integer_sequence<int, S...>) {
        ((kt + S < nk ? step(std::integral_constant<int, S>{}, kt + S) : (void)0), ...);
    }(std::make_integer_sequence<int, NSTAGE - 1>{});

    // ---- epilogue: lane holds, for block (a, bm) and group gq, vocabulary entries
    // v = v0 + wv*WV + 32a + 8gq + 4hi + (0..3) of masked row m0 + wm*WM + 32bm + fr.
    const bool vec_ok = (ldo & 3) == 0;
#pragma unroll
    for (int bm = 0; bm < AM; ++bm) {
        const int row = m0 + wm * WM + bm * 32 + fr;
        if (row >= rows)
            continue;
#pragma unroll
        for (int a = 0; a < AV; ++a) {
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int v = v0 + wv * WV + a * 32 + gq * 8 + hi * 4;
                const float x0 = acc[a][bm][gq * 4 + 0], x1 = acc[a][bm][gq * 4 + 1];
                const float x2 = acc[a][bm][gq * 4 + 2], x3 = acc[a][bm][gq * 4 + 3];
                if constexpr (OUT_BF16) {
                    __bf16 *o = (__bf16 *)out + (int64_t)row * ldo + v;
                    if (vec_ok && v + 3 < V) {
                        uint2 p;
                        p.x = pack_bf16x2(x0, x1);
                        p.y = pack_bf16x2(x2, x3);
                        *(uint2 *)o = p;
                    } else {
                        if (v + 0 < V) o[0] = static_cast<__bf16>(x0);
                        if (v + 1 < V) o[1] = static_cast<__bf16>(x1);
                        if (v + 2 < V) o[2] = static_cast<__bf16>(x2);
                        if (v + 3 < V) o[3] = static_cast<__bf16>(x3);
                    }
                } else {
                    float *o = (float *)out + (int64_t)row * ldo + v;
                    if (vec_ok && v + 3 < V) {
                        *(f32x4_t *)o = f32x4_t{x0, x1, x2, x3};
                    } else {
                        if (v + 0 < V) o[0] = x0;
                        if (v + 1 < V) o[1] = x1;
                        if (v + 2 < V) o[2] = x2;
                        if (v + 3 < V) o[3] = x3;
                    }
                }
            }
        }
    }
}

// bf16 inputs with d % 64 != 0 (any d % 8 == 0): 64 x 64 outputs per workgroup,
// K staged 16 deep through LDS as fp32, fp32 FMA in ascending k.
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void gather_gemm_bf16_simple_kernel(const __bf16 *__restrict__ H,
                                                                      const int32_t *__restrict__ idx,
                                                                      int32_t rows,
                                                                      const __bf16 *__restrict__ W, int32_t V,
                                                                      int32_t d, void *__restrict__ out,
                                                                      int64_t ldo)
{
    constexpr int T = 64, KT = 16;
    __shared__ float hs[KT][T + 4];
    __shared__ float ws[KT][T + 4];
    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;
    const int m0 = blockIdx.x * T, v0 = blockIdx.y * T;
    const int lr = tid >> 2, lq = (tid & 3) * 4;
    const __bf16 *hrow = H + (int64_t)idx[min(m0 + lr, rows - 1)] * d;
    const __bf16 *wrow = W + (int64_t)min(v0 + lr, V - 1) * d;

    float acc[4][4] = {};
    for (int k0 = 0; k0 < d; k0 += KT) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int k = k0 + lq + e;
            hs[lq + e][lr] = k < d ? static_cast<float>(hrow[k]) : 0.f;
            ws[lq + e][lr] = k < d ? static_cast<float>(wrow[k]) : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < KT; ++k) {
            float hm[4], wn[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) hm[i] = hs[k][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) wn[j] = ws[k][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_fmaf(hm[i], wn[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = m0 + ty * 4 + i;
        if (row >= rows)
            continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int v = v0 + tx * 4 + j;
            if (v >= V)
                continue;
            if constexpr (OUT_BF16)
                ((__bf16 *)out)[(int64_t)row * ldo + v] = static_cast<__bf16>(acc[i][j]);
            else
                ((float *)out)[(int64_t)row * ldo + v] = acc[i][j];
        }
    }
}

// fp32 inputs and outputs: 64 x 64 outputs per workgroup of 256 threads (4 x 4 each),
// K staged 16 deep through LDS, fp32 FMA in ascending k.
__global__ __launch_bounds__(256) void gather_gemm_f32_kernel(const float *__restrict__ H,
                                                              const int32_t *__restrict__ idx, int32_t rows,
                                                              const float *__restrict__ W, int32_t V,
                                                              int32_t d, float *__restrict__ out, int64_t ldo)
{
    constexpr int T = 64, KT = 16;
    __shared__ float hs[KT][T + 4];
    __shared__ float ws[KT][T + 4];
    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;
    const int m0 = blockIdx.x * T, v0 = blockIdx.y * T;

    // loader: row lr of the tile, k quad lq
    const int lr = tid >> 2, lq = (tid & 3) * 4;
    const float *hrow = H + (int64_t)idx[min(m0 + lr, rows - 1)] * d;
    const float *wrow = W + (int64_t)min(v0 + lr, V - 1) * d;

    float acc[4][4] = {};
    for (int k0 = 0; k0 < d; k0 += KT) {
        f32x4_t hv = {0.f, 0.f, 0.f, 0.f}, wv = {0.f, 0.f, 0.f, 0.f};
        if (k0 + lq < d) {   // d % 4 == 0: a quad is all in or all out
            hv = *(const f32x4_t *)(hrow + k0 + lq);
            wv = *(const f32x4_t *)(wrow + k0 + lq);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            hs[lq + e][lr] = hv[e];
            ws[lq + e][lr] = wv[e];
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < KT; ++k) {
            float hm[4], wn[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) hm[i] = hs[k][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) wn[j] = ws[k][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_fmaf(hm[i], wn[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = m0 + ty * 4 + i;
        if (row >= rows)
            continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int v = v0 + tx * 4 + j;
            if (v < V)
                out[(int64_t)row * ldo + v] = acc[i][j];
        }
    }
}

template <int BV, int BM, int NSTAGE>
hipError_t launch_bf16(const void *H, const int32_t *idx, int64_t rows, const void *W, int64_t V, int64_t d,
                       void *out, int64_t ldo, bool out_bf16, int group_m, hipStream_t stream)
{
    const int64_t nvt = (V + BV - 1) / BV, nmt = (rows + BM - 1) / BM;
    const dim3 grid((unsigned)(nvt * nmt));
    if (out_bf16)
        hipLaunchKernelGGL((gather_gemm_bf16_kernel<BV, BM, NSTAGE, true>), grid, dim3(256), 0, stream,
                           (const __bf16 *)H, idx, (int32_t)rows, (const __bf16 *)W, (int32_t)V, (int32_t)d, out,
                           ldo, group_m);
    else
        hipLaunchKernelGGL((gather_gemm_bf16_kernel<BV, BM, NSTAGE, false>), grid, dim3(256), 0, stream,
                           (const __bf16 *)H, idx, (int32_t)rows, (const __bf16 *)W, (int32_t)V, (int32_t)d, out,
                           ldo, group_m);
    return hipGetLastError();
}

}  // namespace

bool gather_gemm_grid_fits(int variant, int64_t rows, int64_t V)
{
    switch (variant) {
    case kVariantF32:
    case kVariantBf16Simple:
        return (rows + 63) / 64 <= 0x7fffffffLL && (V + 63) / 64 <= 65535;
    case kVariantBf16Tile256:
        return ((rows + 255) / 256) * ((V + 255) / 256) <= 0x7fffffffLL;
    default:
        return false;
    }
}

hipError_t launch_gather_gemm(int variant, const void *H, const int32_t *idx, int64_t rows, const void *W,
                              int64_t V, int64_t d, void *out, int64_t ldo, bool out_bf16, hipStream_t stream)
{
    switch (variant) {
    case kVariantF32: {
        const dim3 grid((unsigned)((rows + 63) / 64), (unsigned)((V + 63) / 64));
        hipLaunchKernelGGL(gather_gemm_f32_kernel, grid, dim3(256), 0, stream, (const float *)H, idx,
                           (int32_t)rows, (const float *)W, (int32_t)V, (int32_t)d, (float *)out, ldo);
        return hipGetLastError();
    }
    case kVariantBf16Simple: {
        const dim3 grid((unsigned)((rows + 63) / 64), (unsigned)((V + 63) / 64));
        if (out_bf16)
            hipLaunchKernelGGL(gather_gemm_bf16_simple_kernel<true>, grid, dim3(256), 0, stream, (const __bf16 *)H,
                               idx, (int32_t)rows, (const __bf16 *)W, (int32_t)V, (int32_t)d, out, ldo);
        else
            hipLaunchKernelGGL(gather_gemm_bf16_simple_kernel<false>, grid, dim3(256), 0, stream, (const __bf16 *)H,
                               idx, (int32_t)rows, (const __bf16 *)W, (int32_t)V, (int32_t)d, out, ldo);
        return hipGetLastError();
    }
    case kVariantBf16Tile256:
        return launch_bf16<256, 256, 2>(H, idx, rows, W, V, d, out, ldo, out_bf16, 16, stream);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace mosaic

// FP8 (OCP E4M3) LM head for the mask-only logits path.
//
// "扩散大语言模型内存优化：从理论到系统设计", §5 names combining the logits micro-batching
// with FP8 quantization as a next step.  Here: W is quantized once, per vocabulary row,
// and the masked rows of H are quantized per row as each chunk runs; one fp32 scale per
// row, scale = amax / 448, codes = RNE(x * (448 / amax)).  The logits are the fp32 dot
// product of the codes (gfx950 fp8 MFMA) times both row scales, rounded to bf16.
//
//  * quantize_rows_e4m3_kernel: one wave per row (gathered through an index list when
//    given).  Pass 1: |x| max over the row, reduced across the wave.  Pass 2 (the row is
//    in L2 by then): y = x * inv in fp32, then v_cvt_pk_fp8_f32 (round to nearest even;
//    |y| <= 448 by construction, so it never reaches the non-finite codes).
//  * gather_gemm_fp8_kernel: the bf16 tiled kernel's structure with fp8 operands.  A
//    256 x 256 output tile per workgroup; K tiles of 128 codes, i.e. 128-byte rows, so
//    the DMA (global_load_lds_dwordx4), the two 64 KiB LDS stages and the XOR swizzle
//    are the bf16 kernel's.  Each 64-deep k sub-step is one
//    v_mfma_scale_f32_32x32x64_f8f6f4 per 32 x 32 block with unit block scales (E8M0
//    127), which is the plain fp8 product; a lane supplies 32 codes of its row (two
//    16-byte LDS reads).  The epilogue multiplies each fp32 sum by the row scale of H
//    and the row scale of W.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "launch.h"
#include "lowm_epilogue.h"

namespace mosaic {
namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt vmcnt(N) lgkmcnt(0)
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0x0 << 8) | ((N >> 4) << 14));
}

// At most n (0 <= n <= MAXN) DMA tiles of T instructions each still in flight.
template <int T, int MAXN>
__device__ __forceinline__ void wait_tiles_upto_fp8(int n)
{
    if constexpr (MAXN <= 0) {
        wait_vm<0>();
    } else {
        if (n >= MAXN)
            wait_vm<MAXN * T>();
        else
            wait_tiles_upto_fp8<T, MAXN - 1>(n);
    }
}

__device__ __forceinline__ void bar()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

template <bool IN_BF16>
__device__ __forceinline__ void load8(const void *X, int64_t off, float (&x)[8])
{
    if constexpr (IN_BF16) {
        const uint4 u = *(const uint4 *)((const uint16_t *)X + off);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __builtin_bit_cast(float, w[i] << 16);
            x[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xffff0000u);
        }
    } else {
        const f32x4_t a = *(const f32x4_t *)((const float *)X + off);
        const f32x4_t b = *(const f32x4_t *)((const float *)X + off + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = a[i];
            x[4 + i] = b[i];
        }
    }
}

// Row r of the output is source row row_idx[r] (or r).  d % 8 == 0.
template <bool IN_BF16>
__global__ __launch_bounds__(256) void quantize_rows_e4m3_kernel(const void *__restrict__ X, int32_t d,
                                                                const int32_t *__restrict__ row_idx,
                                                                int64_t rows, uint8_t *__restrict__ q,
                                                                float *__restrict__ scale)
{
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= rows)
        return;
    const int64_t src = row_idx ? (int64_t)row_idx[r] : r;
    const int64_t base = src * d;
    float amax = 0.0f;
    for (int k = lane * 8; k < d; k += 512) {
        float x[8];
        load8<IN_BF16>(X, base + k, x);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            amax = fmaxf(amax, fabsf(x[i]));
    }
    amax = wave_max(amax);
    uint8_t *qr = q + r * d;
    if (amax == 0.0f) {
        for (int k = lane * 8; k < d; k += 512)
            *(uint2 *)(qr + k) = make_uint2(0u, 0u);
        if (lane == 0)
            scale[r] = 0.0f;
        return;
    }
    const float inv = 448.0f / amax;
    for (int k = lane * 8; k < d; k += 512) {
        float x[8];
        load8<IN_BF16>(X, base + k, x);
        uint32_t w[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            int p = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * h] * inv, x[4 * h + 1] * inv, 0, false);
            p = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * h + 2] * inv, x[4 * h + 3] * inv, p, true);
            w[h] = (uint32_t)p;
        }
        *(uint2 *)(qr + k) = make_uint2(w[0], w[1]);
    }
    if (lane == 0)
        scale[r] = amax / 448.0f;
}

// logits[i, v] = (sum_k Hq[i, k] Wq[v, k]) * hs[i] * ws[v] for i < rows, v < V; Hq holds
// the chunk's quantized rows contiguously ([rows, d]); d % 128 == 0.
template <int NW>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW), amdgpu_waves_per_eu(NW / 4, NW / 4))) void
gather_gemm_fp8_kernel(const uint8_t *__restrict__ Hq, const float *__restrict__ hs, int32_t rows,
                       const uint8_t *__restrict__ Wq, const float *__restrict__ ws, int32_t V, int32_t d,
                       __bf16 *__restrict__ out, int64_t ldo, int32_t group_m)
{
    constexpr int BV = 256, BM = 256, BK = 128, NSTAGE = 2, NSPREAD = 2;
    constexpr int ROW_BYTES = BK;             // one byte per code
    constexpr int CHUNKS = ROW_BYTES / 16, RPI = 64 / CHUNKS;
    constexpr int W_TILE = BV * ROW_BYTES, H_TILE = BM * ROW_BYTES, STAGE = W_TILE + H_TILE;
    constexpr int WV = BV / 2, WM = BM / (NW / 2);
    constexpr int AV = WV / 32, AM = WM / 32;
    constexpr int LW = BV / RPI / NW, LH = BM / RPI / NW;
    constexpr int NSUB = BK / 64;             // MFMA k sub-steps per K tile (2)
    constexpr int NDMA = LW + LH, PER = NDMA / NSPREAD;
    static_assert(NDMA % NSPREAD == 0 && NSPREAD <= NSUB, "spread");

    // The stages, then the tile's row scales: 256 of W, then 256 of H (fp32).  One
    // allocation: with a second __shared__ array the compiler cannot tell the stage DMA
    // from the fragment reads and waits for the DMA before every read.
    constexpr int SC_BASE = NSTAGE * STAGE;
    __shared__ __attribute__((aligned(1024))) char smem[NSTAGE * STAGE + 2 * BV * 4];
    static_assert(BV == BM, "scale staging assumes square tiles");

    const int nvt = (V + BV - 1) / BV;
    const int nmt = (rows + BM - 1) / BM;
    const int nblk = nvt * nmt;
    // XCD-aware renumbering and grouped order, as in the bf16 tiled kernel
    const int b = blockIdx.x;
    const int qq = nblk >> 3, rem = nblk & 7, xcd = b & 7, slot = b >> 3;
    const int t = (xcd < rem ? xcd * (qq + 1) : rem * (qq + 1) + (xcd - rem) * qq) + slot;
    const int per_group = group_m * nvt;
    const int g = t / per_group;
    const int first_m = g * group_m;
    const int gsz = min(nmt - first_m, group_m);
    const int local = t - g * per_group;
    const int m0 = (first_m + local % gsz) * BM;
    const int v0 = (local / gsz) * BV;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wv = wave & 1, wm = wave >> 1;
    auto swz = [](int r) { return (r >> 1) & 7; };

    // DMA sources: lane i of instruction j fills tile row j*RPI + i/CHUNKS, physical
    // chunk i%CHUNKS (logical chunk (i%CHUNKS) ^ swz(row)).  Rows past V / rows re-read
    // the last valid row; their results are never stored.
    const uint8_t *wsrc[LW];
    const uint8_t *hsrc[LH];
#pragma unroll
    for (int j = 0; j < LW; ++j) {
        const int r = (wave * LW + j) * RPI + lane / CHUNKS;
        wsrc[j] = Wq + (int64_t)min(v0 + r, V - 1) * d + ((lane % CHUNKS) ^ swz(r)) * 16;
    }
#pragma unroll
    for (int j = 0; j < LH; ++j) {
        const int r = (wave * LH + j) * RPI + lane / CHUNKS;
        hsrc[j] = Hq + (int64_t)min(m0 + r, rows - 1) * d + ((lane % CHUNKS) ^ swz(r)) * 16;
    }
    auto issue_part = [&](int so, int kt, int p) {
        const int kb = kt * ROW_BYTES;
#pragma unroll
        for (int i = 0; i < NDMA; ++i) {
            if (i / PER != p)
                continue;
            if (i < LW)
                __builtin_amdgcn_global_load_lds((const void *)(wsrc[i] + kb),
                                                 (lds_void_t *)(smem + so + (wave * LW + i) * 1024), 16, 0, 0);
            else
                __builtin_amdgcn_global_load_lds((const void *)(hsrc[i - LW] + kb),
                                                 (lds_void_t *)(smem + so + W_TILE + (wave * LH + i - LW) * 1024),
                                                 16, 0, 0);
        }
    };

    f32x16_t acc[AV][AM];
#pragma unroll
    for (int a = 0; a < AV; ++a)
#pragma unroll
        for (int bm = 0; bm < AM; ++bm)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[a][bm][e] = 0.0f;

    // Fragment of sub-step s: lane reads codes 64 s + 32 hi + (0..31) of row (lane & 31)
    // of a 32-row block, i.e. logical chunks 4 s + 2 hi and 4 s + 2 hi + 1.
    const int fr = lane & 31, hi = lane >> 5;
    const int lane_chunk = ((2 * hi) ^ swz(fr)) * 16;
    const int a_addr = (wv * WV + fr) * ROW_BYTES + lane_chunk;
    const int b_addr = W_TILE + (wm * WM + fr) * ROW_BYTES + lane_chunk;
    // (native vector loads: the compiler keeps their type-based alias information and so
    // does not wait for the stage DMA before each read; HIP's uint4 struct loads lose it)
    auto frag = [&](int addr, int s) {
        const i32x4_t lo = *(const i32x4_t *)(smem + (addr ^ (64 * s)));
        const i32x4_t up = *(const i32x4_t *)(smem + (addr ^ (64 * s + 16)));
        return i32x8_t{lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]};
    };
    auto load_frags = [&](int so, int s, i32x8_t (&af)[AV], i32x8_t (&bf)[AM]) __attribute__((always_inline)) {
#pragma unroll
        for (int a = 0; a < AV; ++a)
            af[a] = frag(a_addr + so + a * 32 * ROW_BYTES, s);
#pragma unroll
        for (int bm = 0; bm < AM; ++bm)
            bf[bm] = frag(b_addr + so + bm * 32 * ROW_BYTES, s);
    };
    auto mma = [&](const i32x8_t (&af)[AV], const i32x8_t (&bf)[AM]) __attribute__((always_inline)) {
#pragma unroll
        for (int a = 0; a < AV; ++a)
#pragma unroll
            for (int bm = 0; bm < AM; ++bm)
                acc[a][bm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[a], bf[bm], acc[a][bm], 0, 0, 0,
                                                                             127, 0, 127);
    };
    // MFMAs on fragment buffer `cur` while the fragments of k sub-step s of stage so are
    // read.  Four waves: both operands double-buffered.  Eight waves (256 registers per
    // wave): the A fragments are single-buffered, block a's next fragment being read right
    // after the last MFMA of its row, which keeps the wave within its registers.
    constexpr bool ROLL = NW == 8;
    auto mma_load = [&](int so, int s, int cur, i32x8_t (&af)[2][AV], i32x8_t (&bf)[2][AM])
                        __attribute__((always_inline)) {
        if constexpr (ROLL) {
#pragma unroll
            for (int bm = 0; bm < AM; ++bm)
                bf[cur ^ 1][bm] = frag(b_addr + so + bm * 32 * ROW_BYTES, s);
#pragma unroll
            for (int a = 0; a < AV; ++a) {
#pragma unroll
                for (int bm = 0; bm < AM; ++bm)
                    acc[a][bm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[0][a], bf[cur][bm], acc[a][bm], 0,
                                                                                 0, 0, 127, 0, 127);
                af[0][a] = frag(a_addr + so + a * 32 * ROW_BYTES, s);
            }
        } else {
            load_frags(so, s, af[cur ^ 1], bf[cur ^ 1]);
            mma(af[cur], bf[cur]);
        }
    };
    constexpr int NFR = 2 * (AV + AM);
    auto interleave = [&](int nvm) {
#pragma unroll
        for (int i = 0; i < NDMA; ++i) {
            if (i < nvm) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            }
        }
        if constexpr (ROLL) {
            // the B reads early, then each A read after its row's MFMAs
#pragma unroll
            for (int bm = 0; bm < AM; ++bm) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            const int used = nvm + AM;
#pragma unroll
            for (int a = 0; a < AV; ++a) {
#pragma unroll
                for (int c = 0; c < AM; ++c)
                    if (a * AM + c >= used)
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
        } else {
#pragma unroll
            for (int i = 0; i < NFR; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
        }
    };

    // Pipeline as in the bf16 tiled kernel (two stages; the refill of the stage just
    // read is split over the last sub-step of a step and the first of the next).
    const int nk = d / BK;
    i32x8_t af[2][AV], bf[2][AM];
    // The epilogue's row scales reach LDS by DMA ahead of the K loop (8 instructions of
    // 64 x 4 bytes: W scales v0 .. v0+255, then H scales m0 .. m0+255, indices clamped to
    // the last valid row, whose copies are never used), so the epilogue issues no global
    // loads.  They are older than the first stage's DMA, so the first wait covers them.
    for (int j = wave; j < 8; j += NW) {
        const float *src = j < 4 ? ws + min(v0 + j * 64 + lane, V - 1) : hs + min(m0 + (j - 4) * 64 + lane, rows - 1);
        __builtin_amdgcn_global_load_lds((const void *)src, (lds_void_t *)(smem + SC_BASE + j * 256), 4, 0, 0);
    }
    const int npre = min(NSTAGE, nk);
    for (int s = 0; s < npre; ++s)
#pragma unroll
        for (int p = 0; p < NSPREAD; ++p)
            issue_part(s * STAGE, s, p);
    if (npre == 2)
        wait_vm<NDMA>();
    else
        wait_vm<0>();
    bar();
    load_frags(0, 0, af[0], bf[0]);
    int rd = 0, kt = 0, pso = 0, pkt = 0;
    bool pending = false;
    for (; kt + NSTAGE < nk; ++kt) {
        // sub-step 0: the rest of the previous refill, the fragments of sub-step 1
        if (pending)
            issue_part(pso, pkt, 1);
        mma_load(rd, 1, 0, af, bf);
        interleave(pending ? PER : 0);
        __builtin_amdgcn_sched_barrier(0);
        wait_vm<0>();
        bar();
        __builtin_amdgcn_sched_barrier(0);
        issue_part(rd, kt + NSTAGE, 0);
        pso = rd;
        pkt = kt + NSTAGE;
        pending = true;
        const int nx = (rd + STAGE == NSTAGE * STAGE) ? 0 : rd + STAGE;
        mma_load(nx, 0, 1, af, bf);
        interleave(PER);
        __builtin_amdgcn_sched_barrier(0);
        rd = nx;
    }
    for (; kt < nk; ++kt) {
        if (pending)
            issue_part(pso, pkt, 1);
        pending = false;
        mma_load(rd, 1, 0, af, bf);
        if constexpr (ROLL) {
            // one MFMA sequence for both cases; after the last K tile its reads are unused
            if (kt + 1 < nk) {
                wait_vm<0>();
                bar();
                rd = (rd + STAGE == NSTAGE * STAGE) ? 0 : rd + STAGE;
            }
            mma_load(rd, 0, 1, af, bf);
        } else {
            if (kt + 1 < nk) {
                wait_vm<0>();
                bar();
                rd = (rd + STAGE == NSTAGE * STAGE) ? 0 : rd + STAGE;
                load_frags(rd, 0, af[0], bf[0]);
            }
            mma(af[1], bf[1]);
        }
    }

    // epilogue: lane holds vocabulary entries v0 + wv*WV + 32a + 8gq + 4hi + (0..3) of
    // masked row m0 + wm*WM + 32bm + fr.  After scaling and rounding, permlane32_swap gives
    // lanes 0-31 entries 0-7 / 16-23 of a 32-entry block and lanes 32-63 entries 8-15 /
    // 24-31, and every lane stores 16 bytes.
    auto pack2 = [](float x, float y) {
        const __bf16 a = static_cast<__bf16>(x), b = static_cast<__bf16>(y);
        return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
    };
    {
        const bool vec_ok = ((uintptr_t)out & 15) == 0 && (ldo & 7) == 0;
        const float *sc = (const float *)(smem + SC_BASE);
#pragma unroll
        for (int bm = 0; bm < AM; ++bm) {
            const int row = m0 + wm * WM + bm * 32 + fr;
            const bool row_ok = row < rows;
            const float h = sc[BV + wm * WM + bm * 32 + fr];
#pragma unroll
            for (int a = 0; a < AV; ++a) {
                const int vb = v0 + wv * WV + a * 32;
                uint32_t pk[4][2];
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const int v = vb + gq * 8 + hi * 4;
                    const f32x4_t w = *(const f32x4_t *)(sc + (v - v0));
                    pk[gq][0] = pack2(acc[a][bm][gq * 4 + 0] * (h * w[0]), acc[a][bm][gq * 4 + 1] * (h * w[1]));
                    pk[gq][1] = pack2(acc[a][bm][gq * 4 + 2] * (h * w[2]), acc[a][bm][gq * 4 + 3] * (h * w[3]));
                }
#pragma unroll
                for (int pr = 0; pr < 2; ++pr) {
                    const auto s0 = __builtin_amdgcn_permlane32_swap(pk[2 * pr][0], pk[2 * pr + 1][0], false, false);
                    const auto s1 = __builtin_amdgcn_permlane32_swap(pk[2 * pr][1], pk[2 * pr + 1][1], false, false);
                    const int v = vb + 16 * pr + 8 * hi;
                    if (!row_ok)
                        continue;   // (after the swaps: every lane takes part in them)
                    __bf16 *o = out + (int64_t)row * ldo + v;
                    if (vec_ok && v + 7 < V) {
                        *(uint4 *)o = make_uint4(s0[0], s1[0], s0[1], s1[1]);
                    } else {
                        const uint32_t w4[4] = {s0[0], s1[0], s0[1], s1[1]};
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            if (v + e < V)
                                o[e] = __builtin_bit_cast(__bf16, (uint16_t)(w4[e >> 1] >> (16 * (e & 1))));
                    }
                }
            }
        }
    }
}


// The FP8 GEMM's default form: the tile, fragments, MFMA sequence and epilogue of
// gather_gemm_fp8_kernel<8> (so the logits are bit-identical to it), with the K pipeline
// of the bf16 persistent kernel's default:
//  * only waves 0-3, one per SIMD, request K tiles (a quarter each); waves 4-7 run a copy
//    of the K loop with no requests, so each SIMD has one wave whose MFMA issue is never
//    held up by the texture path;
//  * W has three LDS stages and H two (160 KiB): at step k's barrier H's rows of K tile
//    k + 2 are requested into the H stage just freed, and W's rows of K tile k + 3 into the
//    freed W stage at the start of the next step, so each wait leaves one W K tile in
//    flight and W's requests have two steps to land;
//  * the 2 KiB of row scales no longer fit beside the stages: they are requested into the
//    W stage that K tile nk - 2 frees (a stage the tile never uses when nk == 1) and waited
//    for before the epilogue.
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2))) void
gather_gemm_fp8_w3_kernel(const uint8_t *__restrict__ Hq, const float *__restrict__ hs, int32_t rows,
                          const uint8_t *__restrict__ Wq, const float *__restrict__ ws, int32_t V, int32_t d,
                          __bf16 *__restrict__ out, int64_t ldo, int32_t group_m)
{
    constexpr int NW = 8, DMAW = 4;
    constexpr int BV = 256, BM = 256, BK = 128, WST = 3, HST = 2;
    constexpr int ROW_BYTES = BK;             // one byte per code
    constexpr int CHUNKS = ROW_BYTES / 16, RPI = 64 / CHUNKS;
    constexpr int W_TILE = BV * ROW_BYTES, H_TILE = BM * ROW_BYTES;
    constexpr int H_BASE = WST * W_TILE;
    constexpr int WV = BV / 2, WM = BM / (NW / 2);
    constexpr int AV = WV / 32, AM = WM / 32;
    constexpr int LW = BV / RPI / DMAW, LH = BM / RPI / DMAW;   // requests per requesting wave
    constexpr int NDMA = LW + LH;
    static_assert(H_BASE + HST * H_TILE <= 160 * 1024, "LDS");
    static_assert(BV == BM, "scale staging assumes square tiles");
    __shared__ __attribute__((aligned(1024))) char smem[H_BASE + HST * H_TILE];

    const int nvt = (V + BV - 1) / BV;
    const int nmt = (rows + BM - 1) / BM;
    const int nblk = nvt * nmt;
    // XCD-aware renumbering and grouped order, as in gather_gemm_fp8_kernel
    const int b = blockIdx.x;
    const int qq = nblk >> 3, rem = nblk & 7, xcd = b & 7, slot = b >> 3;
    const int t = (xcd < rem ? xcd * (qq + 1) : rem * (qq + 1) + (xcd - rem) * qq) + slot;
    const int per_group = group_m * nvt;
    const int g = t / per_group;
    const int first_m = g * group_m;
    const int gsz = min(nmt - first_m, group_m);
    const int local = t - g * per_group;
    const int m0 = (first_m + local % gsz) * BM;
    const int v0 = (local / gsz) * BV;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wv = wave & 1, wm = wave >> 1;
    const bool dma_wave = wave < DMAW;
    const int dwave = wave % DMAW;
    auto swz = [](int r) { return (r >> 1) & 7; };

    // DMA sources of a requesting wave (layout as in gather_gemm_fp8_kernel)
    const uint8_t *wsrc[LW];
    const uint8_t *hsrc[LH];
#pragma unroll
    for (int j = 0; j < LW; ++j) {
        const int r = (dwave * LW + j) * RPI + lane / CHUNKS;
        wsrc[j] = Wq + (int64_t)min(v0 + r, V - 1) * d + ((lane % CHUNKS) ^ swz(r)) * 16;
    }
#pragma unroll
    for (int j = 0; j < LH; ++j) {
        const int r = (dwave * LH + j) * RPI + lane / CHUNKS;
        hsrc[j] = Hq + (int64_t)min(m0 + r, rows - 1) * d + ((lane % CHUNKS) ^ swz(r)) * 16;
    }
    auto issue_w = [&](int rw, int kt) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < LW; ++j)
            __builtin_amdgcn_global_load_lds((const void *)(wsrc[j] + kt * ROW_BYTES),
                                             (lds_void_t *)(smem + rw + (dwave * LW + j) * 1024), 16, 0, 0);
    };
    auto issue_h = [&](int rh, int kt) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < LH; ++j)
            __builtin_amdgcn_global_load_lds((const void *)(hsrc[j] + kt * ROW_BYTES),
                                             (lds_void_t *)(smem + rh + (dwave * LH + j) * 1024), 16, 0, 0);
    };
    // the tile's row scales (W's 256, then H's 256, fp32; indices clamped to the last valid
    // row, whose copies are never used): instructions dwave and dwave + 4 of 8
    auto issue_scales = [&](int base) __attribute__((always_inline)) {
#pragma unroll
        for (int j = dwave; j < 8; j += DMAW) {
            const float *src = j < 4 ? ws + min(v0 + j * 64 + lane, V - 1) : hs + min(m0 + (j - 4) * 64 + lane, rows - 1);
            __builtin_amdgcn_global_load_lds((const void *)src, (lds_void_t *)(smem + base + j * 256), 4, 0, 0);
        }
    };

    f32x16_t acc[AV][AM];
#pragma unroll
    for (int a = 0; a < AV; ++a)
#pragma unroll
        for (int bm = 0; bm < AM; ++bm)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[a][bm][e] = 0.0f;

    const int fr = lane & 31, hi = lane >> 5;
    const int lane_chunk = ((2 * hi) ^ swz(fr)) * 16;
    const int a_addr = (wv * WV + fr) * ROW_BYTES + lane_chunk;   // from a W stage
    const int b_addr = (wm * WM + fr) * ROW_BYTES + lane_chunk;   // from an H stage
    auto frag = [&](int addr, int s) __attribute__((always_inline)) {
        const i32x4_t lo = *(const i32x4_t *)(smem + (addr ^ (64 * s)));
        const i32x4_t up = *(const i32x4_t *)(smem + (addr ^ (64 * s + 16)));
        return i32x8_t{lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]};
    };
    // MFMAs on B fragment buffer `cur` while sub-step s of the stages at rw (W) and rh (H)
    // is read: the B fragments first, then each block's next A fragment after its row's
    // MFMAs (as gather_gemm_fp8_kernel<8>)
    auto mma_load = [&](int rw, int rh, int s, int cur, i32x8_t (&af)[AV], i32x8_t (&bf)[2][AM])
                        __attribute__((always_inline)) {
#pragma unroll
        for (int bm = 0; bm < AM; ++bm)
            bf[cur ^ 1][bm] = frag(b_addr + rh + bm * 32 * ROW_BYTES, s);
#pragma unroll
        for (int a = 0; a < AV; ++a) {
#pragma unroll
            for (int bm = 0; bm < AM; ++bm)
                acc[a][bm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[a], bf[cur][bm], acc[a][bm], 0, 0, 0,
                                                                             127, 0, 127);
            af[a] = frag(a_addr + rw + a * 32 * ROW_BYTES, s);
        }
    };
    auto interleave = [&](int nvm) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NDMA; ++i) {
            if (i < nvm) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            }
        }
#pragma unroll
        for (int bm = 0; bm < AM; ++bm) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        const int used = nvm + AM;
#pragma unroll
        for (int a = 0; a < AV; ++a) {
#pragma unroll
            for (int c = 0; c < AM; ++c)
                if (a * AM + c >= used)
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
    };
    auto next_w = [](int rw) { return rw + W_TILE == WST * W_TILE ? 0 : rw + W_TILE; };
    auto next_h = [](int rh) { return rh + H_TILE == H_BASE + HST * H_TILE ? H_BASE : rh + H_TILE; };

    const int nk = d / BK;
    const int sc_stage = nk >= 2 ? (nk - 2) % WST : 2;
    i32x8_t af[AV], bf[2][AM];
    auto k_loop = [&](auto dma_tag) __attribute__((always_inline)) {
        constexpr bool DMA_ON = decltype(dma_tag)::value;
        // H0, W0, H1, W1, W2 (the order the waits count on)
        if constexpr (DMA_ON) {
            issue_h(H_BASE, 0);
            issue_w(0, 0);
            if (nk > 1) {
                issue_h(H_BASE + H_TILE, 1);
                issue_w(W_TILE, 1);
            }
            if (nk > 2)
                issue_w(2 * W_TILE, 2);
            else if (nk == 1)
                issue_scales(2 * W_TILE);
        }
        if (nk > 2)
            wait_vm<NDMA + LW>();
        else if (nk == 2)
            wait_vm<NDMA>();
        else
            wait_vm<0>();
        bar();
#pragma unroll
        for (int a = 0; a < AV; ++a)
            af[a] = frag(a_addr + a * 32 * ROW_BYTES, 0);
#pragma unroll
        for (int bm = 0; bm < AM; ++bm)
            bf[0][bm] = frag(b_addr + H_BASE + bm * 32 * ROW_BYTES, 0);
        int rw = 0, rh = H_BASE, kt = 0, pw = 0, pkt = 0;
        bool pend_w = false;
        for (; kt + 2 < nk; ++kt) {
            // sub-step 0: W's rows of K tile kt + 2 (requested for the stage the previous
            // barrier freed), the fragments of sub-step 1
            if (DMA_ON && pend_w)
                issue_w(pw, pkt);
            mma_load(rw, rh, 1, 0, af, bf);
            interleave(DMA_ON && pend_w ? LW : 0);
            __builtin_amdgcn_sched_barrier(0);
            wait_vm<LW>();   // K tile kt + 1 has landed; W's K tile kt + 2 may not have
            bar();
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (DMA_ON)
                issue_h(rh, kt + 2);
            pend_w = kt + 3 < nk;
            pw = rw;
            pkt = kt + 3;
            const int nxw = next_w(rw), nxh = next_h(rh);
            mma_load(nxw, nxh, 0, 1, af, bf);
            interleave(DMA_ON ? LH : 0);
            __builtin_amdgcn_sched_barrier(0);
            rw = nxw;
            rh = nxh;
        }
        for (; kt < nk; ++kt) {
            mma_load(rw, rh, 1, 0, af, bf);
            // one MFMA sequence for both cases; after the last K tile its reads are unused
            if (kt + 1 < nk) {
                wait_vm<0>();
                bar();
                if constexpr (DMA_ON) {
                    if (kt == nk - 2)
                        issue_scales(rw);   // the W stage of K tile nk - 2, free now
                }
                rw = next_w(rw);
                rh = next_h(rh);
            }
            mma_load(rw, rh, 0, 1, af, bf);
        }
    };
    if (dma_wave)
        k_loop(std::true_type{});
    else
        k_loop(std::false_type{});
    wait_vm<0>();
    bar();   // every requesting wave's scales have landed

    // epilogue as in gather_gemm_fp8_kernel
    auto pack2 = [](float x, float y) {
        const __bf16 a = static_cast<__bf16>(x), b = static_cast<__bf16>(y);
        return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
    };
    const bool vec_ok = ((uintptr_t)out & 15) == 0 && (ldo & 7) == 0;
    const float *sc = (const float *)(smem + sc_stage * W_TILE);
#pragma unroll
    for (int bm = 0; bm < AM; ++bm) {
        const int row = m0 + wm * WM + bm * 32 + fr;
        const bool row_ok = row < rows;
        const float h = sc[BV + wm * WM + bm * 32 + fr];
#pragma unroll
        for (int a = 0; a < AV; ++a) {
            const int vb = v0 + wv * WV + a * 32;
            uint32_t pk[4][2];
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int v = vb + gq * 8 + hi * 4;
                const f32x4_t w = *(const f32x4_t *)(sc + (v - v0));
                pk[gq][0] = pack2(acc[a][bm][gq * 4 + 0] * (h * w[0]), acc[a][bm][gq * 4 + 1] * (h * w[1]));
                pk[gq][1] = pack2(acc[a][bm][gq * 4 + 2] * (h * w[2]), acc[a][bm][gq * 4 + 3] * (h * w[3]));
            }
#pragma unroll
            for (int pr = 0; pr < 2; ++pr) {
                const auto s0 = __builtin_amdgcn_permlane32_swap(pk[2 * pr][0], pk[2 * pr + 1][0], false, false);
                const auto s1 = __builtin_amdgcn_permlane32_swap(pk[2 * pr][1], pk[2 * pr + 1][1], false, false);
                const int v = vb + 16 * pr + 8 * hi;
                if (!row_ok)
                    continue;   // (after the swaps: every lane takes part in them)
                __bf16 *o = out + (int64_t)row * ldo + v;
                if (vec_ok && v + 7 < V) {
                    *(uint4 *)o = make_uint4(s0[0], s1[0], s0[1], s1[1]);
                } else {
                    const uint32_t w4[4] = {s0[0], s1[0], s0[1], s1[1]};
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (v + e < V)
                            o[e] = __builtin_bit_cast(__bf16, (uint16_t)(w4[e >> 1] >> (16 * (e & 1))));
                }
            }
        }
    }
}

// Low-M FP8 logits (rows <= 32 * AM): streaming the W codes once.
// The bf16 low-M kernel's design with fp8 operands:
//  * wave w of the grid owns an equal, contiguous range of vocabulary rows (the
//    workgroups of one XCD a contiguous eighth), walked in 32-row blocks, each a full K
//    loop of 128-code K tiles; 128-byte rows, so the DMA, the XOR swizzle and the per-wave
//    LDS ring are the bf16 kernel's;
//  * the 32 * AM quantized masked rows form an H tile shared by the workgroup (each wave
//    DMAs AM 8-row slices), made visible by one barrier per step;
//  * W's requests use the streaming cache policy (read once per launch);
//  * each 64-code k sub-step is one v_mfma_scale_f32_32x32x64_f8f6f4 per block with the
//    fragments and k order of gather_gemm_fp8_kernel, and the epilogue computes
//    sum * (scale_h * scale_w) as it does, so the logits are bit-identical to it;
//  * the row scales reach LDS by DMA (the H scales before the loop, a block's W scales
//    one block ahead), so the K loop's waits count the stream alone;
//  * a finished block's logits are held in registers and stored in bursts.
template <int AM, int NSTAGE>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1))) void
gather_gemm_fp8_lowm_kernel(const uint8_t *__restrict__ Hq, const float *__restrict__ hs, int32_t rows,
                            const uint8_t *__restrict__ Wq, const float *__restrict__ ws, int32_t V, int32_t d,
                            __bf16 *__restrict__ out, int64_t ldo)
{
    constexpr int BK = 128, ROW_BYTES = 128, CHUNKS = 8, RPI = 8, NBK = 8;
    constexpr int W_TILE = 32 * ROW_BYTES;           // 4 KiB: a wave's 32 vocabulary rows
    constexpr int H_TILE = 32 * AM * ROW_BYTES;      // shared by the workgroup
    constexpr int WAVE_W = NSTAGE * W_TILE;
    constexpr int H_BASE = 4 * WAVE_W;
    constexpr int SC_BASE = H_BASE + NSTAGE * H_TILE;
    constexpr int SC_WAVE = 3 * 256;                 // per wave: 64 H scales, two slots of 64 W scales
    constexpr int LW = W_TILE / 1024, LH = AM, T = LW + LH;
    constexpr int kStream = 2;                       // global_load_lds cache policy: NT (streaming)
    static_assert(SC_BASE + 4 * SC_WAVE <= 160 * 1024, "LDS");
    static_assert(NSTAGE >= 3 && (NSTAGE - 2) * T < 64, "vmcnt");

    __shared__ __attribute__((aligned(1024))) char smem[SC_BASE + 4 * SC_WAVE];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wbase = wave * WAVE_W;
    const int sbase = SC_BASE + wave * SC_WAVE;
    const int64_t wg = gridDim.x % 8 == 0 ? (int64_t)(blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8
                                          : (int64_t)blockIdx.x;
    const int64_t nw = (int64_t)gridDim.x * 4, gw = wg * 4 + wave;
    const int v_lo = lowm::range_bound(gw, nw, V);
    const int v_hi = lowm::range_bound(gw + 1, nw, V);
    const int v_max = max(v_hi - 1, 0);              // clamp for padding rows (V >= 1)
    const int nblocks = lowm::range_blocks(nw, V);
    const int nk = d / BK;
    const int ntiles = nblocks * nk;
    auto swz = [](int r) { return (r >> 1) & 7; };

    int wch[LW];
#pragma unroll
    for (int j = 0; j < LW; ++j)
        wch[j] = ((lane % CHUNKS) ^ swz(j * RPI + lane / CHUNKS)) * 16;
    const uint8_t *hsrc[LH];
#pragma unroll
    for (int j = 0; j < LH; ++j) {
        const int r = (j * 4 + wave) * RPI + lane / CHUNKS;
        hsrc[j] = Hq + (int64_t)min(r, rows - 1) * d + ((lane % CHUNKS) ^ swz(r)) * 16;
    }
    auto issue = [&](int slot, int g) {
        const int blk = g / nk, kt = g - blk * nk;
        const int kb = kt * ROW_BYTES;
#pragma unroll
        for (int j = 0; j < LW; ++j) {
            const int v = min(v_lo + blk * 32 + j * RPI + lane / CHUNKS, v_max);
            __builtin_amdgcn_global_load_lds((const void *)(Wq + (int64_t)v * d + kb + wch[j]),
                                             (lds_void_t *)(smem + wbase + slot * W_TILE + j * 1024), 16, 0,
                                             kStream);
        }
#pragma unroll
        for (int j = 0; j < LH; ++j)
            __builtin_amdgcn_global_load_lds((const void *)(hsrc[j] + kb),
                                             (lds_void_t *)(smem + H_BASE + slot * H_TILE + (j * 4 + wave) * 1024),
                                             16, 0, 0);
    };
    // W scales of block blk (64 entries from its first row, clamped) into slot blk & 1
    auto issue_wscale = [&](int blk) {
        __builtin_amdgcn_global_load_lds((const void *)(ws + min(v_lo + blk * 32 + lane, v_max)),
                                         (lds_void_t *)(smem + sbase + 256 + (blk & 1) * 256), 4, 0, 0);
    };

    const int fr = lane & 31, hi = lane >> 5;
    const int lane_chunk = ((2 * hi) ^ swz(fr)) * 16;
    const int a_addr = wbase + fr * ROW_BYTES + lane_chunk;
    const int b_addr = H_BASE + fr * ROW_BYTES + lane_chunk;
    auto frag = [&](int addr, int s) {
        const i32x4_t lo = *(const i32x4_t *)(smem + (addr ^ (64 * s)));
        const i32x4_t up = *(const i32x4_t *)(smem + (addr ^ (64 * s + 16)));
        return i32x8_t{lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]};
    };

    f32x16_t acc[AM], held[NBK][AM];
#pragma unroll
    for (int bm = 0; bm < AM; ++bm)
#pragma unroll
        for (int e = 0; e < 16; ++e)
            acc[bm][e] = 0.0f;

    // the scales first (older than every tile, so the first wait covers them), then
    // NSTAGE - 1 steps of the stream
    __builtin_amdgcn_global_load_lds((const void *)(hs + min(lane, rows - 1)), (lds_void_t *)(smem + sbase), 4, 0,
                                     0);
    issue_wscale(0);
    const int npre = min(NSTAGE - 1, ntiles);
    for (int g = 0; g < npre; ++g)
        issue(g, g);

    const float *sch = (const float *)(smem + sbase);
    int rs = 0;
    for (int g = 0; g < ntiles; ++g) {
        wait_tiles_upto_fp8<T, NSTAGE - 2>(min(NSTAGE - 2, ntiles - 1 - g));
        bar();   // every wave's part of step g landed; every wave is done with step g-1
        if (g + NSTAGE - 1 < ntiles)
            issue(rs == 0 ? NSTAGE - 1 : rs - 1, g + NSTAGE - 1);
        const int blk = g / nk, kt = g - blk * nk;
        if (kt == 0 && blk + 1 < nblocks)
            issue_wscale(blk + 1);   // slot (blk + 1) & 1 was last read at block blk - 1's end
#pragma unroll
        for (int s = 0; s < BK / 64; ++s) {
            const i32x8_t af = frag(a_addr + rs * W_TILE, s);
            i32x8_t bf[AM];
#pragma unroll
            for (int bm = 0; bm < AM; ++bm)
                bf[bm] = frag(b_addr + rs * H_TILE + bm * 32 * ROW_BYTES, s);
#pragma unroll
            for (int bm = 0; bm < AM; ++bm)
                acc[bm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, bf[bm], acc[bm], 0, 0, 0, 127, 0, 127);
        }
        rs = (rs + 1 == NSTAGE) ? 0 : rs + 1;
        if (kt == nk - 1) {
            // This block's W scales were requested at the first step of the previous block,
            // after the refill of step (blk - 1) nk + NSTAGE - 1.  The step waits cover that
            // request once a younger tile has been waited for, i.e. when
            // (blk - 1) nk + NSTAGE <= blk nk + nk - 1; with fewer K tiles per block
            // (d <= 384 here) wait for everything in flight instead.
            if (2 * nk - 1 < NSTAGE)
                wait_vm<0>();
            // sum * (scale_h * scale_w); lane (fr, hi) holds, in accumulators 4 gq .. 4 gq + 3,
            // vocabulary rows 8 gq + 4 hi + (0..3) of the block for masked row 32 bm + fr
            const float *scw = (const float *)(smem + sbase + 256 + (blk & 1) * 256);
#pragma unroll
            for (int bm = 0; bm < AM; ++bm) {
                const float h = sch[bm * 32 + fr];
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const f32x4_t w = *(const f32x4_t *)(scw + gq * 8 + hi * 4);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[bm][gq * 4 + e] = acc[bm][gq * 4 + e] * (h * w[e]);
                }
            }
            lowm::lowm_block_done<AM, NBK, true>(held, acc, blk, nblocks, v_lo, v_hi, rows, fr, hi, out, ldo);
        }
    }
}

}  // namespace

hipError_t launch_quantize_rows_e4m3(const void *X, bool in_bf16, int64_t d, const int32_t *row_idx, int64_t rows,
                                     uint8_t *q, float *scale, hipStream_t stream)
{
    if (rows <= 0)
        return hipSuccess;
    const dim3 grid((unsigned)((rows + 3) / 4));
    if (in_bf16)
        hipLaunchKernelGGL(quantize_rows_e4m3_kernel<true>, grid, dim3(256), 0, stream, X, (int32_t)d, row_idx, rows,
                           q, scale);
    else
        hipLaunchKernelGGL(quantize_rows_e4m3_kernel<false>, grid, dim3(256), 0, stream, X, (int32_t)d, row_idx,
                           rows, q, scale);
    return hipGetLastError();
}

hipError_t launch_gemm_fp8_lowm(const uint8_t *Hq, const float *hs, int64_t rows, const uint8_t *Wq, const float *ws,
                                int64_t V, int64_t d, void *out, int64_t ldo, hipStream_t stream)
{
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    // one workgroup (four streams) per CU, but never fewer than 32 rows per stream
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(cus, (V + 127) / 128));
    if (rows <= 32)
        hipLaunchKernelGGL((gather_gemm_fp8_lowm_kernel<1, 7>), dim3(grid), dim3(256), 0, stream, Hq, hs,
                           (int32_t)rows, Wq, ws, (int32_t)V, (int32_t)d, (__bf16 *)out, ldo);
    else
        hipLaunchKernelGGL((gather_gemm_fp8_lowm_kernel<2, 6>), dim3(grid), dim3(256), 0, stream, Hq, hs,
                           (int32_t)rows, Wq, ws, (int32_t)V, (int32_t)d, (__bf16 *)out, ldo);
    return hipGetLastError();
}

hipError_t launch_gemm_fp8(const uint8_t *Hq, const float *hs, int64_t rows, const uint8_t *Wq, const float *ws,
                           int64_t V, int64_t d, void *out, int64_t ldo, int group_m, int nwaves, hipStream_t stream)
{
    if (group_m <= 0)
        group_m = kDefaultGroupM;
    const int64_t nblk = ((V + 255) / 256) * ((rows + 255) / 256);
    if (nwaves == 4)
        hipLaunchKernelGGL(gather_gemm_fp8_kernel<4>, dim3((unsigned)nblk), dim3(256), 0, stream, Hq, hs,
                           (int32_t)rows, Wq, ws, (int32_t)V, (int32_t)d, (__bf16 *)out, ldo, group_m);
    else if (nwaves == 8)
        hipLaunchKernelGGL(gather_gemm_fp8_kernel<8>, dim3((unsigned)nblk), dim3(512), 0, stream, Hq, hs,
                           (int32_t)rows, Wq, ws, (int32_t)V, (int32_t)d, (__bf16 *)out, ldo, group_m);
    else
        hipLaunchKernelGGL(gather_gemm_fp8_w3_kernel, dim3((unsigned)nblk), dim3(512), 0, stream, Hq, hs,
                           (int32_t)rows, Wq, ws, (int32_t)V, (int32_t)d, (__bf16 *)out, ldo, group_m);
    return hipGetLastError();
}

}  // namespace mosaic

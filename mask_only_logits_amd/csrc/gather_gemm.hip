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
//    of v_mfma_f32_32x32x16_bf16 (fp32 accumulators: 256 per lane), or eight waves (two
//    per SIMD) of 128 x 64, as 4 x 2 such blocks or, in the default bf16-output kernel,
//    8 x 4 blocks of v_mfma_f32_16x16x32_bf16.  W is the MFMA A operand (vocabulary
//    rows) and the gathered H rows are the B operand, so each lane's accumulators hold
//    four consecutive vocabulary entries of one masked row.
//  * Operands reach LDS with global_load_lds_dwordx4 (16 bytes per lane, written to
//    LDS without passing through VGPRs).  The gather is free: each lane's source
//    address is just H + idx[row] * d + k, and a 64-lane instruction fills 8 rows x
//    128 bytes of the tile.  Rows are stored as eight 16-byte chunks whose position is
//    XOR-swizzled by the row, so that the MFMA fragment reads (ds_read_b128, 16 rows
//    per phase at the same logical chunk) hit distinct banks.
//  * K pipeline: NSTAGE LDS buffers.  A stage is refilled as soon as the barrier of
//    the step that used it has passed, with explicit vmcnt waits and a bare s_barrier
//    (no full fence), while MFMAs of the last k sub-step run.  The default bf16-output
//    kernel has only waves 0-3 (one per SIMD) request K tiles and gives W a third stage.
//  * Block mapping: the hardware deals consecutive workgroups round-robin to the 8
//    XCDs.  Workgroup ids are renumbered so each XCD works on a contiguous range of
//    tiles, ordered so that groups of GROUP_M row-tiles share one W slab in that XCD's
//    L2; on large launches the persistent kernel sets the eight XCDs side by side over
//    the vocabulary instead.
//  * Bit-identity across chunks: every output element is one accumulation chain over
//    k in ascending order in the same MFMA positions whatever the chunk, tile or row
//    position, so splitting the rows into chunks never changes a bit.  (The two MFMA
//    shapes were measured to agree bit for bit as well.)
//  * Variants of this design (one tile per workgroup; persistent per-XCD tile lists;
//    deferred epilogue stores) and a low-M streaming kernel share the MFMA, operand
//    roles and k order, so they all produce identical bits.
//
// fp32 path (small fp32 problems): an LDS-tiled FMA kernel, 64 x 64 outputs per
// workgroup, fp32 accumulation in ascending k.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>
#include <utility>

#include "launch.h"
#include "lowm_epilogue.h"

namespace mosaic {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt vmcnt(N) lgkmcnt(0): at most N vector-memory operations of this wave in
// flight, and every LDS access of this wave complete.
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0x0 << 8) | ((N >> 4) << 14));
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

// LDS layout of one operand tile: rows of BK bf16 (BK*2 bytes), each row made of
// 16-byte chunks.  Logical chunk c of tile row r sits at physical chunk c ^ swz(r).
// gfx950 serves a ds_read_b128 16 consecutive lanes per LDS cycle over 64 four-byte
// banks (256 bytes).  A fragment read sends 16 consecutive tile rows (same logical
// chunk) into one cycle; rows 256 bytes apart share banks (every 4th row for 64-byte
// rows, every 2nd for 128-byte rows), so the swizzle gives those rows distinct chunk
// positions.  (Measured on MI355X: this layout reads LDS ~1.75x faster than XOR
// patterns built from other row bits.)
template <int BK>
__device__ __forceinline__ int swz(int r)
{
    if constexpr (BK == 64)
        return (r >> 1) & 7;                      // 8 chunks per row; rows r, r+2, ... r+14
    else
        return (r >> 2) & 3;                      // 4 chunks per row; rows r, r+4, r+8, r+12
}

template <int BV, int BM, int BK, int NSTAGE, int NSPREAD, int NW, bool OUT_BF16>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW), amdgpu_waves_per_eu(NW / 4, NW / 4))) void
gather_gemm_bf16_kernel(const __bf16 *__restrict__ H, const int32_t *__restrict__ idx, int32_t rows,
                        const __bf16 *__restrict__ W, int32_t V, int32_t d, void *__restrict__ out,
                        int64_t ldo, int32_t group_m)
{
    static_assert(BK == 32 || BK == 64, "BK");
    static_assert(NW == 4 || NW == 8, "waves");
    constexpr int ROW_BYTES = BK * 2;         // 64 or 128
    constexpr int CHUNKS = BK / 8;            // 16-byte chunks per row
    constexpr int RPI = 64 / CHUNKS;          // tile rows filled by one 64-lane DMA instruction
    constexpr int W_TILE = BV * ROW_BYTES;
    constexpr int H_TILE = BM * ROW_BYTES;
    constexpr int STAGE = W_TILE + H_TILE;
    // wave sub-tile: 2 waves along V x NW/2 along M (one or two waves per SIMD)
    constexpr int WV = BV / 2, WM = BM / (NW / 2);
    constexpr int AV = WV / 32, AM = WM / 32; // 32 x 32 MFMA blocks per wave
    constexpr int LW = BV / RPI / NW, LH = BM / RPI / NW;   // DMA instructions per wave and K tile
    constexpr int NSUB = BK / 16;             // MFMA k sub-steps per K tile
    static_assert(AV >= 1 && AM >= 1 && LW >= 1 && LH >= 1, "tile too small");
    static_assert(NSTAGE * STAGE <= 160 * 1024, "LDS");
    static_assert(NSTAGE >= 2 && (BK / 16) % 2 == 0, "pipeline");

    __shared__ __attribute__((aligned(1024))) char smem[NSTAGE * STAGE];

    const int nvt = (V + BV - 1) / BV;
    const int nmt = (rows + BM - 1) / BM;
    const int nblk = nvt * nmt;

    // XCD-aware renumbering: hardware block b runs on XCD b % 8, so give XCD x the
    // contiguous range of logical tiles [start_x, start_x + count_x).
    const int b = blockIdx.x;
    const int q = nblk >> 3, rem = nblk & 7, xcd = b & 7, slot = b >> 3;
    const int t = (xcd < rem ? xcd * (q + 1) : rem * (q + 1) + (xcd - rem) * q) + slot;
    // Grouped order: GROUP_M row tiles x all vocabulary tiles, row tiles fastest, so the
    // workgroups resident on one XCD share GROUP_M H slabs and a few W slabs in its L2.
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
    // j*1024 + i*16 of the tile: tile row j*RPI + i/CHUNKS, physical chunk i%CHUNKS,
    // which holds logical chunk (i%CHUNKS) ^ swz(row).  Rows past V or past `rows`
    // re-read the last valid row; their results are never stored.
    const char *wbase = (const char *)(W + (int64_t)v0 * d);
    uint32_t woff[LW];
#pragma unroll
    for (int j = 0; j < LW; ++j) {
        const int r = (wave * LW + j) * RPI + lane / CHUNKS;
        const int vr = min(v0 + r, V - 1) - v0;
        woff[j] = (uint32_t)vr * (uint32_t)d * 2u + (uint32_t)(((lane % CHUNKS) ^ swz<BK>(r)) * 16);
    }
    const char *hsrc[LH];
#pragma unroll
    for (int j = 0; j < LH; ++j) {
        const int r = (wave * LH + j) * RPI + lane / CHUNKS;
        const int m = min(m0 + r, rows - 1);
        hsrc[j] = (const char *)(H + (int64_t)idx[m] * d) + ((lane % CHUNKS) ^ swz<BK>(r)) * 16;
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
    // 2*s + (lane >> 5) for k sub-step s.  swz of that row depends on the lane only and
    // tile rows start at multiples of ROW_BYTES, so the address of sub-step s is the
    // s = 0 address XOR 32*s.
    const int fr = lane & 31, hi = lane >> 5;
    const int lane_chunk = (hi ^ swz<BK>(fr)) * 16;
    const int a_addr = (wv * WV + fr) * ROW_BYTES + lane_chunk;
    const int b_addr = W_TILE + (wm * WM + fr) * ROW_BYTES + lane_chunk;

    // DMA of K tile kt into the stage at byte offset `so` of smem.
    auto issue = [&](int so, int kt) {
        const int kb = kt * ROW_BYTES;
#pragma unroll
        for (int j = 0; j < LW; ++j)
            __builtin_amdgcn_global_load_lds((const void *)(wbase + kb + woff[j]),
                                             (lds_void_t *)(smem + so + (wave * LW + j) * 1024), 16, 0, 0);
#pragma unroll
        for (int j = 0; j < LH; ++j)
            __builtin_amdgcn_global_load_lds((const void *)(hsrc[j] + kb),
                                             (lds_void_t *)(smem + so + W_TILE + (wave * LH + j) * 1024), 16,
                                             0, 0);
    };

    // Part p of NSPREAD of the DMA of K tile kt (W instructions first, then H).
    auto issue_part = [&](int so, int kt, int p) {
        constexpr int PER = (LW + LH) / NSPREAD;
        const int kb = kt * ROW_BYTES;
#pragma unroll
        for (int i = 0; i < LW + LH; ++i) {
            if (i / PER != p)
                continue;
            if (i < LW)
                __builtin_amdgcn_global_load_lds((const void *)(wbase + kb + woff[i]),
                                                 (lds_void_t *)(smem + so + (wave * LW + i) * 1024), 16, 0, 0);
            else
                __builtin_amdgcn_global_load_lds((const void *)(hsrc[i - LW] + kb),
                                                 (lds_void_t *)(smem + so + W_TILE + (wave * LH + i - LW) * 1024),
                                                 16, 0, 0);
        }
    };

    // Fragments of k sub-step s from the stage at byte offset `so`.
    auto load_frags = [&](int so, int s, bf16x8_t (&af)[AV], bf16x8_t (&bf)[AM]) {
        const int ab = (a_addr + so) ^ (32 * s), bb = (b_addr + so) ^ (32 * s);
#pragma unroll
        for (int a = 0; a < AV; ++a)
            af[a] = *(const bf16x8_t *)(smem + ab + a * 32 * ROW_BYTES);
#pragma unroll
        for (int bm = 0; bm < AM; ++bm)
            bf[bm] = *(const bf16x8_t *)(smem + bb + bm * 32 * ROW_BYTES);
    };

    auto mma = [&](const bf16x8_t (&af)[AV], const bf16x8_t (&bf)[AM]) {
#pragma unroll
        for (int a = 0; a < AV; ++a)
#pragma unroll
            for (int bm = 0; bm < AM; ++bm)
                acc[a][bm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a], bf[bm], acc[a][bm], 0, 0, 0);
    };

    // Wait until at most n K tiles of this wave's DMA are still in flight and this wave's
    // LDS reads are complete.
    auto wait_tiles = [&](int n) {
        if (NSTAGE >= 5 && n >= 4) wait_vmcnt<(NSTAGE >= 5 ? 4 : 0) * (LW + LH)>();
        else if (NSTAGE >= 4 && n >= 3) wait_vmcnt<(NSTAGE >= 4 ? 3 : 0) * (LW + LH)>();
        else if (NSTAGE >= 3 && n >= 2) wait_vmcnt<(NSTAGE >= 3 ? 2 : 0) * (LW + LH)>();
        else if (n >= 1) wait_vmcnt<LW + LH>();
        else wait_vmcnt<0>();
    };

    constexpr int NFR = AV + AM;            // ds_read_b128 per sub-step
    constexpr int NDMA = LW + LH;           // DMA instructions per K tile

    // Interleave the MFMAs of one sub-step with `nvm` DMA issues and NFR fragment reads.
    auto interleave = [&](int nvm) {
#pragma unroll
        for (int i = 0; i < NDMA; ++i) {
            if (i < nvm) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            }
        }
#pragma unroll
        for (int i = 0; i < NFR; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
    };

    // Pipeline.  Tile kt lives in stage kt % NSTAGE.  Step kt multiplies tile kt:
    //   sub-steps 0 .. NSUB-2: MFMAs of sub-step s while reading the fragments of s+1;
    //   then: wait for this wave's DMA of tile kt+1 and for its own LDS reads; barrier.
    //         Now tile kt+1 is complete in LDS, and no wave reads tile kt any more (its
    //         last fragments are already in registers), so its stage is refilled at once
    //         with tile kt + NSTAGE;
    //   last sub-step: MFMAs while reading sub-step 0 of tile kt+1.
    bf16x8_t af[2][AV], bf[2][AM];
    const int npre = min(NSTAGE, nk);
    for (int s = 0; s < npre; ++s)
        issue(s * STAGE, s);
    wait_tiles(npre - 1);
    barrier_no_fence();
    load_frags(0, 0, af[0], bf[0]);

    int rd = 0;                               // byte offset of stage kt % NSTAGE
    int kt = 0;
    // Steady state: every step refills a stage.  sched_barrier(0) fences each k sub-step,
    // so at most NFR (8) fragment reads are in flight: lgkmcnt is a 4-bit counter, and a
    // longer run of reads makes the compiler wait for all of them.  The refill's DMA
    // instructions are spread over NSPREAD sub-steps (the last one of this step and the
    // first NSPREAD-1 of the next): a CU's texture path moves ~64 bytes per clock, so a
    // whole 64 KiB refill issued inside one sub-step stalls the wave's MFMA issue.
    static_assert(NSPREAD >= 1 && NSPREAD <= NSUB && (LW + LH) % NSPREAD == 0, "spread");
    constexpr int PER = (LW + LH) / NSPREAD;
    int pso = 0;   // stage of the refill still being issued (parts 1 .. NSPREAD-1)
    bool pending = false;
    for (; kt + NSTAGE < nk; ++kt) {
#pragma unroll
        for (int s = 0; s + 1 < NSUB; ++s) {
            if (s + 1 < NSPREAD && pending)
                issue_part(pso, kt - 1 + NSTAGE, s + 1);
            load_frags(rd, s + 1, af[(s + 1) & 1], bf[(s + 1) & 1]);
            mma(af[s & 1], bf[s & 1]);
            interleave(s + 1 < NSPREAD ? PER : 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        wait_tiles(NSTAGE - 2);
        barrier_no_fence();
        __builtin_amdgcn_sched_barrier(0);
        issue_part(rd, kt + NSTAGE, 0);
        pso = rd;
        pending = NSPREAD > 1;
        const int nx = (rd + STAGE == NSTAGE * STAGE) ? 0 : rd + STAGE;
        load_frags(nx, 0, af[NSUB & 1], bf[NSUB & 1]);
        mma(af[(NSUB - 1) & 1], bf[(NSUB - 1) & 1]);
        interleave(PER);
        __builtin_amdgcn_sched_barrier(0);
        rd = nx;
        // NSUB is even, so af[0] / bf[0] again hold sub-step 0 of the next tile.
    }
    // Drain: no more requests (the parts of the last refill still pending go first).
    for (; kt < nk; ++kt) {
#pragma unroll
        for (int s = 0; s + 1 < NSUB; ++s) {
            if (s + 1 < NSPREAD && pending)
                issue_part(pso, kt - 1 + NSTAGE, s + 1);
            load_frags(rd, s + 1, af[(s + 1) & 1], bf[(s + 1) & 1]);
            mma(af[s & 1], bf[s & 1]);
        }
        pending = false;
        if (kt + 1 < nk) {
            wait_tiles(nk - 2 - kt);
            barrier_no_fence();
            rd = (rd + STAGE == NSTAGE * STAGE) ? 0 : rd + STAGE;
            load_frags(rd, 0, af[NSUB & 1], bf[NSUB & 1]);
        }
        mma(af[(NSUB - 1) & 1], bf[(NSUB - 1) & 1]);
    }

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
                        // plain (write-back) stores: the L2 merges the 8-byte pieces into full
                        // lines; non-temporal stores measured 25% slower here
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

// Persistent form of the tiled kernel: one workgroup per CU walks a list of 256 x 256
// output tiles as one continuous stream of (tile, K tile) steps.
//  * XCD x (hardware block b runs on XCD b % 8) owns a contiguous range of logical tiles
//    in the grouped order; its G/8 workgroups take consecutive tiles of that range in
//    lockstep (tile start_x + slot + i * G/8), so the workgroups resident on one XCD at a
//    time share W slabs and H row blocks in its L2.
//  * The DMA stream runs ahead across tile boundaries: the next tile's first K tiles
//    are in flight while the current tile's last steps and epilogue run, and the next
//    tile's H row indices are loaded a whole tile ahead.
//  * Epilogue stores are 16 bytes per lane for bf16 output: permlane32_swap gives each
//    lane eight consecutive vocabulary entries.
// The k order of every output element is the tiled kernel's, so results are
// bit-identical to it.
template <int BK, int NSTAGE, int NSPREAD, bool OUT_BF16>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1))) void
gather_gemm_bf16_persist_kernel(const __bf16 *__restrict__ H, const int32_t *__restrict__ idx, int32_t rows,
                                const __bf16 *__restrict__ W, int32_t V, int32_t d, void *__restrict__ out,
                                int64_t ldo, int32_t group_m)
{
    constexpr int BV = 256, BM = 256;
    constexpr int ROW_BYTES = BK * 2;
    constexpr int CHUNKS = BK / 8;
    constexpr int RPI = 64 / CHUNKS;
    constexpr int W_TILE = BV * ROW_BYTES;
    constexpr int H_TILE = BM * ROW_BYTES;
    constexpr int STAGE = W_TILE + H_TILE;
    constexpr int WV = BV / 2, WM = BM / 2;
    constexpr int AV = WV / 32, AM = WM / 32;
    constexpr int LW = BV / RPI / 4, LH = BM / RPI / 4;
    constexpr int NSUB = BK / 16;
    constexpr int NDMA = LW + LH;
    constexpr int NFR = AV + AM;
    static_assert(NSTAGE * STAGE <= 160 * 1024, "LDS");
    static_assert(NSTAGE >= 2 && NSUB % 2 == 0, "pipeline");
    static_assert(NSPREAD >= 1 && NSPREAD <= NSUB && NDMA % NSPREAD == 0, "spread");
    constexpr int PER = NDMA / NSPREAD;

    __shared__ __attribute__((aligned(1024))) char smem[NSTAGE * STAGE];

    const int nvt = (V + BV - 1) / BV;
    const int nmt = (rows + BM - 1) / BM;
    const int ntiles = nvt * nmt;
    const int nk = d / BK;

    // ---- this workgroup's tile list
    const int G = gridDim.x;                    // a multiple of 8
    const int per_xcd = G >> 3;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int q = ntiles >> 3, rem = ntiles & 7;
    const int start = xcd < rem ? xcd * (q + 1) : rem * (q + 1) + (xcd - rem) * q;
    const int count = q + (xcd < rem ? 1 : 0);
    const int n_my = slot < count ? (count - slot + per_xcd - 1) / per_xcd : 0;
    const int total = n_my * nk;                // steps of this workgroup
    if (total == 0)
        return;
    auto tile_coords = [&](int i, int &m0, int &v0) {
        const int t = start + slot + i * per_xcd;
        const int per_group = group_m * nvt;
        const int g = t / per_group;
        const int first_m = g * group_m;
        const int gsz = min(nmt - first_m, group_m);
        const int local = t - g * per_group;
        m0 = (first_m + local % gsz) * BM;
        v0 = (local / gsz) * BV;
    };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wv = wave & 1, wm = wave >> 1;

    // ---- per-tile DMA sources, for the current and the next tile of the list
    struct Src {
        const char *wbase;
        uint32_t woff[LW];
        const char *hsrc[LH];
    };
    auto row_w = [&](int j) { return (wave * LW + j) * RPI + lane / CHUNKS; };
    auto row_h = [&](int j) { return (wave * LH + j) * RPI + lane / CHUNKS; };
    auto chunk_of = [&](int r) { return ((lane % CHUNKS) ^ swz<BK>(r)) * 16; };
    int32_t hidx_nxt[LH];                       // H row ids of the next tile (loaded a tile ahead)
    auto load_hidx = [&](int i) {
        if (i >= n_my)
            return;
        int m0, v0;
        tile_coords(i, m0, v0);
#pragma unroll
        for (int j = 0; j < LH; ++j)
            hidx_nxt[j] = idx[min(m0 + row_h(j), rows - 1)];
    };
    auto make_src = [&](int i, Src &sr) {
        int m0, v0;
        tile_coords(min(i, n_my - 1), m0, v0);
        sr.wbase = (const char *)(W + (int64_t)v0 * d);
#pragma unroll
        for (int j = 0; j < LW; ++j) {
            const int vr = min(v0 + row_w(j), V - 1) - v0;
            sr.woff[j] = (uint32_t)vr * (uint32_t)d * 2u + (uint32_t)chunk_of(row_w(j));
        }
#pragma unroll
        for (int j = 0; j < LH; ++j)
            sr.hsrc[j] = (const char *)(H + (int64_t)hidx_nxt[j] * d) + chunk_of(row_h(j));
    };
    Src cur;
    load_hidx(0);
    make_src(0, cur);
    load_hidx(1);

    // DMA of instructions [p*PER, (p+1)*PER) of K tile kt of the output tile whose
    // sources are `sr`, into the stage at byte offset `so`
    auto issue_part = [&](const Src &sr, int so, int kt, int p) {
        const int kb = kt * ROW_BYTES;
#pragma unroll
        for (int i = 0; i < NDMA; ++i) {
            if (i / PER != p)
                continue;
            if (i < LW)
                __builtin_amdgcn_global_load_lds((const void *)(sr.wbase + kb + sr.woff[i]),
                                                 (lds_void_t *)(smem + so + (wave * LW + i) * 1024), 16, 0, 0);
            else
                __builtin_amdgcn_global_load_lds((const void *)(sr.hsrc[i - LW] + kb),
                                                 (lds_void_t *)(smem + so + W_TILE + (wave * LH + i - LW) * 1024),
                                                 16, 0, 0);
        }
    };

    f32x16_t acc[AV][AM];
    auto zero_acc = [&]() {
#pragma unroll
        for (int a = 0; a < AV; ++a)
#pragma unroll
            for (int bm = 0; bm < AM; ++bm)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    acc[a][bm][e] = 0.0f;
    };
    zero_acc();

    const int fr = lane & 31, hi = lane >> 5;
    const int lane_chunk = (hi ^ swz<BK>(fr)) * 16;
    const int a_addr = (wv * WV + fr) * ROW_BYTES + lane_chunk;
    const int b_addr = W_TILE + (wm * WM + fr) * ROW_BYTES + lane_chunk;

    auto load_frags = [&](int so, int s, bf16x8_t (&af)[AV], bf16x8_t (&bf)[AM]) {
        const int ab = (a_addr + so) ^ (32 * s), bb = (b_addr + so) ^ (32 * s);
#pragma unroll
        for (int a = 0; a < AV; ++a)
            af[a] = *(const bf16x8_t *)(smem + ab + a * 32 * ROW_BYTES);
#pragma unroll
        for (int bm = 0; bm < AM; ++bm)
            bf[bm] = *(const bf16x8_t *)(smem + bb + bm * 32 * ROW_BYTES);
    };
    auto mma = [&](const bf16x8_t (&af)[AV], const bf16x8_t (&bf)[AM]) {
#pragma unroll
        for (int a = 0; a < AV; ++a)
#pragma unroll
            for (int bm = 0; bm < AM; ++bm)
                acc[a][bm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a], bf[bm], acc[a][bm], 0, 0, 0);
    };
    auto wait_tiles = [&](int n) {
        if (NSTAGE >= 5 && n >= 4) wait_vmcnt<(NSTAGE >= 5 ? 4 : 0) * NDMA>();
        else if (NSTAGE >= 4 && n >= 3) wait_vmcnt<(NSTAGE >= 4 ? 3 : 0) * NDMA>();
        else if (NSTAGE >= 3 && n >= 2) wait_vmcnt<(NSTAGE >= 3 ? 2 : 0) * NDMA>();
        else if (n >= 1) wait_vmcnt<NDMA>();
        else wait_vmcnt<0>();
    };
    auto interleave = [&](int nvm) {
#pragma unroll
        for (int i = 0; i < NDMA; ++i) {
            if (i < nvm) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            }
        }
#pragma unroll
        for (int i = 0; i < NFR; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
    };

    // Epilogue of tile i: lane holds, for block (a, bm) and group gq, vocabulary entries
    // v = v0 + wv*WV + 32a + 8gq + 4hi + (0..3) of masked row m0 + wm*WM + 32bm + fr.
    // 16-byte stores need a 16-byte aligned row start
    const bool vec_ok = ((uintptr_t)out & 15) == 0 && (ldo & (OUT_BF16 ? 7 : 3)) == 0;
    auto epilogue = [&](int i) {
        int m0, v0;
        tile_coords(i, m0, v0);
#pragma unroll
        for (int bm = 0; bm < AM; ++bm) {
            const int row = m0 + wm * WM + bm * 32 + fr;
            const bool row_ok = row < rows;
#pragma unroll
            for (int a = 0; a < AV; ++a) {
                const int vb = v0 + wv * WV + a * 32;
                if constexpr (OUT_BF16) {
                    uint32_t pk[4][2];
#pragma unroll
                    for (int gq = 0; gq < 4; ++gq) {
                        pk[gq][0] = pack_bf16x2(acc[a][bm][gq * 4 + 0], acc[a][bm][gq * 4 + 1]);
                        pk[gq][1] = pack_bf16x2(acc[a][bm][gq * 4 + 2], acc[a][bm][gq * 4 + 3]);
                    }
                    // lanes 0-31 collect v 0..7 / 16..23, lanes 32-63 v 8..15 / 24..31
#pragma unroll
                    for (int pr = 0; pr < 2; ++pr) {
                        const auto s0 = __builtin_amdgcn_permlane32_swap(pk[2 * pr][0], pk[2 * pr + 1][0], false, false);
                        const auto s1 = __builtin_amdgcn_permlane32_swap(pk[2 * pr][1], pk[2 * pr + 1][1], false, false);
                        const int v = vb + 16 * pr + 8 * hi;
                        __bf16 *o = (__bf16 *)out + (int64_t)row * ldo + v;
                        if (!row_ok)
                            continue;   // (after the swaps: every lane takes part in them)
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
                } else {
#pragma unroll
                    for (int gq = 0; gq < 4; ++gq) {
                        const int v = vb + gq * 8 + hi * 4;
                        float *o = (float *)out + (int64_t)row * ldo + v;
                        const float x0 = acc[a][bm][gq * 4 + 0], x1 = acc[a][bm][gq * 4 + 1];
                        const float x2 = acc[a][bm][gq * 4 + 2], x3 = acc[a][bm][gq * 4 + 3];
                        if (!row_ok)
                            continue;
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
                // this block is stored: restart its accumulation (keeps one block in VGPRs)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    acc[a][bm][e] = 0.0f;
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    // ---- per tile: the tiled kernel's pipeline.  The next tile's first NSTAGE K tiles
    // are requested right after the last MFMAs of a tile have their operands, so they are
    // in flight while the epilogue stores run.
    bf16x8_t af[2][AV], bf[2][AM];
    const int npre = min(NSTAGE, nk);
    for (int s = 0; s < npre; ++s)
#pragma unroll
        for (int p = 0; p < NSPREAD; ++p)
            issue_part(cur, s * STAGE, s, p);

    for (int i = 0; i < n_my; ++i) {
        wait_tiles(npre - 1);
        barrier_no_fence();
        load_frags(0, 0, af[0], bf[0]);
        int rd = 0, pso = 0, pkt = 0;
        bool pending = false;
        int kt = 0;
        for (; kt + NSTAGE < nk; ++kt) {
#pragma unroll
            for (int s = 0; s + 1 < NSUB; ++s) {
                if (s + 1 < NSPREAD && pending)
                    issue_part(cur, pso, pkt, s + 1);
                load_frags(rd, s + 1, af[(s + 1) & 1], bf[(s + 1) & 1]);
                mma(af[s & 1], bf[s & 1]);
                interleave(s + 1 < NSPREAD ? PER : 0);
                __builtin_amdgcn_sched_barrier(0);
            }
            wait_tiles(NSTAGE - 2);
            barrier_no_fence();
            __builtin_amdgcn_sched_barrier(0);
            issue_part(cur, rd, kt + NSTAGE, 0);
            pso = rd;
            pkt = kt + NSTAGE;
            pending = NSPREAD > 1;
            const int nx = (rd + STAGE == NSTAGE * STAGE) ? 0 : rd + STAGE;
            load_frags(nx, 0, af[NSUB & 1], bf[NSUB & 1]);
            mma(af[(NSUB - 1) & 1], bf[(NSUB - 1) & 1]);
            interleave(PER);
            __builtin_amdgcn_sched_barrier(0);
            rd = nx;
        }
        for (; kt < nk; ++kt) {
#pragma unroll
            for (int s = 0; s + 1 < NSUB; ++s) {
                if (s + 1 < NSPREAD && pending)
                    issue_part(cur, pso, pkt, s + 1);
                load_frags(rd, s + 1, af[(s + 1) & 1], bf[(s + 1) & 1]);
                mma(af[s & 1], bf[s & 1]);
            }
            pending = false;
            if (kt + 1 < nk) {
                wait_tiles(nk - 2 - kt);
                barrier_no_fence();
                rd = (rd + STAGE == NSTAGE * STAGE) ? 0 : rd + STAGE;
                load_frags(rd, 0, af[NSUB & 1], bf[NSUB & 1]);
            }
            mma(af[(NSUB - 1) & 1], bf[(NSUB - 1) & 1]);
        }
        // every wave's last fragments are in registers: the stages are free
        wait_vmcnt<63>();
        barrier_no_fence();
        if (i + 1 < n_my) {
            make_src(i + 1, cur);
            for (int s = 0; s < npre; ++s)
#pragma unroll
                for (int p = 0; p < NSPREAD; ++p)
                    issue_part(cur, s * STAGE, s, p);
        }
        epilogue(i);   // also restarts the accumulators
        load_hidx(i + 2);
    }
}

// Persistent eight-wave form with deferred stores (bf16 output).
//  * 256 x 256 tiles, K staged 64 deep in two LDS stages, eight waves: two per SIMD, so
//    while one wave waits (DMA issue, barrier) the other keeps the matrix core busy.  A
//    wave owns 128 vocabulary x 64 masked rows (4 x 2 MFMA blocks, 128 accumulators).
//  * Tile lists per XCD, with the XCDs side by side on large launches (below).
//  * When a tile's K loop ends, its results are rounded to bf16 and arranged for 16-byte
//    stores (permlane32_swap) in registers; NIMM of its stores go out at once and the rest
//    are issued over the first DEFER K steps of the next tile.  Every workgroup reaches a
//    tile boundary at about the same time, so storing whole tiles there sends one burst of
//    all workgroups' results to memory while the matrix cores idle; spreading the stores
//    over MFMA time removes most of that cost.  The last tile stores at once.
// Same MFMA, operand roles and k order as the tiled kernel: results are bit-identical.
//
// REDUCE: the per-row consumer of the logits (largest logit, first index attaining it,
// sum of exp(logit - largest)) is reduced from the fp32 accumulators of every tile
// before they are rounded: each lane walks its 64 entries of a row in ascending
// vocabulary order, the two lanes that share a row combine through permlane32_swap, and
// the two waves that share the row's 256 entries combine through LDS.  One partial per
// (row, vocabulary tile) goes to pmax / parg / psum ([nvt][rows], column-major so a
// wave's 32 rows are consecutive words); mosaic_logits_reduce_finish combines them.
// STORE = false skips the logits stores (consumer-only use: the logits never exist).
//
// M16: the same tile with v_mfma_f32_16x16x32_bf16 (a wave's 128 x 64 as 8 x 4 blocks of
// 16 x 16, k 32 per instruction, so one K tile is two k sub-steps instead of four).  The
// same k order gives results bit-identical to the 32 x 32 x 16 form (measured), and it
// runs about 4% faster.  A sub-step's fragments take twice the registers, which leaves
// no room for deferred stores (they push the K loop into spilling: measured slower, also
// with the deferred words parked in LDS), so the M16 forms store each tile at its end.
// A lane holds four consecutive vocabulary entries of one row per block; permlane16_swap
// pairs the lanes of neighbouring blocks into 16-byte stores, and the four lanes of a row
// combine their consumer partials through permlane16_swap and permlane32_swap.
//
// DMAW: the waves that request K tiles.  8: every wave requests its eighth of each K tile.
// 4 (the 16 x 16 x 32 defaults): only waves 0-3, one per SIMD, request K tiles, a quarter
// each, and waves 4-7 issue no DMA at all, so one wave of each SIMD never waits on the
// texture path and keeps its matrix core fed while the other issues requests.  The two
// kinds of wave run separate instantiations of the K loop (no per-request branch).
// Measured on 4096 rows x 4096 x 126464: moving one launch's K tiles alone takes 1.76 ms
// with 4 requesting waves and 1.94 ms with 8; the GEMM runs 3-5% faster; bit-identical.
//
// DEEP: false: two LDS stages per operand, so the refill issued at step kt's barrier must
// land by the next one (a single batch of requests in flight, and the texture path idles
// between batches).  true: W gets a third stage (160 KiB of LDS in all).  Step kt requests
// W's rows of K tile kt + 2 at its start and H's after its barrier, so W's requests are in
// flight while H's land, and a step's 16 requests are split over its two halves: 3-7%
// faster (4096 x 4096 x 126464: 1448-1452 against 1393-1395 TFLOP/s with W's requested at
// the barrier, K tile kt + 3; requesting them at the next step's start instead gained
// 0.3-1.8% more).  (With the XCDs out of step on large launches it was 5-6% slower there;
// with the tile order below it is not.)  A third H stage instead gained nothing.  REDUCE
// with a third stage keeps its partials in the W stage that is free at each tile's end
// (RED_IN_STAGE): 2-5% faster than two stages.
template <int NSPREAD, int DEFER, int NIMM, bool STORE = true, bool REDUCE = false, bool M16 = false, int DMAW = 8,
          bool DEEP = false>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2))) void
gather_gemm_bf16_defer_kernel(const __bf16 *__restrict__ H, const int32_t *__restrict__ idx, int32_t rows,
                              const __bf16 *__restrict__ W, int32_t V, int32_t d, __bf16 *__restrict__ out,
                              int64_t ldo, int32_t group_m, float *__restrict__ pmax,
                              int32_t *__restrict__ parg, float *__restrict__ psum,
                              const int32_t *__restrict__ rows_dev)
{
    // rows_dev: the row count in device memory, written earlier on the stream (the launch
    // grid was sized for `rows`, the capacity); negative counts are 0, larger ones `rows`.
    // The REDUCE partials keep the capacity as their row stride.
    const int32_t ldp = rows;
    if (rows_dev)
        rows = min(max(*rows_dev, 0), rows);
    constexpr int NW = 8, BV = 256, BM = 256, BK = 64, NSTAGE = 2;
    constexpr int WST = DEEP ? 3 : 2, HST = 2;   // W and H stages
    constexpr int ROW_BYTES = BK * 2;
    constexpr int CHUNKS = BK / 8;
    constexpr int RPI = 64 / CHUNKS;
    constexpr int W_TILE = BV * ROW_BYTES;
    constexpr int H_TILE = BM * ROW_BYTES;
    // LDS: the two W stages (32 KiB each), then the two H stages; a refill requests H's
    // rows before W's.  Against alternating W and H stages with W first, measured on one
    // MI355X: +0.5-1% for the 16 x 16 x 32 form, -2% for the 32 x 32 x 16 form.
    constexpr int H_BASE = WST * W_TILE;
    constexpr int WV = BV / 2, WM = BM / (NW / 2);
    constexpr int MB = M16 ? 16 : 32;         // MFMA block edge
    constexpr int KI = M16 ? 32 : 16;         // k per MFMA
    constexpr int NACC = MB * MB / 64;        // accumulators per lane and block
    constexpr int AV = WV / MB, AM = WM / MB;
    constexpr int LW = BV / RPI / DMAW, LH = BM / RPI / DMAW;   // DMA instructions of a DMA wave
    constexpr int NSUB = BK / KI;
    constexpr int NDMA = LW + LH;
    constexpr int NFR = AV + AM;
    constexpr int NST = M16 ? AV * AM / 2 : AV * AM * 2;   // 16-byte stores per lane and tile
    constexpr int HOOK_S = NSUB > 2 ? 1 : 0;  // k sub-step that issues a step's deferred stores
    constexpr int EARLY = 1;                  // 16 x 16: rows whose next A fragment is read early
    using acc_t = typename std::conditional<M16, f32x4_t, f32x16_t>::type;
    static_assert(NSPREAD >= 1 && NSPREAD <= NSUB && NDMA % NSPREAD == 0, "spread");
    static_assert(NIMM >= 0 && NIMM <= NST && DEFER >= 1 && (NST - NIMM) % DEFER == 0, "defer");
    constexpr int PER = NDMA / NSPREAD;
    constexpr int SPS = (NST - NIMM) / DEFER; // deferred stores per K step

    // The K stages, then (REDUCE) the per-row partials of the upper vocabulary half
    // (wv = 1) of a tile, [3][BM] floats.  One LDS object: with a second one the compiler
    // can no longer tell the stage DMA from the fragment reads and waits for every DMA
    // before each read (measured 17% slower).
    // With a third W stage the five stages take all 160 KiB, and the partials live in the W
    // stage that is free at the tile's end (RED_IN_STAGE, below).
    constexpr bool RED_IN_STAGE = REDUCE && DEEP;
    constexpr int RED_BYTES = REDUCE && !RED_IN_STAGE ? 3 * BM * 4 : 0;
    static_assert(H_BASE + HST * H_TILE + RED_BYTES <= 160 * 1024, "LDS");
    static_assert(!DEEP || (NSPREAD == 1 && M16 && NIMM == NST), "a third stage: 16 x 16 form, no deferral");
    static_assert(!M16 || AV % 4 == 0, "16 x 16 stores: whole 128-byte lines from block-pair pairs");
    __shared__ __attribute__((aligned(1024))) char smem[H_BASE + HST * H_TILE + RED_BYTES];
    float *red_lds = (float *)(smem + H_BASE + HST * H_TILE);
    // W stage of the current tile's K tile 0.  0 except with RED_IN_STAGE, where each tile's
    // ring starts so that the next tile's K tile 2 lands in the stage that held this tile's
    // partials: that request waits for the next tile's first barrier, after every wave has
    // read them.
    int w0 = 0;

    const int nvt = (V + BV - 1) / BV;
    const int nmt = (rows + BM - 1) / BM;
    const int ntiles = nvt * nmt;
    const int nk = d / BK;

    // ---- this workgroup's tile list
    const int G = gridDim.x;                    // a multiple of 8
    const int per_xcd = G >> 3;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int per_group = group_m * nvt;
    // The row tiles come in super-groups of 8 * group_m.  In a full one, XCD x takes row
    // tiles x, x + 8, ... and every vocabulary tile of them in order, so the eight XCDs sweep
    // the vocabulary side by side and read each W slab at about the same time (from HBM
    // once, then from the Infinity Cache).  The tiles of the rows after the last full
    // super-group go to the XCDs in eight contiguous runs of group order (group_m row tiles
    // by every vocabulary tile): XCD x takes the x-th run.  With the XCDs out of step (the
    // runs alone, on 84 and 116 row tiles) the GEMM measured 2-4% slower.
    const int sg = 8 * group_m;
    const int nfull = nmt / sg;
    const int full_tiles = nfull * per_group;  // per XCD
    const int rtiles = ntiles - 8 * full_tiles;
    const int q = rtiles >> 3, rem = rtiles & 7;
    const int start = xcd < rem ? xcd * (q + 1) : rem * (q + 1) + (xcd - rem) * q;
    const int count = full_tiles + q + (xcd < rem ? 1 : 0);
    const int n_my = slot < count ? (count - slot + per_xcd - 1) / per_xcd : 0;
    if (n_my == 0)
        return;
    auto tile_coords = [&](int i, int &m0, int &v0) __attribute__((always_inline)) {
        const int tx = slot + i * per_xcd;
        if (tx < full_tiles) {
            const int s = tx / per_group;
            const int t = 8 * (tx - s * per_group) + xcd;
            m0 = (s * sg + t % sg) * BM;
            v0 = (t / sg) * BV;
            return;
        }
        const int t = start + tx - full_tiles;
        const int g = t / per_group;
        const int first_m = nfull * sg + g * group_m;
        const int gsz = min(nmt - first_m, group_m);
        const int local = t - g * per_group;
        m0 = (first_m + local % gsz) * BM;
        v0 = (local / gsz) * BV;
    };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wv = wave & 1, wm = wave >> 1;

    // ---- DMA sources of the current tile (same layout as the tiled kernel)
    const int dwave = wave % DMAW;              // waves >= DMAW issue no DMA
    const bool dma_wave = wave < DMAW;
    auto row_w = [&](int j) { return (dwave * LW + j) * RPI + lane / CHUNKS; };
    auto row_h = [&](int j) { return (dwave * LH + j) * RPI + lane / CHUNKS; };
    auto chunk_of = [&](int r) { return ((lane % CHUNKS) ^ swz<BK>(r)) * 16; };
    int32_t hidx_nxt[LH];                       // H row ids of the next tile (loaded a tile ahead)
    auto load_hidx = [&](int i) __attribute__((always_inline)) {
        if (i >= n_my)
            return;
        int m0, v0;
        tile_coords(i, m0, v0);
#pragma unroll
        for (int j = 0; j < LH; ++j)
            hidx_nxt[j] = idx[min(m0 + row_h(j), rows - 1)];
    };
    const char *wbase;
    uint32_t woff[LW];
    const char *hsrc[LH];
    auto make_src = [&](int i) __attribute__((always_inline)) {
        int m0, v0;
        tile_coords(i, m0, v0);
        wbase = (const char *)(W + (int64_t)v0 * d);
#pragma unroll
        for (int j = 0; j < LW; ++j) {
            const int vr = min(v0 + row_w(j), V - 1) - v0;
            woff[j] = (uint32_t)vr * (uint32_t)d * 2u + (uint32_t)chunk_of(row_w(j));
        }
#pragma unroll
        for (int j = 0; j < LH; ++j)
            hsrc[j] = (const char *)(H + (int64_t)hidx_nxt[j] * d) + chunk_of(row_h(j));
    };
    load_hidx(0);
    make_src(0);
    load_hidx(1);

    // Part p of the refill with K tile kt: H's rows into the H stage at byte offset rh, then
    // W's into the W stage at rw.
    auto issue_part = [&](int rw, int rh, int kt, int p) __attribute__((always_inline)) {
        const int kb = kt * ROW_BYTES;
#pragma unroll
        for (int i = 0; i < NDMA; ++i) {
            if (i / PER != p)
                continue;
            if (i < LH)
                __builtin_amdgcn_global_load_lds((const void *)(hsrc[i] + kb),
                                                 (lds_void_t *)(smem + rh + (dwave * LH + i) * 1024), 16, 0, 0);
            else
                __builtin_amdgcn_global_load_lds((const void *)(wbase + kb + woff[i - LH]),
                                                 (lds_void_t *)(smem + rw + (dwave * LW + i - LH) * 1024), 16, 0,
                                                 0);
        }
    };
    auto next_w = [](int rw) { return rw + W_TILE == WST * W_TILE ? 0 : rw + W_TILE; };
    auto next_h = [](int rh) { return rh + H_TILE == H_BASE + HST * H_TILE ? H_BASE : rh + H_TILE; };
    // One operand's rows of K tile kt (the 16 x 16 forms with a third stage)
    auto issue_h = [&](int rh, int kt) __attribute__((always_inline)) {
        const int kb = kt * ROW_BYTES;
#pragma unroll
        for (int i = 0; i < LH; ++i)
            __builtin_amdgcn_global_load_lds((const void *)(hsrc[i] + kb),
                                             (lds_void_t *)(smem + rh + (dwave * LH + i) * 1024), 16, 0, 0);
    };
    auto issue_w = [&](int rw, int kt) __attribute__((always_inline)) {
        const int kb = kt * ROW_BYTES;
#pragma unroll
        for (int i = 0; i < LW; ++i)
            __builtin_amdgcn_global_load_lds((const void *)(wbase + kb + woff[i]),
                                             (lds_void_t *)(smem + rw + (dwave * LW + i) * 1024), 16, 0, 0);
    };

    acc_t acc[AV][AM];
    auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int a = 0; a < AV; ++a)
#pragma unroll
            for (int bm = 0; bm < AM; ++bm)
#pragma unroll
                for (int e = 0; e < NACC; ++e)
                    acc[a][bm][e] = 0.0f;
    };
    zero_acc();

    // Fragment lanes.  32 x 32 x 16: lane l reads block row l % 32, k chunk 2s + l / 32 of
    // sub-step s.  16 x 16 x 32: lane l reads block row l % 16, k chunk 4s + l / 16.  The
    // swizzle of a row depends on the lane only (blocks start at multiples of 16 rows), and
    // a sub-step's chunk bits sit above the lane's, so sub-step s is an XOR of the address.
    const int fr = lane & 31, hi = lane >> 5;     // 32 x 32 lanes
    const int r16 = lane & 15, qd = lane >> 4;    // 16 x 16 lanes
    const int lane_row = M16 ? r16 : fr;
    const int lane_chunk = ((M16 ? qd : hi) ^ swz<BK>(lane_row)) * 16;
    const int a_addr = (wv * WV + lane_row) * ROW_BYTES + lane_chunk;
    const int b_addr = (wm * WM + lane_row) * ROW_BYTES + lane_chunk;   // from an H stage
    constexpr int SUB_BYTES = KI * 2;

    auto load_frags = [&](int rw, int rh, int s, bf16x8_t (&af)[AV], bf16x8_t (&bf)[AM]) __attribute__((always_inline)) {
        const int ab = (a_addr + rw) ^ (SUB_BYTES * s), bb = (b_addr + rh) ^ (SUB_BYTES * s);
#pragma unroll
        for (int a = 0; a < AV; ++a)
            af[a] = *(const bf16x8_t *)(smem + ab + a * MB * ROW_BYTES);
#pragma unroll
        for (int bm = 0; bm < AM; ++bm)
            bf[bm] = *(const bf16x8_t *)(smem + bb + bm * MB * ROW_BYTES);
    };
    auto mma = [&](const bf16x8_t (&af)[AV], const bf16x8_t (&bf)[AM]) __attribute__((always_inline)) {
#pragma unroll
        for (int a = 0; a < AV; ++a)
#pragma unroll
            for (int bm = 0; bm < AM; ++bm) {
                if constexpr (M16)
                    acc[a][bm] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[a], bf[bm], acc[a][bm], 0, 0, 0);
                else
                    acc[a][bm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a], bf[bm], acc[a][bm], 0, 0, 0);
            }
    };
    // MFMAs on fragment buffer `cur` while the fragments of k sub-step s of the stages at
    // rw (W) and rh (H) are read.
    // 32 x 32: both operands double-buffered.  16 x 16 (twice the fragment registers per
    // sub-step): the B fragments are double-buffered, the A fragments single: block a's
    // next fragment is read right after the last MFMA of its row.
    auto mma_load = [&](int rw, int rh, int s, int cur, bf16x8_t (&af)[2][AV], bf16x8_t (&bf)[2][AM])
                        __attribute__((always_inline)) {
        if constexpr (M16) {
            const int ab = (a_addr + rw) ^ (SUB_BYTES * s), bb = (b_addr + rh) ^ (SUB_BYTES * s);
#pragma unroll
            for (int bm = 0; bm < AM; ++bm)
                bf[cur ^ 1][bm] = *(const bf16x8_t *)(smem + bb + bm * MB * ROW_BYTES);
#pragma unroll
            for (int a = 0; a < AV; ++a) {
                // the last row reads its next fragment before its MFMAs (into a spare
                // register): the reads of a stage must be complete at the step's barrier, and
                // this way the wave's last read is followed by MFMAs instead of the wait
                // (measured +1.5%; reading the last two or four rows early gains no more)
                const bool early = a >= AV - EARLY;
                bf16x8_t nxt;
                if (early)
                    nxt = *(const bf16x8_t *)(smem + ab + a * MB * ROW_BYTES);
                // odd rows take the B blocks in reverse, so consecutive MFMAs always share
                // one operand (a row's last B block is the next row's first): fewer operand
                // bits change, which lowers the power per MFMA and lets the clock rise
                // (+0.4-0.9% on 1229 to 21399 rows, two MI355Xs; each block's k order, and so
                // every result bit, is unchanged)
#pragma unroll
                for (int c = 0; c < AM; ++c) {
                    const int bm = (a & 1) ? AM - 1 - c : c;
                    acc[a][bm] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[0][a], bf[cur][bm], acc[a][bm], 0, 0, 0);
                }
                af[0][a] = early ? nxt : *(const bf16x8_t *)(smem + ab + a * MB * ROW_BYTES);
            }
        } else {
            load_frags(rw, rh, s, af[cur ^ 1], bf[cur ^ 1]);
            mma(af[cur], bf[cur]);
        }
    };
    // Instruction order of one k sub-step: each refill DMA issue beside an MFMA, then the
    // fragment reads spread over the MFMAs (16 x 16: the B reads first, then each A read
    // after its row's MFMAs, the last row's before them).
    auto interleave = [&](int nvm) {
#pragma unroll
        for (int i = 0; i < NDMA; ++i) {
            if (i < nvm) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            }
        }
        if constexpr (M16) {
#pragma unroll
            for (int bm = 0; bm < AM; ++bm) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            const int used = nvm + AM;
#pragma unroll
            for (int a = 0; a < AV; ++a) {
                if (a >= AV - EARLY)
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
                for (int c = 0; c < AM; ++c)
                    if (a * AM + c >= used)
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (a < AV - EARLY)
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
        } else {
#pragma unroll
            for (int i = 0; i < NFR; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
        }
    };

    // ---- results of the previous tile, as 16-byte store words.  32 x 32: store j covers block
    // (a, bm) = ((j / 2) / AM, (j / 2) % AM), vocabulary entries 16 * (j % 2) + 8 * hi + (0..7)
    // of that block for masked row 32 * bm + fr of the wave's sub-tile.  16 x 16: store j
    // covers the block pair (2 * (j / AM), +1) of row block bm = j % AM; a lane with even qd
    // holds entries 4 * qd + (0..7) of the first block, one with odd qd entries
    // 4 * (qd - 1) + (0..7) of the second, for masked row 16 * bm + r16.
    uint32_t pk[NST][4];
    int pm0 = 0, pv0 = 0;
    const bool vec_ok = ((uintptr_t)out & 15) == 0 && (ldo & 7) == 0;
    auto store_one = [&](int j) __attribute__((always_inline)) {
        int row, v;
        if constexpr (M16) {
            // word (2 q + h) * AM + bm: rows 8 h .. 8 h + 7 of row block bm, block pair
            // 2 q + (r16 >> 3) (see pack)
            const int ap = j / AM, bm = j % AM;
            row = pm0 + wm * WM + bm * 16 + 8 * (ap & 1) + (r16 & 7);
            v = pv0 + wv * WV + (2 * ((ap & ~1) + (r16 >> 3)) + (qd & 1)) * 16 + 4 * (qd & 2);
        } else {
            const int a = (j >> 1) / AM, bm = (j >> 1) % AM, pr = j & 1;
            row = pm0 + wm * WM + bm * 32 + fr;
            v = pv0 + wv * WV + a * 32 + 16 * pr + 8 * hi;
        }
        if (row < rows) {
            __bf16 *o = out + (int64_t)row * ldo + v;
            if (vec_ok && v + 7 < V) {
                *(uint4 *)o = make_uint4(pk[j][0], pk[j][1], pk[j][2], pk[j][3]);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (v + e < V)
                        o[e] = __builtin_bit_cast(__bf16, (uint16_t)(pk[j][e >> 1] >> (16 * (e & 1))));
            }
        }
    };
    // acc -> pk (round to bf16; 32 x 32: lanes 0-31 take entries 0-7 / 16-23 of a block,
    // lanes 32-63 entries 8-15 / 24-31; 16 x 16: permlane16_swap trades the odd-qd lanes'
    // words of the first block of a pair for the even-qd lanes' words of the second), then
    // restart the accumulators
    auto pack = [&]() __attribute__((always_inline)) {
        if constexpr (M16) {
#pragma unroll
            for (int ap = 0; ap < AV / 2; ++ap)
#pragma unroll
                for (int bm = 0; bm < AM; ++bm) {
                    const auto &x = acc[2 * ap][bm], &y = acc[2 * ap + 1][bm];
                    const auto s0 = __builtin_amdgcn_permlane16_swap(pack_bf16x2(x[0], x[1]), pack_bf16x2(y[0], y[1]),
                                                                     false, false);
                    const auto s1 = __builtin_amdgcn_permlane16_swap(pack_bf16x2(x[2], x[3]), pack_bf16x2(y[2], y[3]),
                                                                     false, false);
                    const int j = ap * AM + bm;
                    pk[j][0] = s0[0];
                    pk[j][1] = s1[0];
                    pk[j][2] = s0[1];
                    pk[j][3] = s1[1];
                }
            // Block pairs 2q and 2q + 1 of a row hold its two 64-byte halves of one 128-byte
            // line.  Lanes r16 and r16 ^ 8 trade words so that one store instruction writes
            // whole lines: rows 0-7 of the row block (upper lanes the second halves), then
            // rows 8-15 (lower lanes the first halves).  Each is one DPP move (row rotate by
            // 8) whose bank mask writes only the receiving half of each 16-lane row.  A
            // store-only probe of the two layouts ran at 4.5 and 5.45 TB/s.
#pragma unroll
            for (int q = 0; q < AV / 4; ++q)
#pragma unroll
                for (int bm = 0; bm < AM; ++bm) {
                    const int j0 = 2 * q * AM + bm, j1 = j0 + AM;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int w0 = (int)pk[j0][e], w1 = (int)pk[j1][e];
                        pk[j0][e] = (uint32_t)__builtin_amdgcn_update_dpp(w0, w1, 0x128, 0xf, 0xc, false);
                        pk[j1][e] = (uint32_t)__builtin_amdgcn_update_dpp(w1, w0, 0x128, 0xf, 0x3, false);
                    }
                }
        } else {
#pragma unroll
        for (int a = 0; a < AV; ++a)
#pragma unroll
            for (int bm = 0; bm < AM; ++bm) {
                uint32_t p[4][2];
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    p[gq][0] = pack_bf16x2(acc[a][bm][gq * 4 + 0], acc[a][bm][gq * 4 + 1]);
                    p[gq][1] = pack_bf16x2(acc[a][bm][gq * 4 + 2], acc[a][bm][gq * 4 + 3]);
                }
#pragma unroll
                for (int pr = 0; pr < 2; ++pr) {
                    const auto s0 = __builtin_amdgcn_permlane32_swap(p[2 * pr][0], p[2 * pr + 1][0], false, false);
                    const auto s1 = __builtin_amdgcn_permlane32_swap(p[2 * pr][1], p[2 * pr + 1][1], false, false);
                    const int j = (a * AM + bm) * 2 + pr;
                    pk[j][0] = s0[0];
                    pk[j][1] = s1[0];
                    pk[j][2] = s0[1];
                    pk[j][3] = s1[1];
                }
            }
        }
        zero_acc();
    };

    // ---- per-row consumer partials of the current tile (REDUCE)
    // (max, argmax, sum of exp(x - max)) pairs combine as: larger max wins, equal maxima
    // keep the smaller index, sums are rescaled to the new max.  An empty partial is
    // (-inf, INT32_MAX, 0).
    constexpr float kLog2e = 1.4426950408889634f;
    auto combine = [&](float &m, int &a, float &sm, float m2, int a2, float s2) __attribute__((always_inline)) {
        const float mm = fmaxf(m, m2);
        const bool take = m2 > m || (m2 == m && a2 < a);
        const float e1 = (m == -INFINITY) ? 0.0f : sm * __builtin_amdgcn_exp2f((m - mm) * kLog2e);
        const float e2 = (m2 == -INFINITY) ? 0.0f : s2 * __builtin_amdgcn_exp2f((m2 - mm) * kLog2e);
        sm = e1 + e2;
        a = take ? a2 : a;
        m = mm;
    };
    float rm[AM], rs[AM];
    int ra[AM];
    // Per-lane partials of every row of the wave's sub-tile (entries in ascending
    // vocabulary order), combined over the lanes that share the row (32 x 32: the two lanes
    // l and l ^ 32; 16 x 16: the four lanes l ^ 16, l ^ 32); then the upper vocabulary
    // half's waves leave theirs in LDS.
    const int row_lane = M16 ? r16 : fr;
    const bool row_owner = M16 ? qd == 0 : hi == 0;
    auto reduce_part1 = [&](int v0) __attribute__((always_inline)) {
#pragma unroll
        for (int bm = 0; bm < AM; ++bm) {
            float m = -INFINITY, sm = 0.0f;
            int am = INT32_MAX;
            // entry e of this lane's block a, in ascending vocabulary order
            auto ventry = [&](int a, int e) {
                return M16 ? v0 + wv * WV + a * 16 + 4 * qd + e
                           : v0 + wv * WV + a * 32 + (e >> 2) * 8 + hi * 4 + (e & 3);
            };
#pragma unroll
            for (int a = 0; a < AV; ++a)
#pragma unroll
                for (int e = 0; e < NACC; ++e) {
                    const float x = acc[a][bm][e];
                    if (ventry(a, e) < V && x > m) {
                        m = x;
                        am = ventry(a, e);
                    }
                }
#pragma unroll
            for (int a = 0; a < AV; ++a)
#pragma unroll
                for (int e = 0; e < NACC; ++e)
                    if (ventry(a, e) < V)
                        sm += __builtin_amdgcn_exp2f((acc[a][bm][e] - m) * kLog2e);
            // partner lanes: permlaneN_swap(x, x) gives the upper lane of each pair the
            // lower one's x in [0] and the lower lane the upper one's in [1]
            auto fold_swap32 = [&]() {
                const auto pm = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, m),
                                                                 __builtin_bit_cast(uint32_t, m), false, false);
                const auto pa = __builtin_amdgcn_permlane32_swap((uint32_t)am, (uint32_t)am, false, false);
                const auto ps = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, sm),
                                                                 __builtin_bit_cast(uint32_t, sm), false, false);
                combine(m, am, sm, __builtin_bit_cast(float, hi ? pm[0] : pm[1]), (int)(hi ? pa[0] : pa[1]),
                        __builtin_bit_cast(float, hi ? ps[0] : ps[1]));
            };
            if constexpr (M16) {
                const bool up = qd & 1;
                const auto pm = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, m),
                                                                 __builtin_bit_cast(uint32_t, m), false, false);
                const auto pa = __builtin_amdgcn_permlane16_swap((uint32_t)am, (uint32_t)am, false, false);
                const auto ps = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, sm),
                                                                 __builtin_bit_cast(uint32_t, sm), false, false);
                combine(m, am, sm, __builtin_bit_cast(float, up ? pm[0] : pm[1]), (int)(up ? pa[0] : pa[1]),
                        __builtin_bit_cast(float, up ? ps[0] : ps[1]));
            }
            fold_swap32();
            rm[bm] = m;
            ra[bm] = am;
            rs[bm] = sm;
            if (wv == 1 && row_owner) {
                const int r = wm * WM + bm * MB + row_lane;
                red_lds[r] = m;
                red_lds[BM + r] = __builtin_bit_cast(float, am);
                red_lds[2 * BM + r] = sm;
            }
        }
    };
    // after a barrier: the lower half's waves add the upper half and write the partial
    auto reduce_part2 = [&](int m0, int v0) __attribute__((always_inline)) {
        if (wv != 0 || !row_owner)
            return;
        const int64_t col = (int64_t)(v0 / BV) * ldp;
#pragma unroll
        for (int bm = 0; bm < AM; ++bm) {
            const int r = wm * WM + bm * MB + row_lane;
            float m = rm[bm], sm = rs[bm];
            int am = ra[bm];
            combine(m, am, sm, red_lds[r], __builtin_bit_cast(int, red_lds[BM + r]), red_lds[2 * BM + r]);
            if (m0 + r < rows) {
                pmax[col + m0 + r] = m;
                parg[col + m0 + r] = am;
                psum[col + m0 + r] = sm;
            }
        }
    };

    bf16x8_t af[2][AV], bf[2][AM];
    // A tile's first two K tiles, in the order the waits count on: H0, W0, H1, W1 (with a third
    // stage, W2 is requested by the tile's first step, after the tile's first barrier)
    auto prologue = [&]() __attribute__((always_inline)) {
        for (int s = 0; s < min(NSTAGE, nk); ++s)
#pragma unroll
            for (int p = 0; p < NSPREAD; ++p)
                issue_part((RED_IN_STAGE ? (w0 + s) % WST : s) * W_TILE, H_BASE + s * H_TILE, s, p);
    };
    if (dma_wave)
        prologue();

    auto main_loop = [&](auto dma_tag) __attribute__((always_inline)) {
    constexpr bool DMA_ON = decltype(dma_tag)::value;
    auto issue_part_t = [&](int rw, int rh, int kt, int p) {
        if constexpr (DMA_ON)
            issue_part(rw, rh, kt, p);
    };
    auto prologue_t = [&]() {
        if constexpr (DMA_ON)
            prologue();
    };
    for (int i = 0; i < n_my; ++i) {
        // K tile 0 has landed; K tile 1 may still be in flight
        if (nk > 1)
            wait_vmcnt<NDMA>();
        else
            wait_vmcnt<0>();
        barrier_no_fence();
        int rw = (RED_IN_STAGE ? w0 : 0) * W_TILE, rh = H_BASE;   // stages holding K tile kt
        load_frags(rw, rh, 0, af[0], bf[0]);
        int pw = 0, ph = 0, pkt = 0, kt = 0;
        bool pending = false;
        // One step of the steady state (as in the tiled kernel); `hook` issues the deferred
        // stores of this step in one of its k sub-steps.  The barrier in the middle of step kt
        // needs K tile kt + 1, and the wait before it leaves nothing in flight, so the
        // deferred stores are complete at the barrier, like the DMA.  After it the stages of
        // K tile kt are free and are refilled with K tile kt + 2.
        // With a third W stage (DEEP), W's rows run a step further ahead: step kt requests W's
        // rows of K tile kt + 2 at its start, into the stage K tile kt - 1 freed at the last
        // barrier, and H's rows of K tile kt + 2 after its own barrier; that barrier's wait
        // needs K tile kt + 1 and leaves W's K tile kt + 2 in flight.
        auto steady = [&](auto hook) __attribute__((always_inline)) {
#pragma unroll
            for (int s = 0; s + 1 < NSUB; ++s) {
                if (s + 1 < NSPREAD && pending)
                    issue_part_t(pw, ph, pkt, s + 1);
                if constexpr (DEEP && DMA_ON) {
                    if (s == 0)
                        issue_w(next_w(next_w(rw)), kt + 2);
                }
                if (s == HOOK_S)
                    hook();
                mma_load(rw, rh, s + 1, s & 1, af, bf);
                interleave(s + 1 < NSPREAD ? PER : (DEEP && DMA_ON && s == 0 ? LW : 0));
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (DEEP)
                wait_vmcnt<LW>();
            else
                wait_vmcnt<0>();
            barrier_no_fence();
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (!DEEP)
                issue_part_t(rw, rh, kt + NSTAGE, 0);
            else if constexpr (DMA_ON)
                issue_h(rh, kt + 2);
            pw = rw;
            ph = rh;
            pkt = kt + NSTAGE;
            pending = NSPREAD > 1;
            const int nxw = next_w(rw), nxh = next_h(rh);
            mma_load(nxw, nxh, 0, (NSUB - 1) & 1, af, bf);
            interleave(DEEP ? (DMA_ON ? LH : 0) : PER);
            __builtin_amdgcn_sched_barrier(0);
            rw = nxw;
            rh = nxh;
            ++kt;
        };
        if (STORE && i > 0 && SPS > 0) {
            if (nk >= NSTAGE + DEFER) {
#pragma unroll
                for (int j = 0; j < DEFER; ++j)
                    steady([&] {
#pragma unroll
                        for (int q2 = 0; q2 < SPS; ++q2)
                            store_one(NIMM + j * SPS + q2);
                    });
            } else {
#pragma unroll
                for (int j = NIMM; j < NST; ++j)
                    store_one(j);
            }
        }
        while (kt + NSTAGE < nk)
            steady([] {});
        for (; kt < nk; ++kt) {
#pragma unroll
            for (int s = 0; s + 1 < NSUB; ++s) {
                if (s + 1 < NSPREAD && pending)
                    issue_part_t(pw, ph, pkt, s + 1);
                mma_load(rw, rh, s + 1, s & 1, af, bf);
            }
            pending = false;
            if constexpr (M16) {
                // one MFMA sequence for both cases (two copies of it raise the register
                // pressure); after the last K tile its fragment reads are unused
                if (kt + 1 < nk) {
                    wait_vmcnt<0>();
                    barrier_no_fence();
                    rw = next_w(rw);
                    rh = next_h(rh);
                }
                mma_load(rw, rh, 0, (NSUB - 1) & 1, af, bf);
            } else {
                if (kt + 1 < nk) {
                    wait_vmcnt<0>();
                    barrier_no_fence();
                    rw = next_w(rw);
                    rh = next_h(rh);
                    load_frags(rw, rh, 0, af[NSUB & 1], bf[NSUB & 1]);
                }
                mma(af[(NSUB - 1) & 1], bf[(NSUB - 1) & 1]);
            }
        }
        // every wave's last fragments are in registers: the stages are free
        int cm0, cv0;
        tile_coords(i, cm0, cv0);
        if constexpr (RED_IN_STAGE) {
            // the W stage of K tile nk - 2 (no wave reads it after that step's barrier, and
            // no request targets it), or with one K tile a stage the tile never used
            const int red_stage = (w0 + (nk >= 2 ? nk - 2 : 2)) % WST;
            red_lds = (float *)(smem + red_stage * W_TILE);
            w0 = (red_stage + 1) % WST;
        }
        if constexpr (REDUCE)
            reduce_part1(cv0);
        if constexpr (STORE && !REDUCE && NIMM == NST) {
            // Every store of the tile, then the row ids two tiles ahead, then the next tile's
            // first requests: vmcnt drains in issue order, so the next tile's first wait then
            // leaves exactly its later K tiles in flight instead of also waiting for them
            // behind these stores (+2.5% on a 21399-row launch, neutral on 3687 rows).  All of
            // it but the requests touches no LDS, so it comes before the tile-end barrier
            // (which only guards the stages against the next tile's requests): a wave packs
            // and stores while the other waves finish their last MFMAs.
            pm0 = cm0;
            pv0 = cv0;
            pack();
#pragma unroll
            for (int j = 0; j < NST; ++j)
                store_one(j);
            if (i + 1 < n_my)
                make_src(i + 1);
            load_hidx(i + 2);
            wait_vmcnt<63>();
            barrier_no_fence();
            if (i + 1 < n_my)
                prologue_t();
            continue;
        }
        if constexpr (RED_IN_STAGE && NIMM == NST) {
            // The per-row consumer with a third stage, in the order of the logits path above:
            // what touches no LDS before the tile-end barrier, then the partials (which need
            // the other waves' halves from LDS) and the row ids, then the next tile's first
            // requests, so that its first wait covers its first K tile and not the second.
            if constexpr (STORE) {
                pm0 = cm0;
                pv0 = cv0;
                pack();
#pragma unroll
                for (int j = 0; j < NST; ++j)
                    store_one(j);
            } else {
                zero_acc();
            }
            if (i + 1 < n_my)
                make_src(i + 1);
            wait_vmcnt<63>();
            barrier_no_fence();
            reduce_part2(cm0, cv0);
            load_hidx(i + 2);
            if (i + 1 < n_my)
                prologue_t();
            continue;
        }
        wait_vmcnt<63>();
        barrier_no_fence();
        if (i + 1 < n_my) {
            make_src(i + 1);
            prologue_t();
        }
        if constexpr (REDUCE)
            reduce_part2(cm0, cv0);
        if constexpr (STORE) {
            pm0 = cm0;
            pv0 = cv0;
            pack();
#pragma unroll
            for (int j = 0; j < NIMM; ++j)
                store_one(j);
            if (i + 1 == n_my) {
#pragma unroll
                for (int j = NIMM; j < NST; ++j)
                    store_one(j);
            }
        } else {
            zero_acc();
        }
        load_hidx(i + 2);
        // (REDUCE: red_lds is next written at the next tile's end, and with RED_IN_STAGE its
        // stage is next refilled by the next tile's first step; both come after that tile's
        // first barrier, which every reader of the partials has passed, so no extra barrier
        // is needed here.)
    }
    };
    if (DMAW < 8 && !dma_wave)
        main_loop(std::false_type{});
    else
        main_loop(std::true_type{});
}

// Combine the per-(row, vocabulary tile) partials of the REDUCE kernel into the per-row
// consumer outputs: row_max, row_argmax (the first index attaining the max) and
// row_lse = max + log(sum_v exp(z_v - max)).  A workgroup owns 64 rows (one per lane);
// its 16 waves take 16 contiguous ranges of vocabulary tiles and fold their partials in
// one pass (loads of several tiles in flight per lane), then wave 0 folds the 16 range
// partials in range order through LDS.  The fold order depends on V only, so the result
// does not depend on timing or on how the rows were chunked.
__device__ __forceinline__ void fold_partial(float &m, int &a, float &s, float x, int ax, float sx)
{
    constexpr float kLog2e = 1.4426950408889634f;
    if (x == -INFINITY)
        return;
    if (x > m || (x == m && ax < a)) {
        s = (m == -INFINITY ? 0.0f : s * __builtin_amdgcn_exp2f((m - x) * kLog2e)) + sx;
        m = x;
        a = ax;
    } else {
        s += sx * __builtin_amdgcn_exp2f((x - m) * kLog2e);
    }
}

__global__ __launch_bounds__(1024) void logits_reduce_finish_kernel(const float *__restrict__ pmax,
                                                                   const int32_t *__restrict__ parg,
                                                                   const float *__restrict__ psum, int32_t ncol,
                                                                   int32_t rows, float *__restrict__ row_max,
                                                                   int32_t *__restrict__ row_argmax,
                                                                   float *__restrict__ row_lse,
                                                                   const int32_t *__restrict__ rows_dev)
{
    // rows: the partials' row stride (the launch's capacity); rows_dev, if set, the count of
    // rows to finish, read from device memory and clamped to [0, rows]
    const int nrows = rows_dev ? min(max(*rows_dev, 0), rows) : rows;
    constexpr int NWF = 16;
    constexpr float kLn2 = 0.6931471805599453f;
    __shared__ float sm_m[NWF][64], sm_s[NWF][64];
    __shared__ int32_t sm_a[NWF][64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r = blockIdx.x * 64 + lane;
    const int c0 = (int)((int64_t)ncol * w / NWF), c1 = (int)((int64_t)ncol * (w + 1) / NWF);
    float m = -INFINITY, s = 0.0f;
    int a = INT32_MAX;
    if (r < nrows) {
        int c = c0;
        for (; c + 4 <= c1; c += 4) {
            float x[4], sx[4];
            int ax[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t o = (int64_t)(c + u) * rows + r;
                x[u] = pmax[o];
                ax[u] = parg[o];
                sx[u] = psum[o];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                fold_partial(m, a, s, x[u], ax[u], sx[u]);
        }
        for (; c < c1; ++c) {
            const int64_t o = (int64_t)c * rows + r;
            fold_partial(m, a, s, pmax[o], parg[o], psum[o]);
        }
    }
    sm_m[w][lane] = m;
    sm_a[w][lane] = a;
    sm_s[w][lane] = s;
    __syncthreads();
    if (w == 0 && r < nrows) {
        float mm = -INFINITY, ss = 0.0f;
        int aa = INT32_MAX;
        for (int k = 0; k < NWF; ++k)
            fold_partial(mm, aa, ss, sm_m[k][lane], sm_a[k][lane], sm_s[k][lane]);
        row_max[r] = mm;
        row_argmax[r] = aa;
        row_lse[r] = mm + __builtin_amdgcn_logf(ss) * kLn2;
    }
}

// Cache-policy operand of global_load_lds for data read exactly once: the NT (streaming)
// bit of gfx950's cache policy.  The low-M kernels read W once per launch; with this bit
// on W's requests the 20-row workload's launch went from 195-196 us to 177-179 us
// (rocprofv3, one MI355X), while H, which every step re-reads, keeps the default policy.
constexpr int kLoadStreaming = 2;


// At most n (0 <= n <= MAXN) DMA tiles of T instructions each still in flight.
template <int T, int MAXN>
__device__ __forceinline__ void wait_tiles_upto(int n)
{
    if constexpr (MAXN <= 0) {
        wait_vmcnt<0>();
    } else {
        if (n >= MAXN)
            wait_vmcnt<MAXN * T>();
        else
            wait_tiles_upto<T, MAXN - 1>(n);
    }
}

// Low-M gather-GEMM (M <= 32 * AM): the work is streaming W once from HBM, with the H
// tile shared by the workgroup.
//
// Wave w of the grid owns an equal, contiguous range of vocabulary rows (so every wave
// streams the same number of W bytes) and walks it in 32-row blocks (one MFMA A block),
// each a full K loop, through a private LDS ring filled by its own global_load_lds DMA;
// the ring keeps running across blocks.  The masked rows (at most 32 * AM) are the MFMA B
// operand.  Every wave of the grid runs the same number of
// (block, K tile) steps (waves whose range is short run padding blocks of clamped rows
// that are never stored), so the four waves of a workgroup need the same H tile at the
// same step.  That tile (32 * AM masked rows x 64 k) is fetched once per workgroup into a
// shared ring, each wave DMAing AM of its 8-row slices, and one barrier per step makes it
// visible.  Against a per-wave H copy this reads H from L2 four times less and leaves the
// LDS to a deeper W ring (8 stages for AM = 1: seven 4 KiB W tiles in flight per wave
// while one is consumed).  The barrier also tells each wave that every other wave has
// finished reading the previous step's slot, which is then refilled.
// (Against a per-wave copy of H, measured earlier as its own variant, this reads H from L2
// four times less.)  Same MFMA, operand roles and k order as the tiled kernel: results
// are bit-identical.
template <int AM, int NSTAGE, bool OUT_BF16>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1))) void
gather_gemm_lowm_shared_kernel(const __bf16 *__restrict__ H, const int32_t *__restrict__ idx, int32_t rows,
                               const __bf16 *__restrict__ W, int32_t V, int32_t d, void *__restrict__ out,
                               int64_t ldo)
{
    constexpr int BK = 64, ROW_BYTES = 128, CHUNKS = 8, RPI = 8;
    constexpr int NBK = 8;                        // finished blocks held before a store burst
    constexpr int W_TILE = 32 * ROW_BYTES;        // 4 KiB: a wave's 32 vocabulary rows
    constexpr int H_TILE = 32 * AM * ROW_BYTES;   // 4 or 8 KiB, shared by the workgroup
    constexpr int WAVE_W = NSTAGE * W_TILE;
    constexpr int H_BASE = 4 * WAVE_W;
    constexpr int LW = W_TILE / 1024;             // W DMA instructions per wave per step
    constexpr int LH = AM;                        // H DMA instructions per wave per step
    constexpr int T = LW + LH;
    static_assert(H_BASE + NSTAGE * H_TILE <= 160 * 1024, "LDS");
    static_assert(NSTAGE >= 3 && (NSTAGE - 2) * T < 64, "vmcnt");

    __shared__ __attribute__((aligned(1024))) char smem[H_BASE + NSTAGE * H_TILE];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wbase = wave * WAVE_W;
    // The workgroups of one XCD (hardware block b runs on XCD b % 8) take one contiguous
    // eighth of the vocabulary rows, so the output lines at the boundary between two
    // workgroups' ranges are completed in one L2 instead of being written back partially
    // by two (measured about 1% faster on the 20-row workload).
    const int64_t wg = gridDim.x % 8 == 0 ? (int64_t)(blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8
                                          : (int64_t)blockIdx.x;
    const int64_t nw = (int64_t)gridDim.x * 4, gw = wg * 4 + wave;
    const int v_lo = lowm::range_bound(gw, nw, V);
    const int v_hi = lowm::range_bound(gw + 1, nw, V);
    const int v_max = max(v_hi - 1, 0);           // clamp for padding rows (V >= 1)
    // the same block count for all waves (that of the longest range)
    const int nblocks = lowm::range_blocks(nw, V);
    const int nk = d / BK;
    const int ntiles = nblocks * nk;

    // DMA lanes: an instruction fills 8 tile rows (lane / 8) x 8 physical chunks (lane % 8).
    int wch[LW];
#pragma unroll
    for (int j = 0; j < LW; ++j)
        wch[j] = ((lane % CHUNKS) ^ swz<BK>(j * RPI + lane / CHUNKS)) * 16;
    // H slice q = j * 4 + wave holds masked rows 8q .. 8q + 7 of the tile
    const char *hsrc[LH];
#pragma unroll
    for (int j = 0; j < LH; ++j) {
        const int r = (j * 4 + wave) * RPI + lane / CHUNKS;
        hsrc[j] = (const char *)(H + (int64_t)idx[min(r, rows - 1)] * d) + ((lane % CHUNKS) ^ swz<BK>(r)) * 16;
    }

    auto issue = [&](int slot, int g) {
        const int blk = g / nk, kt = g - blk * nk;
        const int kb = kt * ROW_BYTES;
#pragma unroll
        for (int j = 0; j < LW; ++j) {
            const int v = min(v_lo + blk * 32 + j * RPI + lane / CHUNKS, v_max);
            __builtin_amdgcn_global_load_lds((const void *)((const char *)(W + (int64_t)v * d) + kb + wch[j]),
                                             (lds_void_t *)(smem + wbase + slot * W_TILE + j * 1024), 16, 0,
                                             kLoadStreaming);
        }
#pragma unroll
        for (int j = 0; j < LH; ++j)
            __builtin_amdgcn_global_load_lds((const void *)(hsrc[j] + kb),
                                             (lds_void_t *)(smem + H_BASE + slot * H_TILE + (j * 4 + wave) * 1024),
                                             16, 0, 0);
    };

    const int fr = lane & 31, hi = lane >> 5;
    const int lane_chunk = (hi ^ swz<BK>(fr)) * 16;
    const int a_addr = wbase + fr * ROW_BYTES + lane_chunk;
    const int b_addr = H_BASE + fr * ROW_BYTES + lane_chunk;

    f32x16_t acc[AM], held[NBK][AM];
#pragma unroll
    for (int bm = 0; bm < AM; ++bm)
#pragma unroll
        for (int e = 0; e < 16; ++e)
            acc[bm][e] = 0.0f;

    // NSTAGE - 1 steps ahead; the last slot is filled once the first step's barrier has
    // passed
    const int npre = min(NSTAGE - 1, ntiles);
    for (int g = 0; g < npre; ++g)
        issue(g, g);

    int rs = 0;   // slot of step g
    for (int g = 0; g < ntiles; ++g) {
        // this wave's part of step g has landed (younger: steps g+1 .. g+NSTAGE-2)
        wait_tiles_upto<T, NSTAGE - 2>(min(NSTAGE - 2, ntiles - 1 - g));
        barrier_no_fence();   // every wave's part landed; every wave is done with step g-1
        if (g + NSTAGE - 1 < ntiles)
            issue(rs == 0 ? NSTAGE - 1 : rs - 1, g + NSTAGE - 1);
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
            const bf16x8_t af = *(const bf16x8_t *)(smem + ((a_addr + rs * W_TILE) ^ (32 * s)));
            bf16x8_t bf[AM];
#pragma unroll
            for (int bm = 0; bm < AM; ++bm)
                bf[bm] = *(const bf16x8_t *)(smem + ((b_addr + rs * H_TILE + bm * 32 * ROW_BYTES) ^ (32 * s)));
#pragma unroll
            for (int bm = 0; bm < AM; ++bm)
                acc[bm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf[bm], acc[bm], 0, 0, 0);
        }
        rs = (rs + 1 == NSTAGE) ? 0 : rs + 1;

        const int blk = g / nk;
        if (g - blk * nk == nk - 1)
            lowm::lowm_block_done<AM, NBK, OUT_BF16>(held, acc, blk, nblocks, v_lo, v_hi, rows, fr, hi, out, ldo);
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

template <int BV, int BM, int BK, int NSTAGE, int NSPREAD = 1, int NW = 4>
hipError_t launch_bf16(const void *H, const int32_t *idx, int64_t rows, const void *W, int64_t V, int64_t d,
                       void *out, int64_t ldo, bool out_bf16, int group_m, hipStream_t stream)
{
    const int64_t nvt = (V + BV - 1) / BV, nmt = (rows + BM - 1) / BM;
    const dim3 grid((unsigned)(nvt * nmt));
    if (out_bf16)
        hipLaunchKernelGGL((gather_gemm_bf16_kernel<BV, BM, BK, NSTAGE, NSPREAD, NW, true>), grid, dim3(64 * NW), 0,
                           stream, (const __bf16 *)H, idx, (int32_t)rows, (const __bf16 *)W, (int32_t)V, (int32_t)d,
                           out, ldo, group_m);
    else
        hipLaunchKernelGGL((gather_gemm_bf16_kernel<BV, BM, BK, NSTAGE, NSPREAD, NW, false>), grid, dim3(64 * NW), 0,
                           stream, (const __bf16 *)H, idx, (int32_t)rows, (const __bf16 *)W, (int32_t)V, (int32_t)d,
                           out, ldo, group_m);
    return hipGetLastError();
}

template <int BK, int NSTAGE, int NSPREAD>
hipError_t launch_persist(const void *H, const int32_t *idx, int64_t rows, const void *W, int64_t V, int64_t d,
                          void *out, int64_t ldo, bool out_bf16, int group_m, hipStream_t stream)
{
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const int64_t ntiles = ((V + 255) / 256) * ((rows + 255) / 256);
    // one workgroup per CU (a multiple of 8: one set per XCD), no more than there are tiles
    int64_t grid = std::max<int64_t>(8, (cus / 8) * 8);
    grid = std::min<int64_t>(grid, ((ntiles + 7) / 8) * 8);
    if (out_bf16)
        hipLaunchKernelGGL((gather_gemm_bf16_persist_kernel<BK, NSTAGE, NSPREAD, true>), dim3((unsigned)grid), dim3(256),
                           0, stream, (const __bf16 *)H, idx, (int32_t)rows, (const __bf16 *)W, (int32_t)V, (int32_t)d,
                           out, ldo, group_m);
    else
        hipLaunchKernelGGL((gather_gemm_bf16_persist_kernel<BK, NSTAGE, NSPREAD, false>), dim3((unsigned)grid), dim3(256),
                           0, stream, (const __bf16 *)H, idx, (int32_t)rows, (const __bf16 *)W, (int32_t)V, (int32_t)d,
                           out, ldo, group_m);
    return hipGetLastError();
}

template <int NSPREAD, int DEFER, int NIMM, bool STORE = true, bool REDUCE = false, bool M16 = false,
          int DMAW = 8, bool DEEP = false>
hipError_t launch_defer(const void *H, const int32_t *idx, int64_t rows, const void *W, int64_t V, int64_t d,
                        void *out, int64_t ldo, int group_m, hipStream_t stream, float *pmax = nullptr,
                        int32_t *parg = nullptr, float *psum = nullptr, const int32_t *rows_dev = nullptr)
{
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const int64_t ntiles = ((V + 255) / 256) * ((rows + 255) / 256);
    int64_t grid = std::max<int64_t>(8, (cus / 8) * 8);
    grid = std::min<int64_t>(grid, ((ntiles + 7) / 8) * 8);
    hipLaunchKernelGGL((gather_gemm_bf16_defer_kernel<NSPREAD, DEFER, NIMM, STORE, REDUCE, M16, DMAW, DEEP>),
                       dim3((unsigned)grid), dim3(512), 0, stream, (const __bf16 *)H, idx, (int32_t)rows, (const __bf16 *)W, (int32_t)V,
                       (int32_t)d, (__bf16 *)out, ldo, group_m, pmax, parg, psum, rows_dev);
    return hipGetLastError();
}

template <int AM>
hipError_t launch_lowm_shared(const void *H, const int32_t *idx, int64_t rows, const void *W, int64_t V, int64_t d,
                              void *out, int64_t ldo, bool out_bf16, hipStream_t stream)
{
    constexpr int NSTAGE = AM == 1 ? 8 : 6;   // 160 / 144 KiB of LDS
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    // one workgroup (four streams) per CU, but never fewer than 32 rows per stream
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(cus, (V + 127) / 128));
    if (out_bf16)
        hipLaunchKernelGGL((gather_gemm_lowm_shared_kernel<AM, NSTAGE, true>), dim3(grid), dim3(256), 0, stream,
                           (const __bf16 *)H, idx, (int32_t)rows, (const __bf16 *)W, (int32_t)V, (int32_t)d, out, ldo);
    else
        hipLaunchKernelGGL((gather_gemm_lowm_shared_kernel<AM, NSTAGE, false>), dim3(grid), dim3(256), 0, stream,
                           (const __bf16 *)H, idx, (int32_t)rows, (const __bf16 *)W, (int32_t)V, (int32_t)d, out, ldo);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gather_gemm_device_rows(const void *H, const int32_t *idx, const int32_t *rows_dev,
                                          int64_t max_rows, const void *W, int64_t V, int64_t d, void *out,
                                          int64_t ldo, int group_m, hipStream_t stream)
{
    if (group_m <= 0)
        group_m = kDefaultGroupM;
    return launch_defer<1, 1, 16, true, false, true, 4, true>(H, idx, max_rows, W, V, d, out, ldo, group_m, stream,
                                                              nullptr, nullptr, nullptr, rows_dev);
}

bool gather_gemm_grid_fits(int variant, int64_t rows, int64_t V)
{
    switch (variant) {
    case kVariantF32:
    case kVariantBf16Simple:
        return (rows + 63) / 64 <= 0x7fffffffLL && (V + 63) / 64 <= 65535;
    case kVariantBf16W8K64S2:
    case kVariantBf16PersistK32:
    case kVariantBf16DeferS4I8:
    case kVariantBf16M16S1:
    case kVariantBf16M16Dma4:
    case kVariantBf16M16Dma4W3:
        return ((rows + 255) / 256) * ((V + 255) / 256) <= 0x7fffffffLL;
    case kVariantBf16LowMShared:
        return rows <= 64;
    default:
        return false;
    }
}

hipError_t launch_logits_argmax_lse(const void *H, const int32_t *idx, int64_t rows, const void *W, int64_t V,
                                    int64_t d, void *out, int64_t ldo, float *pmax, int32_t *parg, float *psum,
                                    float *row_max, int32_t *row_argmax, float *row_lse, int group_m,
                                    bool m16, hipStream_t stream, const int32_t *rows_dev)
{
    if (group_m <= 0)
        group_m = kDefaultGroupM;
    hipError_t e;
    if (m16)
        e = out ? launch_defer<1, 1, 16, true, true, true, 4, true>(H, idx, rows, W, V, d, out, ldo, group_m,
                                                                 stream, pmax, parg, psum, rows_dev)
                : launch_defer<1, 1, 16, false, true, true, 4, true>(H, idx, rows, W, V, d, nullptr, ldo, group_m,
                                                                  stream, pmax, parg, psum, rows_dev);
    else
        e = out ? launch_defer<2, 4, 8, true, true>(H, idx, rows, W, V, d, out, ldo, group_m, stream, pmax, parg, psum,
                                                    rows_dev)
                : launch_defer<2, 4, 8, false, true>(H, idx, rows, W, V, d, nullptr, ldo, group_m, stream, pmax, parg,
                                                     psum, rows_dev);
    if (e != hipSuccess)
        return e;
    const int ncol = (int)((V + 255) / 256);
    hipLaunchKernelGGL(logits_reduce_finish_kernel, dim3((unsigned)((rows + 63) / 64)), dim3(1024), 0, stream, pmax,
                       parg, psum, ncol, (int32_t)rows, row_max, row_argmax, row_lse, rows_dev);
    return hipGetLastError();
}

hipError_t launch_gather_gemm(int variant, const void *H, const int32_t *idx, int64_t rows, const void *W,
                              int64_t V, int64_t d, void *out, int64_t ldo, bool out_bf16, int group_m,
                              hipStream_t stream)
{
    if (group_m <= 0)
        group_m = kDefaultGroupM;
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
    case kVariantBf16W8K64S2:
        return launch_bf16<256, 256, 64, 2, 2, 8>(H, idx, rows, W, V, d, out, ldo, out_bf16, group_m, stream);
    case kVariantBf16DeferS4I8:
        return out_bf16 ? launch_defer<2, 4, 8>(H, idx, rows, W, V, d, out, ldo, group_m, stream) : hipErrorInvalidValue;
    case kVariantBf16M16S1:
        return out_bf16 ? launch_defer<1, 1, 16, true, false, true>(H, idx, rows, W, V, d, out, ldo, group_m, stream)
                        : hipErrorInvalidValue;
    case kVariantBf16M16Dma4:
        return out_bf16 ? launch_defer<1, 1, 16, true, false, true, 4, false>(H, idx, rows, W, V, d, out, ldo, group_m,
                                                                         stream)
                        : hipErrorInvalidValue;
    case kVariantBf16M16Dma4W3:
        return out_bf16 ? launch_defer<1, 1, 16, true, false, true, 4, true>(H, idx, rows, W, V, d, out, ldo, group_m,
                                                                         stream)
                        : hipErrorInvalidValue;
    case kVariantBf16PersistK32:
        return launch_persist<32, 4, 2>(H, idx, rows, W, V, d, out, ldo, out_bf16, group_m, stream);
    case kVariantBf16LowMShared:
        if (rows <= 32)
            return launch_lowm_shared<1>(H, idx, rows, W, V, d, out, ldo, out_bf16, stream);
        return launch_lowm_shared<2>(H, idx, rows, W, V, d, out, ldo, out_bf16, stream);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace mosaic

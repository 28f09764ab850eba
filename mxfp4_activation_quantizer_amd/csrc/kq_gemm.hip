// kq_gemm.hip — the W4A4 consumer: Y = dequant(A) * dequant(W)^T on the gfx950
// block-scaled matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4 with E2M1
// operands and E8M0 scales), fp32 accumulation, bf16 output.
//
// A (activations, [M][K]) and W (weights, [N][K]) are both MXFP4 in the
// quantizer's layout: codes [rows][K/2] with element k in nibble k%2 of byte
// k/2, scales [rows][K/32].  For the 32x32x64 FP4 MFMA, lane l holds row l%32
// and the 32 elements 32*(l/32) .. +31 of a 64-wide K step: exactly one
// 16-byte chunk of a code row plus its one scale byte, so both operands come
// from the quantizer's output as is.
//
// The MFMA computes the transposed tile Y^T = W A^T (first operand W): the
// accumulator register r of lane l then holds Y[m = l%32][n = 8*(r/4) +
// 4*(l/32) + r%4], four consecutive columns of one output row per group of
// four registers; the epilogue gathers the bf16 tile in LDS and stores it a
// whole row at a time.
//
// Tiling: 8 waves (2 along M x 4 along N) compute a 128 x 256 tile of Y, each
// wave 64 x 64 (2 x 2 MFMA tiles).  K advances in tiles of 256 (four MFMA
// steps; 128 code bytes and 8 scale bytes per row).  The operand tiles go
// from global memory straight into LDS (global_load_lds_dwordx4 for codes,
// _dword for scales) through three LDS stages: two K tiles are in flight
// while a third is multiplied, and no registers hold them on the way.
// In LDS a code row is eight 16-byte chunks stored at slot
// c ^ ((row >> 1) & 7): the 16 lanes that one LDS cycle serves read 16
// consecutive rows at the same chunk and hit 16 distinct slots of a
// 256-byte bank window.  A DMA lane writes 16 bytes at (region base +
// 16 * lane), so that layout is made on the global side: the lane that
// lands in slot s of a row fetches chunk s ^ ((row >> 1) & 7).  A row's 8
// scale bytes are read as one 8-byte word per tile (byte reads conflict on
// gfx950) and the MFMA's scale operand select picks the byte of each step.
//
// Waits are explicit: before tile kt is read, vmcnt(one tile's DMAs)
// retires tile kt's DMAs and leaves tile kt + 1's in flight; the barrier
// after it also tells every wave that the stage of tile kt - 1 is free, and
// the DMAs of tile kt + 2 go into that stage.  The stages are three separate
// LDS arrays, so the compiler sees that the pending DMAs (into the other
// two) do not alias the reads and adds no waits of its own, except where it
// merges the two ways into a loop head; the loop body therefore holds 15
// steps (one pass for K up to 3328).
//
// Workgroup order: XCD x (workgroups go to the 8 XCDs round-robin) takes a
// contiguous range of an order that walks eight M tiles for each N tile, so
// each W tile is fetched into that XCD's L2 once for eight workgroups.
// A K that is a multiple of 128 but not of 256 ends with a half tile: its
// missing half re-reads the valid half (never used) and only its first two
// MFMA steps run.
//
// Epilogue: the bf16 tile is written into two of the (then free) stages, in
// an XOR slot layout that keeps the 32-row accumulator stores conflict-free,
// and every wave stores two whole 512-byte tile rows per instruction.
//
// All of the above describes the per-tile kernel, which takes any K that is
// a multiple of 128.  A K that is a multiple of 512, with 16-byte aligned
// scale arrays, takes the pipelined kernel further down: the same tiles,
// MFMAs and epilogue, with the K pipeline carried across output tiles and
// the scales in a ring of their own.

#include <stdint.h>
#include <stdlib.h>

#include <hip/hip_runtime.h>

#include "kq.h"
#include "kq_device.h"
#include "kq_host.h"
#include "kq_gemm_wide.h"

namespace kq {

// Sweep builds only: -DKQ_GEMM_WPX=n fixes the workgroups per XCD (0: one per
// CU); -DKQ_GEMM_PIPE=0 keeps every call on the per-tile kernel.
#ifndef KQ_GEMM_WPX
#define KQ_GEMM_WPX 0
#endif
#ifndef KQ_GEMM_PIPE
#define KQ_GEMM_PIPE 1
#endif
// -DKQ_GEMM_WIDE=0 keeps large problems off the 256 x 256-tile kernel.
#ifndef KQ_GEMM_WIDE
#define KQ_GEMM_WIDE 1
#endif
static_assert(KQ_GEMM_WPX >= 0, "KQ_GEMM_WPX must be >= 0");

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16g __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2g __attribute__((ext_vector_type(2)));

constexpr int kGemmWM = 2, kGemmWN = 4;          // waves along M and N
constexpr int kBM = 64 * kGemmWM, kBN = 64 * kGemmWN;
constexpr int kGemmThreads = 64 * kGemmWM * kGemmWN;
constexpr int kBK = 256;                          // K elements per LDS tile
constexpr int kRowBytes = kBK / 2;                // 128 code bytes per row per tile
constexpr int kMGroup = 8;                        // M tiles that share a W tile
constexpr int kAB = kBM * kRowBytes, kWB = kBN * kRowBytes;

__device__ __forceinline__ int swz_slot(int row, int c) { return c ^ ((row >> 1) & 7); }

constexpr int kDScale = 8 * (kBM + kBN);         // 8 scale bytes per A and W row
constexpr int kDStage = kAB + kWB + kDScale;     // 52224 bytes
constexpr int kDA = kAB / 1024 / (kGemmThreads / 64);     // A DMAs (1 KB per wave) per wave
constexpr int kDW = kWB / 1024 / (kGemmThreads / 64);     // W DMAs per wave
constexpr int kDSRegions = kDScale / 256;                 // 256-byte scale regions
constexpr int kDS = (kDSRegions + kGemmThreads / 64 - 1) / (kGemmThreads / 64);
constexpr int kDPerTile = kDA + kDW + kDS;                // DMAs per thread per K tile
static_assert(kAB % (1024 * (kGemmThreads / 64)) == 0 && kWB % (1024 * (kGemmThreads / 64)) == 0,
              "whole 1 KB regions per wave");
static_assert(kDPerTile < 16, "vmcnt immediate");

__shared__ __attribute__((aligned(16))) uint8_t gemm_st0[kDStage];
__shared__ __attribute__((aligned(16))) uint8_t gemm_st1[kDStage];
__shared__ __attribute__((aligned(16))) uint8_t gemm_st2[kDStage];

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void dma16(const void *g, uint8_t *l) {
    __builtin_amdgcn_global_load_lds(g, (lds_void *)l, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void *g, uint8_t *l) {
    __builtin_amdgcn_global_load_lds(g, (lds_void *)l, 4, 0, 0);
}
// s_waitcnt with vmcnt(n) and no expcnt / lgkmcnt wait (gfx9 encoding)
#define KQ_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

// This lane's DMA sources (byte offsets at K tile 0) and, per DMA, whether
// a half tile has no data there.
struct DmaPlan {
    int ga[kDA], gw[kDW], gs[kDS], rs[kDS];
    bool hia[kDA], hiw[kDW], his[kDS];
    const uint8_t *sb[kDS];
};

// Tile kt of both operands into stage st (one of the three stage arrays:
// with the stages as separate objects the compiler's wait insertion sees
// that these DMAs do not alias reads of the other two).
__device__ __forceinline__ void gemm_issue(const DmaPlan &pl, const uint8_t *ac, const uint8_t *wc,
                                           int kt, bool half, int wave, uint8_t *__restrict__ st) {
#pragma unroll
    for (int q = 0; q < kDA; ++q)
        dma16(ac + pl.ga[q] + kt * kRowBytes - (half && pl.hia[q] ? 64 : 0),
              st + (q * (kGemmThreads / 64) + wave) * 1024);
#pragma unroll
    for (int q = 0; q < kDW; ++q)
        dma16(wc + pl.gw[q] + kt * kRowBytes - (half && pl.hiw[q] ? 64 : 0),
              st + kAB + (q * (kGemmThreads / 64) + wave) * 1024);
#pragma unroll
    for (int q = 0; q < kDS; ++q)
        dma4(pl.sb[q] + pl.gs[q] + kt * 8 - (half && pl.his[q] ? 4 : 0), st + kAB + kWB + pl.rs[q] * 256);
}

// One K step of 64: the lane's A and W fragments (chunk 2 KS + kg of its
// rows) and the scale bytes, which sit at byte 2 KS of each row's scale
// word pair (see gemm_compute); the MFMA's scale operand select (0..3)
// takes the byte, so no shifts per step.
template <int KS>
__device__ __forceinline__ void gemm_kstep(const uint8_t *__restrict__ b, int wm, int wn, int i32, int kg,
                                           const u32x2g (&sa)[2], const u32x2g (&sw)[2],
                                           f32x16g (&acc)[2][2]) {
    constexpr int kSel = 2 * (KS & 1), kWord = KS >> 1;
    const int ch = 2 * KS + kg;
    i32x8 fa[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int row = wm * 64 + j * 32 + i32;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(b + row * kRowBytes + 16 * swz_slot(row, ch));
        fa[j] = (i32x8)__builtin_shufflevector(v, v, 0, 1, 2, 3, -1, -1, -1, -1);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = wn * 64 + i * 32 + i32;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(b + kAB + row * kRowBytes + 16 * swz_slot(row, ch));
        const i32x8 fw = (i32x8)__builtin_shufflevector(v, v, 0, 1, 2, 3, -1, -1, -1, -1);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                fw, fa[j], acc[i][j], 4, 4, kSel, (int)sw[i][kWord], kSel, (int)sa[j][kWord]);
    }
}

// nks K steps of 64 from stage b into the wave's 2 x 2 accumulator tiles.
// Scales: one 8-byte read per row per tile (byte reads conflict on gfx950:
// two extra cycles each), shifted right one byte for the lanes of the upper
// 32 K values (kg = 1), so that K step ks finds its byte at 2 ks for every
// lane.
__device__ __forceinline__ void gemm_compute(const uint8_t *__restrict__ b, int nks, int wm, int wn,
                                             int i32, int kg, f32x16g (&acc)[2][2]) {
    const uint8_t *sc = b + kAB + kWB;
    u32x2g sa[2], sw[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const uint64_t v = *reinterpret_cast<const uint64_t *>(sc + (wm * 64 + j * 32 + i32) * 8) >> (8 * kg);
        sa[j] = u32x2g{(uint32_t)v, (uint32_t)(v >> 32)};
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const uint64_t v = *reinterpret_cast<const uint64_t *>(sc + (kBM + wn * 64 + i * 32 + i32) * 8) >> (8 * kg);
        sw[i] = u32x2g{(uint32_t)v, (uint32_t)(v >> 32)};
    }
    gemm_kstep<0>(b, wm, wn, i32, kg, sa, sw, acc);
    gemm_kstep<1>(b, wm, wn, i32, kg, sa, sw, acc);
    if (nks > 2) {
        gemm_kstep<2>(b, wm, wn, i32, kg, sa, sw, acc);
        gemm_kstep<3>(b, wm, wn, i32, kg, sa, sw, acc);
    }
}

// Workgroup tile lin of the order that walks kMGroup M tiles for each N tile.
__device__ __forceinline__ void tile_origin(int lin, int mtc, int ntc, int &m0, int &n0) {
    const int blk = lin / (kMGroup * ntc), rem = lin - blk * kMGroup * ntc;
    const int grp = mtc - blk * kMGroup < kMGroup ? mtc - blk * kMGroup : kMGroup;
    const int nt = rem / grp, mt = blk * kMGroup + rem - nt * grp;
    m0 = mt * kBM;
    n0 = nt * kBN;
}

// This lane's DMA sources for the tile at (m0, n0): a 1 KB region is 8 rows
// of 128 bytes; lane p of it fetches the chunk that slot p & 7 of row p >> 3
// holds.  Rows past M or N repeat the last row.
__device__ __forceinline__ void make_plan(DmaPlan &pl, int m0, int n0, int M, int N, int K2, int K32,
                                          int wave, int lane, const uint8_t *as, const uint8_t *ws) {
#pragma unroll
    for (int q = 0; q < kDA; ++q) {
        const int p = (q * (kGemmThreads / 64) + wave) * 64 + lane;  // 16-byte slot in the A tile
        const int row = p >> 3, c = (p & 7) ^ ((row >> 1) & 7);
        pl.ga[q] = (m0 + row < M ? m0 + row : M - 1) * K2 + 16 * c;
        pl.hia[q] = c >= 4;
    }
#pragma unroll
    for (int q = 0; q < kDW; ++q) {
        const int p = (q * (kGemmThreads / 64) + wave) * 64 + lane;
        const int row = p >> 3, c = (p & 7) ^ ((row >> 1) & 7);
        pl.gw[q] = (n0 + row < N ? n0 + row : N - 1) * K2 + 16 * c;
        pl.hiw[q] = c >= 4;
    }
#pragma unroll
    for (int q = 0; q < kDS; ++q) {
        int r = q * (kGemmThreads / 64) + wave;
        r = r < kDSRegions ? r : r - (kGemmThreads / 64);  // past the last: a repeat
        pl.rs[q] = r;
        const int dw = r * 64 + lane, v = dw >> 1, hf = dw & 1;  // row slot, dword of its 8 bytes
        const int ra = m0 + v < M ? m0 + v : M - 1;
        const int rw = n0 + (v - kBM) < N ? n0 + (v - kBM) : N - 1;
        pl.sb[q] = v < kBM ? as : ws;
        pl.gs[q] = (v < kBM ? ra : rw) * K32 + 4 * hf;
        pl.his[q] = hf;
    }
}

// Half j of the output tile at (m0, n0): rows wm * 64 + j * 32 + (0..31) of
// both row blocks wm = 0, 1 (64 rows), bf16 (nearest even), through LDS
// buffer ob (64 rows x 512 bytes).  Every wave writes its 32 rows of the
// half (LDS row wm * 32 + r) in the 8-byte slot layout (c / 4) ^ (r & 31),
// so all eight waves share the write phase; then every thread stores 16
// bytes, two whole rows per wave instruction.  The caller places a barrier
// between the write and the read phase (barrier_mid) and after the reads
// before ob is reused.
template <class Barrier>
__device__ __forceinline__ void store_half(const f32x16g (&acc)[2][2], int j, uint8_t *ob, int wm,
                                           int wn, int i32, int kg, int tid, int m0, int n0, int M,
                                           int N, int64_t ldy, uint16_t *y, Barrier barrier_mid) {
    const int lr = wm * 32 + i32;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int s8 = wn * 16 + i * 8 + 2 * q + kg;
            const uint32_t lo = __builtin_bit_cast(
                uint32_t, __builtin_convertvector(f32x2{acc[i][j][4 * q], acc[i][j][4 * q + 1]}, bf16x2));
            const uint32_t hi = __builtin_bit_cast(
                uint32_t, __builtin_convertvector(f32x2{acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]}, bf16x2));
            *reinterpret_cast<u32x2g *>(ob + lr * (kBN * 2) + 8 * (s8 ^ i32)) = u32x2g{lo, hi};
        }
    }
    barrier_mid();
    constexpr int kRowChunks = kBN * 2 / 16;
#pragma unroll
    for (int k = 0; k < 64 * kRowChunks / kGemmThreads; ++k) {
        const int f = tid + k * kGemmThreads;
        const int row = f / kRowChunks, ch = f % kRowChunks, g = row & 31;
        u32x4 v = *reinterpret_cast<const u32x4 *>(ob + row * (kBN * 2) + 16 * (ch ^ (g >> 1)));
        if (g & 1) v = u32x4{v[2], v[3], v[0], v[1]};
        const int gr = m0 + (row >> 5) * 64 + j * 32 + g, col = n0 + 8 * ch;
        if (gr >= M || col >= N) continue;
        uint16_t *yp = y + (int64_t)gr * ldy + col;
        if (col + 7 < N) {
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(yp));
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (col + e < N) yp[e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
        }
    }
}

__global__ __launch_bounds__(kGemmThreads) void w4a4_gemm_kernel(
    const uint8_t *__restrict__ ac, const uint8_t *__restrict__ as,
    const uint8_t *__restrict__ wc, const uint8_t *__restrict__ ws, uint16_t *__restrict__ y,
    int M, int N, int K, int64_t ldy, int mtc, int ntc) {
    // ---- persistent: workgroup w of XCD x (workgroups go to the XCDs
    //      round-robin) takes tiles w, w + wpx, ... of that XCD's contiguous
    //      range of an order that walks kMGroup M tiles for each N tile; its
    //      output stores drain while the next tile's first DMAs are in flight
    const int tiles = mtc * ntc, per = (tiles + 7) / 8, wpx = gridDim.x >> 3;
    for (int t = blockIdx.x >> 3; t < per; t += wpx) {
        const int lin = (blockIdx.x & 7) * per + t;
        if (lin >= tiles) break;
        int m0, n0;
        tile_origin(lin, mtc, ntc, m0, n0);

        const int tid = threadIdx.x, lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int wm = wave / kGemmWN, wn = wave % kGemmWN;
        const int i32 = lane & 31, kg = lane >> 5;
        const int K2 = K / 2, K32 = K / 32;
        const int KT = (K + kBK - 1) / kBK;
        const bool half_tail = (K % kBK) != 0;

        // ---- DMA plan: source offsets of this lane, one region per DMA ----
        DmaPlan pl;
        make_plan(pl, m0, n0, M, N, K2, K32, wave, lane, as, ws);

        auto issue = [&](int kt, uint8_t *st) {
            gemm_issue(pl, ac, wc, kt, half_tail && kt == KT - 1, wave, st);
        };

        f32x16g acc[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[i][j] = f32x16g{};

        auto compute = [&](const uint8_t *b, int kt) {
            gemm_compute(b, half_tail && kt == KT - 1 ? 2 : kBK / 64, wm, wn, i32, kg, acc);
        };

        // ---- three stages: step s issues tile s and multiplies tile s - 2 ----
        // Step s: vmcnt(one tile) retires tile s - 2 (tile s - 1 stays in
        // flight); the barrier makes every wave's DMAs of tile s - 2 visible and
        // frees the stage of tile s - 3, which takes tile s.  Steps past the last
        // tile issue a repeat of it (never read).  The compiler's wait insertion
        // keeps pending DMAs apart from reads of another stage except where it
        // merges the two ways into the loop head (there it drains), so the loop
        // body holds kSteps steps: K up to 3328 (13 tiles, 15 steps) takes one
        // pass with no drain.
        constexpr int kSteps = 15;
        static_assert(kSteps % 3 == 0, "stages rotate with the step");
        for (int s0 = 0; s0 < KT + 2; s0 += kSteps) {
#pragma unroll
            for (int u = 0; u < kSteps; ++u) {
                const int st = s0 + u;
                if (st >= KT + 2) break;
                uint8_t *in = u % 3 == 0 ? gemm_st0 : u % 3 == 1 ? gemm_st1 : gemm_st2;
                const uint8_t *rd = u % 3 == 2 ? gemm_st0 : u % 3 == 0 ? gemm_st1 : gemm_st2;
                KQ_WAIT_VM(kDPerTile);
                __builtin_amdgcn_s_barrier();
                issue(st < KT ? st : KT - 1, in);
                if (st >= 2) compute(rd, st - 2);
            }
        }
        // the repeats of the last tile may still be landing: drain, then the
        // stages hold the output tile (rows 0..63 in stage 0, 64..127 in stage 1)
        KQ_WAIT_VM(0);
        __syncthreads();

        // ---- epilogue: bf16 (nearest even) through LDS, whole rows per store ----
        static_assert(kBM == 128 && 64 * kBN * 2 <= kDStage, "two halves of the output tile");
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int row = wm * 64 + j * 32 + i32;
            uint8_t *ob = wm == 0 ? gemm_st0 : gemm_st1;
            const int lr = row & 63;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int s8 = wn * 16 + i * 8 + 2 * q + kg;
                    const uint32_t lo = __builtin_bit_cast(
                        uint32_t, __builtin_convertvector(f32x2{acc[i][j][4 * q], acc[i][j][4 * q + 1]}, bf16x2));
                    const uint32_t hi = __builtin_bit_cast(
                        uint32_t, __builtin_convertvector(f32x2{acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]}, bf16x2));
                    *reinterpret_cast<u32x2g *>(ob + lr * (kBN * 2) + 8 * (s8 ^ i32)) = u32x2g{lo, hi};
                }
            }
        }
        __syncthreads();
        constexpr int kRowChunks = kBN * 2 / 16;
#pragma unroll
        for (int k = 0; k < kBM * kRowChunks / kGemmThreads; ++k) {
            const int f = tid + k * kGemmThreads;
            const int row = f / kRowChunks, ch = f % kRowChunks, g = row & 31;
            const uint8_t *ob = row < 64 ? gemm_st0 : gemm_st1;
            u32x4 v = *reinterpret_cast<const u32x4 *>(ob + (row & 63) * (kBN * 2) + 16 * (ch ^ (g >> 1)));
            if (g & 1) v = u32x4{v[2], v[3], v[0], v[1]};
            const int gr = m0 + row, col = n0 + 8 * ch;
            if (gr >= M || col >= N) continue;
            uint16_t *yp = y + (int64_t)gr * ldy + col;
            if (col + 7 < N) {
                __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(yp));
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (col + e < N) yp[e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
            }
        }
        // every wave is done reading the staged output before the next
        // tile's DMAs land in those stages
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Pipelined form for K a multiple of two K tiles (K % 512 == 0) and 16-byte
// aligned scale arrays: the K pipeline runs on across the output tiles of a
// workgroup.  K tile g of the workgroup's running sequence sits in stage
// g % 3, so a tile's first K tile is in stage (its index * KT) % 3.  The last
// two steps of a tile issue the next tile's first two K tiles, and the
// epilogue runs in the stage of its last K tile (free once multiplied) while
// those are in flight: no pipeline fill per tile and no idle epilogue.
//
// Scales travel apart from the codes.  One row's scale bytes for two
// consecutive K tiles are 16 contiguous bytes, so with every even K tile one
// 16-byte DMA per wave (48 active lanes, one row each) brings the 384 rows
// of both operands for that pair into one slot of a two-slot ring: 8 wave
// instructions per two K tiles where per-tile 4-byte DMAs took 32, each of
// those touching 32 cache lines for 256 bytes.  Pair n of the workgroup's
// running sequence sits in slot n % 2; it is fetched with its first K tile,
// two steps before it is read, after the barrier that ends the reads of
// pair n - 2 in that slot.
//
// This kernel issues its DMAs through inline assembly, so the compiler
// neither sees them nor adds waits for them (it cannot tell the ring slots
// apart and would drain at every read).  The waits are explicit: before K
// tile s is read, vmcnt(the DMAs of the step before) retires it; a step
// issues six code DMAs, plus the scale DMA when its K tile is even.  At a
// tile's first two steps the outstanding operations also include the
// previous epilogue's stores, which are younger than the K tile waited for,
// so the same count still retires it.
// ---------------------------------------------------------------------------
constexpr int kPStage = kAB + kWB;                               // codes of one K tile: 49152
constexpr int kRingRows = kBM + kBN;                             // A rows, then W rows
constexpr int kRingSlot = 16 * kRingRows;                        // 6144
constexpr int kRingRowsPerWave = kRingRows / (kGemmThreads / 64);  // 48
constexpr int kPipeK = 2 * kBK;                                  // K granule of this kernel
static_assert(kRingRows % (kGemmThreads / 64) == 0 && kRingRowsPerWave <= 64, "one scale DMA per wave");
static_assert(3 * kPStage + 2 * kRingSlot <= 160 * 1024, "LDS of the pipelined kernel");
static_assert(kDA + kDW == 6, "six code DMAs per step");

__shared__ __attribute__((aligned(16))) uint8_t gp_st[3 * kPStage];
__shared__ __attribute__((aligned(16))) uint8_t gp_ring[2 * kRingSlot];

__device__ __forceinline__ uint32_t lds_u32(const uint8_t *l) {
    return (uint32_t)(uintptr_t)(lds_void *)l;
}
// A 16-byte LDS DMA the compiler does not track.  M0 holds the LDS base
// (lane l writes at M0 + 16 l); one wait state must separate the write of
// M0 from the DMA that reads it.  The compiler reserves M0 and does not
// preserve it around inline assembly (hence its warning, silenced here):
// this is sound only while nothing else in the kernel uses M0, which a test
// checks in the kernel's assembly.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16_raw(const void *g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(g), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop

struct PipePlan {
    int ga[kDA], gw[kDW];   // code offsets at K tile 0, as in DmaPlan
    const uint8_t *sp;      // this lane's scale row (lanes < kRingRowsPerWave)
};

__device__ __forceinline__ void make_pipe_plan(PipePlan &pl, int m0, int n0, int M, int N, int K2,
                                               int K32, int wave, int lane, const uint8_t *as,
                                               const uint8_t *ws) {
#pragma unroll
    for (int q = 0; q < kDA; ++q) {
        const int p = (q * (kGemmThreads / 64) + wave) * 64 + lane;
        const int row = p >> 3, c = (p & 7) ^ ((row >> 1) & 7);
        pl.ga[q] = (m0 + row < M ? m0 + row : M - 1) * K2 + 16 * c;
    }
#pragma unroll
    for (int q = 0; q < kDW; ++q) {
        const int p = (q * (kGemmThreads / 64) + wave) * 64 + lane;
        const int row = p >> 3, c = (p & 7) ^ ((row >> 1) & 7);
        pl.gw[q] = (n0 + row < N ? n0 + row : N - 1) * K2 + 16 * c;
    }
    const int r = wave * kRingRowsPerWave + (lane < kRingRowsPerWave ? lane : 0);
    pl.sp = r < kBM ? as + (int64_t)(m0 + r < M ? m0 + r : M - 1) * K32
                    : ws + (int64_t)(n0 + r - kBM < N ? n0 + r - kBM : N - 1) * K32;
}

// K tile kt of both operands into stage st; with an even kt also the scale
// pair kt / 2 into ring slot `slot`.
__device__ __forceinline__ void pipe_issue(const PipePlan &pl, const uint8_t *ac, const uint8_t *wc,
                                           int kt, int wave, int lane, const uint8_t *st, int slot) {
    if ((kt & 1) == 0 && lane < kRingRowsPerWave)
        dma16_raw(pl.sp + 8 * kt, lds_u32(gp_ring + slot * kRingSlot + wave * kRingRowsPerWave * 16));
#pragma unroll
    for (int q = 0; q < kDA; ++q)
        dma16_raw(ac + pl.ga[q] + kt * kRowBytes, lds_u32(st + (q * (kGemmThreads / 64) + wave) * 1024));
#pragma unroll
    for (int q = 0; q < kDW; ++q)
        dma16_raw(wc + pl.gw[q] + kt * kRowBytes,
                  lds_u32(st + kAB + (q * (kGemmThreads / 64) + wave) * 1024));
}

// The 16 scale bytes (two K tiles) of this lane's four rows (A rows j = 0, 1,
// then W rows i = 0, 1) from ring slot rs.  One 16-byte read per row and
// pair: sixteen lanes read sixteen consecutive rows, 256 contiguous bytes,
// where 8-byte reads of one half of each 16-byte slot would pair rows 16
// apart on the same banks.
__device__ __forceinline__ void pipe_scales(const uint8_t *rs, int wm, int wn, int i32, u32x4 (&sc)[4]) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
        sc[j] = *reinterpret_cast<const u32x4 *>(rs + (wm * 64 + j * 32 + i32) * 16);
#pragma unroll
    for (int i = 0; i < 2; ++i)
        sc[2 + i] = *reinterpret_cast<const u32x4 *>(rs + (kBM + wn * 64 + i * 32 + i32) * 16);
}

// One K tile from stage b; its scale word per row is half `odd` of the
// row's pair in sc, shifted one byte for the upper 32 K values of a step, as
// in gemm_compute.  The step's DMAs (issue) go out after the second of the
// four K steps: issued right after the barrier, every wave first queues its
// DMAs and only then starts multiplying; issued half a step later they still
// have a step and a half to land, and the MFMAs of the first two K steps run
// meanwhile (2-3% faster than either end of the step).
template <class Issue>
__device__ __forceinline__ void pipe_compute(const uint8_t *__restrict__ b, const u32x4 (&sc)[4], int odd,
                                             int wm, int wn, int i32, int kg, f32x16g (&acc)[2][2],
                                             Issue issue) {
    u32x2g sa[2], sw[2];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint64_t w = odd ? ((uint64_t)sc[r][3] << 32 | sc[r][2]) : ((uint64_t)sc[r][1] << 32 | sc[r][0]);
        const uint64_t v = w >> (8 * kg);
        const u32x2g x = u32x2g{(uint32_t)v, (uint32_t)(v >> 32)};
        if (r < 2) sa[r] = x;
        else sw[r - 2] = x;
    }
    gemm_kstep<0>(b, wm, wn, i32, kg, sa, sw, acc);
    gemm_kstep<1>(b, wm, wn, i32, kg, sa, sw, acc);
    issue();
    gemm_kstep<2>(b, wm, wn, i32, kg, sa, sw, acc);
    gemm_kstep<3>(b, wm, wn, i32, kg, sa, sw, acc);
}

// kFixedStages: KT is a multiple of 3, so every tile's K tile 0 is in
// stage 0 and the stage of each unrolled step is a constant.
template <bool kFixedStages>
__global__ __launch_bounds__(kGemmThreads) void w4a4_gemm_pipe_kernel(
    const uint8_t *__restrict__ ac, const uint8_t *__restrict__ as,
    const uint8_t *__restrict__ wc, const uint8_t *__restrict__ ws, uint16_t *__restrict__ y,
    int M, int N, int K, int64_t ldy, int mtc, int ntc) {
    const int tiles = mtc * ntc, per = (tiles + 7) / 8, wpx = gridDim.x >> 3;
    const int xcd = blockIdx.x & 7;
    int t = blockIdx.x >> 3;
    if (t >= per || xcd * per + t >= tiles) return;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / kGemmWN, wn = wave % kGemmWN;
    const int i32 = lane & 31, kg = lane >> 5;
    const int K2 = K / 2, K32 = K / 32;
    const int KT = K / kBK;              // even
    const int flip = (KT / 2) & 1;       // ring slot change from one tile's pair 0 to the next's

    int m0, n0;
    tile_origin(xcd * per + t, mtc, ntc, m0, n0);
    PipePlan pc;
    make_pipe_plan(pc, m0, n0, M, N, K2, K32, wave, lane, as, ws);
    int pb = 0;                          // ring slot of this tile's scale pair 0
    int sb = 0;                          // stage of this tile's K tile 0
    const int sstep = kFixedStages ? 0 : KT % 3;  // stage change from one tile's K tile 0 to the next's
    pipe_issue(pc, ac, wc, 0, wave, lane, gp_st, pb);
    pipe_issue(pc, ac, wc, 1, wave, lane, gp_st + kPStage, pb);

    f32x16g acc[2][2];
    u32x4 sc[4];  // scale words of the current pair, rows A j = 0, 1 and W i = 0, 1
    auto barrier = [] { __builtin_amdgcn_s_barrier(); };
    for (;;) {
        // the next tile of this workgroup, if any (else the DMAs of the last
        // two steps repeat this tile's first K tiles, never read)
        const int tn = t + wpx;
        const bool has_next = tn < per && xcd * per + tn < tiles;
        int m1 = m0, n1 = n0;
        if (has_next) tile_origin(xcd * per + tn, mtc, ntc, m1, n1);
        PipePlan pn;
        make_pipe_plan(pn, m1, n1, M, N, K2, K32, wave, lane, as, ws);
        const int pbn = pb ^ flip;

#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[i][j] = f32x16g{};

        // step s: retire K tile s, multiply K tile s from stage (sb + s) % 3
        // and, halfway through, issue K tile s + 2 (or the next tile's
        // s + 2 - KT) into stage (sb + s + 2) % 3.  Twelve steps per pass
        // keep the parity of s and the stage offset (s % 3) of each unrolled
        // step fixed; the pass's three stage addresses are taken once.
        constexpr int kSteps = 12;
        for (int s0 = 0; s0 < KT; s0 += kSteps) {
            const int r0 = kFixedStages ? 0 : (sb + s0) % 3;
            const uint8_t *sp[3] = {gp_st + r0 * kPStage, gp_st + (r0 == 2 ? 0 : r0 + 1) * kPStage,
                                    gp_st + (r0 == 0 ? 2 : r0 - 1) * kPStage};
#pragma unroll
            for (int u = 0; u < kSteps; ++u) {
                const int st = s0 + u;
                if (st >= KT) break;
                const uint8_t *in = sp[(u + 2) % 3];
                const uint8_t *rd = sp[u % 3];
                // the step before issued 6 DMAs, 7 when its K tile (s + 1) was even
                if (u & 1) KQ_WAIT_VM(kDA + kDW + 1);
                else KQ_WAIT_VM(kDA + kDW);
                __builtin_amdgcn_s_barrier();
                const int f = st + 2;
                // a pair's scale words are read at its first K tile, after
                // the barrier that follows its arrival, and kept for the second
                if ((u & 1) == 0) pipe_scales(gp_ring + ((pb + (st >> 1)) & 1) * kRingSlot, wm, wn, i32, sc);
                pipe_compute(rd, sc, u & 1, wm, wn, i32, kg, acc, [&] {
                                 if (f < KT) pipe_issue(pc, ac, wc, f, wave, lane, in, (pb + (f >> 1)) & 1);
                                 else pipe_issue(pn, ac, wc, f - KT, wave, lane, in,
                                                 (pbn + ((f - KT) >> 1)) & 1);
                             });
            }
        }
        // epilogue in the stage of K tile KT - 1, two passes of 64 rows
        // (j = 0: rows 0-31 and 64-95, j = 1: the others); the other two
        // stages take the next tile's first K tiles
        uint8_t *ep = gp_st + (kFixedStages ? 2 : (sb + KT - 1) % 3) * kPStage;
        __builtin_amdgcn_s_barrier();
        store_half(acc, 0, ep, wm, wn, i32, kg, tid, m0, n0, M, N, ldy, y, barrier);
        __builtin_amdgcn_s_barrier();
        store_half(acc, 1, ep, wm, wn, i32, kg, tid, m0, n0, M, N, ldy, y, barrier);
        if (!has_next) break;
        sb = (sb + sstep) % 3;
        t = tn;
        m0 = m1;
        n0 = n1;
        pc = pn;
        pb = pbn;
    }
    // the last repeats may still be landing in LDS: finish before the
    // workgroup's LDS is handed to another
    KQ_WAIT_VM(0);
}

static kq_status launch_gemm(const uint8_t *ac, const uint8_t *as, const uint8_t *wc,
                             const uint8_t *ws, uint16_t *y, int M, int N, int K, int64_t ldy,
                             void *stream) {
    const int mtc = (M + kBM - 1) / kBM, ntc = (N + kBN - 1) / kBN;
    const int64_t tiles = (int64_t)mtc * ntc;
    if (tiles > INT32_MAX) return KQ_ERR_SHAPE;
    // one workgroup per CU (the LDS holds one), a multiple of the 8 XCDs;
    // a sweep build may fix the workgroups per XCD with -DKQ_GEMM_WPX=n
    const int wpx_env = KQ_GEMM_WPX;
    static std::atomic<int> wpx_dev[64];  // per device; 0 = not yet known
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return KQ_ERR_HIP;
    int wpx = dev >= 0 && dev < 64 ? wpx_dev[dev].load(std::memory_order_relaxed) : 0;
    if (wpx == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return KQ_ERR_HIP;
        wpx = wpx_env > 0 ? wpx_env : (cus / 8 > 0 ? cus / 8 : 1);
        if (dev >= 0 && dev < 64) wpx_dev[dev].store(wpx, std::memory_order_relaxed);
    }
    // Large problems with K a multiple of 256 take the 256 x 256-tile kernel
    // (less LDS traffic per MFMA); it needs a few tiles per compute unit to
    // fill the chip.
    if (KQ_GEMM_WIDE && K % 256 == 0 &&
        (int64_t)((M + 255) / 256) * ((N + 255) / 256) >= 2 * 8 * wpx) {
        static const bool wide_ok = [] {
            hipFuncAttributes fa;
            return hipFuncGetAttributes(&fa, (const void *)wide_kernel_symbol()) == hipSuccess &&
                   fa.localSizeBytes == 0;
        }();
        if (!wide_ok) return KQ_ERR_HIP;
        return launch_gemm_wide(ac, as, wc, ws, y, M, N, K, ldy, 8 * wpx, stream);
    }
    const int64_t per = (tiles + 7) / 8;
    const int64_t grid = 8 * (per < wpx ? per : wpx);
    void *args[] = {(void *)&ac, (void *)&as, (void *)&wc, (void *)&ws, (void *)&y, (void *)&M,
                    (void *)&N, (void *)&K, (void *)&ldy, (void *)&mtc, (void *)&ntc};
    const bool pipe_env = KQ_GEMM_PIPE != 0;
    // the pipelined kernel fetches two K tiles' scale bytes per row with one
    // 16-byte DMA: it needs 16-byte aligned scale rows (K % 512 == 0 and
    // 16-byte aligned arrays); otherwise the per-tile kernel runs
    const bool pipe = pipe_env && K % kPipeK == 0 && (uintptr_t)as % 16 == 0 &&
                      (uintptr_t)ws % 16 == 0;
    const void *fn = !pipe ? (const void *)w4a4_gemm_kernel
                     : (K / kBK) % 3 == 0 ? (const void *)w4a4_gemm_pipe_kernel<true>
                                         : (const void *)w4a4_gemm_pipe_kernel<false>;
    // The explicit vmcnt waits count this kernel's DMAs; register spills would
    // add scratch loads and stores to that count and let a stage be read
    // before it has landed.  A build that gives the kernel scratch memory is
    // refused rather than run.
    static const bool no_scratch = [] {
        const void *kernels[] = {(const void *)w4a4_gemm_kernel,
                                 (const void *)w4a4_gemm_pipe_kernel<true>,
                                 (const void *)w4a4_gemm_pipe_kernel<false>};
        for (const void *k : kernels) {
            hipFuncAttributes fa;
            if (hipFuncGetAttributes(&fa, k) != hipSuccess || fa.localSizeBytes != 0) return false;
        }
        return true;
    }();
    if (!no_scratch) return KQ_ERR_HIP;
    const hipError_t e = hipLaunchKernel(fn, dim3((unsigned)grid), dim3(kGemmThreads), args, 0,
                                         (hipStream_t)stream);
    return e == hipSuccess ? KQ_OK : KQ_ERR_HIP;
}

}  // namespace kq

using namespace kq;

extern "C" kq_status kq_w4a4_gemm(const uint8_t *a_codes, const uint8_t *a_scales,
                                  const uint8_t *w_codes, const uint8_t *w_scales, int64_t M,
                                  int64_t N, int64_t K, void *y, int64_t ld_y, void *stream) {
    if (M < 0 || N < 0 || K < 0 || M >= (int64_t(1) << 30) || N >= (int64_t(1) << 30) ||
        K >= (int64_t(1) << 24) || K % 128 != 0 || ld_y < N)
        return KQ_ERR_SHAPE;
    if (M == 0 || N == 0) return KQ_OK;
    if (K == 0) return KQ_ERR_SHAPE;
    // byte offsets inside an operand are 32-bit
    if ((M > N ? M : N) * (K / 2) >= (int64_t(1) << 31)) return KQ_ERR_SHAPE;
    if (!a_codes || !a_scales || !w_codes || !w_scales || !y) return KQ_ERR_NULL;
    if (((uintptr_t)a_codes % 16) || ((uintptr_t)w_codes % 16) || ((uintptr_t)a_scales % 4) ||
        ((uintptr_t)w_scales % 4) || ((uintptr_t)y % 16) || (ld_y % 8))
        return KQ_ERR_ALIGN;
    return launch_gemm(a_codes, a_scales, w_codes, w_scales, (uint16_t *)y, (int)M, (int)N, (int)K,
                       ld_y, stream);
}

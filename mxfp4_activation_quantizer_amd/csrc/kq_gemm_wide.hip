// kq_gemm_wide.hip — the W4A4 consumer with 256 x 256 output tiles: the
// same product as kq_gemm.hip (Y = dequant(A) dequant(W)^T on the gfx950
// block-scaled FP4 MFMA, fp32 accumulation, bf16 out), arranged so that the
// LDS traffic per MFMA is lower.
//
// Why.  With 128 x 256 tiles and 64 x 64 per wave, every MFMA needs one
// 16-byte fragment read per lane from LDS and the tile's operand DMAs write
// LDS as well: per K tile and CU that is about 1.3 times the matrix cores'
// own time, so the LDS, not the MFMA, sets the pace.  Here a workgroup of
// four waves (one per SIMD) computes a 256 x 256 tile, each wave 128 x 128
// as 4 x 4 MFMA tiles (256 accumulator registers, in the AGPRs): per 64-wide
// K step a wave reads 8 fragments for 16 MFMAs, and per K element the tile
// fetches 512 rows for 65536 outputs instead of 384 for 32768.  A build
// with -DKQ_GEMM_WIDE_WAVES=8 runs eight waves (two per SIMD, 128 x 64
// each, 128 accumulators): correct, and no faster.
//
// K runs in tiles of 256 (128 code bytes per row, whole cache lines per
// DMA) through two LDS stages of 64 KB: one K tile is in flight while the
// other is multiplied.  A stage holds A and W codes, 256 rows x 128 bytes
// each.  A code row is eight 16-byte chunks at slot c ^ ((row >> 1) & 7):
// the 16 lanes an LDS cycle serves read 16 consecutive rows at one chunk
// and so cover all 64 banks once.  A DMA lane writes 16 bytes at
// (region base + 16 lane), so the layout is made on the global side: the
// lane landing in slot s of a row fetches chunk s ^ ((row >> 1) & 7).
//
// Scale bytes come in chunks of four K tiles (32 bytes per row, 8 lanes of
// 4 bytes per row, so a DMA reads 8 rows' contiguous bytes) into two 16 KB
// buffers; a quarter of the next chunk is fetched during each K tile.  In
// the LDS, row r keeps K tile q's 8 bytes at unit q ^ ((r >> 3) & 3) (the
// DMA lanes fetch their words in that order), so that reading one K tile's
// bytes of 32 consecutive rows touches every bank once.  One
// 4-byte DMA per row and K tile, the first form, touched a separate cache
// line per lane and made half of all L2 requests.
//
// Per K tile: wait for this wave's DMAs (explicit vmcnt), barrier (every
// wave's DMAs of the tile have landed, and every wave has finished reading
// the previous tile), then four K steps of 16 MFMAs with the 20 DMAs of the
// next K tile issued one at a time between the MFMAs of the first three
// steps.  The DMAs are written as inline assembly and the waits are
// explicit (see dma16).
//
// Epilogue: the bf16 tile (128 KB) goes through the two stages (128 rows
// each, 8-byte slots at (column / 4) ^ (row & 31)), then every wave stores
// two whole 512-byte rows per instruction.
//
// Tiles are persistent per workgroup, XCD-contiguous, walking eight M tiles
// for each N tile (as in kq_gemm.hip).

#include <stdint.h>

#include <utility>

#include <hip/hip_runtime.h>

#include "kq.h"
#include "kq_device.h"
#include "kq_gemm_wide.h"

namespace kq {
namespace wide {

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

// Waves per workgroup: 4 (one per SIMD, 128 x 128 each) or 8 (two per
// SIMD, 128 x 64 each); -DKQ_GEMM_WIDE_WAVES selects it.
#ifndef KQ_GEMM_WIDE_WAVES
#define KQ_GEMM_WIDE_WAVES 4
#endif
constexpr int kWaves = KQ_GEMM_WIDE_WAVES;
static_assert(kWaves == 4 || kWaves == 8, "KQ_GEMM_WIDE_WAVES must be 4 or 8");
constexpr int kThreads = 64 * kWaves;
constexpr int kWN = kWaves / 2;          // wave columns; wave rows: 2
constexpr int kTI = 256 / kWN / 32;      // 32-column MFMA tiles per wave (4 or 2)
constexpr int kCodeDma = 64 / kWaves;    // code DMAs per wave per K tile (16 or 8)
constexpr int kScaleDma = 16 / kWaves;   // scale DMAs per wave per K tile (4 or 2)
constexpr int kBM = 256, kBN = 256;      // output tile
constexpr int kBK = 256;                 // K elements per stage
constexpr int kRow = kBK / 2;            // 128 code bytes per row per stage
constexpr int kCodesA = kBM * kRow;      // 32768
constexpr int kCodesW = kBN * kRow;      // 32768
constexpr int kStage = kCodesA + kCodesW;  // 65536 code bytes per stage
constexpr int kChunkKT = 4;                // K tiles per scale chunk
constexpr int kSRow = 8 * kChunkKT;        // 32 scale bytes per row per chunk
constexpr int kSBuf = (kBM + kBN) * kSRow; // 16384: A rows, then W rows
constexpr int kMGroup = 8;
static_assert(2 * kStage + 2 * kSBuf <= 160 * 1024, "two stages and two scale chunks fit the LDS");
static_assert(128 * 512 <= kStage, "128 output rows of bf16 fit one stage");

__shared__ __attribute__((aligned(16))) uint8_t st0[kStage];
__shared__ __attribute__((aligned(16))) uint8_t st1[kStage];
__shared__ __attribute__((aligned(16))) uint8_t sc0[kSBuf];
__shared__ __attribute__((aligned(16))) uint8_t sc1[kSBuf];

// s_waitcnt vmcnt(n), no expcnt / lgkmcnt wait (gfx9 encoding)
#define KQW_WAIT_VM(n) \
    __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

// LDS DMAs the compiler does not see.  Written with the builtin, each DMA
// into one stage made the compiler's wait insertion retire every DMA in
// flight before the next LDS read; so they are issued here and the waits are
// explicit.  They are buffer loads: the operand's bounds (num_records) make
// rows past M or N read as zeros with no clamping (the range check applies
// to the lane offset, which therefore carries the row; see Plan).  M0 holds
// the LDS base (lane l writes at
// M0 + size * l); one wait state separates the write of M0 from the DMA.
// The compiler reserves M0 and does not preserve it around inline assembly
// (hence its warning, silenced here): this is sound only while nothing else
// in the kernel uses M0, which a test checks in the kernel's assembly.
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds"
                 :: "v"(voff), "s"(rsrc), "s"(lds), "s"(soff) : "memory", "m0");
}
__device__ __forceinline__ void dma4(i32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, %3 offen lds"
                 :: "v"(voff), "s"(rsrc), "s"(lds), "s"(soff) : "memory", "m0");
}
#pragma clang diagnostic pop

// Raw buffer resource over [base, base + bytes): loads past the end read 0.
__device__ __forceinline__ i32x4 buffer_rsrc(const void *base, uint32_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    return i32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                 __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu)),
                 __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000};
}

// Two accumulator values, read from their AGPRs here and converted to a bf16
// pair (nearest even, first value in the low half).  Written out so that the
// epilogue reads each accumulator where it converts it: left to the compiler,
// all 256 accumulators were first copied into VGPRs, which spilled.  The
// caller keeps enough wait states between the last MFMA and these reads.
__device__ __forceinline__ uint32_t acc_bf16x2(float a, float b) {
    uint32_t r, t;
    asm volatile("v_accvgpr_read_b32 %0, %2\n\tv_accvgpr_read_b32 %1, %3\n\t"
                 "v_cvt_pk_bf16_f32 %0, %0, %1"
                 : "=&v"(r), "=&v"(t) : "a"(a), "a"(b));
    return r;
}

__device__ __forceinline__ uint32_t lds_addr(const uint8_t *l) {
    return (uint32_t)(uintptr_t)(lds_void *)l;
}

// This lane's DMA sources for one output tile, as byte offsets at K 0: of
// its first code chunk in A and W (DMA q is 32 q rows further) and of its
// first scale word (8 lanes per row; DMA i of a part is 8 i rows further).
// The buffer range check sees the lane offset (not the scalar offset), so
// every row step goes into the lane offset and the scalar offset holds only
// a position inside the row: rows past the operand's end read zeros and no
// DMA reads past it.  Every operand is under 2 GiB.
struct Plan {
    uint32_t va, vw;    // code offsets (A, W)
    uint32_t sa, sw;    // scale offsets (A, W)
    i32x4 ra, rw, rsa, rsw;
    uint32_t row32;     // bytes of 8 kWaves code rows (one DMA step)
    uint32_t srow8;     // bytes of 8 scale rows
    uint32_t sword;     // this lane's byte in a row's 32 scale bytes, before the swizzle
};

__device__ __forceinline__ void make_plan(Plan &pl, const uint8_t *ac, const uint8_t *as,
                                          const uint8_t *wc, const uint8_t *ws, int m0, int n0,
                                          int M, int N, int K2, int K32, int wave, int lane) {
    // DMA q writes 1 KB region q * kWaves + wave: rows (q * kWaves + wave) * 8
    // + lane / 8 (= the lane's row + 8 kWaves q), slot lane % 8, which holds
    // chunk slot ^ ((row >> 1) & 7); row + 8 kWaves q has the same low bits
    const int r0 = wave * 8 + (lane >> 3);
    const uint32_t c16 = 16 * ((lane & 7) ^ ((r0 >> 1) & 7));
    pl.va = (uint32_t)(m0 + r0) * (uint32_t)K2 + c16;
    pl.vw = (uint32_t)(n0 + r0) * (uint32_t)K2 + c16;
    const int srow = wave * (128 / kWaves) + (lane >> 3);
    pl.sa = (uint32_t)(m0 + srow) * (uint32_t)K32;
    pl.sw = (uint32_t)(n0 + srow) * (uint32_t)K32;
    pl.sword = 4 * (lane & 7);
    pl.ra = buffer_rsrc(ac, (uint32_t)M * (uint32_t)K2);
    pl.rw = buffer_rsrc(wc, (uint32_t)N * (uint32_t)K2);
    pl.rsa = buffer_rsrc(as, (uint32_t)M * (uint32_t)K32);
    pl.rsw = buffer_rsrc(ws, (uint32_t)N * (uint32_t)K32);
    pl.row32 = __builtin_amdgcn_readfirstlane(8 * kWaves * K2);
    pl.srow8 = __builtin_amdgcn_readfirstlane(8 * K32);
}

// The DMAs a wave issues during K tile kt (20 with four waves, 10 with
// eight): D < kCodeDma are the code rows of K tile kt + 1 (A for even D, W
// for odd D, 8 kWaves (D / 2) rows further down), the next kScaleDma a
// quarter of the scale chunk after the current one: chunk c covers K tiles
// 4c .. 4c + 3 (32 bytes per row), and during K tile kt, part kt % 4 of
// chunk kt / 4 + 1 is fetched, 128 rows (rows 0 .. 255 of A for parts 0 and
// 1, of W for parts 2 and 3), 128 / kWaves per wave, 8 per DMA.  An empty
// resource (num_records 0) turns every DMA it serves into zeros written to
// the LDS with no memory read (past the last K tile or chunk).
struct Dma {
    i32x4 ra, rw, rs;
    uint32_t va, vw, vs, row32, srow8, ko, sword, skey;
    uint32_t st, ss;  // LDS: this wave's first code region, its scale rows
};

__device__ __forceinline__ i32x4 with_records(const i32x4 &r, bool live) {
    return i32x4{r[0], r[1], r[2] & (live ? -1 : 0), r[3]};
}

__device__ __forceinline__ void make_dma(Dma &dm, const Plan &pl, int kt, int KT, int wave,
                                         uint8_t *__restrict__ st) {
    const bool live = kt + 1 < KT;
    dm.ra = with_records(pl.ra, live);
    dm.rw = with_records(pl.rw, live);
    dm.va = pl.va;
    dm.vw = pl.vw;
    dm.row32 = pl.row32;
    dm.srow8 = pl.srow8;
    dm.sword = pl.sword;
    dm.ko = __builtin_amdgcn_readfirstlane((uint32_t)(kt + 1) * kRow);
    dm.st = __builtin_amdgcn_readfirstlane(lds_addr(st) + wave * 1024);
    dm.skey = (wave * (16 / kWaves)) & 3;
    const int chunk = (kt >> 2) + 1, part = kt & 3;
    dm.rs = with_records(part < 2 ? pl.rsa : pl.rsw, chunk * kChunkKT < KT);
    dm.vs = (part < 2 ? pl.sa : pl.sw) + (uint32_t)chunk * kSRow + (uint32_t)(part & 1) * 16 * pl.srow8;
    dm.ss = __builtin_amdgcn_readfirstlane(lds_addr(chunk & 1 ? sc1 : sc0) +
                                           (part * 128 + wave * (128 / kWaves)) * kSRow);
}

template <int D>
__device__ __forceinline__ void issue_one(const Dma &dm) {
    if constexpr (D < kCodeDma) {
        constexpr int q = D >> 1;
        // region q * kWaves + wave of 1 KB
        if constexpr ((D & 1) == 0)
            dma16(dm.ra, dm.va + q * dm.row32, dm.ko, dm.st + q * kWaves * 1024);
        else
            dma16(dm.rw, dm.vw + q * dm.row32, dm.ko, dm.st + kCodesA + q * kWaves * 1024);
    } else {
        // rows of DMA i: (row >> 3) & 3 = skey ^ i (skey even when i < 2)
        constexpr int i = D - kCodeDma;
        dma4(dm.rs, dm.vs + i * dm.srow8 + (dm.sword ^ (8 * (dm.skey ^ i))), 0, dm.ss + i * 8 * kSRow);
    }
}

// The first K tile of an output tile into stage 0 and the whole first scale
// chunk into its buffer, all at once.
__device__ __forceinline__ void issue_first(const Plan &pl, int wave) {
    const uint32_t st = __builtin_amdgcn_readfirstlane(lds_addr(st0) + wave * 1024);
#pragma unroll
    for (int q = 0; q < kCodeDma / 2; ++q) {
        dma16(pl.ra, pl.va + q * pl.row32, 0, st + q * kWaves * 1024);
        dma16(pl.rw, pl.vw + q * pl.row32, 0, st + kCodesA + q * kWaves * 1024);
    }
    const int skey = (wave * (16 / kWaves)) & 3;
#pragma unroll
    for (int part = 0; part < 4; ++part) {
        const uint32_t ss = __builtin_amdgcn_readfirstlane(lds_addr(sc0) +
                                                           (part * 128 + wave * (128 / kWaves)) * kSRow);
        const uint32_t vs = (part < 2 ? pl.sa : pl.sw) + (uint32_t)(part & 1) * 16 * pl.srow8;
#pragma unroll
        for (int i = 0; i < kScaleDma; ++i)
            dma4(part < 2 ? pl.rsa : pl.rsw, vs + i * pl.srow8 + (pl.sword ^ (8 * (skey ^ i))), 0,
                 ss + i * 8 * kSRow);
    }
}

__device__ __forceinline__ i32x8 frag(const uint8_t *b, int row, int ch) {
    const u32x4 v = *reinterpret_cast<const u32x4 *>(b + row * kRow + 16 * (ch ^ ((row >> 1) & 7)));
    return (i32x8)__builtin_shufflevector(v, v, 0, 1, 2, 3, -1, -1, -1, -1);
}

// The fragments of one K step: rows wm*128 + j*32 + (lane % 32) of A and
// wn*32*kTI + i*32 + (lane % 32) of W, chunk 2 KS + kg.
struct Frags {
    i32x8 a[4], w[kTI];
};

template <int KS>
__device__ __forceinline__ void load_frags(const uint8_t *__restrict__ b, int wm, int wn, int i32, int kg,
                                           Frags &f) {
    const int ch = 2 * KS + kg;
#pragma unroll
    for (int j = 0; j < 4; ++j) f.a[j] = frag(b, wm * 128 + j * 32 + i32, ch);
#pragma unroll
    for (int i = 0; i < kTI; ++i) f.w[i] = frag(b + kCodesA, wn * 32 * kTI + i * 32 + i32, ch);
}

// The DMA issued after MFMA m of K step ks, or -1: the code DMAs after the
// odd MFMAs of steps 0 and 1, the scale DMAs in step 2 after every fourth.
// Spread out so that the wave never waits long to hand a DMA over while its
// MFMAs could issue; issued all at once after the barrier, they held the
// matrix cores idle for a good part of every K tile.
constexpr int kNM = 4 * kTI;  // MFMAs per wave per K step
static_assert(kCodeDma == kNM && kScaleDma * 4 == kNM, "the DMA slots of dma_after");
constexpr int dma_after(int ks, int m) {
    return ks < 2 ? ((m & 1) ? ks * (kNM / 2) + (m >> 1) : -1)
                  : (ks == 2 && (m & 3) == 3 ? kCodeDma + (m >> 2) : -1);
}

// MFMA m = 4 i + j of K step KS (its scale byte is byte 2 (KS % 2) of word
// KS / 2, see compute), then its DMA if it has one; the scheduling barriers
// keep the DMA where it is placed.
template <int KS, int MI>
__device__ __forceinline__ void mfma_one(const Frags &f, const u32x2 (&sa)[4], const u32x2 (&sw)[kTI],
                                         f32x16 (&acc)[kTI][4], const Dma &dm) {
    constexpr int kSel = 2 * (KS & 1), kWord = KS >> 1, i = MI >> 2, j = MI & 3;
    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
        f.w[i], f.a[j], acc[i][j], 4, 4, kSel, (int)sw[i][kWord], kSel, (int)sa[j][kWord]);
    constexpr int d = dma_after(KS, MI);
    if constexpr (d >= 0) {
        __builtin_amdgcn_sched_barrier(0);
        issue_one<d>(dm);
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int KS, int... MI>
__device__ __forceinline__ void mfma_seq(const Frags &f, const u32x2 (&sa)[4], const u32x2 (&sw)[kTI],
                                         f32x16 (&acc)[kTI][4], const Dma &dm,
                                         std::integer_sequence<int, MI...>) {
    (mfma_one<KS, MI>(f, sa, sw, acc, dm), ...);
}

// The MFMAs of K step KS, with their share of the next K tile's DMAs.
template <int KS>
__device__ __forceinline__ void mfma16(const Frags &f, const u32x2 (&sa)[4], const u32x2 (&sw)[kTI],
                                       f32x16 (&acc)[kTI][4], const Dma &dm) {
    mfma_seq<KS>(f, sa, sw, acc, dm, std::make_integer_sequence<int, kNM>{});
}

// The four K steps of stage b.  A row's 8 scale bytes (the stage's eight
// 32-element groups) are shifted right one byte for the lanes of the upper
// 32 K values of a step (kg = 1), so that K step ks finds its byte at 2 ks
// for every lane: byte 2 (ks % 2) of word ks / 2 (the MFMA's scale select).
// The fragments of step ks + 1 are read while the MFMAs of step ks run; the
// scheduling barriers keep it to two fragment sets in registers (left free,
// the compiler read all four steps' fragments ahead and ran out of
// registers).
__device__ __forceinline__ void compute(const uint8_t *__restrict__ b, const uint8_t *__restrict__ sc,
                                        int kq, int wm, int wn, int i32, int kg, f32x16 (&acc)[kTI][4],
                                        const Dma &dm) {
    // sc: the scale chunk; kq: the K tile within it.  Row r holds its four
    // K tiles' 8-byte groups at unit q ^ ((r >> 3) & 3) (so that 32
    // consecutive rows' reads of one K tile cover all banks); every row this
    // lane reads has (r >> 3) & 3 = (i32 >> 3) & 3.
    const int sx = 8 * (kq ^ ((i32 >> 3) & 3));
    u32x2 sa[4], sw[kTI];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = wm * 128 + j * 32 + i32;
        const uint64_t v = *reinterpret_cast<const uint64_t *>(sc + r * kSRow + sx) >> (8 * kg);
        sa[j] = u32x2{(uint32_t)v, (uint32_t)(v >> 32)};
    }
#pragma unroll
    for (int i = 0; i < kTI; ++i) {
        const int r = kBM + wn * 32 * kTI + i * 32 + i32;
        const uint64_t v = *reinterpret_cast<const uint64_t *>(sc + r * kSRow + sx) >> (8 * kg);
        sw[i] = u32x2{(uint32_t)v, (uint32_t)(v >> 32)};
    }
    Frags f0, f1;
    load_frags<0>(b, wm, wn, i32, kg, f0);
    __builtin_amdgcn_sched_barrier(0);
    load_frags<1>(b, wm, wn, i32, kg, f1);
    mfma16<0>(f0, sa, sw, acc, dm);
    __builtin_amdgcn_sched_barrier(0);
    load_frags<2>(b, wm, wn, i32, kg, f0);
    mfma16<1>(f1, sa, sw, acc, dm);
    __builtin_amdgcn_sched_barrier(0);
    load_frags<3>(b, wm, wn, i32, kg, f1);
    mfma16<2>(f0, sa, sw, acc, dm);
    __builtin_amdgcn_sched_barrier(0);
    mfma16<3>(f1, sa, sw, acc, dm);
}

__device__ __forceinline__ void tile_origin(int lin, int mtc, int ntc, int &m0, int &n0) {
    const int blk = lin / (kMGroup * ntc), rem = lin - blk * kMGroup * ntc;
    const int grp = mtc - blk * kMGroup < kMGroup ? mtc - blk * kMGroup : kMGroup;
    const int nt = rem / grp, mt = blk * kMGroup + rem - nt * grp;
    m0 = mt * kBM;
    n0 = nt * kBN;
}

// One K tile step U (0, 1) of the unrolled body: stage U is read, the other
// stage receives K tile kt + 1.
template <int U>
__device__ __forceinline__ void kstep(const Plan &pl, int kt, int KT, int wave, int wm, int wn,
                                      int i32, int kg, f32x16 (&acc)[kTI][4]) {
    uint8_t *const rd = U == 0 ? st0 : st1;
    uint8_t *const in = U == 0 ? st1 : st0;
    // this wave's DMAs of tile kt have landed (none younger are in flight:
    // tile kt + 1 is issued during compute)
    KQW_WAIT_VM(0);
    __builtin_amdgcn_s_barrier();
    // K tile kt + 1 into the other stage and a quarter of the next scale
    // chunk, or, past the last ones, zeros with no memory read (no branch
    // around the accumulating steps)
    Dma dm;
    make_dma(dm, pl, kt, KT, wave, in);
    compute(rd, (kt >> 2) & 1 ? sc1 : sc0, kt & 3, wm, wn, i32, kg, acc, dm);
}

__global__ __launch_bounds__(kThreads) void gemm_wide_kernel(
    const uint8_t *__restrict__ ac, const uint8_t *__restrict__ as,
    const uint8_t *__restrict__ wc, const uint8_t *__restrict__ ws, uint16_t *__restrict__ y,
    int M, int N, int K, int64_t ldy, int mtc, int ntc) {
    const int tiles = mtc * ntc, per = (tiles + 7) / 8, wpx = gridDim.x >> 3;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / kWN, wn = wave % kWN;
    const int i32 = lane & 31, kg = lane >> 5;
    const int K2 = K / 2, K32 = K / 32, KT = K / kBK;
    for (int t = blockIdx.x >> 3; t < per; t += wpx) {
        const int lin = (blockIdx.x & 7) * per + t;
        if (lin >= tiles) break;
        int m0, n0;
        tile_origin(lin, mtc, ntc, m0, n0);
        Plan pl;
        make_plan(pl, ac, as, wc, ws, m0, n0, M, N, K2, K32, wave, lane);
        issue_first(pl, wave);

        f32x16 acc[kTI][4];
#pragma unroll
        for (int i = 0; i < kTI; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

        // two K tiles per pass with no branch around a step (a merge of two
        // paths made the compiler copy the 256 accumulators); an odd last
        // K tile, in stage 0, after the loop
        int kt = 0;
        for (; kt + 1 < KT; kt += 2) {
            kstep<0>(pl, kt, KT, wave, wm, wn, i32, kg, acc);
            kstep<1>(pl, kt + 1, KT, wave, wm, wn, i32, kg, acc);
        }
        if (kt < KT) kstep<0>(pl, kt, KT, wave, wm, wn, i32, kg, acc);

        // ---- epilogue: the last zero DMAs have landed and every wave is
        //      done reading the stages; the wait states cover the last
        //      MFMAs' results before their reads ----
        KQW_WAIT_VM(0);
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
        __builtin_amdgcn_s_barrier();
        // accumulator (i, j) register 4g + e of lane l: row wm*128 + j*32 + l%32,
        // column wn*32*kTI + i*32 + 8g + 4kg + e.  Stage s holds output rows
        // 128 s .. 128 s + 127, 512 bytes each, as 8-byte slots (col / 4) ^ (row & 31).
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint8_t *ob = (wm == 0 ? st0 : st1) + (j * 32 + i32) * 512;
#pragma unroll
            for (int i = 0; i < kTI; ++i) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    // slot (wn*8*kTI + i*8 + 2g + kg) ^ (row & 31), row & 31 = i32
                    const int phys = (wn * 8 * kTI + i * 8 + 2 * g + kg) ^ i32;
                    const uint32_t lo = acc_bf16x2(acc[i][j][4 * g], acc[i][j][4 * g + 1]);
                    const uint32_t hi = acc_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
                    *reinterpret_cast<u32x2 *>(ob + 8 * phys) = u32x2{lo, hi};
                }
            }
        }
        __syncthreads();
        // 256 rows x 32 chunks of 16 bytes; a wave stores two rows per instruction
#pragma unroll 4
        for (int k = 0; k < kBM * 32 / kThreads; ++k) {
            const int f = tid + k * kThreads;
            const int row = f >> 5, ch = f & 31, lr = row & 127, x = lr & 31;
            const uint8_t *ob = row < 128 ? st0 : st1;
            u32x4 v = *reinterpret_cast<const u32x4 *>(ob + lr * 512 + 16 * (ch ^ (x >> 1)));
            if (x & 1) v = u32x4{v[2], v[3], v[0], v[1]};
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
        // tile's DMAs land in the stages
        __syncthreads();
    }
}

}  // namespace wide

const void *wide_kernel_symbol() { return (const void *)wide::gemm_wide_kernel; }

kq_status launch_gemm_wide(const uint8_t *ac, const uint8_t *as, const uint8_t *wc,
                           const uint8_t *ws, uint16_t *y, int M, int N, int K, int64_t ldy,
                           int cus, void *stream) {
    using namespace wide;
    const int mtc = (M + kBM - 1) / kBM, ntc = (N + kBN - 1) / kBN;
    const int64_t tiles = (int64_t)mtc * ntc;
    if (tiles > INT32_MAX) return KQ_ERR_SHAPE;
    const int wpx = cus / 8 > 0 ? cus / 8 : 1;
    const int64_t per = (tiles + 7) / 8;
    const int64_t grid = 8 * (per < wpx ? per : wpx);
    void *args[] = {(void *)&ac, (void *)&as, (void *)&wc, (void *)&ws, (void *)&y, (void *)&M,
                    (void *)&N, (void *)&K, (void *)&ldy, (void *)&mtc, (void *)&ntc};
    const hipError_t e = hipLaunchKernel((const void *)gemm_wide_kernel, dim3((unsigned)grid),
                                         dim3(kThreads), args, 0, (hipStream_t)stream);
    return e == hipSuccess ? KQ_OK : KQ_ERR_HIP;
}

}  // namespace kq

// kq_device.h — device-side building blocks of the gfx950 quantizer kernels.
//
// Everything here is written for CDNA4 (gfx950, wave64): 16-byte global
// loads, the hardware E2M1 pack-convert with an E8M0 scale operand
// (v_cvt_scalef32_pk_fp4_f32) and the NaN-propagating three-input maximum
// (v_maximum3_f32).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kq {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// bf16 -> fp32 is exact: a bf16 is the upper half of a binary32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Largest |y| over a 32-value block.  llvm.maximum propagates NaN (unlike
// fmaxf), so a NaN anywhere in the block makes amax NaN.  Written as a chain
// that folds two new values per step, which gfx950 issues as one
// v_maximum3_f32 with |.| source modifiers per step.
__device__ __forceinline__ float block_amax(const float (&y)[32]) {
    float m = __builtin_elementwise_maximum(__builtin_fabsf(y[0]), __builtin_fabsf(y[1]));
#pragma unroll
    for (int k = 2; k < 32; k += 2)
        m = __builtin_elementwise_maximum(__builtin_elementwise_maximum(m, __builtin_fabsf(y[k])),
                                          __builtin_fabsf(y[k + 1]));
    return m;
}

// floor(n / d) for 0 <= n < 2^31 by one 32x32 -> 64-bit multiply and a
// shift: with s = 31 + ceil(log2 d) and m = ceil(2^s / d) (< 2^32, made once
// on the host by div_magic), n*m / 2^s exceeds n/d by less than 2^-ceil(log2 d)
// <= 1/d, which never reaches the next integer.
struct DivMagic {
    uint32_t m, s;
};
__host__ __device__ inline DivMagic div_magic(uint32_t d) {
    uint32_t l = 0;
    while ((uint64_t(1) << l) < d) ++l;
    const uint64_t p = uint64_t(1) << (31 + l);
    return DivMagic{(uint32_t)((p + d - 1) / d), 31 + l};
}
__device__ __forceinline__ uint32_t udiv31(uint32_t n, DivMagic dm) {
    return (uint32_t)(((uint64_t)n * dm.m) >> dm.s);
}

// LDS position (in 16-B chunks) of chunk i (0..7) of block j's 32-float
// slice of a per-channel vector staged in LDS.  Lane j reads its block's
// eight chunks with a 128-B stride between lanes; XOR-ing the chunk index
// with bits 1..3 of j spreads any 16 consecutive lanes over all 64 banks (no
// conflicts), and staging writes of eight consecutive chunks per block stay
// conflict-free.
__device__ __forceinline__ int vec_chunk(int j, int i) { return j * 8 + (i ^ ((j >> 1) & 7)); }

// Correctly rounded fp32 reciprocal.  For |u| in [2^-126, 2^126) (biased
// exponent 1..252) one fused correction of the hardware estimate,
// r + r*(1 - u*r), equals IEEE 1/u bit for bit (checked exhaustively over
// that range on gfx950 against the correctly rounded quotient); any other u
// takes the IEEE division.
__device__ __forceinline__ float rcp_rn(float u) {
    const uint32_t ex = (__float_as_uint(u) >> 23) & 0xffu;
    if (__builtin_expect(ex - 1u < 252u, 1)) {
        const float r = __builtin_amdgcn_rcpf(u);
        return __builtin_fmaf(__builtin_fmaf(-u, r, 1.0f), r, r);
    }
    return 1.0f / u;
}

// The five reciprocals of a block's factor expansion, each equal to IEEE
// 1/u_b: the corrected hardware estimate when every |u_b| lies in
// [2^-126, 2^126) (one range test for all five, NaN failing it through the
// NaN-propagating minimum/maximum), else the IEEE division for all five.
__device__ __forceinline__ void rcp5_rn(const float (&u)[5], float (&iu)[5]) {
#pragma unroll
    for (int b = 0; b < 5; ++b) {
        const float r = __builtin_amdgcn_rcpf(u[b]);
        iu[b] = __builtin_fmaf(__builtin_fmaf(-u[b], r, 1.0f), r, r);
    }
    const float a0 = __builtin_fabsf(u[0]), a1 = __builtin_fabsf(u[1]), a2 = __builtin_fabsf(u[2]),
                a3 = __builtin_fabsf(u[3]), a4 = __builtin_fabsf(u[4]);
    const float mn = __builtin_elementwise_minimum(__builtin_elementwise_minimum(
        __builtin_elementwise_minimum(a0, a1), a2), __builtin_elementwise_minimum(a3, a4));
    const float mx = __builtin_elementwise_maximum(__builtin_elementwise_maximum(
        __builtin_elementwise_maximum(a0, a1), a2), __builtin_elementwise_maximum(a3, a4));
    if (__builtin_expect(!(mn >= 0x1p-126f && mx < 0x1p126f), 0)) {
#pragma unroll
        for (int b = 0; b < 5; ++b) iu[b] = 1.0f / u[b];
    }
}

// E8M0 scale byte of the MXFP4 block: e = floor(log2 amax) - 2 clamped to
// [-127, 127], stored as e + 127.  For a normal amax with biased exponent E,
// floor(log2 amax) = E - 127, so the byte is E - 2; E < 2 (tiny, subnormal
// or zero amax) clamps to 0; E = 255 (Inf or NaN) gives the NaN byte 0xFF.
__device__ __forceinline__ uint32_t e8m0_from_amax(float amax) {
    uint32_t E = (__float_as_uint(amax) >> 23) & 0xffu;
    uint32_t s = E > 2u ? E - 2u : 0u;
    return E == 255u ? 255u : s;
}

// Eight values -> one dword of E2M1 codes.  The gfx950 convert divides its
// two inputs by the scale operand, whose exponent field carries the E8M0
// byte (1.0 * 2^(s-127)), rounds to nearest even with saturation and writes
// one byte (first input in the low nibble) into the byte lane `sel` of `old`.
__device__ __forceinline__ uint32_t pack8_fp4(const float *y, float scale) {
    uint32_t w = 0;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[0], y[1], scale, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2], y[3], scale, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[4], y[5], scale, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[6], y[7], scale, 3);
    return w;
}

// Quantize one 32-value block to 16 code bytes (4 dwords of 8 codes) and one
// scale byte.  Non-finite blocks store all-zero codes next to the 0xFF scale.
__device__ __forceinline__ void mxfp4_block(const float (&y)[32], u32x4 &codes,
                                            uint32_t &sbyte) {
    const float amax = block_amax(y);
    const uint32_t s = e8m0_from_amax(amax);
    const float scale = __uint_as_float(s << 23);
    uint32_t c[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) c[q] = pack8_fp4(&y[8 * q], scale);
    const bool nonfinite = (s == 255u);
    codes = u32x4{nonfinite ? 0u : c[0], nonfinite ? 0u : c[1], nonfinite ? 0u : c[2],
                  nonfinite ? 0u : c[3]};
    sbyte = s;
}

// MXFP4 decode of one block: 16 code bytes (4 dwords of 8 codes, element 0 in
// the low nibble) times 2^(s-127) by the gfx950 scaled convert; a NaN scale
// byte makes the whole block NaN.
__device__ __forceinline__ void mxfp4_decode(const u32x4 &c, uint32_t s, float (&z)[32]) {
    const float scale = __uint_as_float(s << 23);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const f32x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c[q], scale, 0);
        const f32x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c[q], scale, 1);
        const f32x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c[q], scale, 2);
        const f32x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c[q], scale, 3);
        z[8 * q + 0] = v0[0]; z[8 * q + 1] = v0[1];
        z[8 * q + 2] = v1[0]; z[8 * q + 3] = v1[1];
        z[8 * q + 4] = v2[0]; z[8 * q + 5] = v2[1];
        z[8 * q + 6] = v3[0]; z[8 * q + 7] = v3[1];
    }
    if (s == 255u) {
#pragma unroll
        for (int k = 0; k < 32; ++k) z[k] = __builtin_nanf("");
    }
}

// Orders the LDS accesses of one wave around a wave-level exchange: the
// lanes of a wave reach LDS in issue order, so a compiler barrier and
// wavefront-scope fences are all that is needed (no s_barrier).
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Wave-cooperative store of one 64-B unit per lane (w[0..16), bound for dst;
// dst == nullptr stores nothing).  Stored lane by lane, each of the four
// 16-B store instructions of a wave would write a quarter of each of 32
// cache lines (lanes 64 B apart), which halves HBM write throughput on
// gfx950 (28 MB of bf16 output: 13.5 us that way, 6.0 us whole-line).  So
// the units go through LDS first and store instruction c writes units
// 16c .. 16c+15 whole: lane L stores 16-B chunk L & 3 of unit 16c + L/4.
// Chunk k of unit u sits at slot 4u + (k ^ ((u >> 2) & 3)), which keeps the
// writes and the reads free of bank conflicts.  ROUNDS = 1 exchanges all 64
// units at once (4.5 KB of LDS per wave); ROUNDS = 2 or 4 exchange 32 or 16
// at a time through a buffer of 1/ROUNDS that size.  Every lane of the wave
// must make the call.
template <int ROUNDS>
struct WaveStoreBuf {
    u32x4 chunk[256 / ROUNDS];
    uint64_t addr[64 / ROUNDS];
};

template <int ROUNDS>
__device__ __forceinline__ void wave_store64(WaveStoreBuf<ROUNDS> &b, const uint32_t (&w)[16],
                                             void *dst) {
    constexpr int kUnits = 64 / ROUNDS;  // units per round
    const int L = threadIdx.x & 63;
    const int q = L & 3;
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
        const int ul = L - r * kUnits;  // this lane's unit within the round
        if (ROUNDS == 1 || (ul >= 0 && ul < kUnits)) {
            const int sw = (ul >> 2) & 3;
#pragma unroll
            for (int k = 0; k < 4; ++k)
                b.chunk[4 * ul + (k ^ sw)] = u32x4{w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]};
            b.addr[ul] = (uint64_t)(uintptr_t)dst;
        }
        wave_sync();
        // all reads first (kept ahead of the conditional stores, which the
        // compiler would otherwise sink them into, one LDS round trip each)
        u32x4 v[4 / ROUNDS];
        uint64_t a[4 / ROUNDS];
#pragma unroll
        for (int c = 0; c < 4 / ROUNDS; ++c) {
            const int u = 16 * c + (L >> 2);
            v[c] = b.chunk[4 * u + (q ^ ((u >> 2) & 3))];
            a[c] = b.addr[u];
        }
#pragma unroll
        for (int c = 0; c < 4 / ROUNDS; ++c) asm volatile("" : "+v"(v[c]), "+v"(a[c]));
#pragma unroll
        for (int c = 0; c < 4 / ROUNDS; ++c)
            if (a[c]) __builtin_nontemporal_store(v[c], reinterpret_cast<u32x4 *>((uintptr_t)a[c]) + q);
        if (ROUNDS > 1) wave_sync();
    }
}

}  // namespace kq

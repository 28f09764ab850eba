// kq_mfma.hip — the KroQuant quantizer with the block transform as a dense
// 32x32 product on the gfx950 matrix cores (the formulation of the KroQuant
// summary, "Approach": one matrix-core GEMM per block), for comparison with
// the register butterfly of kq_quant.hip.
//
// Per wave: one 32-channel block j and a few 32-token tiles.  The transposed
// product Y^T = T_j^T X^T runs as v_mfma_f32_32x32x16_bf16 with
//   A = T_j^T (32 outputs x 32 inputs), B = X^T (32 inputs x 32 tokens),
// so lane l's B operand (token l%32, input channels 8*(l/32)+16c .. +7) is one
// 16-byte load of the bf16 activation, used as is.  T_j is materialised in
// fp32 from its five factors and split into three bf16 terms hi + mid + lo
// (24 significand bits), so 6 MFMAs per tile give an fp32-accurate product
// with fp32 accumulation.  The order of the fp32 sums is the hardware's, so
// this arm matches the exact definition within rounding, not the butterfly's
// fixed order.  In the accumulator lane l holds token l%32's outputs
// k = 8*(r/4) + 4*(l/32) + r%4, r = 0..15; lanes l and l^32 share a token.
//
// Workgroups: 8 waves on 8 consecutive blocks and the same NT token tiles, so
// one workgroup reads 512 contiguous bytes per row; each wave builds its
// block's A fragments once and reuses them for its NT tiles.  The waves leave
// their code and scale bytes in LDS, and after one barrier the workgroup
// writes each row's 128 bytes of codes with 8 lanes x 16 bytes and its 8
// scale bytes with one 8-byte store: scattered 8-byte and 1-byte stores from
// the accumulator layout cost more than the whole read stream.  The
// workgroup index is mapped so that all block groups of a tile range run on
// the same XCD (workgroups go to the 8 XCDs round-robin), so the 8-byte scale
// pieces of a row meet in one L2.

#include <stdint.h>
#include <stdlib.h>

#include <hip/hip_runtime.h>

#include "kq.h"
#include "kq_device.h"
#include "kq_host.h"

namespace kq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kMfmaWaves = 8;
constexpr int kMfmaThreads = 64 * kMfmaWaves;
constexpr int kXcds = 8;

// Value of lane l^32's v in every lane (v_permlane32_swap exchanges the
// upper half of its first operand with the lower half of its second).
__device__ __forceinline__ uint32_t swap_halves(uint32_t v, int h) {
    auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return h ? r[0] : r[1];
}

// Three-term bf16 split of an fp32 value: t = hi + mid + lo to 24 bits.
__device__ __forceinline__ void split3(float t0, float t1, uint32_t &hi, uint32_t &mid, uint32_t &lo) {
    bf16x2 h = __builtin_convertvector(f32x2{t0, t1}, bf16x2);
    f32x2 hf = __builtin_convertvector(h, f32x2);
    const float r0 = t0 - hf[0], r1 = t1 - hf[1];  // exact
    bf16x2 m = __builtin_convertvector(f32x2{r0, r1}, bf16x2);
    f32x2 mf = __builtin_convertvector(m, f32x2);
    bf16x2 l = __builtin_convertvector(f32x2{r0 - mf[0], r1 - mf[1]}, bf16x2);
    hi = __builtin_bit_cast(uint32_t, h);
    mid = __builtin_bit_cast(uint32_t, m);
    lo = __builtin_bit_cast(uint32_t, l);
}

template <int NT>
__global__ __launch_bounds__(kMfmaThreads) void kron_mfma_kernel(
    const uint16_t *__restrict__ x, int64_t ld, const float *__restrict__ lu,
    uint8_t *__restrict__ codes, uint8_t *__restrict__ scales, int tokens, int nb, int tiles,
    int nranges, int ngroups) {
    // Workgroup -> (tile range, block group); every block group of a tile
    // range on the same XCD.
    const int b = blockIdx.x;
    const int slot = b / kXcds;
    const int grp = slot % ngroups;
    const int range = (slot / ngroups) * kXcds + b % kXcds;
    if (range >= nranges) return;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // Waves past the last block stay for the barrier and compute a copy of
    // the last block, which is never stored.
    const int jw = grp * kMfmaWaves + wave;
    const int j = jw < nb ? jw : nb - 1;
    const int lane = threadIdx.x & 63;
    const int h = lane >> 5, n = lane & 31;
    const int64_t d = (int64_t)nb * 32;

    // ---- all loads first: this wave's NT tiles, two 16-byte pieces each ----
    u32x4 xb[NT][2];
#pragma unroll
    for (int k = 0; k < NT; ++k) {
        int tile = range * NT + k;
        tile = tile < tiles ? tile : tiles - 1;
        int row = tile * 32 + n;
        row = row < tokens ? row : tokens - 1;
        const u32x4 *p = reinterpret_cast<const u32x4 *>(x + (int64_t)row * ld + (int64_t)j * 32 + 8 * h);
        xb[k][0] = p[0];  // input channels 8h .. 8h+7
        xb[k][1] = p[2];  // input channels 16 + 8h .. 16 + 8h + 7
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- A fragments: T_j^T[k_out = n][i], i = 16c + 8h + e, three terms ----
    // T[i][k] = prod_b F_b[bit b of i][bit b of k], F = [[u, v], [l*u, l*v + 1/u]].
    const float *p = lu + (int64_t)j * 15;
    float r0[5], r1[5];  // F_b[0][k_b], F_b[1][k_b] for this lane's output k = n
#pragma unroll
    for (int bb = 0; bb < 5; ++bb) {
        const float l_ = p[3 * bb], u = p[3 * bb + 1], v = p[3 * bb + 2];
        const float f00 = u, f01 = v, f10 = l_ * u, f11 = __builtin_fmaf(l_, v, rcp_rn(u));
        const bool kb = (n >> bb) & 1;
        r0[bb] = kb ? f01 : f00;
        r1[bb] = kb ? f11 : f10;
    }
    float q01[4] = {r0[0] * r0[1], r1[0] * r0[1], r0[0] * r1[1], r1[0] * r1[1]};
    const float f3 = h ? r1[3] : r0[3];
    uint32_t A[3][2][4];  // [term][chunk][bf16 pair]
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const float f4 = c ? r1[4] : r0[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const float t0 = q01[e & 3] * ((e & 4) ? r1[2] : r0[2]) * f3 * f4;
            const float t1 = q01[(e + 1) & 3] * (((e + 1) & 4) ? r1[2] : r0[2]) * f3 * f4;
            split3(t0, t1, A[0][c][e / 2], A[1][c][e / 2], A[2][c][e / 2]);
        }
    }

    // Staged outputs: codes [NT][32 rows][136 B] (128 B + pad: 34-dword row
    // stride keeps the 8-byte writes of 32 rows on distinct banks), scales
    // [NT][32][8].
    __shared__ uint64_t lds_codes[NT][32][17];
    __shared__ uint64_t lds_scales[NT][32];
    uint8_t *lsc = reinterpret_cast<uint8_t *>(lds_scales);

    // ---- per tile: 6 MFMAs, then amax / scale / convert / stage ----
#pragma unroll
    for (int k = 0; k < NT; ++k) {
        f32x16 acc = {};
#pragma unroll
        for (int term = 2; term >= 0; --term)  // smallest terms first
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const u32x4 av = {A[term][c][0], A[term][c][1], A[term][c][2], A[term][c][3]};
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                              __builtin_bit_cast(bf16x8, xb[k][c]),
                                                              acc, 0, 0, 0);
            }
        float y[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) y[r] = acc[r];
        float m = __builtin_elementwise_maximum(__builtin_fabsf(y[0]), __builtin_fabsf(y[1]));
#pragma unroll
        for (int r = 2; r < 16; r += 2)
            m = __builtin_elementwise_maximum(__builtin_elementwise_maximum(m, __builtin_fabsf(y[r])),
                                              __builtin_fabsf(y[r + 1]));
        const float mo = __uint_as_float(swap_halves(__float_as_uint(m), h));
        const float amax = __builtin_elementwise_maximum(m, mo);
        const uint32_t s = e8m0_from_amax(amax);
        const float scale = __uint_as_float(s << 23);
        const uint32_t P = pack8_fp4(&y[0], scale);  // code bytes 4a+2h, 4a+2h+1, a = 0, 1
        const uint32_t Q = pack8_fp4(&y[8], scale);  // a = 2, 3
        const uint32_t R = swap_halves(h ? P : Q, h);
        const uint32_t mine = h ? Q : P;
        const uint32_t lo = h ? R : mine, hi = h ? mine : R;
        uint32_t d0 = (lo & 0xffffu) | (hi << 16);
        uint32_t d1 = (lo >> 16) | (hi & 0xffff0000u);
        if (s == 255u) d0 = d1 = 0u;
        lds_codes[k][n][2 * wave + h] = (uint64_t)d0 | ((uint64_t)d1 << 32);
        if (h == 0) lsc[(k * 32 + n) * 8 + wave] = (uint8_t)s;
    }
    __syncthreads();

    // ---- cooperative stores: 16 B per lane, 8 lanes per 128-byte row ----
    const int nblk = nb - grp * kMfmaWaves < kMfmaWaves ? nb - grp * kMfmaWaves : kMfmaWaves;
    for (int c = threadIdx.x; c < NT * 32 * 8; c += kMfmaThreads) {
        const int k = c >> 8, r = (c >> 3) & 31, q = c & 7;
        if (q >= nblk) continue;
        int tile = range * NT + k;
        tile = tile < tiles ? tile : tiles - 1;
        int row = tile * 32 + r;
        row = row < tokens ? row : tokens - 1;
        const uint64_t a0 = lds_codes[k][r][2 * q], a1 = lds_codes[k][r][2 * q + 1];
        __builtin_nontemporal_store(
            u32x4{(uint32_t)a0, (uint32_t)(a0 >> 32), (uint32_t)a1, (uint32_t)(a1 >> 32)},
            reinterpret_cast<u32x4 *>(codes + (int64_t)row * (d / 2) + (int64_t)(grp * kMfmaWaves + q) * 16));
    }
    for (int c = threadIdx.x; c < NT * 32; c += kMfmaThreads) {
        const int k = c >> 5, r = c & 31;
        int tile = range * NT + k;
        tile = tile < tiles ? tile : tiles - 1;
        int row = tile * 32 + r;
        row = row < tokens ? row : tokens - 1;
        uint8_t *dst = scales + (int64_t)row * nb + grp * kMfmaWaves;
        if (nblk == kMfmaWaves && ((uintptr_t)dst & 7) == 0) {
            *reinterpret_cast<uint64_t *>(dst) = lds_scales[k][r];  // partial line: plain store
        } else {
            for (int q = 0; q < nblk; ++q) dst[q] = lsc[c * 8 + q];
        }
    }
}

// Token tiles per wave: each wave builds its block's A fragments once for
// its tiles.  One tile per wave (more waves, more setup) measured faster up
// to about a million units: 9.1 against 9.6 us on 4608 x 3072; two tiles
// faster beyond: 29.2 against 32.4 us on 4608 x 12288.
// Building with -DKQ_MFMA_TILES_PER_WAVE=1, 2, 4 or 8 overrides it for sweeps.
#ifndef KQ_MFMA_TILES_PER_WAVE
#define KQ_MFMA_TILES_PER_WAVE 0
#endif
static_assert(KQ_MFMA_TILES_PER_WAVE == 0 || KQ_MFMA_TILES_PER_WAVE == 1 ||
                  KQ_MFMA_TILES_PER_WAVE == 2 || KQ_MFMA_TILES_PER_WAVE == 4 ||
                  KQ_MFMA_TILES_PER_WAVE == 8,
              "KQ_MFMA_TILES_PER_WAVE must be 1, 2, 4 or 8");
static int mfma_tiles_per_wave(int64_t units) {
    if (KQ_MFMA_TILES_PER_WAVE) return KQ_MFMA_TILES_PER_WAVE;
    return units <= (int64_t(1) << 20) ? 1 : 2;
}

}  // namespace kq

using namespace kq;

extern "C" kq_status kq_transform_quant_mfma(const void *x, int64_t tokens, int64_t d,
                                             int64_t ld_x, const float *lu, uint8_t *codes,
                                             uint8_t *scales, void *stream) {
    if (tokens < 0 || tokens >= (int64_t(1) << 30)) return KQ_ERR_SHAPE;
    if (d <= 0 || d % 32 != 0 || d > (int64_t(1) << 26) || ld_x < d) return KQ_ERR_SHAPE;
    if (tokens == 0) return KQ_OK;
    if (!x || !lu || !codes || !scales) return KQ_ERR_NULL;
    if (((uintptr_t)x % 16) || (ld_x * 2) % 16 || ((uintptr_t)codes % 16) || ((uintptr_t)lu % 4))
        return KQ_ERR_ALIGN;
    const int nb = (int)(d / 32);
    const int tiles = (int)((tokens + 31) / 32);
    const int nt = mfma_tiles_per_wave(tokens * nb);
    const int nranges = (tiles + nt - 1) / nt;
    const int ngroups = (nb + kMfmaWaves - 1) / kMfmaWaves;
    const int64_t grid = (int64_t)((nranges + kXcds - 1) / kXcds) * kXcds * ngroups;
    if (grid > INT32_MAX) return KQ_ERR_SHAPE;
    const uint16_t *xp = (const uint16_t *)x;
    const int t = (int)tokens;
    void *args[] = {(void *)&xp, (void *)&ld_x, (void *)&lu, (void *)&codes, (void *)&scales,
                    (void *)&t, (void *)&nb, (void *)&tiles, (void *)&nranges, (void *)&ngroups};
    const void *fn = nt == 1 ? (const void *)kron_mfma_kernel<1>
                   : nt == 2 ? (const void *)kron_mfma_kernel<2>
                   : nt == 8 ? (const void *)kron_mfma_kernel<8>
                             : (const void *)kron_mfma_kernel<4>;
    hipError_t e = hipLaunchKernel(fn, dim3((unsigned)grid), dim3(kMfmaThreads), args, 0,
                                   (hipStream_t)stream);
    return e == hipSuccess ? KQ_OK : KQ_ERR_HIP;
}

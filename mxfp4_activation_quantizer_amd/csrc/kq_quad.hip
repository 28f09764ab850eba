// kq_quad.hip — the KroQuant quantizer with four lanes per unit and the two
// upper butterfly stages exchanged between lanes, kept as a measured
// alternative to the one-lane-per-unit kernel of kq_quant.hip.
//
// Lane L of a workgroup holds elements 8q .. 8q+7 (q = L & 3) of unit
// u = (workgroup's first unit) + L/4, so every 16-byte load of a wave reads
// 1 KB of contiguous input (16 whole units) and every 4-byte code store
// writes 256 contiguous bytes.  Bits 0..2 of the in-block index are in-lane;
// bits 3 and 4 pair lanes q and q^1, q and q^2 of a quad, exchanged with DPP
// quad permutations.  The arithmetic is the one fixed fp32 order of
// kq_transform_quant: for a cross-lane pair (p in the lane with the bit
// clear, q in its partner) the p lane forms r = fma(l, q, p) from its
// partner's q, then the q lane forms s = fma(w, r, q) from its partner's r,
// each half under its own exec mask, so codes and scales equal the
// one-lane kernel's bit for bit.  Each lane builds only its eight d_k.
//
// Cost: the per-unit constants are built by four lanes instead of one and
// each cross-lane stage takes two exchanges and two masked multiply-adds per
// element, so the VALU work per element is about twice the one-lane kernel's.

#include <stdint.h>

#include <hip/hip_runtime.h>

#include "kq.h"
#include "kq_device.h"

namespace kq {

constexpr int kQuadThreads = 256;  // 64 units per workgroup

// Lane l ^ 1 (CTRL 0xB1) or l ^ 2 (CTRL 0x4E) of the lane's quad.
template <int CTRL>
__device__ __forceinline__ float quad_xchg(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL,
                                                                0xf, 0xf, true));
}

// One cross-lane shear stage over the lane's eight values: the lanes with
// the stage's bit clear hold p and form r = fma(l, q, p); their partners then
// form s = fma(w, r, q).  The exchanges run with every lane active.
template <int CTRL>
__device__ __forceinline__ void cross_stage(float (&z)[8], bool hi, float l, float w) {
    float o[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) o[m] = quad_xchg<CTRL>(z[m]);
    if (!hi) {
#pragma unroll
        for (int m = 0; m < 8; ++m) z[m] = __builtin_fmaf(l, o[m], z[m]);
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) o[m] = quad_xchg<CTRL>(z[m]);
    if (hi) {
#pragma unroll
        for (int m = 0; m < 8; ++m) z[m] = __builtin_fmaf(w, o[m], z[m]);
    }
}

__global__ __launch_bounds__(kQuadThreads) void kron_quad_kernel(
    const uint16_t *__restrict__ x, int64_t ld, const float *__restrict__ lu,
    uint8_t *__restrict__ codes, uint8_t *__restrict__ scales, int tokens, int nb,
    DivMagic nbm) {
    const int q = threadIdx.x & 3;
    const int u = (int)(((int64_t)blockIdx.x * kQuadThreads + threadIdx.x) >> 2);
    const int t = (int)udiv31((uint32_t)u, nbm);
    // a quad is wholly in or out
    if (t >= tokens) return;
    const int j = u - t * nb;
    const float *pp = lu + (int64_t)j * 15;
    float p[15];
#pragma unroll
    for (int i = 0; i < 15; ++i) p[i] = pp[i];
    const u32x4 raw = *reinterpret_cast<const u32x4 *>(x + (int64_t)t * ld + (int64_t)j * 32 + 8 * q);
    __builtin_amdgcn_sched_barrier(0);
    float l[5], w[5], uu[5], iu[5];
#pragma unroll
    for (int b = 0; b < 5; ++b) {
        l[b] = p[3 * b];
        uu[b] = p[3 * b + 1];
        w[b] = uu[b] * p[3 * b + 2];
    }
    rcp5_rn(uu, iu);
    // d_k for k = 8q + m: the left-to-right product over b = 0..4
    float dk[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) dk[m] = (m & 1) ? iu[0] : uu[0];
#pragma unroll
    for (int b = 1; b < 3; ++b)
#pragma unroll
        for (int m = 0; m < 8; ++m) dk[m] = dk[m] * (((m >> b) & 1) ? iu[b] : uu[b]);
    const float a3 = (q & 1) ? iu[3] : uu[3];
    const float a4 = (q & 2) ? iu[4] : uu[4];
#pragma unroll
    for (int m = 0; m < 8; ++m) dk[m] = dk[m] * a3;
#pragma unroll
    for (int m = 0; m < 8; ++m) dk[m] = dk[m] * a4;

    float z[8];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        z[2 * c] = bf16_lo(raw[c]);
        z[2 * c + 1] = bf16_hi(raw[c]);
    }
#pragma unroll
    for (int b = 0; b < 3; ++b) {
        const int h = 1 << b;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (i & h) continue;
            const float r = __builtin_fmaf(l[b], z[i | h], z[i]);
            const float s = __builtin_fmaf(w[b], r, z[i | h]);
            z[i] = r;
            z[i | h] = s;
        }
    }
    cross_stage<0xB1>(z, (q & 1) != 0, l[3], w[3]);
    cross_stage<0x4E>(z, (q & 2) != 0, l[4], w[4]);
#pragma unroll
    for (int m = 0; m < 8; ++m) z[m] = z[m] * dk[m];

    // block amax: in-lane, then across the quad (NaN-propagating maximum)
    float a = __builtin_elementwise_maximum(__builtin_fabsf(z[0]), __builtin_fabsf(z[1]));
#pragma unroll
    for (int m = 2; m < 8; m += 2)
        a = __builtin_elementwise_maximum(
            __builtin_elementwise_maximum(a, __builtin_fabsf(z[m])), __builtin_fabsf(z[m + 1]));
    a = __builtin_elementwise_maximum(a, quad_xchg<0xB1>(a));
    a = __builtin_elementwise_maximum(a, quad_xchg<0x4E>(a));
    const uint32_t s = e8m0_from_amax(a);
    uint32_t cw = pack8_fp4(z, __uint_as_float(s << 23));
    if (s == 255u) cw = 0;
    const int64_t unit = (int64_t)t * nb + j;
    __builtin_nontemporal_store(cw, reinterpret_cast<uint32_t *>(codes) + unit * 4 + q);
    if (q == 0) __builtin_nontemporal_store((uint8_t)s, scales + unit);
}

}  // namespace kq

using namespace kq;

extern "C" kq_status kq_transform_quant_quad(const void *x, int64_t tokens, int64_t d,
                                             int64_t ld_x, const float *lu, uint8_t *codes,
                                             uint8_t *scales, void *stream) {
    if (tokens < 0 || tokens >= (int64_t(1) << 30)) return KQ_ERR_SHAPE;
    if (d <= 0 || d % 32 != 0 || d > (int64_t(1) << 26) || ld_x < d) return KQ_ERR_SHAPE;
    if (tokens == 0) return KQ_OK;
    if (!x || !lu || !codes || !scales) return KQ_ERR_NULL;
    if (((uintptr_t)x % 16) || (ld_x * 2) % 16 || ((uintptr_t)codes % 16) || ((uintptr_t)lu % 4))
        return KQ_ERR_ALIGN;
    const int64_t nb = d / 32;
    const int64_t units = tokens * nb;
    // unit indices stay below 2^31 (the index arithmetic is 32-bit)
    if (units >= (int64_t(1) << 31) - kQuadThreads) return KQ_ERR_SHAPE;
    const int grid = (int)((units * 4 + kQuadThreads - 1) / kQuadThreads);
    const uint16_t *xp = (const uint16_t *)x;
    const int t = (int)tokens, n = (int)nb;
    const DivMagic nbm = div_magic((uint32_t)nb);
    void *args[] = {(void *)&xp, (void *)&ld_x, (void *)&lu, (void *)&codes, (void *)&scales,
                    (void *)&t, (void *)&n, (void *)&nbm};
    hipError_t e = hipLaunchKernel((const void *)kron_quad_kernel, dim3(grid), dim3(kQuadThreads),
                                   args, 0, (hipStream_t)stream);
    return e == hipSuccess ? KQ_OK : KQ_ERR_HIP;
}

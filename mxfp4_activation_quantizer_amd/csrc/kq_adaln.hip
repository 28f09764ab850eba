// kq_adaln.hip — the quantizer fused with the adaptive LayerNorm that feeds
// it in a diffusion-transformer block (KroQuant summary, "Problem": AdaLN is
// why the transform cannot be folded into the previous layer and has to run
// online).  One pass over the activation:
//   h = LN(x) * (1 + scale_s) + shift_s,  y = h T_j per 32-channel block,
//   MXFP4(y),
// so the modulated tensor never goes to memory.  kq_adaln_modulate is the
// same pass with a bf16 h output instead of the transform and quantizer (the
// first half of the unfused two-kernel pipeline).
//
// Work decomposition.  A workgroup owns ROWS = G * U whole rows of one
// sample: thread i handles block j = i mod nb of rows U*(i / nb) ..
// U*(i / nb) + U - 1 (U = 1 by default).
// The sample's modulation vectors (1 + scale and shift, fp32) are staged in
// LDS.  The row statistics use a fixed order, so the result is reproducible
// bit for bit:
//   block partial   sequential sum over the block's 32 values;
//   row total       wave-wide: lane l starts from partial l (0 past nb) and
//                   adds partials l + 64, l + 128, ...; then for m = 1, 2, 4,
//                   8, 16, 32 each lane adds lane l ^ m's value (DPP moves
//                   and lane reads; every wave reduces the rows it needs, so
//                   a launch has two workgroup barriers);
//   mean = total / d; c = x - mean;
//   block partial   fma(c_31, c_31, ... fma(c_0, c_0, 0));
//   var = total / d; rstd = 1 / sqrt(var + eps) (correctly rounded steps);
//   h = fma(c * rstd, 1 + scale, shift).
// Two-pass variance: the centered values stay in registers between passes.

#include <stdint.h>
#include <stdlib.h>

#include <hip/hip_runtime.h>

#include "kq.h"
#include "kq_device.h"
#include "kq_host.h"
#include "kq_kron.h"

namespace kq {

constexpr int kAdalnMaxD = 8192;  // the modulation vectors of one sample live in LDS
                                  // (and d/32 <= 256 fits one 512-thread workgroup)

struct AdalnArgs {
    const uint16_t *x;
    int64_t ld;
    const float *shift, *scale;  // [samples][d]
    int64_t rps;                 // rows per sample
    float eps;
    const float *lu;             // [nb][5][3] (quantizing variant)
    uint8_t *codes, *scales;     // quantizing variant
    uint16_t *h;                 // bf16 output (modulate variant)
    int64_t ldh;
    int64_t tokens;
    int d, nb, G, wps;           // row groups per workgroup, workgroups per sample
    DivMagic nbm;                // division by nb
};

// Sum over the 64 lanes of a wave in the exchange order m = 1, 2, 4, 8, 16,
// 32 (each lane adds lane l ^ m's value).  Steps 1 and 2 are quad
// permutations; after them the four lanes of a quad agree, so the mirror
// within eight lanes (lane 7 - i) supplies lane i ^ 4's value, and after that
// the mirror within sixteen lanes supplies lane i ^ 8's.  The last two steps
// combine the four row values (lanes 0, 16, 32, 48) as (R0 + R1) + (R2 + R3),
// which is what every lane holds after the exchanges with l ^ 16 and l ^ 32.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float a) {
    const int t = __builtin_amdgcn_update_dpp(0, __float_as_int(a), CTRL, 0xF, 0xF, false);
    return a + __int_as_float(t);
}

__device__ __forceinline__ float wave_total(float a) {
    a = dpp_add<0xB1>(a);   // quad_perm [1,0,3,2]: lane l ^ 1
    a = dpp_add<0x4E>(a);   // quad_perm [2,3,0,1]: lane l ^ 2
    a = dpp_add<0x141>(a);  // row_half_mirror
    a = dpp_add<0x140>(a);  // row_mirror
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 48));
    return (r0 + r1) + (r2 + r3);
}

// Row totals of the block partials part[r][0..nb) for the rows this lane
// owns (rows g*U .. g*U + U - 1).  Each wave reduces every row any of its
// lanes needs (all 64 lanes take part; the loops are wave-uniform), so no
// wave waits for another.
template <int U>
__device__ __forceinline__ void own_row_totals(const float *part, int nb, DivMagic nbm, int G, int g,
                                               int nrows, float (&tot)[U]) {
    const int lane = threadIdx.x & 63;
    const uint32_t base = __builtin_amdgcn_readfirstlane(threadIdx.x & ~63);
    const int g_lo = (int)udiv31(base, nbm), g_top = (int)udiv31(base + 63, nbm);
    const int g_hi = g_top < G - 1 ? g_top : G - 1;
#pragma unroll
    for (int k = 0; k < U; ++k) tot[k] = 0.0f;
    for (int gg = g_lo; gg <= g_hi; ++gg) {
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int r = gg * U + k;
            if (r >= nrows) break;
            const float *pr = part + r * nb;
            float v = lane < nb ? pr[lane] : 0.0f;
            for (int jj = lane + 64; jj < nb; jj += 64) v = v + pr[jj];
            const float t = wave_total(v);
            if (gg == g) tot[k] = t;
        }
    }
}

// bf16 form: the wave exchange runs in four rounds of 16 units (1.1 KB of LDS
// per wave next to the sample vectors; one round of 64 measured slower).
constexpr int kModRounds = 4;

template <int U, bool QUANT>
__global__ __launch_bounds__(512) void adaln_kernel(AdalnArgs a) {
    extern __shared__ float lds[];
    const int d = a.d, nb = a.nb, ROWS = a.G * U;
    float *onep = lds;                  // [d] 1 + scale (chunks placed by vec_chunk)
    float *shv = lds + d;               // [d] shift (chunks placed by vec_chunk)
    float *part = lds + 2 * d;          // [ROWS][nb] block sums
    float *part2 = part + ROWS * nb;    // [ROWS][nb] block sums of squares

    const int s = blockIdx.x / a.wps, w = blockIdx.x - s * a.wps;
    const int64_t row0 = (int64_t)s * a.rps + (int64_t)w * ROWS;
    int64_t rend = (int64_t)(s + 1) * a.rps;
    if (rend > a.tokens) rend = a.tokens;
    if (row0 >= rend) return;  // whole workgroup
    const int nrows = rend - row0 < ROWS ? (int)(rend - row0) : ROWS;

    const int tid = threadIdx.x;
    const int g = (int)udiv31((uint32_t)tid, a.nbm), j = tid - g * nb;
    const bool act = g < a.G;

    // ---- parameters, then this thread's U units, then the sample vectors ----
    KronStage ks = KronStage::from(a.lu);
    if (QUANT) ks.fetch(j);
    u32x4 raw[U][4];
#pragma unroll
    for (int k = 0; k < U; ++k) {
        const int r = g * U + k;
        const int64_t row = row0 + (act && r < nrows ? r : 0);
        const u32x4 *p = reinterpret_cast<const u32x4 *>(a.x + row * a.ld + (int64_t)j * 32);
#pragma unroll
        for (int i = 0; i < 4; ++i) raw[k][i] = p[i];
    }
    {
        const f32x4 *sc4 = reinterpret_cast<const f32x4 *>(a.scale + (int64_t)s * d);
        const f32x4 *sh4 = reinterpret_cast<const f32x4 *>(a.shift + (int64_t)s * d);
        for (int i = tid; i < d / 4; i += blockDim.x) {
            const f32x4 c = sc4[i], b = sh4[i];
            const int at = vec_chunk(i >> 3, i & 7);
            reinterpret_cast<f32x4 *>(onep)[at] = f32x4{1.0f + c[0], 1.0f + c[1], 1.0f + c[2], 1.0f + c[3]};
            reinterpret_cast<f32x4 *>(shv)[at] = b;
        }
    }

    // ---- pass 1: block sums -> row means ----
    float z[U][32];
#pragma unroll
    for (int k = 0; k < U; ++k) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                z[k][8 * i + 2 * c] = bf16_lo(raw[k][i][c]);
                z[k][8 * i + 2 * c + 1] = bf16_hi(raw[k][i][c]);
            }
        float acc = z[k][0];
#pragma unroll
        for (int e = 1; e < 32; ++e) acc = acc + z[k][e];
        const int r = g * U + k;
        if (act && r < nrows) part[r * nb + j] = acc;
    }
    __syncthreads();
    float mu[U];
    own_row_totals<U>(part, nb, a.nbm, a.G, g, nrows, mu);

    // ---- pass 2: centered sums of squares -> 1/sqrt(var + eps) ----
#pragma unroll
    for (int k = 0; k < U; ++k) {
        const int r = g * U + k;
        const float m = mu[k] / (float)d;
        float q = 0.0f;
#pragma unroll
        for (int e = 0; e < 32; ++e) {
            z[k][e] = z[k][e] - m;
            q = __builtin_fmaf(z[k][e], z[k][e], q);
        }
        if (act && r < nrows) part2[r * nb + j] = q;
    }
    __syncthreads();
    float rs[U];
    own_row_totals<U>(part2, nb, a.nbm, a.G, g, nrows, rs);
#pragma unroll
    for (int k = 0; k < U; ++k) rs[k] = 1.0f / __builtin_sqrtf(rs[k] / (float)d + a.eps);

    // ---- modulate, then transform + quantize (or store bf16 h) ----
    // The bf16 form stores through the wave exchange, so every lane of a
    // wave stays to the end (lanes without a row store nothing).
    if (QUANT && !act) return;
    if (QUANT) ks.setup();
    const f32x4 *op4 = reinterpret_cast<const f32x4 *>(onep);
    const f32x4 *sv4 = reinterpret_cast<const f32x4 *>(shv);
#pragma unroll
    for (int k = 0; k < U; ++k) {
        const int r = g * U + k;
        if (QUANT && r >= nrows) break;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const f32x4 o = op4[vec_chunk(j, i)], b = sv4[vec_chunk(j, i)];
#pragma unroll
            for (int e = 0; e < 4; ++e) z[k][4 * i + e] = __builtin_fmaf(z[k][4 * i + e] * rs[k], o[e], b[e]);
        }
        const int64_t row = row0 + r;
        if (QUANT) {
            ks.apply(z[k]);
            u32x4 c;
            uint32_t sb;
            mxfp4_block(z[k], c, sb);
            const int64_t unit = row * nb + j;
            __builtin_nontemporal_store(c, reinterpret_cast<u32x4 *>(a.codes) + unit);
            __builtin_nontemporal_store((uint8_t)sb, a.scales + unit);
        } else {
            __shared__ WaveStoreBuf<kModRounds> wsb[512 / 64];
            uint32_t hw[16];
#pragma unroll
            for (int m = 0; m < 16; ++m)
                hw[m] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{z[k][2 * m], z[k][2 * m + 1]}, bf16x2));
            const bool valid = act && r < nrows;
            wave_store64(wsb[tid >> 6], hw, valid ? (void *)(a.h + row * a.ldh + (int64_t)j * 32) : nullptr);
        }
    }
}

// Rows per thread: 1 by default.  Two or four rows share the constant setup
// but hold two or four blocks of centered values in registers (occupancy 3
// or 2 instead of 7); on 4608 x 3072 one row per thread in workgroups of
// about 384 threads measured fastest (17.0 us against 20.0 and 25.5 us).
// Building with -DKQ_ADALN_ROWS_PER_THREAD=2 or 4 overrides it for sweeps.
#ifndef KQ_ADALN_ROWS_PER_THREAD
#define KQ_ADALN_ROWS_PER_THREAD 1
#endif
static_assert(KQ_ADALN_ROWS_PER_THREAD == 1 || KQ_ADALN_ROWS_PER_THREAD == 2 ||
                  KQ_ADALN_ROWS_PER_THREAD == 4,
              "KQ_ADALN_ROWS_PER_THREAD must be 1, 2 or 4");
static int adaln_rows_per_thread() { return KQ_ADALN_ROWS_PER_THREAD; }

// Row groups per workgroup: among G with G * nb <= 512 threads, the one whose
// G * nb threads fill whole waves best; ties go to the G whose workgroup is
// closest to KQ_ADALN_THREADS threads (384 unless a sweep build sets it with
// -DKQ_ADALN_THREADS=64..512).
#ifndef KQ_ADALN_THREADS
#define KQ_ADALN_THREADS 384
#endif
static_assert(KQ_ADALN_THREADS >= 64 && KQ_ADALN_THREADS <= 512, "KQ_ADALN_THREADS out of range");
static int adaln_groups(int nb) {
    const int target = KQ_ADALN_THREADS;
    int best = 1;
    double best_util = -1.0;
    int best_dist = 1 << 30;
    for (int G = 1; G * nb <= 512; ++G) {
        const int th = (G * nb + 63) / 64 * 64;
        const double util = (double)(G * nb) / th;
        const int dist = th > target ? th - target : target - th;
        if (util > best_util + 1e-9 || (util > best_util - 1e-9 && dist < best_dist)) {
            best_util = util;
            best_dist = dist;
            best = G;
        }
    }
    return best;
}

template <int U, bool QUANT>
static kq_status launch_adaln(AdalnArgs a, void *stream) {
    const int ROWS = a.G * U;
    const int threads = (a.G * a.nb + 63) / 64 * 64;
    const int64_t span = a.rps < a.tokens ? a.rps : a.tokens;
    const int64_t wps = (span + ROWS - 1) / ROWS;
    const int64_t samples = (a.tokens + a.rps - 1) / a.rps;
    if (wps > INT32_MAX || samples * wps > INT32_MAX) return KQ_ERR_SHAPE;
    a.wps = (int)wps;
    const size_t lds = sizeof(float) * (2 * (size_t)a.d + 2 * (size_t)ROWS * a.nb);
    auto kern = adaln_kernel<U, QUANT>;
    static DeviceOnce attr_set;  // the attribute is per device
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return KQ_ERR_HIP;
    if (!attr_set.done(dev)) {
        if (hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                96 * 1024) != hipSuccess)
            return KQ_ERR_HIP;
        attr_set.set(dev);
    }
    void *argv[] = {(void *)&a};
    const hipError_t e = hipLaunchKernel((const void *)kern, dim3((unsigned)(samples * wps)),
                                         dim3(threads), argv, lds, (hipStream_t)stream);
    return e == hipSuccess ? KQ_OK : KQ_ERR_HIP;
}

template <bool QUANT>
static kq_status run_adaln(AdalnArgs a, void *stream) {
    a.G = adaln_groups(a.nb);
    a.nbm = div_magic((uint32_t)a.nb);
    switch (adaln_rows_per_thread()) {
        case 1: return launch_adaln<1, QUANT>(a, stream);
        case 4: return launch_adaln<4, QUANT>(a, stream);
        default: return launch_adaln<2, QUANT>(a, stream);
    }
}

static kq_status check_adaln(const void *x, int64_t tokens, int64_t d, int64_t ld_x,
                             const float *shift, const float *scale, int64_t rps, float eps) {
    if (tokens < 0 || tokens >= (int64_t(1) << 30)) return KQ_ERR_SHAPE;
    if (d <= 0 || d % 32 != 0 || d > kAdalnMaxD || ld_x < d) return KQ_ERR_SHAPE;
    if (rps < 1 || !(eps >= 0.0f) || eps > 3.0e38f) return KQ_ERR_SHAPE;
    if (tokens == 0) return KQ_OK;
    if (!x || !shift || !scale) return KQ_ERR_NULL;
    if (((uintptr_t)x % 16) || (ld_x * 2) % 16 || ((uintptr_t)shift % 16) || ((uintptr_t)scale % 16))
        return KQ_ERR_ALIGN;
    return KQ_OK;
}

}  // namespace kq

using namespace kq;

extern "C" {

kq_status kq_adaln_transform_quant(const void *x, int64_t tokens, int64_t d, int64_t ld_x,
                                   const float *shift, const float *scale, int64_t rows_per_sample,
                                   float eps, const float *lu, uint8_t *codes, uint8_t *scales,
                                   void *stream) {
    kq_status st = check_adaln(x, tokens, d, ld_x, shift, scale, rows_per_sample, eps);
    if (st != KQ_OK || tokens == 0) return st;
    if (!lu || !codes || !scales) return KQ_ERR_NULL;
    if (((uintptr_t)lu % 4) || ((uintptr_t)codes % 16)) return KQ_ERR_ALIGN;
    AdalnArgs a{(const uint16_t *)x, ld_x, shift, scale, rows_per_sample, eps, lu, codes, scales,
                nullptr, 0, tokens, (int)d, (int)(d / 32), 0, 0};
    return run_adaln<true>(a, stream);
}

kq_status kq_adaln_modulate(const void *x, int64_t tokens, int64_t d, int64_t ld_x,
                            const float *shift, const float *scale, int64_t rows_per_sample,
                            float eps, void *h, int64_t ld_h, void *stream) {
    kq_status st = check_adaln(x, tokens, d, ld_x, shift, scale, rows_per_sample, eps);
    if (st != KQ_OK || tokens == 0) return st;
    if (!h) return KQ_ERR_NULL;
    if (ld_h < d) return KQ_ERR_SHAPE;
    if (((uintptr_t)h % 16) || (ld_h * 2) % 16) return KQ_ERR_ALIGN;
    AdalnArgs a{(const uint16_t *)x, ld_x, shift, scale, rows_per_sample, eps, nullptr, nullptr,
                nullptr, (uint16_t *)h, ld_h, tokens, (int)d, (int)(d / 32), 0, 0};
    return run_adaln<false>(a, stream);
}

}  // extern "C"

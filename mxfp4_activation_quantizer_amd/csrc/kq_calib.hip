// kq_calib.hip — calibration of the block parameters (KroQuant summary,
// "Approach": the five factors of every block are learned layer-wise from the
// Hadamard start with an output loss).
//
// Objective of block j over a calibration set of tokens:
//   f_j = sum_t r_t G_j r_t^T,  r_t = dequant(MXFP4(x_t T_j)) T_j^-1 - x_t,
// with G_j = I (the quantizer's round-trip error) or the block's weight Gram
// W_j^T W_j (the block-diagonal part of the output error of X W^T).  The
// objective is separable over blocks, so one launch scores a candidate
// parameter set for every block at once, and the per-block (1+1) evolution
// strategy (kq_calib_es_update) keeps or rejects each block's candidate on its
// own.  The strategy sees the true quantized objective; no gradient through
// the rounding is needed.
//
// kq_calib_objective: one workgroup per block.  Each thread takes tokens
// tid, tid + 256, ...: forward transform (the quantizer's fixed fp32 order),
// MXFP4 quantize and decode, inverse transform, residual, weighted square;
// per-thread sums in fp32, then a fixed-order reduction (wave exchange tree,
// then the four wave totals in order), so repeated calls give identical
// values and an unchanged candidate never counts as an improvement.

#include <stdint.h>
#include <stdlib.h>

#include <hip/hip_runtime.h>

#include "kq.h"
#include "kq_device.h"
#include "kq_kron.h"

namespace kq {

constexpr int kCalThreads = 256;

__device__ __forceinline__ float cal_wave_sum(float a) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) a = a + __shfl_xor(a, m, 64);
    return a;
}

__global__ __launch_bounds__(kCalThreads) void calib_objective_kernel(
    const uint16_t *__restrict__ x, int64_t ld, int64_t tokens, const float *__restrict__ lu,
    const float *__restrict__ gram, float *__restrict__ f) {
    __shared__ float G[32 * 32];
    __shared__ float wsum[kCalThreads / 64];
    const int j = blockIdx.x, tid = threadIdx.x;
    if (gram) {
        for (int i = tid; i < 1024; i += kCalThreads) G[i] = gram[(int64_t)j * 1024 + i];
    }
    KronStage fw = KronStage::from(lu);
    KronInverseStage iv = KronInverseStage::from(lu);
    fw.fetch(j);
    iv.fetch(j);
    fw.setup();
    iv.setup();
    __syncthreads();

    float acc = 0.0f;
    for (int64_t t = tid; t < tokens; t += kCalThreads) {
        const u32x4 *p = reinterpret_cast<const u32x4 *>(x + t * ld + (int64_t)j * 32);
        float xv[32], z[32];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u32x4 v = p[i];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                xv[8 * i + 2 * c] = bf16_lo(v[c]);
                xv[8 * i + 2 * c + 1] = bf16_hi(v[c]);
            }
        }
#pragma unroll
        for (int k = 0; k < 32; ++k) z[k] = xv[k];
        fw.apply(z);
        u32x4 codes;
        uint32_t sb;
        mxfp4_block(z, codes, sb);
        mxfp4_decode(codes, sb, z);
        iv.apply(z);
#pragma unroll
        for (int k = 0; k < 32; ++k) z[k] = z[k] - xv[k];
        float e = 0.0f;
        if (gram) {
            for (int a = 0; a < 32; ++a) {
                float ga = 0.0f;
#pragma unroll
                for (int b = 0; b < 32; ++b) ga = __builtin_fmaf(G[a * 32 + b], z[b], ga);
                e = __builtin_fmaf(z[a], ga, e);
            }
        } else {
#pragma unroll
            for (int k = 0; k < 32; ++k) e = __builtin_fmaf(z[k], z[k], e);
        }
        acc = acc + e;
    }
    acc = cal_wave_sum(acc);
    if ((tid & 63) == 0) wsum[tid >> 6] = acc;
    __syncthreads();
    if (tid == 0) {
        float s = wsum[0];
#pragma unroll
        for (int w = 1; w < kCalThreads / 64; ++w) s = s + wsum[w];
        f[j] = s;
    }
}

// One (1+1)-ES step per block, in this fp32 order: accept the evaluated
// candidate if it is strictly better (sigma * 1.5, at most 0.5), otherwise
// sigma * 0.90360200 (1.5^-1/4, at least 1e-4), so that one success in five
// keeps sigma fixed; then the next candidate fma(sigma, noise, theta), kept
// at theta when any u would come within 0.1 of zero.
__global__ void calib_es_update_kernel(int nb, float *__restrict__ theta, float *__restrict__ sigma,
                                       float *__restrict__ fbest, float *__restrict__ cand,
                                       const float *__restrict__ fcand,
                                       const float *__restrict__ noise) {
    const int j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= nb) return;
    float *th = theta + (int64_t)j * 15, *cd = cand + (int64_t)j * 15;
    const float *nz = noise + (int64_t)j * 15;
    float s = sigma[j];
    if (fcand[j] < fbest[j]) {
#pragma unroll
        for (int i = 0; i < 15; ++i) th[i] = cd[i];
        fbest[j] = fcand[j];
        s = s * 1.5f;
        s = s < 0.5f ? s : 0.5f;
    } else {
        s = s * 0.90360200f;
        s = s > 1e-4f ? s : 1e-4f;
    }
    sigma[j] = s;
    float c[15];
    bool ok = true;
#pragma unroll
    for (int i = 0; i < 15; ++i) {
        c[i] = __builtin_fmaf(s, nz[i], th[i]);
        if (i % 3 == 1 && __builtin_fabsf(c[i]) < 0.1f) ok = false;
    }
#pragma unroll
    for (int i = 0; i < 15; ++i) cd[i] = ok ? c[i] : th[i];
}

}  // namespace kq

using namespace kq;

extern "C" {

kq_status kq_calib_objective(const void *x, int64_t tokens, int64_t d, int64_t ld_x,
                             const float *lu, const float *gram, float *f, void *stream) {
    if (tokens < 0 || tokens >= (int64_t(1) << 30) || d <= 0 || d % 32 != 0 ||
        d > (int64_t(1) << 26) || ld_x < d)
        return KQ_ERR_SHAPE;
    if (!lu || !f || (tokens > 0 && !x)) return KQ_ERR_NULL;
    if (((uintptr_t)x % 16) || (ld_x * 2) % 16 || ((uintptr_t)lu % 4) || ((uintptr_t)f % 4) ||
        ((uintptr_t)gram % 4))
        return KQ_ERR_ALIGN;
    const int nb = (int)(d / 32);
    const uint16_t *xp = (const uint16_t *)x;
    void *args[] = {(void *)&xp, (void *)&ld_x, (void *)&tokens, (void *)&lu, (void *)&gram, (void *)&f};
    const hipError_t e = hipLaunchKernel((const void *)calib_objective_kernel, dim3(nb),
                                         dim3(kCalThreads), args, 0, (hipStream_t)stream);
    return e == hipSuccess ? KQ_OK : KQ_ERR_HIP;
}

kq_status kq_calib_es_update(int64_t nb, float *theta, float *sigma, float *fbest, float *cand,
                             const float *fcand, const float *noise, void *stream) {
    if (nb < 0 || nb >= (int64_t(1) << 26)) return KQ_ERR_SHAPE;
    if (nb == 0) return KQ_OK;
    if (!theta || !sigma || !fbest || !cand || !fcand || !noise) return KQ_ERR_NULL;
    if (((uintptr_t)theta % 4) || ((uintptr_t)sigma % 4) || ((uintptr_t)fbest % 4) ||
        ((uintptr_t)cand % 4) || ((uintptr_t)fcand % 4) || ((uintptr_t)noise % 4))
        return KQ_ERR_ALIGN;
    int n = (int)nb;
    void *args[] = {(void *)&n, (void *)&theta, (void *)&sigma, (void *)&fbest, (void *)&cand,
                    (void *)&fcand, (void *)&noise};
    const hipError_t e = hipLaunchKernel((const void *)calib_es_update_kernel, dim3((n + 63) / 64),
                                         dim3(64), args, 0, (hipStream_t)stream);
    return e == hipSuccess ? KQ_OK : KQ_ERR_HIP;
}

}  // extern "C"

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

__device__ __forceinline__ void load15(const float *src, float (&v)[15]) {
#pragma unroll
    for (int i = 0; i < 15; ++i) v[i] = src[i];
}

__device__ __forceinline__ void load_row32(const uint16_t *src, u32x4 (&v)[4]) {
    const u32x4 *p = reinterpret_cast<const u32x4 *>(src);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = p[i];
}

// Objective of block j = blockIdx.x over all tokens, for the parameters pr
// (the block's 15 values, already in registers); the total lands in thread 0
// (the other threads return an unspecified partial value).  Each thread's
// next token is loaded one iteration ahead, the first one before the
// parameter set-up.
__device__ __forceinline__ float calib_block_objective(const uint16_t *__restrict__ x, int64_t ld,
                                                       int64_t tokens, const float (&pr)[15],
                                                       const float *__restrict__ gram) {
    __shared__ float G[32 * 32];
    __shared__ float wsum[kCalThreads / 64];
    const int j = blockIdx.x, tid = threadIdx.x;
    const uint16_t *xb = x + (int64_t)j * 32;
    u32x4 nx[4] = {};
    if (tid < tokens) load_row32(xb + (int64_t)tid * ld, nx);
    if (gram) {
        for (int i = tid; i < 1024; i += kCalThreads) G[i] = gram[(int64_t)j * 1024 + i];
    }
    KronStage fw = KronStage::from(nullptr);
    KronInverseStage iv = KronInverseStage::from(nullptr);
#pragma unroll
    for (int i = 0; i < 15; ++i) fw.p[i] = iv.p[i] = pr[i];
    fw.setup();
    iv.setup();
    __syncthreads();

    float acc = 0.0f;
    for (int64_t t = tid; t < tokens; t += kCalThreads) {
        u32x4 cur[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) cur[i] = nx[i];
        if (t + kCalThreads < tokens) load_row32(xb + (t + kCalThreads) * ld, nx);
        float xv[32], z[32];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                xv[8 * i + 2 * c] = bf16_lo(cur[i][c]);
                xv[8 * i + 2 * c + 1] = bf16_hi(cur[i][c]);
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
    float s = wsum[0];
#pragma unroll
    for (int w = 1; w < kCalThreads / 64; ++w) s = s + wsum[w];
    return s;
}

__global__ __launch_bounds__(kCalThreads) void calib_objective_kernel(
    const uint16_t *__restrict__ x, int64_t ld, int64_t tokens, const float *__restrict__ lu,
    const float *__restrict__ gram, float *__restrict__ f) {
    float pr[15];
    load15(lu + (int64_t)blockIdx.x * 15, pr);
    const float s = calib_block_objective(x, ld, tokens, pr, gram);
    if (threadIdx.x == 0) f[blockIdx.x] = s;
}

// One (1+1)-ES step of one block on values in registers, in this fp32 order:
// keep the evaluated candidate cd if its objective fc is strictly below the
// kept fb (sigma * 1.5, at most 0.5), otherwise sigma * 0.90360200
// (1.5^-1/4, at least 1e-4), so that one success in five keeps sigma fixed;
// then the next candidate fma(sigma, noise, theta), or theta itself when any
// u would come within 0.1 of zero.  Returns whether cd was kept (th then
// holds it).
__device__ __forceinline__ bool es_update_regs(float fc, float fb, float &s, float (&th)[15],
                                               const float (&cd)[15], const float (&nz)[15],
                                               float (&next)[15]) {
    const bool keep = fc < fb;
    if (keep) {
#pragma unroll
        for (int i = 0; i < 15; ++i) th[i] = cd[i];
        s = s * 1.5f;
        s = s < 0.5f ? s : 0.5f;
    } else {
        s = s * 0.90360200f;
        s = s > 1e-4f ? s : 1e-4f;
    }
    bool ok = true;
#pragma unroll
    for (int i = 0; i < 15; ++i) {
        next[i] = __builtin_fmaf(s, nz[i], th[i]);
        if (i % 3 == 1 && __builtin_fabsf(next[i]) < 0.1f) ok = false;
    }
#pragma unroll
    for (int i = 0; i < 15; ++i) next[i] = ok ? next[i] : th[i];
    return keep;
}

// Writes the outcome of es_update_regs for block j.
__device__ __forceinline__ void es_store(int j, bool keep, float fc, float s, const float (&th)[15],
                                         const float (&next)[15], float *theta, float *sigma,
                                         float *fbest, float *cand) {
    if (keep) {
#pragma unroll
        for (int i = 0; i < 15; ++i) theta[(int64_t)j * 15 + i] = th[i];
        fbest[j] = fc;
    }
    sigma[j] = s;
#pragma unroll
    for (int i = 0; i < 15; ++i) cand[(int64_t)j * 15 + i] = next[i];
}

__global__ void calib_es_update_kernel(int nb, float *__restrict__ theta, float *__restrict__ sigma,
                                       float *__restrict__ fbest, float *__restrict__ cand,
                                       const float *__restrict__ fcand,
                                       const float *__restrict__ noise) {
    const int j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= nb) return;
    float th[15], cd[15], nz[15], next[15];
    load15(theta + (int64_t)j * 15, th);
    load15(cand + (int64_t)j * 15, cd);
    load15(noise + (int64_t)j * 15, nz);
    float s = sigma[j];
    const float fc = fcand[j];
    const bool keep = es_update_regs(fc, fbest[j], s, th, cd, nz, next);
    es_store(j, keep, fc, s, th, next, theta, sigma, fbest, cand);
}

// One whole iteration: block j's workgroup scores cand_j, then its thread 0
// applies the update of block j (which touches only block j's entries) and
// records the kept objective.  Everything the update reads is loaded at the
// start, so its latency hides behind the objective, and every write comes
// after the workgroup's last barrier.
__global__ __launch_bounds__(kCalThreads) void calib_es_step_kernel(
    const uint16_t *__restrict__ x, int64_t ld, int64_t tokens, const float *__restrict__ gram,
    float *theta, float *sigma, float *fbest, float *cand, const float *noise, float *fhist) {
    const int j = blockIdx.x;
    float cd[15], th[15], nz[15], next[15];
    load15(cand + (int64_t)j * 15, cd);
    load15(theta + (int64_t)j * 15, th);
    load15(noise + (int64_t)j * 15, nz);
    float s = sigma[j];
    const float fb = fbest[j];
    const float fc = calib_block_objective(x, ld, tokens, cd, gram);
    if (threadIdx.x != 0) return;
    const bool keep = es_update_regs(fc, fb, s, th, cd, nz, next);
    es_store(j, keep, fc, s, th, next, theta, sigma, fbest, cand);
    if (fhist) fhist[j] = keep ? fc : fb;
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

kq_status kq_calib_es_run(const void *x, int64_t tokens, int64_t d, int64_t ld_x,
                          const float *gram, float *theta, float *sigma, float *fbest, float *cand,
                          const float *noise, int64_t iterations, float *fhist, void *stream) {
    if (tokens < 0 || tokens >= (int64_t(1) << 30) || d <= 0 || d % 32 != 0 ||
        d > (int64_t(1) << 26) || ld_x < d || iterations < 0 || iterations > (int64_t(1) << 24))
        return KQ_ERR_SHAPE;
    if (iterations == 0) return KQ_OK;
    if (!theta || !sigma || !fbest || !cand || !noise || (tokens > 0 && !x)) return KQ_ERR_NULL;
    if (((uintptr_t)x % 16) || (ld_x * 2) % 16 || ((uintptr_t)gram % 4) ||
        ((uintptr_t)theta % 4) || ((uintptr_t)sigma % 4) || ((uintptr_t)fbest % 4) ||
        ((uintptr_t)cand % 4) || ((uintptr_t)noise % 4) || ((uintptr_t)fhist % 4))
        return KQ_ERR_ALIGN;
    const int nb = (int)(d / 32);
    const uint16_t *xp = (const uint16_t *)x;
    for (int64_t i = 0; i < iterations; ++i) {
        const float *nz = noise + i * nb * 15;
        float *fh = fhist ? fhist + i * nb : nullptr;
        void *args[] = {(void *)&xp,    (void *)&ld_x,  (void *)&tokens, (void *)&gram,
                        (void *)&theta, (void *)&sigma, (void *)&fbest,  (void *)&cand,
                        (void *)&nz,    (void *)&fh};
        const hipError_t e = hipLaunchKernel((const void *)calib_es_step_kernel, dim3(nb),
                                             dim3(kCalThreads), args, 0, (hipStream_t)stream);
        if (e != hipSuccess) return KQ_ERR_HIP;
    }
    return KQ_OK;
}

kq_status kq_calib_es_step(const void *x, int64_t tokens, int64_t d, int64_t ld_x,
                           const float *gram, float *theta, float *sigma, float *fbest,
                           float *cand, const float *noise, float *fhist, void *stream) {
    return kq_calib_es_run(x, tokens, d, ld_x, gram, theta, sigma, fbest, cand, noise, 1, fhist,
                           stream);
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

// kq_kron.h — the Kronecker block transform and its inverse as register
// stages, shared by the quantizer kernels (plain, AdaLN-fused, inverse side,
// calibration objective).
#pragma once

#include "kq_device.h"

namespace kq {

// The Kronecker-structured block transform (KroQuant summary, "Approach").
// F_b = [[1,0],[l,1]] [[u,v],[0,1/u]] = G_b D_b with the shear pair
// G_b = [[1,w],[l,1+l*w]], w = u*v, and D_b = diag(u, 1/u).  The Kronecker
// mixed-product rule turns T = (x)_b F_b into (x)_b G_b times the diagonal
// (x)_b D_b, so the kernel runs two fused multiply-adds per index pair and
// bit, then one multiply per element by d_k = prod_b (bit b of k ? 1/u_b : u_b).
struct KronStage {
    const float *lu;  // [nb][5][3]
    // kernels take only the parameter pointer and build the lane state here
    __device__ __forceinline__ static KronStage from(const float *p) {
        KronStage s;
        s.lu = p;
        return s;
    }
    float p[15];      // raw (l, u, v) x 5 of this lane's block
    float l[5], w[5], dk[32];
    __device__ __forceinline__ void fetch(int j) {
        const float *src = lu + (int64_t)j * 15;
#pragma unroll
        for (int i = 0; i < 15; ++i) p[i] = src[i];
    }
    __device__ __forceinline__ void setup() {
        float u[5], iu[5];
#pragma unroll
        for (int b = 0; b < 5; ++b) {
            l[b] = p[3 * b + 0];
            u[b] = p[3 * b + 1];
            w[b] = u[b] * p[3 * b + 2];
        }
        rcp5_rn(u, iu);  // = IEEE 1/u
        // d_k as the running product over b = 0..4, built bit by bit.
        dk[0] = u[0];
        dk[1] = iu[0];
#pragma unroll
        for (int b = 1; b < 5; ++b) {
            const int h = 1 << b;
#pragma unroll
            for (int k = 0; k < h; ++k) {
                dk[k + h] = dk[k] * iu[b];
                dk[k] = dk[k] * u[b];
            }
        }
    }
    __device__ __forceinline__ void apply(float (&z)[32]) const {
#pragma unroll
        for (int b = 0; b < 5; ++b) {
            const int h = 1 << b;
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                if (i & h) continue;
                const float r = __builtin_fmaf(l[b], z[i | h], z[i]);
                const float s = __builtin_fmaf(w[b], r, z[i | h]);
                z[i] = r;
                z[i | h] = s;
            }
        }
#pragma unroll
        for (int k = 0; k < 32; ++k) z[k] = z[k] * dk[k];
    }
};

// Inverse of the block transform: T^-1 = (D_4 (x)...(x) D_0)^-1 (G_4 (x)...(x) G_0)^-1
// (the inverse of y = x * T, KroQuant abstract: "invertible" transform, its
// inverse applied to the weights).  First z_k = y_k * e_k with e_k the running
// product over b = 0..4 of (bit b of k ? u_b : 1/u_b); then bits b = 4..0 map
// each pair (r, s) back by q = s - w*r, p = r - l*q (two fused multiply-adds).
// Constants shared by the inverse and the weight-side stages: l_b, w_b and
// e_k = running product over b = 0..4 of (bit b of k ? u_b : 1/u_b), the
// diagonal of (D_4 (x)...(x) D_0)^-1.
struct KronInvConsts {
    const float *lu;
    float p[15];
    float l[5], w[5], ek[32];
    __device__ __forceinline__ void fetch(int j) {
        const float *src = lu + (int64_t)j * 15;
#pragma unroll
        for (int i = 0; i < 15; ++i) p[i] = src[i];
    }
    __device__ __forceinline__ void setup() {
        float u[5], iu[5];
#pragma unroll
        for (int b = 0; b < 5; ++b) {
            l[b] = p[3 * b + 0];
            u[b] = p[3 * b + 1];
            w[b] = u[b] * p[3 * b + 2];
        }
        rcp5_rn(u, iu);
        ek[0] = iu[0];
        ek[1] = u[0];
#pragma unroll
        for (int b = 1; b < 5; ++b) {
            const int h = 1 << b;
#pragma unroll
            for (int k = 0; k < h; ++k) {
                ek[k + h] = ek[k] * u[b];
                ek[k] = ek[k] * iu[b];
            }
        }
    }
};

struct KronInverseStage : KronInvConsts {
    __device__ __forceinline__ static KronInverseStage from(const float *p) {
        KronInverseStage s;
        s.lu = p;
        return s;
    }
    __device__ __forceinline__ void apply(float (&z)[32]) const {
#pragma unroll
        for (int k = 0; k < 32; ++k) z[k] = z[k] * ek[k];
#pragma unroll
        for (int b = 4; b >= 0; --b) {
            const int h = 1 << b;
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                if (i & h) continue;
                const float r = z[i], s = z[i | h];
                const float q = __builtin_fmaf(-w[b], r, s);
                const float pv = __builtin_fmaf(-l[b], q, r);
                z[i] = pv;
                z[i | h] = q;
            }
        }
    }
};

}  // namespace kq

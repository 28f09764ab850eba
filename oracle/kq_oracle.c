/*
 * kq_oracle.c — CPU oracle for the KroQuant online activation quantizer.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark, never by the product path.  Plain C99,
 * built with -O2 -ffp-contract=off so that every fp32 operation written here
 * is one correctly rounded IEEE operation and every fused multiply-add is an
 * explicit fmaf().  Citations use the source keys defined in kq_oracle.h.
 */
#include "kq_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ======================================================================== */
/* Number formats                                                            */
/* ======================================================================== */

static float f32_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_from_f32(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* bf16 is the top half of an IEEE binary32; widening is exact. */
float kqo_bf16_to_f32(uint16_t bits) { return f32_from_bits((uint32_t)bits << 16); }

/* Round a double to the nearest bfloat16 (8 significant bits, binary32
 * exponent range), ties to even, by scaling to the bf16 quantum at the value's
 * binade and calling rint() (the default rounding mode is nearest-even). */
static uint16_t bf16_from_double_rne(double v) {
    if (isnan(v)) return (uint16_t)(signbit(v) ? 0xFFC0u : 0x7FC0u);
    double a = fabs(v);
    double r;
    if (isinf(a)) {
        r = a;
    } else if (a == 0.0) {
        r = 0.0;
    } else {
        int e;
        frexp(a, &e);                   /* a = m * 2^e, m in [0.5, 1) */
        int qexp = e - 8;               /* 8 significant bits */
        if (qexp < -133) qexp = -133;   /* bf16 subnormal spacing 2^-133 */
        r = ldexp(rint(ldexp(a, -qexp)), qexp);
        if (r >= ldexp(1.0, 128)) r = INFINITY;
    }
    uint32_t u = bits_from_f32((float)r); /* r is representable in binary32 */
    uint16_t h = (uint16_t)(u >> 16);
    if (signbit(v)) h |= 0x8000u;
    return h;
}

uint16_t kqo_f32_to_bf16_rne(float f) { return bf16_from_double_rne((double)f); }

/* E2M1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit.  Exponent
 * field 0 is subnormal: 0.5 * m.  Otherwise 2^(E-1) * (1 + m/2). */
double kqo_e2m1_value(uint8_t code) {
    int s = (code >> 3) & 1, E = (code >> 1) & 3, m = code & 1;
    double mag = (E == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, E - 1);
    return s ? -mag : mag;
}

/* Round-to-nearest-even onto the E2M1 grid with saturation: choose the
 * representable magnitude nearest |q|; on a tie prefer the code whose
 * mantissa bit is 0; anything above the largest magnitude (6) becomes 6.
 * The sign is kept, so a negative value rounding to zero gives 0x8. */
uint8_t kqo_e2m1_encode(double q) {
    uint8_t sign = signbit(q) ? 0x8 : 0x0;
    double a = fabs(q);
    if (isnan(q)) return sign;          /* only reached inside NaN blocks */
    if (a >= kqo_e2m1_value(7)) return (uint8_t)(sign | 7);
    uint8_t best = 0;
    double best_dist = a;               /* distance to magnitude 0 */
    for (uint8_t c = 1; c < 8; ++c) {
        double dist = fabs(a - kqo_e2m1_value(c));
        if (dist < best_dist || (dist == best_dist && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            best_dist = dist;
        }
    }
    return (uint8_t)(sign | best);
}

/* Shared-scale rule of MXFP4: the largest power of two 2^e such that
 * amax * 2^-e stays below 8, i.e. e = floor(log2 amax) - emax(E2M1) with
 * emax = 2; clamped to the E8M0 range.  floor(log2) is read off frexp(),
 * which is exact for normal and subnormal inputs. */
uint8_t kqo_e8m0_from_amax(float amax) {
    if (isnan(amax) || isinf(amax)) return 0xFF;
    int e;
    if (amax == 0.0f) {
        e = -127;
    } else {
        int ex;
        frexp((double)amax, &ex);       /* amax = m * 2^ex, m in [0.5,1) */
        e = (ex - 1) - 2;
        if (e < -127) e = -127;
        if (e > 127) e = 127;
    }
    return (uint8_t)(e + 127);
}

double kqo_e8m0_value(uint8_t byte) {
    if (byte == 0xFF) return NAN;
    return ldexp(1.0, (int)byte - 127);
}

void kqo_mxfp4_block(const float y[32], uint8_t codes[16], uint8_t *scale) {
    /* amax propagates NaN explicitly (a NaN anywhere makes the block NaN). */
    float amax = 0.0f;
    int nonfinite = 0;
    for (int k = 0; k < 32; ++k) {
        if (!isfinite(y[k])) nonfinite = 1;
        float a = fabsf(y[k]);
        if (a > amax) amax = a;
    }
    if (nonfinite) {
        *scale = 0xFF;
        memset(codes, 0, 16);
        return;
    }
    uint8_t b = kqo_e8m0_from_amax(amax);
    *scale = b;
    int e = (int)b - 127;
    for (int m = 0; m < 16; ++m) {
        /* y * 2^-e is exact in fp64 for every fp32 y. */
        uint8_t lo = kqo_e2m1_encode(ldexp((double)y[2 * m], -e));
        uint8_t hi = kqo_e2m1_encode(ldexp((double)y[2 * m + 1], -e));
        codes[m] = (uint8_t)(lo | (hi << 4));
    }
}

/* ======================================================================== */
/* The block transform                                                       */
/* ======================================================================== */

/* [KQ-sum] "Approach": each 2x2 factor is a unit-determinant LU product.
 * F = [[1,0],[l,1]] * [[u,v],[0,1/u]] = [[u, v], [l*u, l*v + 1/u]]. */
void kqo_lu_factor(const float p[3], double F[4]) {
    double l = p[0], u = p[1], v = p[2];
    double L[4] = {1.0, 0.0, l, 1.0};
    double U[4] = {u, v, 0.0, 1.0 / u};
    for (int r = 0; r < 2; ++r)
        for (int c = 0; c < 2; ++c)
            F[r * 2 + c] = L[r * 2 + 0] * U[0 * 2 + c] + L[r * 2 + 1] * U[1 * 2 + c];
}

/* Kronecker product: (A (x) B)[ia*rb + ib][ja*cb + jb] = A[ia][ja] * B[ib][jb]. */
void kqo_kron(const double *A, int ra, int ca, const double *B, int rb, int cb,
              double *C) {
    int cc = ca * cb;
    for (int ia = 0; ia < ra; ++ia)
        for (int ja = 0; ja < ca; ++ja)
            for (int ib = 0; ib < rb; ++ib)
                for (int jb = 0; jb < cb; ++jb)
                    C[(ia * rb + ib) * cc + (ja * cb + jb)] = A[ia * ca + ja] * B[ib * cb + jb];
}

/* Fold F4 (x) (F3 (x) (F2 (x) (F1 (x) F0))) from the right. */
static void kron_chain(const double F[5][4], double T[1024]) {
    double acc[1024], tmp[1024];
    int n = 2;
    memcpy(acc, F[0], sizeof(double) * 4);
    for (int b = 1; b < 5; ++b) {
        kqo_kron(F[b], 2, 2, acc, n, n, tmp);
        n *= 2;
        memcpy(acc, tmp, sizeof(double) * (size_t)(n * n));
    }
    memcpy(T, acc, sizeof(double) * 1024);
}

/* [KQ-sum] "Approach": the 32x32 block is the Kronecker product of the
 * five LU factors; F_b is the factor on bit b of the in-block index. */
void kqo_block_matrix(const float p[15], double T[1024]) {
    double F[5][4];
    for (int b = 0; b < 5; ++b) kqo_lu_factor(p + 3 * b, F[b]);
    kron_chain(F, T);
}

/* Inverse: (A (x) B)^-1 = A^-1 (x) B^-1, and for det F = 1 the inverse of
 * [[a,b],[c,d]] is its adjugate [[d,-b],[-c,a]]. */
void kqo_block_inverse_matrix(const float p[15], double Ti[1024]) {
    double F[5][4], A[5][4];
    for (int b = 0; b < 5; ++b) {
        kqo_lu_factor(p + 3 * b, F[b]);
        A[b][0] = F[b][3];
        A[b][1] = -F[b][1];
        A[b][2] = -F[b][2];
        A[b][3] = F[b][0];
    }
    kron_chain(A, Ti);
}

/* [LRQ] Eq. (3): H_2 = (1/sqrt2)[[1,1],[1,-1]], H_{2^n} = H_2 (x) H_{2^(n-1)}. */
void kqo_hadamard32(double H[1024]) {
    double H2[5][4];
    double s = 1.0 / sqrt(2.0);
    for (int b = 0; b < 5; ++b) {
        H2[b][0] = s; H2[b][1] = s; H2[b][2] = s; H2[b][3] = -s;
    }
    kron_chain(H2, H);
}

/* [KQ-sum] "Approach": factors start at the Hadamard.  H_2 itself has
 * determinant -1, so the unit-determinant start is H_2 * diag(1,-1) =
 * (1/sqrt2)[[1,-1],[1,1]]: u = F00 = 1/sqrt2, v = F01 = -1/sqrt2,
 * l = F10 / u = 1.  T_init = H_32 * diag((-1)^popcount(k)). */
void kqo_hadamard_init_params(float p[15]) {
    float r = (float)(1.0 / sqrt(2.0));
    for (int b = 0; b < 5; ++b) {
        p[3 * b + 0] = 1.0f;
        p[3 * b + 1] = r;
        p[3 * b + 2] = -r;
    }
}

void kqo_block_transform_dense64(const float x[32], const float p[15], float y[32]) {
    double T[1024];
    kqo_block_matrix(p, T);
    for (int k = 0; k < 32; ++k) {
        double acc = 0.0;
        for (int i = 0; i < 32; ++i) acc += (double)x[i] * T[i * 32 + k];
        y[k] = (float)acc;
    }
}

/*
 * Fixed fp32 order of the Kronecker factor applications.
 *
 * Write U = [[u,v],[0,1/u]] = N * D with N = [[1, u*v],[0,1]] and
 * D = diag(u, 1/u).  Then F = L * N * D = G * D, G = [[1, w],[l, 1 + l*w]],
 * w = u*v.  By the mixed-product rule of the Kronecker product,
 * T = (G4 (x) ... (x) G0) * (D4 (x) ... (x) D0): the five shears act on
 * their own index bit and commute, and the diagonal part is one diagonal
 * matrix with entries d_k = prod_b (bit b of k ? 1/u_b : u_b).
 *
 * For a row vector, multiplying by G on bit b maps each pair (p, q) =
 * (z[i], z[i | 2^b]) with bit b of i clear to (r, s):
 *     r = p + l*q          (one fused multiply-add)
 *     s = q + w*r          (one fused multiply-add)
 * The order fixed here: w_b = fl(u_b*v_b), 1/u_b by IEEE division, bits
 * b = 0,1,2,3,4 in turn, then d_k as the running product over b = 0..4 of
 * the per-bit entries (fp32, left to right) and y_k = fl(z_k * d_k).
 */
void kqo_block_transform_staged32(const float x[32], const float p[15], float y[32]) {
    float l[5], w[5], u[5], iu[5];
    for (int b = 0; b < 5; ++b) {
        l[b] = p[3 * b + 0];
        u[b] = p[3 * b + 1];
        w[b] = p[3 * b + 1] * p[3 * b + 2];
        iu[b] = 1.0f / p[3 * b + 1];
    }
    float z[32];
    memcpy(z, x, sizeof z);
    for (int b = 0; b < 5; ++b) {
        int h = 1 << b;
        for (int i = 0; i < 32; ++i) {
            if (i & h) continue;
            float pv = z[i], qv = z[i | h];
            float r = fmaf(l[b], qv, pv);
            float s = fmaf(w[b], r, qv);
            z[i] = r;
            z[i | h] = s;
        }
    }
    for (int k = 0; k < 32; ++k) {
        float dk = (k & 1) ? iu[0] : u[0];
        for (int b = 1; b < 5; ++b) dk = dk * (((k >> b) & 1) ? iu[b] : u[b]);
        y[k] = z[k] * dk;
    }
}

void kqo_block_inverse_dense64(const float y[32], const float p[15], float x[32]) {
    double Ti[1024];
    kqo_block_inverse_matrix(p, Ti);
    for (int k = 0; k < 32; ++k) {
        double acc = 0.0;
        for (int i = 0; i < 32; ++i) acc += (double)y[i] * Ti[i * 32 + k];
        x[k] = (float)acc;
    }
}

/*
 * Inverse in the mirrored fp32 order: T^-1 = D^-1 * (G4 (x) ... (x) G0)^-1.
 * First z_k = fl(y_k * e_k) with e_k the running product over b = 0..4 of
 * (bit b of k ? u_b : 1/u_b); then bits b = 4,3,2,1,0, each pair (r, s)
 * mapped back by q = s - w*r, p = r - l*q (two fused multiply-adds).
 */
void kqo_block_inverse_staged32(const float y[32], const float p[15], float x[32]) {
    float l[5], w[5], u[5], iu[5];
    for (int b = 0; b < 5; ++b) {
        l[b] = p[3 * b + 0];
        u[b] = p[3 * b + 1];
        w[b] = p[3 * b + 1] * p[3 * b + 2];
        iu[b] = 1.0f / p[3 * b + 1];
    }
    float z[32];
    for (int k = 0; k < 32; ++k) {
        float ek = (k & 1) ? u[0] : iu[0];
        for (int b = 1; b < 5; ++b) ek = ek * (((k >> b) & 1) ? u[b] : iu[b]);
        z[k] = y[k] * ek;
    }
    for (int b = 4; b >= 0; --b) {
        int h = 1 << b;
        for (int i = 0; i < 32; ++i) {
            if (i & h) continue;
            float r = z[i], s = z[i | h];
            float q = fmaf(-w[b], r, s);
            float pv = fmaf(-l[b], q, r);
            z[i] = pv;
            z[i | h] = q;
        }
    }
    memcpy(x, z, sizeof z);
}

void kqo_block_weight_dense64(const float w[32], const float p[15], float y[32]) {
    double Ti[1024];
    kqo_block_inverse_matrix(p, Ti);
    for (int k = 0; k < 32; ++k) {
        /* y = w * Ti^T: y_k = sum_i w_i * Ti[k][i] */
        double acc = 0.0;
        for (int i = 0; i < 32; ++i) acc += (double)w[i] * Ti[k * 32 + i];
        y[k] = (float)acc;
    }
}

/*
 * Fixed fp32 order of w * T^-T.  With T = (G4 (x)...(x) G0)(D4 (x)...(x) D0):
 * T^-T = (G4^-T (x)...(x) G0^-T)(D4^-1 (x)...(x) D0^-1), and
 * G^-T = [[1,-l],[0,1]] * [[1,0],[-w,1]].  A row vector pair (p, q) on bit b
 * therefore maps to s = q - l*p, then r = p - w*s (two fused multiply-adds),
 * bits b = 0..4 in turn; then y_k = z_k * e_k with e_k the running product over
 * b = 0..4 of (bit b of k ? u_b : 1/u_b).
 */
void kqo_block_weight_staged32(const float w[32], const float p[15], float y[32]) {
    float l[5], ww[5], u[5], iu[5];
    for (int b = 0; b < 5; ++b) {
        l[b] = p[3 * b + 0];
        u[b] = p[3 * b + 1];
        ww[b] = p[3 * b + 1] * p[3 * b + 2];
        iu[b] = 1.0f / p[3 * b + 1];
    }
    float z[32];
    memcpy(z, w, sizeof z);
    for (int b = 0; b < 5; ++b) {
        int h = 1 << b;
        for (int i = 0; i < 32; ++i) {
            if (i & h) continue;
            float pv = z[i], qv = z[i | h];
            float s = fmaf(-l[b], pv, qv);
            float r = fmaf(-ww[b], s, pv);
            z[i] = r;
            z[i | h] = s;
        }
    }
    for (int k = 0; k < 32; ++k) {
        float ek = (k & 1) ? u[0] : iu[0];
        for (int b = 1; b < 5; ++b) ek = ek * (((k >> b) & 1) ? u[b] : iu[b]);
        y[k] = z[k] * ek;
    }
}

/* ======================================================================== */
/* Row-parallel driver                                                       */
/* ======================================================================== */

typedef void (*row_fn)(void *ctx, int64_t t);

typedef struct {
    row_fn fn;
    void *ctx;
    int64_t begin, end;
} row_job;

static void *row_worker(void *arg) {
    row_job *j = (row_job *)arg;
    for (int64_t t = j->begin; t < j->end; ++t) j->fn(j->ctx, t);
    return NULL;
}

static void parallel_rows(row_fn fn, void *ctx, int64_t rows, int threads) {
    if (threads < 1) threads = 1;
    if (threads > 256) threads = 256;
    if (rows < threads) threads = rows > 0 ? (int)rows : 1;
    if (threads == 1) {
        for (int64_t t = 0; t < rows; ++t) fn(ctx, t);
        return;
    }
    pthread_t tid[256];
    row_job jobs[256];
    int64_t chunk = (rows + threads - 1) / threads;
    int started = 0;
    for (int i = 0; i < threads; ++i) {
        jobs[i].fn = fn;
        jobs[i].ctx = ctx;
        jobs[i].begin = (int64_t)i * chunk;
        jobs[i].end = jobs[i].begin + chunk < rows ? jobs[i].begin + chunk : rows;
        if (jobs[i].begin >= jobs[i].end) break;
        if (pthread_create(&tid[i], NULL, row_worker, &jobs[i]) != 0) {
            row_worker(&jobs[i]);   /* no thread available: run it here */
            jobs[i].fn = NULL;
        }
        started = i + 1;
    }
    for (int i = 0; i < started; ++i)
        if (jobs[i].fn) pthread_join(tid[i], NULL);
}

static int bad_shape(int64_t tokens, int64_t d, int64_t ld) {
    return tokens < 0 || d <= 0 || d % 32 != 0 || ld < d;
}

/* ---- transform (+ quantize) ---- */
typedef struct {
    const uint16_t *x;
    int64_t d, ld;
    const float *lu;
    int mode;
    float *y;
    uint8_t *codes, *scales;
    double *bound;
    const float *mult;
} tq_ctx;

static void load_block(const tq_ctx *c, int64_t t, int64_t j, float xb[32]) {
    const uint16_t *src = c->x + t * c->ld + j * 32;
    for (int i = 0; i < 32; ++i) xb[i] = kqo_bf16_to_f32(src[i]);
}

static void transform_block(const tq_ctx *c, int64_t t, int64_t j, float yb[32]) {
    float xb[32];
    load_block(c, t, j, xb);
    const float *p = c->lu + j * 15;
    if (c->mode == KQO_DENSE64)
        kqo_block_transform_dense64(xb, p, yb);
    else
        kqo_block_transform_staged32(xb, p, yb);
}

static void row_transform(void *vc, int64_t t) {
    tq_ctx *c = (tq_ctx *)vc;
    for (int64_t j = 0; j < c->d / 32; ++j) transform_block(c, t, j, c->y + t * c->d + j * 32);
}

static void row_transform_quant(void *vc, int64_t t) {
    tq_ctx *c = (tq_ctx *)vc;
    int64_t nb = c->d / 32;
    for (int64_t j = 0; j < nb; ++j) {
        float yb[32];
        transform_block(c, t, j, yb);
        kqo_mxfp4_block(yb, c->codes + t * (c->d / 2) + j * 16, c->scales + t * nb + j);
    }
}

static void row_absbound(void *vc, int64_t t) {
    tq_ctx *c = (tq_ctx *)vc;
    for (int64_t j = 0; j < c->d / 32; ++j) {
        double T[1024];
        float xb[32];
        kqo_block_matrix(c->lu + j * 15, T);
        load_block(c, t, j, xb);
        for (int k = 0; k < 32; ++k) {
            double acc = 0.0;
            for (int i = 0; i < 32; ++i) acc += fabs((double)xb[i]) * fabs(T[i * 32 + k]);
            c->bound[t * c->d + j * 32 + k] = acc;
        }
    }
}

int kqo_transform(const uint16_t *x, int64_t tokens, int64_t d, int64_t ld,
                  const float *lu, int mode, float *y, int threads) {
    if (!x || !lu || !y || bad_shape(tokens, d, ld)) return -1;
    tq_ctx c = {x, d, ld, lu, mode, y, NULL, NULL, NULL, NULL};
    parallel_rows(row_transform, &c, tokens, threads);
    return 0;
}

int kqo_transform_absbound(const uint16_t *x, int64_t tokens, int64_t d, int64_t ld,
                           const float *lu, double *bound, int threads) {
    if (!x || !lu || !bound || bad_shape(tokens, d, ld)) return -1;
    tq_ctx c = {x, d, ld, lu, KQO_DENSE64, NULL, NULL, NULL, bound, NULL};
    parallel_rows(row_absbound, &c, tokens, threads);
    return 0;
}

int kqo_transform_quant(const uint16_t *x, int64_t tokens, int64_t d, int64_t ld,
                        const float *lu, int mode, uint8_t *codes, uint8_t *scales,
                        int threads) {
    if (!x || !lu || !codes || !scales || bad_shape(tokens, d, ld)) return -1;
    tq_ctx c = {x, d, ld, lu, mode, NULL, codes, scales, NULL, NULL};
    parallel_rows(row_transform_quant, &c, tokens, threads);
    return 0;
}

/* ---- plain MXFP4 of an fp32 tensor ---- */
typedef struct {
    const float *y;
    int64_t d;
    uint8_t *codes, *scales;
} q_ctx;

static void row_quant(void *vc, int64_t t) {
    q_ctx *c = (q_ctx *)vc;
    int64_t nb = c->d / 32;
    for (int64_t j = 0; j < nb; ++j)
        kqo_mxfp4_block(c->y + t * c->d + j * 32, c->codes + t * (c->d / 2) + j * 16,
                        c->scales + t * nb + j);
}

int kqo_mxfp4_quant(const float *y, int64_t tokens, int64_t d, uint8_t *codes,
                    uint8_t *scales, int threads) {
    if (!y || !codes || !scales || bad_shape(tokens, d, d)) return -1;
    q_ctx c = {y, d, codes, scales};
    parallel_rows(row_quant, &c, tokens, threads);
    return 0;
}

/* ---- per-channel scaling baseline ([KQ-abs]: SmoothQuant-style scaling) ---- */
static void row_smooth_quant(void *vc, int64_t t) {
    tq_ctx *c = (tq_ctx *)vc;
    int64_t nb = c->d / 32;
    for (int64_t j = 0; j < nb; ++j) {
        float xb[32], yb[32];
        load_block(c, t, j, xb);
        for (int k = 0; k < 32; ++k) yb[k] = xb[k] * c->mult[j * 32 + k];
        kqo_mxfp4_block(yb, c->codes + t * (c->d / 2) + j * 16, c->scales + t * nb + j);
    }
}

int kqo_smooth_quant(const uint16_t *x, int64_t tokens, int64_t d, int64_t ld,
                     const float *mult, uint8_t *codes, uint8_t *scales, int threads) {
    if (!x || !mult || !codes || !scales || bad_shape(tokens, d, ld)) return -1;
    tq_ctx c = {x, d, ld, NULL, 0, NULL, codes, scales, NULL, mult};
    parallel_rows(row_smooth_quant, &c, tokens, threads);
    return 0;
}

/* ---- fixed 32-point Hadamard baseline ([KQ-sum] "Experimental setup":
 *      Hadamard (32x32) block transform and FWHT baselines) ---- */
static void fwht32_block(const float xb[32], int mode, float yb[32]) {
    if (mode == KQO_DENSE64) {
        double H[1024];
        kqo_hadamard32(H);
        for (int k = 0; k < 32; ++k) {
            double acc = 0.0;
            for (int i = 0; i < 32; ++i) acc += (double)xb[i] * H[i * 32 + k];
            yb[k] = (float)acc;
        }
        return;
    }
    float z[32];
    memcpy(z, xb, sizeof z);
    for (int b = 0; b < 5; ++b) {
        int h = 1 << b;
        for (int i = 0; i < 32; ++i) {
            if (i & h) continue;
            float pv = z[i], qv = z[i | h];
            z[i] = pv + qv;
            z[i | h] = pv - qv;
        }
    }
    float c = (float)(1.0 / sqrt(32.0));
    for (int k = 0; k < 32; ++k) yb[k] = z[k] * c;
}

static void row_fwht(void *vc, int64_t t) {
    tq_ctx *c = (tq_ctx *)vc;
    for (int64_t j = 0; j < c->d / 32; ++j) {
        float xb[32];
        load_block(c, t, j, xb);
        fwht32_block(xb, c->mode, c->y + t * c->d + j * 32);
    }
}

static void row_fwht_quant(void *vc, int64_t t) {
    tq_ctx *c = (tq_ctx *)vc;
    int64_t nb = c->d / 32;
    for (int64_t j = 0; j < nb; ++j) {
        float xb[32], yb[32];
        load_block(c, t, j, xb);
        fwht32_block(xb, c->mode, yb);
        kqo_mxfp4_block(yb, c->codes + t * (c->d / 2) + j * 16, c->scales + t * nb + j);
    }
}

int kqo_fwht32(const uint16_t *x, int64_t tokens, int64_t d, int64_t ld, int mode,
               float *y, int threads) {
    if (!x || !y || bad_shape(tokens, d, ld)) return -1;
    tq_ctx c = {x, d, ld, NULL, mode, y, NULL, NULL, NULL, NULL};
    parallel_rows(row_fwht, &c, tokens, threads);
    return 0;
}

int kqo_fwht32_quant(const uint16_t *x, int64_t tokens, int64_t d, int64_t ld,
                     int mode, uint8_t *codes, uint8_t *scales, int threads) {
    if (!x || !codes || !scales || bad_shape(tokens, d, ld)) return -1;
    tq_ctx c = {x, d, ld, NULL, mode, NULL, codes, scales, NULL, NULL};
    parallel_rows(row_fwht_quant, &c, tokens, threads);
    return 0;
}

/* ---- weight side ---- */
static void weight_block(const tq_ctx *c, int64_t t, int64_t j, float yb[32]) {
    float xb[32];
    load_block(c, t, j, xb);
    const float *p = c->lu + j * 15;
    if (c->mode == KQO_DENSE64)
        kqo_block_weight_dense64(xb, p, yb);
    else
        kqo_block_weight_staged32(xb, p, yb);
}

static void row_weight(void *vc, int64_t t) {
    tq_ctx *c = (tq_ctx *)vc;
    for (int64_t j = 0; j < c->d / 32; ++j) weight_block(c, t, j, c->y + t * c->d + j * 32);
}

static void row_weight_quant(void *vc, int64_t t) {
    tq_ctx *c = (tq_ctx *)vc;
    int64_t nb = c->d / 32;
    for (int64_t j = 0; j < nb; ++j) {
        float yb[32];
        weight_block(c, t, j, yb);
        kqo_mxfp4_block(yb, c->codes + t * (c->d / 2) + j * 16, c->scales + t * nb + j);
    }
}

int kqo_weight_transform(const uint16_t *w, int64_t rows, int64_t k, int64_t ld,
                         const float *lu, int mode, float *y, int threads) {
    if (!w || !lu || !y || bad_shape(rows, k, ld)) return -1;
    tq_ctx c = {w, k, ld, lu, mode, y, NULL, NULL, NULL, NULL};
    parallel_rows(row_weight, &c, rows, threads);
    return 0;
}

int kqo_weight_quant(const uint16_t *w, int64_t rows, int64_t k, int64_t ld,
                     const float *lu, int mode, uint8_t *codes, uint8_t *scales, int threads) {
    if (!w || !lu || !codes || !scales || bad_shape(rows, k, ld)) return -1;
    tq_ctx c = {w, k, ld, lu, mode, NULL, codes, scales, NULL, NULL};
    parallel_rows(row_weight_quant, &c, rows, threads);
    return 0;
}

/* ---- decode and inverse ([KQ-abs]: the transform is invertible; its inverse
 *      is applied to the weights) ---- */
int kqo_mxfp4_dequant(const uint8_t *codes, const uint8_t *scales, int64_t tokens,
                      int64_t d, float *xhat) {
    if (!codes || !scales || !xhat || bad_shape(tokens, d, d)) return -1;
    int64_t nb = d / 32;
    for (int64_t t = 0; t < tokens; ++t)
        for (int64_t k = 0; k < d; ++k) {
            uint8_t byte = codes[t * (d / 2) + k / 2];
            uint8_t code = (k & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 0xF);
            double s = kqo_e8m0_value(scales[t * nb + k / 32]);
            xhat[t * d + k] = (float)(kqo_e2m1_value(code) * s);
        }
    return 0;
}

typedef struct {
    const uint8_t *codes, *scales;
    int64_t d;
    const float *lu;
    int mode;
    uint16_t *out;
} di_ctx;

static void row_dequant_inverse(void *vc, int64_t t) {
    di_ctx *c = (di_ctx *)vc;
    int64_t nb = c->d / 32;
    for (int64_t j = 0; j < nb; ++j) {
        float yb[32], xb[32];
        double s = kqo_e8m0_value(c->scales[t * nb + j]);
        for (int k = 0; k < 32; ++k) {
            uint8_t byte = c->codes[t * (c->d / 2) + j * 16 + k / 2];
            uint8_t code = (k & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 0xF);
            yb[k] = (float)(kqo_e2m1_value(code) * s);
        }
        const float *p = c->lu + j * 15;
        uint16_t *dst = c->out + t * c->d + j * 32;
        if (c->mode == KQO_DENSE64) {
            double Ti[1024];
            kqo_block_inverse_matrix(p, Ti);
            for (int k = 0; k < 32; ++k) {
                double acc = 0.0;
                for (int i = 0; i < 32; ++i) acc += (double)yb[i] * Ti[i * 32 + k];
                dst[k] = bf16_from_double_rne(acc);
            }
        } else {
            kqo_block_inverse_staged32(yb, p, xb);
            for (int k = 0; k < 32; ++k) dst[k] = kqo_f32_to_bf16_rne(xb[k]);
        }
    }
}

int kqo_dequant_inverse(const uint8_t *codes, const uint8_t *scales, int64_t tokens,
                        int64_t d, const float *lu, int mode, uint16_t *x_out,
                        int threads) {
    if (!codes || !scales || !lu || !x_out || bad_shape(tokens, d, d)) return -1;
    di_ctx c = {codes, scales, d, lu, mode, x_out};
    parallel_rows(row_dequant_inverse, &c, tokens, threads);
    return 0;
}

/* ---- fp64 reference product for the W4A4 consumer ([LRQ] Eq. (2)) ---- */
typedef struct {
    const float *A, *W;
    int64_t N, K;
    double *Y;
} mm_ctx;

static void row_matmul(void *vc, int64_t m) {
    mm_ctx *c = (mm_ctx *)vc;
    for (int64_t n = 0; n < c->N; ++n) {
        double acc = 0.0;
        for (int64_t k = 0; k < c->K; ++k)
            acc += (double)c->A[m * c->K + k] * (double)c->W[n * c->K + k];
        c->Y[m * c->N + n] = acc;
    }
}

int kqo_matmul_nt(const float *A, const float *W, int64_t M, int64_t N, int64_t K,
                  double *Y, int threads) {
    if (!A || !W || !Y || M < 0 || N < 0 || K < 0) return -1;
    mm_ctx c = {A, W, N, K, Y};
    parallel_rows(row_matmul, &c, M, threads);
    return 0;
}

/* ======================================================================== */
/* AdaLN-modulated input ([KQ-sum] "Problem": adaptive LayerNorm in the      */
/* diffusion-transformer blocks is why the transform has to run online)      */
/* ======================================================================== */
/*
 * h = LN(x) * (1 + scale_s) + shift_s per row, LN over the row's d channels
 * with no affine part, population variance and eps inside the square root;
 * row t uses the modulation vectors of sample s = t / rows_per_sample.
 *
 * DENSE64 is the definition: mean and variance (two passes) in fp64,
 * n = (x - mean) / sqrt(var + eps), h = n * (1 + scale) + shift, all fp64.
 *
 * STAGED32 is the fixed fp32 order of the GPU kernel:
 *   block partial  s_j = (((x_0 + x_1) + x_2) + ...) + x_31 of block j;
 *   row total      64 lanes: lane l starts from s_l (0 when l >= nb), adds
 *                  s_{l+64}, s_{l+128}, ... in turn; then six exchange
 *                  steps: for m = 1, 2, 4, 8, 16, 32 every lane adds
 *                  the value of lane l ^ m; the total is lane 0's value;
 *   mean           = total / d;
 *   c_k            = x_k - mean;
 *   block partial  q_j = fma(c_31, c_31, ... fma(c_1, c_1, fma(c_0, c_0, 0)));
 *   row total      as above, var = total / d;
 *   rstd           = 1 / sqrt(var + eps) (each step correctly rounded);
 *   h_k            = fma(c_k * rstd, 1 + scale_k, shift_k), 1 + scale_k in fp32.
 */
static float staged_row_total(const float *part, int64_t nb) {
    float acc[64], nxt[64];
    for (int l = 0; l < 64; ++l) {
        float a = l < nb ? part[l] : 0.0f;
        for (int64_t j = l + 64; j < nb; j += 64) a = a + part[j];
        acc[l] = a;
    }
    for (int m = 1; m < 64; m <<= 1) {
        for (int l = 0; l < 64; ++l) nxt[l] = acc[l] + acc[l ^ m];
        memcpy(acc, nxt, sizeof acc);
    }
    return acc[0];
}

typedef struct {
    const uint16_t *x;
    int64_t d, ld, rps;
    const float *shift, *scale, *lu;
    float eps;
    int mode;
    float *h, *mean, *rstd;
    uint8_t *codes, *scales;
    double *bound;
} ad_ctx;

/* Row t: the modulated values, fp64 (DENSE64) or fp32 (STAGED32), plus the
 * row statistics in the same mode. */
static void adaln_row(const ad_ctx *c, int64_t t, double *h64, float *h32, double *mu_out,
                      double *rstd_out) {
    const uint16_t *xr = c->x + t * c->ld;
    const int64_t d = c->d, nb = d / 32, s = t / c->rps;
    const float *sh = c->shift + s * d, *sc = c->scale + s * d;
    if (c->mode == KQO_DENSE64) {
        double sum = 0.0, sq = 0.0;
        for (int64_t k = 0; k < d; ++k) sum += (double)kqo_bf16_to_f32(xr[k]);
        const double mu = sum / (double)d;
        for (int64_t k = 0; k < d; ++k) {
            const double cdev = (double)kqo_bf16_to_f32(xr[k]) - mu;
            sq += cdev * cdev;
        }
        const double rstd = 1.0 / sqrt(sq / (double)d + (double)c->eps);
        for (int64_t k = 0; k < d; ++k) {
            const double n = ((double)kqo_bf16_to_f32(xr[k]) - mu) * rstd;
            h64[k] = n * (1.0 + (double)sc[k]) + (double)sh[k];
        }
        if (mu_out) *mu_out = mu;
        if (rstd_out) *rstd_out = rstd;
        return;
    }
    float *part = (float *)calloc((size_t)nb, sizeof(float));
    for (int64_t j = 0; j < nb; ++j) {
        float a = kqo_bf16_to_f32(xr[j * 32]);
        for (int k = 1; k < 32; ++k) a = a + kqo_bf16_to_f32(xr[j * 32 + k]);
        part[j] = a;
    }
    const float mean = staged_row_total(part, nb) / (float)d;
    for (int64_t j = 0; j < nb; ++j) {
        float q = 0.0f;
        for (int k = 0; k < 32; ++k) {
            const float cdev = kqo_bf16_to_f32(xr[j * 32 + k]) - mean;
            q = fmaf(cdev, cdev, q);
        }
        part[j] = q;
    }
    const float var = staged_row_total(part, nb) / (float)d;
    const float rstd = 1.0f / sqrtf(var + c->eps);
    free(part);
    for (int64_t k = 0; k < d; ++k) {
        const float cdev = kqo_bf16_to_f32(xr[k]) - mean;
        h32[k] = fmaf(cdev * rstd, 1.0f + sc[k], sh[k]);
    }
    if (mu_out) *mu_out = mean;
    if (rstd_out) *rstd_out = rstd;
}

static void row_adaln_modulate(void *vc, int64_t t) {
    ad_ctx *c = (ad_ctx *)vc;
    double *h64 = (double *)malloc((size_t)c->d * sizeof(double));
    double mu, rstd;
    adaln_row(c, t, h64, c->h + t * c->d, &mu, &rstd);
    if (c->mode == KQO_DENSE64)
        for (int64_t k = 0; k < c->d; ++k) c->h[t * c->d + k] = (float)h64[k];
    if (c->mean) c->mean[t] = (float)mu;
    if (c->rstd) c->rstd[t] = (float)rstd;
    free(h64);
}

static void row_adaln_quant(void *vc, int64_t t) {
    ad_ctx *c = (ad_ctx *)vc;
    const int64_t d = c->d, nb = d / 32;
    double *h64 = (double *)malloc((size_t)d * sizeof(double));
    float *h32 = (float *)malloc((size_t)d * sizeof(float));
    adaln_row(c, t, h64, h32, NULL, NULL);
    for (int64_t j = 0; j < nb; ++j) {
        const float *p = c->lu + j * 15;
        float yb[32];
        if (c->mode == KQO_DENSE64) {
            double T[1024];
            kqo_block_matrix(p, T);
            for (int k = 0; k < 32; ++k) {
                double acc = 0.0;
                for (int i = 0; i < 32; ++i) acc += h64[j * 32 + i] * T[i * 32 + k];
                yb[k] = (float)acc;
            }
        } else {
            kqo_block_transform_staged32(h32 + j * 32, p, yb);
        }
        kqo_mxfp4_block(yb, c->codes + t * (d / 2) + j * 16, c->scales + t * nb + j);
    }
    free(h64);
    free(h32);
}

/* Forward-error scale of the STAGED32 values against DENSE64, per output:
 * sum_i (|1 + scale_i| (|n_i| + mean_j |x_j| * rstd) + |h_i|) |T_ik| (fp64). */
static void row_adaln_bound(void *vc, int64_t t) {
    ad_ctx *c = (ad_ctx *)vc;
    const int64_t d = c->d, nb = d / 32, s = t / c->rps;
    const uint16_t *xr = c->x + t * c->ld;
    const float *sc = c->scale + s * d;
    double *h64 = (double *)malloc((size_t)d * sizeof(double));
    double mu, rstd, amean = 0.0;
    ad_ctx cd = *c;
    cd.mode = KQO_DENSE64;
    adaln_row(&cd, t, h64, NULL, &mu, &rstd);
    for (int64_t k = 0; k < d; ++k) amean += fabs((double)kqo_bf16_to_f32(xr[k]));
    amean /= (double)d;
    for (int64_t j = 0; j < nb; ++j) {
        double T[1024], e[32];
        kqo_block_matrix(c->lu + j * 15, T);
        for (int i = 0; i < 32; ++i) {
            const int64_t k = j * 32 + i;
            const double n = ((double)kqo_bf16_to_f32(xr[k]) - mu) * rstd;
            e[i] = fabs(1.0 + (double)sc[k]) * (fabs(n) + amean * rstd) + fabs(h64[k]);
        }
        for (int k = 0; k < 32; ++k) {
            double acc = 0.0;
            for (int i = 0; i < 32; ++i) acc += e[i] * fabs(T[i * 32 + k]);
            c->bound[t * d + j * 32 + k] = acc;
        }
    }
    free(h64);
}

static int bad_adaln(const uint16_t *x, int64_t tokens, int64_t d, int64_t ld,
                     const float *shift, const float *scale, int64_t rps, float eps) {
    return !x || !shift || !scale || bad_shape(tokens, d, ld) || rps < 1 || !(eps >= 0.0f);
}

int kqo_adaln_modulate(const uint16_t *x, int64_t tokens, int64_t d, int64_t ld,
                       const float *shift, const float *scale, int64_t rows_per_sample,
                       float eps, int mode, float *h, float *mean, float *rstd, int threads) {
    if (bad_adaln(x, tokens, d, ld, shift, scale, rows_per_sample, eps) || !h) return -1;
    ad_ctx c = {x, d, ld, rows_per_sample, shift, scale, NULL, eps, mode, h, mean, rstd,
                NULL, NULL, NULL};
    parallel_rows(row_adaln_modulate, &c, tokens, threads);
    return 0;
}

int kqo_adaln_transform_quant(const uint16_t *x, int64_t tokens, int64_t d, int64_t ld,
                              const float *shift, const float *scale, int64_t rows_per_sample,
                              float eps, const float *lu, int mode, uint8_t *codes,
                              uint8_t *scales, int threads) {
    if (bad_adaln(x, tokens, d, ld, shift, scale, rows_per_sample, eps) || !lu || !codes ||
        !scales)
        return -1;
    ad_ctx c = {x, d, ld, rows_per_sample, shift, scale, lu, eps, mode, NULL, NULL, NULL,
                codes, scales, NULL};
    parallel_rows(row_adaln_quant, &c, tokens, threads);
    return 0;
}

int kqo_adaln_bound(const uint16_t *x, int64_t tokens, int64_t d, int64_t ld,
                    const float *shift, const float *scale, int64_t rows_per_sample, float eps,
                    const float *lu, double *bound, int threads) {
    if (bad_adaln(x, tokens, d, ld, shift, scale, rows_per_sample, eps) || !lu || !bound)
        return -1;
    ad_ctx c = {x, d, ld, rows_per_sample, shift, scale, lu, eps, KQO_DENSE64, NULL, NULL,
                NULL, NULL, NULL, bound};
    parallel_rows(row_adaln_bound, &c, tokens, threads);
    return 0;
}

/* ======================================================================== */
/* Calibration of the block parameters ([KQ-sum] "Approach": the factors     */
/* are learned layer-wise from the Hadamard start with an output loss)       */
/* ======================================================================== */
/*
 * Objective of block j over a calibration set:
 *   f_j = sum_t r_t G_j r_t^T,  r_t = dequant(MXFP4(x_t T_j)) T_j^-1 - x_t,
 * x_t the block's 32 values of token t, G_j a 32x32 weighting (the identity
 * when gram is NULL: the round-trip error of the quantizer; W_j^T W_j for the
 * block-diagonal part of the output error of X W^T).  The MXFP4 decisions are
 * taken on the fixed-fp32-order transform (the kernel's values); the decoded
 * values, the inverse (adjugate Kronecker factors) and the sums are fp64.
 * A block whose scale byte is NaN makes f_j NaN.
 */
typedef struct {
    const uint16_t *x;
    int64_t tokens, d, ld;
    const float *lu, *gram;
    double *f;
} cal_ctx;

static void block_objective(void *vc, int64_t j) {
    const cal_ctx *c = (const cal_ctx *)vc;
    const float *p = c->lu + j * 15;
    double Ti[1024];
    kqo_block_inverse_matrix(p, Ti);
    const float *G = c->gram ? c->gram + j * 1024 : NULL;
    double acc = 0.0;
    for (int64_t t = 0; t < c->tokens; ++t) {
        float xb[32], yb[32];
        const uint16_t *src = c->x + t * c->ld + j * 32;
        for (int i = 0; i < 32; ++i) xb[i] = kqo_bf16_to_f32(src[i]);
        kqo_block_transform_staged32(xb, p, yb);
        uint8_t codes[16], sbyte;
        kqo_mxfp4_block(yb, codes, &sbyte);
        const double sc = kqo_e8m0_value(sbyte);
        double q[32], r[32];
        for (int k = 0; k < 32; ++k) {
            const uint8_t code = (codes[k / 2] >> (4 * (k & 1))) & 0xF;
            q[k] = kqo_e2m1_value(code) * sc;
        }
        for (int i = 0; i < 32; ++i) {
            double v = 0.0;
            for (int k = 0; k < 32; ++k) v += q[k] * Ti[k * 32 + i];
            r[i] = v - (double)xb[i];
        }
        double e = 0.0;
        if (G) {
            for (int a = 0; a < 32; ++a)
                for (int b = 0; b < 32; ++b) e += r[a] * (double)G[a * 32 + b] * r[b];
        } else {
            for (int a = 0; a < 32; ++a) e += r[a] * r[a];
        }
        acc += e;
    }
    c->f[j] = acc;
}

int kqo_calib_objective(const uint16_t *x, int64_t tokens, int64_t d, int64_t ld,
                        const float *lu, const float *gram, double *f, int threads) {
    if (!x || !lu || !f || bad_shape(tokens, d, ld)) return -1;
    cal_ctx c = {x, tokens, d, ld, lu, gram, f};
    parallel_rows(block_objective, &c, d / 32, threads);
    return 0;
}

/*
 * One step of the per-block (1+1) evolution strategy with the 1/5 success
 * rule (all fp32, in this order):
 *   if fcand < fbest:  theta = cand, fbest = fcand, sigma = min(sigma * 1.5, 0.5)
 *   else:              sigma = max(sigma * 0.90360200 (= 1.5^-1/4), 1e-4)
 *   cand = fma(sigma, noise, theta) per parameter; if any u (parameter 3b+1)
 *   of cand has |u| < 0.1, cand = theta (no move: the next comparison fails).
 */
void kqo_calib_es_update(int64_t nb, float *theta, float *sigma, float *fbest, float *cand,
                         const float *fcand, const float *noise) {
    for (int64_t j = 0; j < nb; ++j) {
        float *th = theta + j * 15, *cd = cand + j * 15;
        const float *nz = noise + j * 15;
        if (fcand[j] < fbest[j]) {
            memcpy(th, cd, 15 * sizeof(float));
            fbest[j] = fcand[j];
            const float s = sigma[j] * 1.5f;
            sigma[j] = s < 0.5f ? s : 0.5f;
        } else {
            const float s = sigma[j] * 0.90360200f;
            sigma[j] = s > 1e-4f ? s : 1e-4f;
        }
        int ok = 1;
        for (int i = 0; i < 15; ++i) {
            cd[i] = fmaf(sigma[j], nz[i], th[i]);
            if (i % 3 == 1 && fabsf(cd[i]) < 0.1f) ok = 0;
        }
        if (!ok) memcpy(cd, th, 15 * sizeof(float));
    }
}

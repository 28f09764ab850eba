/*
 * kq_oracle.h — CPU oracle for the KroQuant online activation quantizer.
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the slow, plain, obviously
 * correct reference that the GPU library is checked against.  It shares no
 * code, header, table or constant with the GPU library.  Only the test suite,
 * the smoke check and the CPU-baseline leg of the benchmark may load it.
 *
 * Sources (cited by page title and section, never by anything else):
 *  [KQ-sum]  "KroQuant: Kronecker-Structured Block Transforms for Efficient
 *            Post-Training Quantization of Diffusion Transformers",
 *            research-map summary page, sections "Problem", "Approach",
 *            "Key results", "Limitations".
 *  [KQ-abs]  the KroQuant abstract (thelatestinai.com paper-card pages).
 *  [LRQ]     "LRQ-DiT: Log-Rotation Post-Training Quantization of Diffusion
 *            Transformers for Image and Video Generation" (arXiv 2508.03485v2),
 *            Sec. 3.2 Eq. (2) and Eq. (3), Sec. 4.3 Lemma 1,
 *            Sec. 5.1 "Implementation Details and Baselines".
 *  [MX]      the pages name the element format only ("W4A4 MXFP4",
 *            "MXFP4e2" in [KQ-sum] and [KQ-abs]).  The element and scale rules
 *            below are the OCP Microscaling (MX) v1.0 definitions of MXFP4:
 *            E2M1 elements, one E8M0 scale per 32 elements.
 *
 * Conventions fixed here (readings of the pages; each is listed in the design
 * notes of the repository):
 *  - Row-vector transform y = x * T, as in [LRQ] Eq. (2) (the activation
 *    is multiplied on the right: XH).
 *  - A block is 32 consecutive channels.  T = F4 (x) F3 (x) F2 (x) F1 (x) F0,
 *    so factor F_b acts on bit b of the in-block channel index.
 *  - A factor is the unit-determinant LU product F = L * U with
 *    L = [[1,0],[l,1]], U = [[u,v],[0,1/u]] and parameters (l,u,v)
 *    ([KQ-sum] "Approach": five 2x2 unit-determinant LU factors, 15
 *    parameters per block).  Parameters are stored params[block][b][0..2] =
 *    (l, u, v).
 *  - Hadamard initialisation ([KQ-sum] "Approach"; [LRQ] Eq. (3)):
 *    (l,u,v) = (1, 1/sqrt2, -1/sqrt2), i.e. F = H2 * diag(1,-1), the
 *    unit-determinant factor closest to the normalised H2 (whose own
 *    determinant is -1).
 *  - MXFP4: scale exponent e = floor(log2(amax)) - 2 clamped to [-127,127],
 *    stored as the byte e+127; 0xFF (NaN) when the block holds NaN or Inf.
 *    Element code = E2M1 round-to-nearest-even of y * 2^-e with saturation
 *    at +-6 and the sign kept (a negative value that rounds to zero is 0x8).
 *  - Packing: codes[t][k/2] holds element k in its low nibble when k is even
 *    and in its high nibble when k is odd; scales[t][j] is block j's byte.
 */
#ifndef KQ_ORACLE_H
#define KQ_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Evaluation modes of the transform. */
enum {
    /* The definition: materialise T (fp64) and form y = x*T in fp64, then
     * round each output once to fp32. */
    KQO_DENSE64 = 0,
    /* The Kronecker factors applied one after another in fp32, in the fixed
     * operation order documented at kqo_block_transform_staged32(). */
    KQO_STAGED32 = 1
};

/* ---- number formats ------------------------------------------------------ */
float    kqo_bf16_to_f32(uint16_t bits);
uint16_t kqo_f32_to_bf16_rne(float f);
double   kqo_e2m1_value(uint8_t code);          /* code in 0..15 */
uint8_t  kqo_e2m1_encode(double q);             /* RNE, saturating, signed zero */
uint8_t  kqo_e8m0_from_amax(float amax);        /* floor rule, 0xFF for NaN/Inf */
double   kqo_e8m0_value(uint8_t byte);          /* 2^(byte-127); NaN for 0xFF */

/* One MXFP4 block: 32 fp32 values -> 16 packed code bytes + 1 scale byte. */
void kqo_mxfp4_block(const float y[32], uint8_t codes[16], uint8_t *scale);

/* ---- the block transform -------------------------------------------------- */
/* F = L(l) * U(u,v) in fp64, F[r*2+c]. */
void kqo_lu_factor(const float p[3], double F[4]);
/* Generic Kronecker product C = A (x) B, all row-major. */
void kqo_kron(const double *A, int ra, int ca, const double *B, int rb, int cb,
              double *C);
/* T = F4 (x) F3 (x) F2 (x) F1 (x) F0 (32x32, row-major, fp64). */
void kqo_block_matrix(const float p[15], double T[1024]);
/* T^-1 = adj(F4) (x) ... (x) adj(F0); adj is the inverse because det F = 1. */
void kqo_block_inverse_matrix(const float p[15], double Ti[1024]);
/* Orthonormal Sylvester Hadamard H_32 by the recursion of [LRQ] Eq. (3). */
void kqo_hadamard32(double H[1024]);
/* Hadamard-initialised parameters (l,u,v) = (1, 1/sqrt2, -1/sqrt2) x 5. */
void kqo_hadamard_init_params(float p[15]);

/* y = x * T for one block. */
void kqo_block_transform_dense64(const float x[32], const float p[15], float y[32]);
void kqo_block_transform_staged32(const float x[32], const float p[15], float y[32]);
/* x = y * T^-1 for one block (inverse transform). */
void kqo_block_inverse_dense64(const float y[32], const float p[15], float x[32]);
void kqo_block_inverse_staged32(const float y[32], const float p[15], float x[32]);

/* ---- tensor drivers --------------------------------------------------------
 * x is bf16 bits, row-major [tokens][ld] with ld >= d, d % 32 == 0.
 * lu is [d/32][5][3].  Outputs are packed: y [tokens][d], codes
 * [tokens][d/2], scales [tokens][d/32].  threads <= 1 runs single-threaded.
 * Return 0 on success, -1 on bad arguments.                                  */
int kqo_transform(const uint16_t *x, int64_t tokens, int64_t d, int64_t ld,
                  const float *lu, int mode, float *y, int threads);
/* Forward-error scale: sum_i |x_i| * |T_ik| in fp64, per output element. */
int kqo_transform_absbound(const uint16_t *x, int64_t tokens, int64_t d, int64_t ld,
                           const float *lu, double *bound, int threads);
int kqo_transform_quant(const uint16_t *x, int64_t tokens, int64_t d, int64_t ld,
                        const float *lu, int mode, uint8_t *codes, uint8_t *scales,
                        int threads);
/* MXFP4 of an fp32 tensor [tokens][d]. */
int kqo_mxfp4_quant(const float *y, int64_t tokens, int64_t d, uint8_t *codes,
                    uint8_t *scales, int threads);
/* Per-channel scaling baseline: y_c = fl32(x_c * mult_c), then MXFP4. */
int kqo_smooth_quant(const uint16_t *x, int64_t tokens, int64_t d, int64_t ld,
                     const float *mult, uint8_t *codes, uint8_t *scales, int threads);
/* Fixed 32-point orthonormal Hadamard baseline y = x * H_32, then MXFP4.
 * DENSE64: fp64 product with the Eq. (3) matrix.  STAGED32: five fp32
 * add/subtract stages (bits 0..4) then one multiply by fl32(1/sqrt(32)). */
int kqo_fwht32(const uint16_t *x, int64_t tokens, int64_t d, int64_t ld, int mode,
               float *y, int threads);
int kqo_fwht32_quant(const uint16_t *x, int64_t tokens, int64_t d, int64_t ld,
                     int mode, uint8_t *codes, uint8_t *scales, int threads);
/* MXFP4 decode: xhat = value(code) * 2^(scale-127) (fp32; exact). */
int kqo_mxfp4_dequant(const uint8_t *codes, const uint8_t *scales, int64_t tokens,
                      int64_t d, float *xhat);
/* Dequantise then undo the block transform, bf16 output (RNE). */
int kqo_dequant_inverse(const uint8_t *codes, const uint8_t *scales, int64_t tokens,
                        int64_t d, const float *lu, int mode, uint16_t *x_out,
                        int threads);
/* Weight side of the invariance (XT)(W T^-T)^T = X W^T ([LRQ] Eq. (2) with
 * an invertible T; [KQ-abs]: the inverse goes to the weights): every
 * 32-channel block of every weight row (K axis) is multiplied by T_j^-T, then
 * quantized to MXFP4 along K.  w bf16 [rows][ld], codes [rows][k/2], scales
 * [rows][k/32].  DENSE64: the fp64 product with the transposed adjugate
 * Kronecker inverse.  STAGED32: see kqo_block_weight_staged32(). */
void kqo_block_weight_dense64(const float w[32], const float p[15], float y[32]);
void kqo_block_weight_staged32(const float w[32], const float p[15], float y[32]);
int kqo_weight_transform(const uint16_t *w, int64_t rows, int64_t k, int64_t ld,
                         const float *lu, int mode, float *y, int threads);
int kqo_weight_quant(const uint16_t *w, int64_t rows, int64_t k, int64_t ld,
                     const float *lu, int mode, uint8_t *codes, uint8_t *scales, int threads);

/* AdaLN-modulated quantizer input ([KQ-sum] "Problem": adaptive LayerNorm
 * in the transformer blocks is why the transform runs online):
 * h = LN(x) * (1 + scale_s) + shift_s, LN over the d channels of a row (no
 * affine part, population variance, eps inside the square root), s = t /
 * rows_per_sample; shift and scale are fp32 [samples][d].  DENSE64 is fp64
 * throughout; STAGED32 follows the fixed fp32 order of the GPU kernel (see
 * the comment at adaln_row() in kq_oracle.c).  kqo_adaln_modulate writes h
 * (fp32; DENSE64 rounds the fp64 value once) and, when the pointers are not
 * NULL, each row's mean and 1/sqrt(var + eps).  kqo_adaln_transform_quant
 * quantizes h * T to MXFP4 (DENSE64: fp64 h and fp64 product, rounded once to
 * fp32 before the MXFP4 decisions).  kqo_adaln_bound is the forward-error
 * scale of STAGED32 against DENSE64 per output element:
 * sum_i (|1 + scale_i| (|n_i| + mean|x| * rstd) + |h_i|) |T_ik|. */
int kqo_adaln_modulate(const uint16_t *x, int64_t tokens, int64_t d, int64_t ld,
                       const float *shift, const float *scale, int64_t rows_per_sample,
                       float eps, int mode, float *h, float *mean, float *rstd, int threads);
int kqo_adaln_transform_quant(const uint16_t *x, int64_t tokens, int64_t d, int64_t ld,
                              const float *shift, const float *scale, int64_t rows_per_sample,
                              float eps, const float *lu, int mode, uint8_t *codes,
                              uint8_t *scales, int threads);
int kqo_adaln_bound(const uint16_t *x, int64_t tokens, int64_t d, int64_t ld,
                    const float *shift, const float *scale, int64_t rows_per_sample, float eps,
                    const float *lu, double *bound, int threads);

/* Calibration of the block parameters ([KQ-sum] "Approach": learned from the
 * Hadamard start with an output loss).  Per block j over the calibration
 * tokens: f_j = sum_t r_t G_j r_t^T with r_t = dequant(MXFP4(x_t T_j)) T_j^-1
 * - x_t; G_j = identity when gram is NULL (fp32 [nb][32][32] otherwise).  The
 * MXFP4 decisions use the fixed-fp32-order transform; the rest is fp64. */
int kqo_calib_objective(const uint16_t *x, int64_t tokens, int64_t d, int64_t ld,
                        const float *lu, const float *gram, double *f, int threads);
/* One step of the per-block (1+1) evolution strategy with the 1/5 success
 * rule; see kq_oracle.c for the exact fp32 operations. */
void kqo_calib_es_update(int64_t nb, float *theta, float *sigma, float *fbest, float *cand,
                         const float *fcand, const float *noise);

/* Y[m][n] = sum_k A[m][k] * W[n][k] in fp64 (A, W fp32 row-major). */
int kqo_matmul_nt(const float *A, const float *W, int64_t M, int64_t N, int64_t K,
                  double *Y, int threads);

#ifdef __cplusplus
}
#endif
#endif /* KQ_ORACLE_H */

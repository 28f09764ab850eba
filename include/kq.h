/*
 * kq.h — C ABI of libkq, the MI355X (gfx950) KroQuant activation quantizer.
 *
 * KroQuant multiplies every 32-channel block of a bf16 activation by a
 * learned invertible 32x32 matrix T_j and quantizes the result to MXFP4
 * (source: "KroQuant: Kronecker-Structured Block Transforms for Efficient
 * Post-Training Quantization of Diffusion Transformers", research-map summary,
 * sections "Problem" and "Approach"; the KroQuant abstract).  T_j is the
 * Kronecker product of five 2x2 unit-determinant LU factors, 15 parameters per
 * block ("Approach").  Because AdaLN/normalisation sits in front of every
 * linear layer, this transform runs online at every denoising step (summary,
 * "Problem"; abstract).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All buffer pointers are DEVICE pointers (HIP global memory) owned by the
 *    caller.  The library never allocates, frees or synchronises; every call
 *    enqueues its kernel on `stream` (a hipStream_t passed as void*, NULL for
 *    the default stream) and returns.  Errors of the asynchronous work surface
 *    at the caller's next synchronisation.  Calls are stateless and may be
 *    issued from several host threads.
 *  - Activations are row-major bf16 [tokens][ld] (element stride 1, row stride
 *    ld elements), of which the first d channels are used; d % 32 == 0.
 *    Channel block j is channels 32j .. 32j+31.
 *  - Transform parameters `lu` are fp32 [d/32][5][3]: for block j and factor
 *    b = 0..4 the triple (l, u, v) of F_b = [[1,0],[l,1]] * [[u,v],[0,1/u]];
 *    T_j = F_4 (x) F_3 (x) F_2 (x) F_1 (x) F_0, so F_b acts on bit b of the
 *    in-block channel index, and y = x * T_j (row vector, as X*H in LRQ-DiT
 *    Sec. 3.2 Eq. (2)).  The Hadamard start of the summary's "Approach" is
 *    (l,u,v) = (1, 1/sqrt2, -1/sqrt2) for every factor.
 *  - MXFP4 output (the pages' W4A4 MXFP4 setting; element and scale rules
 *    of the OCP MX v1.0 format):
 *      codes  uint8 [tokens][d/2]: element k of a row in the low nibble of
 *             byte k/2 when k is even, in the high nibble when k is odd;
 *             each nibble is an E2M1 code (sign<<3 | magnitude index,
 *             magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6).
 *      scales uint8 [tokens][d/32]: E8M0 byte s of block j, value 2^(s-127).
 *    s = clamp(floor(log2(amax)) - 2, -127, 127) + 127 where amax is the
 *    largest |y| of the block (s = 0 for an all-zero block); codes are y*2^-e
 *    rounded to nearest-even on the E2M1 grid, saturating at +-6, sign kept.
 *    A block holding NaN or Inf gets s = 0xFF and all-zero codes.
 *  - Arithmetic is fp32 in a fixed order (see kq_transform_quant), with fp32
 *    denormals kept, so results are deterministic and bit-reproducible.
 *  - Status: validation happens on the host before any HIP call, in the order
 *    shape -> empty (tokens == 0 returns KQ_OK, launches nothing, and may pass
 *    NULL pointers) -> NULL pointers -> alignment.  A failed launch returns
 *    KQ_ERR_HIP.  Nothing throws across this boundary.
 */
#ifndef KQ_H
#define KQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The library is built with hidden visibility; the entry points declared
 * here are its only exported symbols. */
#pragma GCC visibility push(default)

typedef enum kq_status {
    KQ_OK = 0,
    KQ_ERR_NULL = 1,   /* a required pointer is NULL                         */
    KQ_ERR_SHAPE = 2,  /* tokens < 0 or >= 2^31, d <= 0, d % 32, ld < d, ... */
    KQ_ERR_ALIGN = 3,  /* x, codes or a stride not 16-byte aligned, ...      */
    KQ_ERR_HIP = 4     /* the HIP runtime rejected the launch                */
} kq_status;

/* Human-readable name of a status code (static string, never NULL). */
const char *kq_status_str(int status);

/* Library version: major * 10000 + minor * 100 + patch. */
int kq_version(void);

/*
 * kq_transform_quant — the online KroQuant quantizer: y = x * T_j for every
 * (token, block), then MXFP4.  Source: summary "Approach" (Kronecker product
 * of five 2x2 unit-determinant LU factors, 15 parameters per block, Hadamard
 * start); abstract (invertible per-32-element block transform, then MXFP4
 * quantization of the activations).
 *
 *   x       bf16 [tokens][ld_x], 16-byte aligned, ld_x % 8 == 0, ld_x >= d
 *   lu      fp32 [d/32][5][3] (4-byte aligned)
 *   codes   uint8 [tokens][d/2], 16-byte aligned (written)
 *   scales  uint8 [tokens][d/32] (written)
 *
 * Fixed fp32 order (every step one IEEE operation): per block, w_b = u_b*v_b
 * and 1/u_b (IEEE division); for bits b = 0..4 each index pair (i, i|2^b)
 * with bit b of i clear maps (p, q) to r = fma(l_b, q, p), s = fma(w_b, r, q);
 * then y_k = z_k * d_k, d_k the left-to-right product over b = 0..4 of
 * (bit b of k ? 1/u_b : u_b).  This is T = (G_4 (x)...(x) G_0)(D_4 (x)...(x) D_0)
 * with F_b = G_b D_b, G_b = [[1,w],[l,1+l*w]], D_b = diag(u, 1/u).
 */
kq_status kq_transform_quant(const void *x, int64_t tokens, int64_t d, int64_t ld_x,
                             const float *lu, uint8_t *codes, uint8_t *scales,
                             void *stream);

/*
 * kq_transform_quant_mfma — the same quantizer with the block transform run
 * as a dense 32x32 product on the matrix cores, the formulation of the
 * KroQuant summary (Approach: one matrix-core GEMM per block) and
 * abstract (small matrix-core GEMMs).  Same arguments, layouts and errors
 * as kq_transform_quant.  T_j is materialised in fp32 and split into three
 * bf16 terms; the products accumulate in fp32 in the matrix core's own order,
 * so values agree with the exact y = x * T_j to within fp32 rounding (not
 * bit-for-bit with kq_transform_quant), and codes may differ from it only at
 * E2M1 rounding ties.
 */
kq_status kq_transform_quant_mfma(const void *x, int64_t tokens, int64_t d, int64_t ld_x,
                                  const float *lu, uint8_t *codes, uint8_t *scales,
                                  void *stream);

/*
 * kq_transform_quant_quad — the same quantizer with another work split:
 * four lanes per unit (token, block), each holding 8 consecutive elements,
 * the in-block index bits 3 and 4 exchanged between the lanes of a quad by
 * DPP permutations (every wave load reads 1 KB of contiguous input).  Same
 * transform (KroQuant summary, "Approach"), same fixed fp32 order and the
 * same outputs, bit for bit, as kq_transform_quant; kept as the measured
 * alternative layout.  Same arguments, layouts and errors as
 * kq_transform_quant, and KQ_ERR_SHAPE when tokens * d/32 >= 2^31 - 256.
 */
kq_status kq_transform_quant_quad(const void *x, int64_t tokens, int64_t d, int64_t ld_x,
                                  const float *lu, uint8_t *codes, uint8_t *scales,
                                  void *stream);

/*
 * kq_transform_f32 — the same device transform as kq_transform_quant with an
 * fp32 store instead of the quantizer: y fp32 [tokens][d], 16-byte aligned.
 * For checking the transform stage on its own.
 */
kq_status kq_transform_f32(const void *x, int64_t tokens, int64_t d, int64_t ld_x,
                           const float *lu, float *y, void *stream);

/*
 * kq_smooth_quant — per-channel scaling baseline (SmoothQuant, named as the
 * baseline in the summary's "Key results" and in the abstract):
 * y_c = x_c * mult_c (one fp32 multiply), then MXFP4 as above.
 *   mult  fp32 [d], 16-byte aligned.
 */
kq_status kq_smooth_quant(const void *x, int64_t tokens, int64_t d, int64_t ld_x,
                          const float *mult, uint8_t *codes, uint8_t *scales,
                          void *stream);

/*
 * kq_fwht32_quant — fixed 32-point Hadamard baseline (summary "Surprising
 * findings" and "Experimental setup": Hadamard 32x32 block transform, FWHT):
 * y = x * H_32 with H_32 the orthonormal Sylvester matrix of LRQ-DiT
 * Sec. 3.2 Eq. (3), computed as five add/subtract stages over bits 0..4,
 * (p, q) -> (p + q, p - q), then one multiply by fl32(1/sqrt(32)); then MXFP4.
 */
kq_status kq_fwht32_quant(const void *x, int64_t tokens, int64_t d, int64_t ld_x,
                          uint8_t *codes, uint8_t *scales, void *stream);

/*
 * kq_mxfp4_quant_f32 — MXFP4 of an fp32 tensor without a transform (the
 * quantizer stage alone).  y fp32 [tokens][ld_y], 16-byte aligned,
 * ld_y % 4 == 0.
 */
kq_status kq_mxfp4_quant_f32(const float *y, int64_t tokens, int64_t d, int64_t ld_y,
                             uint8_t *codes, uint8_t *scales, void *stream);

/*
 * kq_weight_quant — weight preparation for the W4A4 consumer: every
 * 32-channel block (along K) of every weight row is multiplied by T_j^-T and
 * the result is quantized to MXFP4 along K, so that
 * (X T)(W T^-T)^T = X W^T (LRQ-DiT Sec. 3.2 Eq. (2) with an invertible T;
 * KroQuant abstract: the inverse transform goes to the weights).  Runs once
 * per weight matrix, offline.
 *
 *   w       bf16 [rows = N][ld_w] (row-major, K = k contiguous), as for x
 *   lu      fp32 [k/32][5][3], the activation side's parameters
 *   codes   uint8 [rows][k/2], scales uint8 [rows][k/32] (written)
 *
 * Fixed fp32 order: for bits b = 0..4 each pair (p, q) maps to
 * s = fma(-l_b, p, q), r = fma(-w_b, s, p); then y_k = z_k * e_k with e_k the
 * left-to-right product over b = 0..4 of (bit b of k ? u_b : 1/u_b).
 */
kq_status kq_weight_quant(const void *w, int64_t rows, int64_t k, int64_t ld_w,
                          const float *lu, uint8_t *codes, uint8_t *scales, void *stream);

/*
 * kq_dequant_inverse — the inverse side: decode MXFP4 and undo the block
 * transform, x = dequant(codes, scales) * T_j^-1, rounded to bf16 (nearest
 * even).  The transform is invertible with unit determinant (KroQuant
 * summary, "Approach"; abstract: the activations take the invertible
 * transform and the weights its inverse).
 *
 *   codes   uint8 [tokens][d/2], 16-byte aligned (layout as above)
 *   scales  uint8 [tokens][d/32]
 *   lu      fp32 [d/32][5][3], the parameters that produced the codes
 *   x_out   bf16 [tokens][ld_out], 16-byte aligned, ld_out % 8 == 0 (written)
 *
 * Fixed fp32 order: the decoded value is code value * 2^(s-127) (exact; a
 * 0xFF scale makes the whole block NaN); then z_k = y_k * e_k, e_k the
 * left-to-right product over b = 0..4 of (bit b of k ? u_b : 1/u_b); then bits
 * b = 4..0 map each pair (r, s) to q = fma(-w_b, r, s), p = fma(-l_b, q, r).
 */
kq_status kq_dequant_inverse(const uint8_t *codes, const uint8_t *scales, int64_t tokens,
                             int64_t d, const float *lu, void *x_out, int64_t ld_out,
                             void *stream);

/*
 * kq_w4a4_gemm — the W4A4 consumer of the quantized activations:
 * Y = dequant(A) * dequant(W)^T with fp32 accumulation and bf16 output
 * (nearest even), on the gfx950 block-scaled matrix cores (E2M1 operands,
 * E8M0 scales).  The pages' setting is W4A4 MXFP4 (KroQuant summary and
 * abstract): A from kq_transform_quant, W from kq_weight_quant, so
 * that Y approximates X * W_original^T (LRQ-DiT Sec. 3.2 Eq. (2)).
 *
 *   a_codes uint8 [M][K/2] (16-byte aligned), a_scales uint8 [M][K/32] (4-byte aligned)
 *   w_codes uint8 [N][K/2] (16-byte aligned), w_scales uint8 [N][K/32] (4-byte aligned)
 *   y       bf16 [M][ld_y], 16-byte aligned, ld_y % 8 == 0, ld_y >= N (written)
 *
 * K % 128 == 0; M and N are arbitrary, with max(M, N) * K/2 < 2^31 (one
 * operand's codes under 2 GiB).  M == 0 or N == 0 returns KQ_OK.
 * One of three kernels runs, by shape and alignment: with K % 256 == 0 and
 * at least two 256 x 256 output tiles per compute unit, 256 x 256 tiles;
 * otherwise, with K % 512 == 0 and both scale arrays 16-byte aligned,
 * 128 x 256 tiles with the K pipeline continuing across output tiles;
 * otherwise 128 x 256 tiles one at a time.  All three accumulate every
 * output over K in the same order (one MFMA per 64 K values, in K order), so
 * the choice does not change the result.
 * KQ_ERR_HIP also if the library was built so that the kernel needs scratch
 * memory (its load waits count its own loads and would be wrong then).
 */
kq_status kq_w4a4_gemm(const uint8_t *a_codes, const uint8_t *a_scales,
                       const uint8_t *w_codes, const uint8_t *w_scales, int64_t M, int64_t N,
                       int64_t K, void *y, int64_t ld_y, void *stream);

/*
 * kq_adaln_transform_quant — the quantizer fused with the adaptive LayerNorm
 * that produces its input in a diffusion-transformer block (KroQuant summary,
 * "Problem": AdaLN blocks are why the transform runs online).  One pass:
 *   h = LN(x) * (1 + scale_s) + shift_s,  then y = h * T_j and MXFP4(y),
 * LN over the d channels of each row with no affine part, population
 * variance and eps inside the square root; row t belongs to sample
 * s = t / rows_per_sample.  The modulated tensor is never stored.
 *
 *   x        bf16 [tokens][ld_x], 16-byte aligned, ld_x % 8 == 0
 *   shift    fp32 [ceil(tokens / rows_per_sample)][d], 16-byte aligned
 *   scale    fp32, same shape (the modulation multiplies by 1 + scale)
 *   rows_per_sample >= 1; eps >= 0 and finite
 *   lu, codes, scales as for kq_transform_quant
 *
 * d % 32 == 0 and d <= 8192 (one sample's modulation vectors are staged in
 * LDS); anything else returns KQ_ERR_SHAPE.
 * Fixed fp32 order (results reproducible bit for bit): per 32-value block a
 * sequential sum; per row, 64 lanes where lane l starts from block l's sum
 * (0 when l >= d/32) and adds blocks l + 64, l + 128, ... in turn, then for
 * m = 1, 2, 4, 8, 16, 32 every lane adds lane l ^ m's value; mean = total / d;
 * c = x - mean; per block q = fma(c, c, q) from q = 0 over the 32 values in
 * order, row total as before, var = total / d; rstd = 1 / sqrt(var + eps);
 * h = fma(c * rstd, 1 + scale, shift); then the transform in the order of
 * kq_transform_quant.
 */
kq_status kq_adaln_transform_quant(const void *x, int64_t tokens, int64_t d, int64_t ld_x,
                                   const float *shift, const float *scale,
                                   int64_t rows_per_sample, float eps, const float *lu,
                                   uint8_t *codes, uint8_t *scales, void *stream);

/*
 * kq_adaln_modulate — the same modulation alone, h rounded to bf16 (nearest
 * even): the first kernel of the unfused pipeline (modulate, then
 * kq_transform_quant), kept for comparison and for callers that need h.
 *   h   bf16 [tokens][ld_h], 16-byte aligned, ld_h % 8 == 0, ld_h >= d (written)
 * Other arguments and the operation order as for kq_adaln_transform_quant.
 */
kq_status kq_adaln_modulate(const void *x, int64_t tokens, int64_t d, int64_t ld_x,
                            const float *shift, const float *scale, int64_t rows_per_sample,
                            float eps, void *h, int64_t ld_h, void *stream);

/*
 * kq_calib_objective — calibration objective of every block (KroQuant
 * summary, "Approach": the factors are learned layer-wise from the Hadamard
 * start with an output loss; the loss and optimiser are not given, so this
 * library takes the quantizer's own error):
 *   f_j = sum_t r_t G_j r_t^T,  r_t = dequant(MXFP4(x_t T_j)) T_j^-1 - x_t,
 * over the tokens of a calibration set, x_t the 32 values of block j.
 *
 *   x      bf16 [tokens][ld_x], as for kq_transform_quant
 *   lu     fp32 [d/32][5][3], the parameters to score (one candidate per block)
 *   gram   fp32 [d/32][32][32] weighting G_j, or NULL for the identity (the
 *          round-trip error); W_j^T W_j gives the block-diagonal part of the
 *          output error of X W^T
 *   f      fp32 [d/32] (written)
 *
 * The MXFP4 decisions and both transforms follow the quantizer's fixed fp32
 * orders; per-thread fp32 sums are reduced in a fixed order, so the value is
 * reproducible bit for bit.  tokens == 0 writes zeros.
 */
kq_status kq_calib_objective(const void *x, int64_t tokens, int64_t d, int64_t ld_x,
                             const float *lu, const float *gram, float *f, void *stream);

/*
 * kq_calib_es_update — one step of the per-block (1+1) evolution strategy
 * with the 1/5 success rule, on device arrays (fp32, in place):
 *   theta [nb][15] kept parameters, sigma [nb] step sizes, fbest [nb] kept
 *   objectives, cand [nb][15] the candidate just scored (replaced by the next
 *   one), fcand [nb] its objective, noise [nb][15] standard normal draws.
 * If fcand < fbest the candidate is kept and sigma grows by 1.5 (at most 0.5);
 * otherwise sigma shrinks by 1.5^-1/4 = 0.90360200 (at least 1e-4).  The next
 * candidate is fma(sigma, noise, theta), or theta itself when any u would
 * fall within 0.1 of zero.
 */
kq_status kq_calib_es_update(int64_t nb, float *theta, float *sigma, float *fbest, float *cand,
                             const float *fcand, const float *noise, void *stream);

/*
 * kq_calib_es_step — one whole iteration of the calibration in one launch:
 * the same result, bit for bit, as kq_calib_objective on cand (writing
 * fcand) followed by kq_calib_es_update with that fcand, for every block.
 * The update of block j depends only on block j's objective, so each block's
 * workgroup applies it as soon as its own sum is known.
 *   x, tokens, d, ld_x, gram   as for kq_calib_objective
 *   theta, sigma, fbest, cand, noise   as for kq_calib_es_update, nb = d/32
 *   fhist  fp32 [d/32] (written with the kept objectives after the update),
 *          or NULL
 * The candidate's objective itself is not stored.  Errors as for the two
 * separate calls.
 */
kq_status kq_calib_es_step(const void *x, int64_t tokens, int64_t d, int64_t ld_x,
                           const float *gram, float *theta, float *sigma, float *fbest,
                           float *cand, const float *noise, float *fhist, void *stream);

/*
 * kq_calib_es_run — `iterations` calls of kq_calib_es_step issued from the
 * library in one call, so a long calibration is not paced by the caller's
 * per-launch overhead:
 *   noise  fp32 [iterations][d/32][15]; iteration i uses noise + i*(d/32)*15
 *   fhist  fp32 [iterations][d/32], row i written after iteration i, or NULL
 * Other arguments as for kq_calib_es_step.  iterations == 0 does nothing;
 * iterations < 0 or above 2^24 is KQ_ERR_SHAPE.  The launches are queued on
 * `stream` and the call returns without waiting.  If a launch fails,
 * KQ_ERR_HIP is returned and the state holds the iterations queued before it.
 */
kq_status kq_calib_es_run(const void *x, int64_t tokens, int64_t d, int64_t ld_x,
                          const float *gram, float *theta, float *sigma, float *fbest, float *cand,
                          const float *noise, int64_t iterations, float *fhist, void *stream);

/*
 * kq_copy_ceiling — not a quantizer: moves the same bytes as
 * kq_transform_quant (reads the bf16 tensor, writes d/2 + d/32 bytes per row)
 * with almost no arithmetic, to measure the achievable bandwidth of this
 * access pattern.  Output bytes are a fold of the input, not MXFP4.
 */
kq_status kq_copy_ceiling(const void *x, int64_t tokens, int64_t d, int64_t ld_x,
                          uint8_t *codes, uint8_t *scales, void *stream);

/*
 * kq_stream_ceiling — not a quantizer: an HBM reference with the
 * quantizer's byte counts and a wave-contiguous access pattern of its own
 * (each wave reads 4 KB as four 1 KB loads and writes 1 KB + 64 B), for
 * measuring what the memory system sustains independently of the
 * quantizer's one-lane-per-unit mapping.
 *   src     16-byte aligned, units * 64 bytes, read
 *   codes   units * 16 bytes (16-byte aligned), written with a fold of the
 *           input; NULL for a read-only pass
 *   scales  units bytes, written; for a read-only pass at least 1 byte, of
 *           which byte 0 may be written
 * 0 <= units <= 2^36; units == 0 returns KQ_OK.  Output bytes are no
 * quantization.
 */
kq_status kq_stream_ceiling(const void *src, int64_t units, uint8_t *codes, uint8_t *scales,
                            void *stream);

#pragma GCC visibility pop

#ifdef __cplusplus
}
#endif
#endif /* KQ_H */

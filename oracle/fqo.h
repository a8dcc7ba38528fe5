/*
 * FoldQuant CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU implementation of what the FoldQuant
 * integer linear layer computes, written from the vla.cpp pull request page
 * "FoldQuant W8A8/W4A4 inference and FoldQuantVLA quantized-model converter"
 * (its runtime summary, the dequant-mode commit that defines the fold algebra,
 * and the OpenVINO commit that lists the act-node steps).  Only the tests, the
 * package's smoke check and the benchmark's CPU-baseline leg may load it.  It
 * shares no code, header, table or helper with the HIP library.
 *
 * Readings of the pages that the functions below fix (each is listed with its
 * justification in the design notes of the repository):
 *   - R_b = blockdiag(H_b)/sqrt(b) over contiguous blocks of b along K, H_b the
 *     Sylvester Hadamard matrix in natural order, H_b[i][j] = (-1)^popcount(i&j).
 *     The butterfly runs its stages with span 1, 2, 4, ..., b/2 in that order and
 *     then multiplies by the float32 value nearest to 1/sqrt(b).
 *   - Codes are symmetric: +-127 for 8 bits, +-7 for 4 bits ("15 activation
 *     levels"); rounding is half-to-even; scale = amax / qmax.
 *   - 4-bit codes are packed two per byte, the even k in the low nibble.
 *   - The activation prologue computes in float32 (IEEE divide and sqrt, no
 *     contraction), except the sum of squares of the RMSNorm, which adds the
 *     exact float32 squares in float64; mean = (float)(sum / K).
 *   - The weight packer computes in float64; the stored per-row scale is the
 *     float32 rounding of max|u|/qmax and the codes are rounded against it.
 *   - The epilogue computes acc * s_a * s_w (+ bias) (+ residual) in float64
 *     and rounds once to bfloat16, nearest-even.
 *
 * All functions are synchronous and return 0 on success, a negative value on
 * a bad argument (nothing written) and, for fqo_gemm_i32, 1 when a sum does not
 * fit in int32.
 */
#ifndef FQO_H
#define FQO_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* H_b entry (-1)^popcount(i & j); b a power of two, 0 <= i, j < b. */
int fqo_hadamard_entry(int32_t b, int32_t i, int32_t j);

/* In-place R_b on a float64 vector of length n (n % b == 0): butterfly then 1/sqrt(b). */
int fqo_rotate_f64(double* v, int64_t n, int32_t b);

/* In-place unnormalised butterfly (H_b per block) in float32, stage order 1..b/2. */
int fqo_butterfly_f32(float* v, int64_t n, int32_t b);

/* gamma' = gamma / a in float32 (norm sites carry the smoothing vector in the gain). */
int fqo_fold_gain(const float* gamma, const float* ascale, int32_t K, float* gamma_out);

/* Folded weight rows in float64 (no quantisation):
 *   fold_after == 0: u_n = R_b(a (.) w_n);  fold_after == 1: u_n = a (.) R_b(w_n).
 * ascale may be NULL (a = 1).  W [N][K] float32, U [N][K] float64. */
int fqo_fold_weights(const float* W, int32_t N, int32_t K, const float* ascale,
                     int32_t fold_after, int32_t hblock, double* U);

/* Weight packer: fold as above, then per-row s_n = (float)(max|u|/qmax),
 * q = clamp(rint(u / s_n), -qmax, qmax); codes [N][K] int8 (wbits 8) or
 * [N][K/2] bytes (wbits 4). */
int fqo_pack_weights(const float* W, int32_t N, int32_t K, const float* ascale,
                     int32_t fold_after, int32_t hblock, int32_t wbits,
                     void* codes, float* wscale);

/* Dequantised weight rows in the original frame, float64:
 *   fold_after == 0: W_n = R_b(s_n q_n) / a;  fold_after == 1: W_n = R_b(s_n q_n / a). */
int fqo_unfold_weights(const void* codes, const float* wscale, int32_t N, int32_t K,
                       const float* ascale, int32_t fold_after, int32_t hblock,
                       int32_t wbits, double* Wout);

/* Activation frame before quantisation (float32): RMSNorm with the folded gain
 * (gamma NULL: no norm), explicit a before or after the rotation (ascale NULL:
 * none), rotation.  x [M][ldx] bf16 bits, h [M][K]. */
int fqo_act_frame(const uint16_t* x, int32_t M, int32_t K, int64_t ldx,
                  const float* gamma, float eps, const float* ascale, int32_t fold_after,
                  int32_t hblock, float* h);

/* Full prologue: frame as above, then per-token amax, s_m = amax/qmax,
 * q = clamp(rint(h/s_m)).  codes [M][K] int8 or [M][K/2] bytes; act_scale [M]. */
int fqo_prologue(const uint16_t* x, int32_t M, int32_t K, int64_t ldx,
                 const float* gamma, float eps, const float* ascale, int32_t fold_after,
                 int32_t hblock, int32_t abits, void* codes, float* act_scale);

/* Integer contraction acc[m][n] = sum_k qa[m][k] * qw[n][k] (exact, int64, then
 * checked to fit int32).  Returns 1 (acc still written, saturated) on overflow. */
int fqo_gemm_i32(const void* act_codes, int32_t M, int32_t abits,
                 const void* w_codes, int32_t N, int32_t K, int32_t wbits, int32_t* acc);

/* Epilogue: y = bf16_rne(acc * s_a[m] * s_w[n] + bias[n] + residual[m][n]) from
 * float64.  bias / residual may be NULL.  y_f64 (optional) receives the
 * value before rounding. */
int fqo_epilogue(const int32_t* acc, int32_t M, int32_t N, const float* act_scale,
                 const float* wscale, const float* bias, const uint16_t* residual,
                 int64_t ldr, uint16_t* y, double* y_f64);

/* Nearest-even bfloat16 of a float64 value (one rounding). */
uint16_t fqo_bf16_from_f64(double v);

/* GeGLU of a gate+up output row [gate F | up F] (bf16) into h (bf16):
 * h = bf16_rne(gelu_tanh(gate) * up) from float64; h_f64 (optional) receives
 * the value before rounding. */
int fqo_geglu(const uint16_t* gu, int32_t M, int32_t F, int64_t ld_in, uint16_t* h, int64_t ld_out,
              double* h_f64);

/* Threads the oracle's parallel loops use (OpenMP max threads). */
int fqo_num_threads(void);

/* Integer value of code k of a row (int8 or packed 4-bit). */
int32_t fqo_code_at(const void* row, int32_t k, int32_t bits);

#ifdef __cplusplus
}
#endif
#endif

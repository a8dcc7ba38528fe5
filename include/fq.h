/*
 * fq.h -- C ABI of libfq, FoldQuant integer linear layers on AMD Instinct MI355X (gfx950).
 *
 * The operation is the FoldQuant linear site of the vla.cpp pull request page
 * "FoldQuant W8A8/W4A4 inference and FoldQuantVLA quantized-model converter":
 *
 *   prologue (the page's "act" node; OpenVINO commit lists its steps):
 *     f  = float(x_m)                                   bf16 token, widened exactly
 *     r  = f * (1/sqrt(mean(f^2) + eps)) * gamma'       RMSNorm with the folded gain
 *                                                       (skipped when gamma' is NULL)
 *     r  = r / a            (explicit smoothing, fold before; dequant-mode commit)
 *     h  = R_b r            R_b = blockdiag(H_b)/sqrt(b), Sylvester H_b, contiguous blocks
 *     h  = h / a            (explicit smoothing, fold after)
 *     s_m = max|h| / qmax;  q = clamp(round_half_even(h / s_m), -qmax, qmax)
 *   GEMM (the page's "gemm" node): acc[m][n] = sum_k q_a[m][k] * q_w[n][k] (exact int32)
 *   epilogue: y[m][n] = bf16_rne(acc * (s_m * s_n) [+ bias[n]] [+ residual[m][n]])
 *
 * qmax is 127 for 8-bit codes and 7 for 4-bit codes (the page's "15 activation
 * levels").  4-bit codes are packed two per byte with the even k in the low
 * nibble.  Code width FQ_CODES_E2M3 (6) is a second storage of the same 4-bit
 * codes (see below).  Weight rows are folded into the same frame on the host by
 * fq_pack_weights: u_n = R_b(a . w_n) (fold before) or a . R_b(w_n) (fold
 * after), then per-row symmetric round-to-nearest-even with s_n = max|u_n|/qmax.
 *
 * Arithmetic of the prologue: float32 with IEEE divide and sqrt and no
 * contraction; the RMSNorm sum of squares adds the (exact) float32 squares in
 * float64 and mean = (float)(sum / K); the butterfly runs its stages with span
 * 1, 2, ..., b/2 and then multiplies by (float)(1/sqrt(b)).  The epilogue runs in
 * float32 with one round-to-nearest-even to bf16.
 *
 * Conventions for every entry point
 *   - Status codes: FQ_OK on success.  On any failure the call returns a code,
 *     sets a thread-local message (fq_last_error) that names the call, the
 *     argument and the arithmetic, writes nothing and queues no device work.
 *     The one exception is a launch refused by the HIP runtime after an
 *     earlier launch of the same call was queued (fq_linear's GEMM after its
 *     prologue): FQ_ERR_DEVICE then reports it, and the workspace may hold
 *     the prologue's codes.  Every host-side step that can fail runs before
 *     the first launch.  No C++ exception crosses this ABI; nothing aborts.
 *   - Ownership: the caller allocates and frees every buffer.  The library
 *     allocates no device memory and never synchronises.  Inputs are read
 *     only; outputs are overwritten.
 *   - State kept by the library: the thread-local error message; per device,
 *     a record made once per process on the first device call there (or by
 *     fq_device_init): the compute-unit and LDS sizes, and the streaming
 *     GEMV kernels' register-limited residency after raising their
 *     dynamic-LDS limit, and the address of its fq_linear_noalloc scratch
 *     array; and the process-wide test hooks (fq_test_hook).
 *     No call depends on an earlier call's data.
 *   - Device entry points are asynchronous on `stream` (a hipStream_t passed as
 *     void*; NULL is the null stream) and take device pointers.
 *   - Shapes: M, N >= 1; N a multiple of 8; K <= 65536, a multiple of 32 for
 *     fq_prologue (of 64 when K > 32768) and of 128 for fq_pack_weights,
 *     fq_dequant_rows, fq_gemm and fq_linear;
 *     hblock a power of two in [1, 256] dividing K (1 = no rotation); bits in
 *     {4, 8} for both weights and activations (W8A8, W4A4, W4A8, W8A4), or 6
 *     (FQ_CODES_E2M3) for both of a GEMM's operands.
 *   - Alignment: bf16 rows (x, residual, y) need a 16-byte aligned base and a
 *     leading dimension that is a multiple of 8 elements; code buffers, gamma,
 *     ascale, scales and bias need a 16-byte aligned base.
 *   - Inputs must be finite.  A token (or weight row) whose scale is zero, or
 *     underflows to zero, gets all-zero codes.
 */
#ifndef FQ_H
#define FQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FQ_ABI_VERSION 2

/* Code width 6: the 4-bit codes (integers in [-7, 7], qmax 7, quantised exactly
 * as with width 4) stored as OCP FP6 E2M3 numbers -- sign bit 5, exponent bits
 * 4..3 with bias 1, mantissa bits 2..0 -- which hold each of those integers
 * exactly.  Value k of a row occupies bits 6k .. 6k+5 of the row's bytes read
 * as one little-endian bit string: 3K/4 bytes per row.  In this form a W4A4
 * GEMM runs on gfx950's FP6 matrix instruction (v_mfma_scale_f32_16x16x128_f8f6f4,
 * twice the rate of the int8 one) with float32 sums that stay exact integers
 * (|sum| <= 49 K < 2^24), so its results equal the 4-bit path's bit for bit.
 * Accepted by fq_pack_weights, fq_dequant_rows, fq_prologue, and by the GEMM
 * entry points when both abits and wbits are 6 (mixing 6 with 4 or 8 is
 * FQ_ERR_UNSUPPORTED).  Every M runs on the tiled kernel: for decode-sized M
 * the 4-bit storage streams a third fewer weight bytes. */
#define FQ_CODES_E2M3 6

typedef enum {
    FQ_OK = 0,
    FQ_ERR_ARG = 1,          /* NULL pointer or out-of-range scalar */
    FQ_ERR_SHAPE = 2,        /* M, N, K, leading dimensions or hblock inconsistent */
    FQ_ERR_UNSUPPORTED = 3,  /* a bit width or size this build does not handle */
    FQ_ERR_ALIGN = 4,        /* pointer or leading dimension misaligned */
    FQ_ERR_DEVICE = 5        /* a HIP call failed; the message holds hipGetErrorString */
} fq_status;

/* Message of the last failed call on this thread ("" if none).  Valid until the
 * next fq_* call on the same thread. */
const char* fq_last_error(void);

/* FQ_ABI_VERSION of the built library. */
int fq_abi_version(void);

/* Optional set-up of the current HIP device: the per-device record described
 * under "State kept by the library" above.  Every device entry point makes it
 * itself on its first call on a device; calling this first keeps those HIP
 * queries (attribute, occupancy) out of a graph capture that would otherwise
 * contain the first call.  Idempotent; FQ_ERR_DEVICE if a query fails. */
fq_status fq_device_init(void);

/* Test hook, for the tests only: forces kernel choices that the shape would
 * not get, so that every kernel variant can be checked against the oracle.
 * spec: comma-separated key=value items, each call replacing the whole hook
 * state; "" or NULL restores the defaults.
 *   gemm_tile=<128x128|128x144|128x112|128x96|64x128|64x224|64x256|64x288|64x128x2|auto>
 *   gemm_mfma=<16|32>     (8-bit x 8-bit codes on v_mfma_i32_32x32x32_i8 with 32)
 *   gemv=<split|auto>     (decode-sized M always on the split-K GEMV kernel)
 *   decode1=<off|auto>    (one-token fq_linear as two launches, not the fused kernel)
 * The environment variable FQ_TEST_HOOK, read once per process at the hooks'
 * first use, takes the same spec.  FQ_ERR_ARG on an unknown key or value (state kept).
 * Process-wide; a call while another thread launches races with it. */
fq_status fq_test_hook(const char* spec);

/* ------------------------------------------------------------------ host, synchronous */

/* Bytes of one code matrix of rows x K codes at `bits` bits (rows*K, rows*K/2,
 * or rows*3K/4 for FQ_CODES_E2M3); 0 on bad arguments. */
size_t fq_weight_bytes(int32_t N, int32_t K, int32_t wbits);
size_t fq_act_bytes(int32_t M, int32_t K, int32_t abits);

/* gamma_out[k] = gamma[k] / ascale[k] in float32 (host).  Norm sites carry the
 * smoothing vector inside the RMSNorm gain (dequant-mode commit of the page).
 * ascale NULL copies gamma. */
fq_status fq_fold_gain(const float* gamma, const float* ascale, int32_t K, float* gamma_out);

/* Host weight packer (the page's converter and bring-up export: rotation and
 * per-row round-to-nearest, no calibration).
 *   W          host float32 [N][K], nn.Linear layout (row n = output feature n)
 *   ascale     host float32 [K] smoothing vector, or NULL (a = 1)
 *   fold_after 0: u_n = R_b(a . w_n); 1: u_n = a . R_b(w_n) -- must match the
 *              prologue's fold order (or the gain fold, which is fold before)
 *   hblock     Hadamard block b (1 = no rotation)
 *   codes_out  host, fq_weight_bytes(N, K, wbits) bytes: int8 [N][K], packed [N][K/2],
 *              or E2M3 [N][3K/4] (wbits 6)
 *   wscale_out host float32 [N]: s_n = (float)(max|u_n| / qmax)
 * The fold runs in float64; codes are rounded (ties to even) against the stored
 * float32 scale and clamped to +-qmax. */
fq_status fq_pack_weights(const float* W, int32_t N, int32_t K, const float* ascale,
                          int32_t fold_after, int32_t hblock, int32_t wbits,
                          void* codes_out, float* wscale_out);

/* Dequantised float weight rows in the original frame: the page's dequant mode,
 * which rebuilds every site as a float GEMM weight for backends without the
 * integer nodes (dequant-mode commit: row n of the float weight is R(w_n)/a or
 * R(w_n/a)).  With v = wscale[n] * q_n (the stored codes):
 *   fold_after 0: W_out[n] = R_b(v) / a      fold_after 1: W_out[n] = R_b(v / a)
 * which undoes fq_pack_weights' fold exactly (R_b is its own inverse), leaving
 * only the rounding of the codes.  ascale NULL means a = 1; at norm sites the
 * smoothing vector lives in the folded gain, so there the float path uses the
 * folded gain with these rows.
 *   codes, wscale  host, as written by fq_pack_weights (same N, K, hblock, wbits)
 *   W_out          host float32 [N][K]
 * Float64 inside, one rounding to float32.  Same argument rules as
 * fq_pack_weights; wscale must be finite and >= 0. */
fq_status fq_dequant_rows(const void* codes, const float* wscale, int32_t N, int32_t K,
                          const float* ascale, int32_t fold_after, int32_t hblock, int32_t wbits,
                          float* W_out);

/* ------------------------------------------------------------------ device, asynchronous */

/* Prologue: quantise M bf16 tokens into codes and per-token scales.
 *   x_bf16       device bf16 [M][ldx]
 *   gamma_folded device float32 [K] (gamma / a at norm sites) or NULL: no RMSNorm
 *   eps          RMSNorm epsilon (ignored without gamma)
 *   ascale       device float32 [K] explicit smoothing divide, or NULL
 *   fold_after   0: divide before the rotation; 1: after it
 *   act_codes    device, fq_act_bytes(M, K, abits) bytes, row stride K, K/2 or 3K/4 bytes
 *   act_scale    device float32 [M] */
fq_status fq_prologue(const void* x_bf16, int32_t M, int32_t K, int64_t ldx,
                      const float* gamma_folded, float eps, const float* ascale,
                      int32_t fold_after, int32_t hblock, int32_t abits,
                      void* act_codes, float* act_scale, void* stream);

/* Integer GEMM with the fused epilogue (the page's gemm node: integer GEMM,
 * per-row weight scale, residual add).
 *   act_codes/act_scale  device, as written by fq_prologue (row stride K or K/2 bytes)
 *   w_codes/wscale       device, as written by fq_pack_weights
 *   bias                 device float32 [N] or NULL
 *   residual_bf16        device bf16 [M][ldr] or NULL
 *   y_bf16               device bf16 [M][ldy]
 *   acc_i32              device int32 [M][N] (row stride N) receiving the exact
 *                        accumulators, or NULL (diagnostic output)
 * M <= 32 runs the weight-streaming GEMV kernel, larger M the tiled MFMA kernel;
 * both give identical results.  E2M3 codes (abits = wbits = 6) run the FP6
 * tiled kernel for every M, with the same results as the 4-bit codes. */
fq_status fq_gemm(const void* act_codes, const float* act_scale, int32_t M, int32_t abits,
                  const void* w_codes, const float* wscale, int32_t N, int32_t K, int32_t wbits,
                  const float* bias, const void* residual_bf16, int64_t ldr,
                  void* y_bf16, int64_t ldy, int32_t* acc_i32, void* stream);

/* Workspace of fq_linear: the activation codes and scales (256-byte aligned parts). */
size_t fq_linear_workspace_bytes(int32_t M, int32_t K, int32_t abits);

/* Prologue then GEMM on one stream; arguments as in fq_prologue and fq_gemm.
 * workspace: device, at least fq_linear_workspace_bytes(M, K, abits) bytes,
 * 256-byte aligned; it holds the codes and scales after the call.  A single
 * token (M = 1, K <= 4096, hblock 32, 64 or 128) runs as one launch in which
 * every workgroup quantises the token while its weight loads are in flight;
 * codes, scale and outputs are those of the two launches, bit for bit. */
fq_status fq_linear(const void* x_bf16, int32_t M, int32_t K, int64_t ldx,
                    const float* gamma_folded, float eps, const float* ascale,
                    int32_t fold_after, int32_t hblock, int32_t abits,
                    const void* w_codes, const float* wscale, int32_t N, int32_t wbits,
                    const float* bias, const void* residual_bf16, int64_t ldr,
                    void* y_bf16, int64_t ldy,
                    void* workspace, size_t workspace_bytes, void* stream);

/* fq_linear without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation).  The codes and scales that pass from the prologue
 * to the GEMM live in a fixed device array of the library, one per GPU,
 * created when the library's code is loaded on that GPU and held until the
 * process ends; its size is fq_linear_noalloc_max_bytes() (24 MiB), and a
 * call needing more than fq_linear_workspace_bytes(M, K, abits) allows
 * returns FQ_ERR_UNSUPPORTED before any work.  The call allocates nothing
 * (no hipMalloc, no allocating library routine) and clears nothing: the
 * prologue overwrites every byte the GEMM then reads.  All calls on one GPU
 * share that GPU's array, so calls that may overlap on one GPU (other
 * streams, other threads) race and must be ordered by the caller.  Other
 * arguments, results and errors as in fq_linear. */
fq_status fq_linear_noalloc(const void* x_bf16, int32_t M, int32_t K, int64_t ldx,
                            const float* gamma_folded, float eps, const float* ascale,
                            int32_t fold_after, int32_t hblock, int32_t abits,
                            const void* w_codes, const float* wscale, int32_t N, int32_t wbits,
                            const float* bias, const void* residual_bf16, int64_t ldr,
                            void* y_bf16, int64_t ldy, void* stream);
size_t fq_linear_noalloc_max_bytes(void);

/* GeGLU between the sites of a chained MLP block (gate+up site -> GeGLU -> down
 * site with the residual, the Gemma-style MLP of the page's pi0.5 backbone):
 *   h[m][j] = bf16_rne(gelu_tanh(g) * u),  g = gateup[m][j], u = gateup[m][F + j],
 *   gelu_tanh(g) = g/2 * (1 + tanh(sqrt(2/pi) * (g + 0.044715 g^3)))
 * in float32 (device tanh).  gateup_bf16: device bf16 [M][ld_in] holding
 * [gate F | up F] per row (the gate+up site's output); h_bf16: device bf16
 * [M][ld_out].  F a positive multiple of 8; ld_in >= 2F and ld_out >= F,
 * multiples of 8; 16-byte aligned bases. */
fq_status fq_geglu(const void* gateup_bf16, int32_t M, int32_t F, int64_t ld_in,
                   void* h_bf16, int64_t ld_out, void* stream);

/* Head-layout variants (the page's CUDA path fuses "the head layout" into the
 * epilogue; the SYCL path keeps plain outputs and so has none): the output of
 * feature n = h * head_dim + d for token m goes to y[h][m][d], i.e. y is
 * [N / head_dim][M][head_dim], each head a dense [M][head_dim] block (the
 * layout attention consumes per head).  head_dim must be a positive multiple
 * of 8 dividing N; everything else, including the row-major [M][ldr]
 * residual, is as in fq_gemm / fq_linear. */
fq_status fq_gemm_heads(const void* act_codes, const float* act_scale, int32_t M, int32_t abits,
                        const void* w_codes, const float* wscale, int32_t N, int32_t K, int32_t wbits,
                        const float* bias, const void* residual_bf16, int64_t ldr,
                        int32_t head_dim, void* y_bf16, int32_t* acc_i32, void* stream);

fq_status fq_linear_heads(const void* x_bf16, int32_t M, int32_t K, int64_t ldx,
                          const float* gamma_folded, float eps, const float* ascale,
                          int32_t fold_after, int32_t hblock, int32_t abits,
                          const void* w_codes, const float* wscale, int32_t N, int32_t wbits,
                          const float* bias, const void* residual_bf16, int64_t ldr,
                          int32_t head_dim, void* y_bf16,
                          void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* FQ_H */

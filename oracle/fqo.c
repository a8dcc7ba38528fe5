/*
 * FoldQuant CPU oracle -- TEST INFRASTRUCTURE ONLY (see fqo.h).
 *
 * Source of every step: the vla.cpp pull request page "FoldQuant W8A8/W4A4
 * inference and FoldQuantVLA quantized-model converter":
 *   - runtime summary: per-row INT8/INT4 weight codes in a block-Hadamard,
 *     SmoothQuant-folded frame; activations quantised per token; integer GEMMs;
 *     a fused RMSNorm + butterfly + quant prologue; residual add in the epilogue.
 *   - dequant-mode commit: x' = R(x/a) (fold before) or R(x)/a (fold after),
 *     R the block-normalised Sylvester-Hadamard butterfly (symmetric,
 *     orthonormal); the float weight row is R(w_n)/a or R(w_n/a); at LLM sites
 *     the smoothing vector lives in the norm gain.
 *   - OpenVINO commit: the act node is RMSNorm with the folded gain, the ascale
 *     divide, the block rotation, a per-token amax scale, round-half-even and a
 *     clamp; 4-bit activations have 15 levels; weights are dequantised by the
 *     per-row scale.
 *   - SYCL commit: integer sums are exact in any order; the reference builds
 *     with -ffp-contract=off and correctly rounded divide / sqrt.
 * Build: gcc -O2 -ftree-vectorize -fopenmp -ffp-contract=off (no fast-math).
 * The loops are parallel over independent tokens or rows only.
 */
#include "fqo.h"

#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdlib.h>
#include <string.h>

static int is_pow2(int32_t b) { return b >= 1 && (b & (b - 1)) == 0; }

static float bf16_to_f32(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

int fqo_hadamard_entry(int32_t b, int32_t i, int32_t j) {
    if (!is_pow2(b) || i < 0 || j < 0 || i >= b || j >= b) return 0;
    return (__builtin_popcount((unsigned)(i & j)) & 1) ? -1 : 1;
}

/* H_b per contiguous block, stages with span 1, 2, ..., b/2: (p, q) -> (p + q, p - q). */
static void butterfly_f64(double* v, int64_t n, int32_t b) {
    for (int64_t s = 0; s < n; s += b)
        for (int32_t h = 1; h < b; h <<= 1)
            for (int32_t i = 0; i < b; ++i)
                if ((i & h) == 0) {
                    double p = v[s + i], q = v[s + i + h];
                    v[s + i] = p + q;
                    v[s + i + h] = p - q;
                }
}

static void butterfly_f32(float* v, int64_t n, int32_t b) {
    for (int64_t s = 0; s < n; s += b)
        for (int32_t h = 1; h < b; h <<= 1)
            for (int32_t i = 0; i < b; ++i)
                if ((i & h) == 0) {
                    float p = v[s + i], q = v[s + i + h];
                    v[s + i] = p + q;
                    v[s + i + h] = p - q;
                }
}

int fqo_rotate_f64(double* v, int64_t n, int32_t b) {
    if (!v || !is_pow2(b) || n < 0 || n % b) return -1;
    butterfly_f64(v, n, b);
    const double rs = 1.0 / sqrt((double)b);
    for (int64_t k = 0; k < n; ++k) v[k] *= rs;
    return 0;
}

int fqo_butterfly_f32(float* v, int64_t n, int32_t b) {
    if (!v || !is_pow2(b) || n < 0 || n % b) return -1;
    butterfly_f32(v, n, b);
    return 0;
}

int fqo_fold_gain(const float* gamma, const float* ascale, int32_t K, float* out) {
    if (!gamma || !out || K < 1) return -1;
    for (int32_t k = 0; k < K; ++k) out[k] = ascale ? gamma[k] / ascale[k] : gamma[k];
    return 0;
}

static int qmax_of(int32_t bits) { return bits == 8 ? 127 : (bits == 4 ? 7 : 0); }

int32_t fqo_code_at(const void* row, int32_t k, int32_t bits) {
    const uint8_t* r = (const uint8_t*)row;
    if (bits == 8) return (int32_t)(int8_t)r[k];
    int32_t v = (k & 1) ? (r[k >> 1] >> 4) : (r[k >> 1] & 0xF);
    return v >= 8 ? v - 16 : v;
}

static void store_code(uint8_t* row, int32_t k, int32_t bits, int32_t q) {
    if (bits == 8) {
        row[k] = (uint8_t)(int8_t)q;
    } else {
        uint8_t nib = (uint8_t)(q & 0xF);
        if (k & 1) row[k >> 1] = (uint8_t)((row[k >> 1] & 0x0F) | (nib << 4));
        else row[k >> 1] = (uint8_t)((row[k >> 1] & 0xF0) | nib);
    }
}

static int64_t row_bytes(int32_t K, int32_t bits) { return bits == 8 ? K : K / 2; }

/* one folded weight row in float64 */
static void fold_row(const float* w, int32_t K, const float* a, int32_t fold_after,
                     int32_t b, double* u) {
    for (int32_t k = 0; k < K; ++k) u[k] = (double)w[k];
    if (a && !fold_after)
        for (int32_t k = 0; k < K; ++k) u[k] *= (double)a[k];
    fqo_rotate_f64(u, K, b);
    if (a && fold_after)
        for (int32_t k = 0; k < K; ++k) u[k] *= (double)a[k];
}

int fqo_fold_weights(const float* W, int32_t N, int32_t K, const float* ascale,
                     int32_t fold_after, int32_t hblock, double* U) {
    if (!W || !U || N < 1 || K < 1 || !is_pow2(hblock) || K % hblock) return -1;
#pragma omp parallel for schedule(static)
    for (int32_t n = 0; n < N; ++n)
        fold_row(W + (int64_t)n * K, K, ascale, fold_after, hblock, U + (int64_t)n * K);
    return 0;
}

int fqo_pack_weights(const float* W, int32_t N, int32_t K, const float* ascale,
                     int32_t fold_after, int32_t hblock, int32_t wbits,
                     void* codes, float* wscale) {
    const int qmax = qmax_of(wbits);
    if (!W || !codes || !wscale || N < 1 || K < 2 || K % 2 || !qmax || !is_pow2(hblock) ||
        K % hblock)
        return -1;
    const int64_t rb = row_bytes(K, wbits);
#pragma omp parallel
    {
        double* u = (double*)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(static)
        for (int32_t n = 0; n < N; ++n) {
            fold_row(W + (int64_t)n * K, K, ascale, fold_after, hblock, u);
            double amax = 0.0;
            for (int32_t k = 0; k < K; ++k) amax = fmax(amax, fabs(u[k]));
            const float s = (float)(amax / (double)qmax);
            uint8_t* row = (uint8_t*)codes + (int64_t)n * rb;
            memset(row, 0, (size_t)rb);
            for (int32_t k = 0; k < K; ++k) {
                double q = s > 0.0f ? rint(u[k] / (double)s) : 0.0;
                if (q > qmax) q = qmax;
                if (q < -qmax) q = -qmax;
                store_code(row, k, wbits, (int32_t)q);
            }
            wscale[n] = s;
        }
        free(u);
    }
    return 0;
}

int fqo_unfold_weights(const void* codes, const float* wscale, int32_t N, int32_t K,
                       const float* ascale, int32_t fold_after, int32_t hblock,
                       int32_t wbits, double* Wout) {
    if (!codes || !wscale || !Wout || N < 1 || K < 2 || !qmax_of(wbits) || !is_pow2(hblock) ||
        K % hblock)
        return -1;
    const int64_t rb = row_bytes(K, wbits);
#pragma omp parallel for schedule(static)
    for (int32_t n = 0; n < N; ++n) {
        const uint8_t* row = (const uint8_t*)codes + (int64_t)n * rb;
        double* w = Wout + (int64_t)n * K;
        for (int32_t k = 0; k < K; ++k) w[k] = (double)wscale[n] * (double)fqo_code_at(row, k, wbits);
        if (ascale && fold_after)
            for (int32_t k = 0; k < K; ++k) w[k] /= (double)ascale[k];
        fqo_rotate_f64(w, K, hblock);
        if (ascale && !fold_after)
            for (int32_t k = 0; k < K; ++k) w[k] /= (double)ascale[k];
    }
    return 0;
}

/* one token's activation frame in float32 */
static void act_row(const uint16_t* xr, int32_t K, const float* gamma, float eps,
                    const float* a, int32_t fold_after, int32_t b, float* h) {
    for (int32_t k = 0; k < K; ++k) h[k] = bf16_to_f32(xr[k]);
    if (gamma) {
        double ss = 0.0;
        for (int32_t k = 0; k < K; ++k) ss += (double)h[k] * (double)h[k];
        const float ms = (float)(ss / (double)K);
        const float rinv = 1.0f / sqrtf(ms + eps);
        for (int32_t k = 0; k < K; ++k) h[k] = (h[k] * rinv) * gamma[k];
    }
    if (a && !fold_after)
        for (int32_t k = 0; k < K; ++k) h[k] = h[k] / a[k];
    butterfly_f32(h, K, b);
    const float rs = (float)(1.0 / sqrt((double)b));
    for (int32_t k = 0; k < K; ++k) h[k] = h[k] * rs;
    if (a && fold_after)
        for (int32_t k = 0; k < K; ++k) h[k] = h[k] / a[k];
}

int fqo_act_frame(const uint16_t* x, int32_t M, int32_t K, int64_t ldx,
                  const float* gamma, float eps, const float* ascale, int32_t fold_after,
                  int32_t hblock, float* h) {
    if (!x || !h || M < 1 || K < 1 || ldx < K || !is_pow2(hblock) || K % hblock) return -1;
#pragma omp parallel for schedule(static)
    for (int32_t m = 0; m < M; ++m)
        act_row(x + (int64_t)m * ldx, K, gamma, eps, ascale, fold_after, hblock, h + (int64_t)m * K);
    return 0;
}

int fqo_prologue(const uint16_t* x, int32_t M, int32_t K, int64_t ldx,
                 const float* gamma, float eps, const float* ascale, int32_t fold_after,
                 int32_t hblock, int32_t abits, void* codes, float* act_scale) {
    const int qmax = qmax_of(abits);
    if (!x || !codes || !act_scale || M < 1 || K < 2 || K % 2 || ldx < K || !qmax ||
        !is_pow2(hblock) || K % hblock)
        return -1;
    const int64_t rb = row_bytes(K, abits);
#pragma omp parallel
    {
        float* h = (float*)malloc(sizeof(float) * (size_t)K);
#pragma omp for schedule(static)
        for (int32_t m = 0; m < M; ++m) {
            act_row(x + (int64_t)m * ldx, K, gamma, eps, ascale, fold_after, hblock, h);
            float amax = 0.0f;
            for (int32_t k = 0; k < K; ++k) amax = fmaxf(amax, fabsf(h[k]));
            const float s = amax / (float)qmax;
            uint8_t* row = (uint8_t*)codes + (int64_t)m * rb;
            memset(row, 0, (size_t)rb);
            for (int32_t k = 0; k < K; ++k) {
                float q = s > 0.0f ? rintf(h[k] / s) : 0.0f;
                if (q > (float)qmax) q = (float)qmax;
                if (q < (float)-qmax) q = (float)-qmax;
                store_code(row, k, abits, (int32_t)q);
            }
            act_scale[m] = s;
        }
        free(h);
    }
    return 0;
}

int fqo_gemm_i32(const void* act_codes, int32_t M, int32_t abits,
                 const void* w_codes, int32_t N, int32_t K, int32_t wbits, int32_t* acc) {
    if (!act_codes || !w_codes || !acc || M < 1 || N < 1 || K < 2 || K % 2 ||
        !qmax_of(abits) || !qmax_of(wbits))
        return -1;
    /* widen both operands to one int8 per code, then plain dot products */
    int8_t* A = (int8_t*)malloc((size_t)M * K);
    int8_t* B = (int8_t*)malloc((size_t)N * K);
    if (!A || !B) { free(A); free(B); return -2; }
    const int64_t ra = row_bytes(K, abits), rw = row_bytes(K, wbits);
#pragma omp parallel for schedule(static)
    for (int32_t m = 0; m < M; ++m)
        for (int32_t k = 0; k < K; ++k)
            A[(int64_t)m * K + k] = (int8_t)fqo_code_at((const uint8_t*)act_codes + m * ra, k, abits);
#pragma omp parallel for schedule(static)
    for (int32_t n = 0; n < N; ++n)
        for (int32_t k = 0; k < K; ++k)
            B[(int64_t)n * K + k] = (int8_t)fqo_code_at((const uint8_t*)w_codes + n * rw, k, wbits);
    int overflow = 0;
#pragma omp parallel for schedule(dynamic, 4) reduction(| : overflow)
    for (int32_t m = 0; m < M; ++m) {
        const int8_t* a = A + (int64_t)m * K;
        for (int32_t n = 0; n < N; ++n) {
            const int8_t* w = B + (int64_t)n * K;
            int64_t s = 0;
            /* exact: partial sums of 4096 products stay below 2^31 */
            for (int32_t k0 = 0; k0 < K; k0 += 4096) {
                const int32_t k1 = k0 + 4096 < K ? k0 + 4096 : K;
                int32_t p = 0;
                for (int32_t k = k0; k < k1; ++k) p += (int32_t)a[k] * (int32_t)w[k];
                s += p;
            }
            if (s > INT32_MAX) { s = INT32_MAX; overflow = 1; }
            if (s < INT32_MIN) { s = INT32_MIN; overflow = 1; }
            acc[(int64_t)m * N + n] = (int32_t)s;
        }
    }
    free(A);
    free(B);
    return overflow ? 1 : 0;
}

uint16_t fqo_bf16_from_f64(double v) {
    if (isnan(v)) return 0x7FC0;
    const uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0) return sign;
    if (isinf(a)) return sign | 0x7F80;
    int e;
    frexp(a, &e);                    /* a = f * 2^e, 0.5 <= f < 1 */
    if (e < -125) e = -125;          /* below 2^-126 the quantum stays 2^-133 */
    const double quantum = ldexp(1.0, e - 8);
    const double r = rint(a / quantum) * quantum;  /* 8 significant bits, ties to even */
    if (r >= ldexp(1.0, 128)) return sign | 0x7F80;
    const float f = (float)r;        /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(sign | (u >> 16));
}

int fqo_epilogue(const int32_t* acc, int32_t M, int32_t N, const float* act_scale,
                 const float* wscale, const float* bias, const uint16_t* residual,
                 int64_t ldr, uint16_t* y, double* y_f64) {
    if (!acc || !act_scale || !wscale || !y || M < 1 || N < 1 || (residual && ldr < N)) return -1;
#pragma omp parallel for schedule(static)
    for (int32_t m = 0; m < M; ++m)
        for (int32_t n = 0; n < N; ++n) {
            double t = (double)acc[(int64_t)m * N + n] * ((double)act_scale[m] * (double)wscale[n]);
            if (bias) t += (double)bias[n];
            if (residual) t += (double)bf16_to_f32(residual[(int64_t)m * ldr + n]);
            if (y_f64) y_f64[(int64_t)m * N + n] = t;
            y[(int64_t)m * N + n] = fqo_bf16_from_f64(t);
        }
    return 0;
}

/* GeGLU between the MLP sites of the chained block (gate+up site, GeGLU,
 * down site with the residual): h = bf16(gelu_tanh(gate) * up), float64 inside,
 * one rounding; gelu_tanh(g) = g/2 * (1 + tanh(sqrt(2/pi) * (g + 0.044715 g^3))). */
int fqo_geglu(const uint16_t* gu, int32_t M, int32_t F, int64_t ld_in, uint16_t* h, int64_t ld_out,
              double* h_f64) {
    if (!gu || !h || M < 1 || F < 1 || ld_in < 2 * (int64_t)F || ld_out < F) return -1;
    const double c = sqrt(2.0 / 3.14159265358979323846);
#pragma omp parallel for schedule(static)
    for (int32_t m = 0; m < M; ++m)
        for (int32_t j = 0; j < F; ++j) {
            const double g = (double)bf16_to_f32(gu[(int64_t)m * ld_in + j]);
            const double u = (double)bf16_to_f32(gu[(int64_t)m * ld_in + F + j]);
            const double t = 0.5 * g * (1.0 + tanh(c * (g + 0.044715 * g * g * g))) * u;
            if (h_f64) h_f64[(int64_t)m * F + j] = t;
            h[(int64_t)m * ld_out + j] = fqo_bf16_from_f64(t);
        }
    return 0;
}

int fqo_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

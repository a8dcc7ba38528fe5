// FoldQuant activation quantisation of one token (gfx950, wave64), the body
// of the prologue kernel, kept apart so that another kernel can quantise a
// token the same way, bit for bit.  The arithmetic and its bit-exactness
// argument are described with the prologue kernel.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <type_traits>

#include "fq_device.h"

namespace fq {

// Per-launch constants of a token's arithmetic, computed on the host in
// float64 and correctly rounded: rs = 1/sqrt(b) (float) and rk = 1/K (the
// mean's divide, below).
struct TokenConsts {
    float rs;
    double rk;
};

// Whole-wave reductions on the VALU: DPP within rows of 16 lanes (xor 1,
// xor 2, half-row mirror, row mirror), then the gfx950 row swaps (lanes
// l <-> l ^ 16 and l <-> l ^ 32).  Each step combines two complete partial
// results, so every lane ends with the same value, in a fixed order.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}

// Maximum over the wave of a value that is >= 0 and not NaN: for such floats
// the order of the bit patterns as unsigned integers is the order of the
// values, and the integer max needs none of the quieting maxes that fmaxf
// compiles to here.
__device__ __forceinline__ float wave_max_nonneg(float x) {
    uint32_t v = __float_as_uint(x);
    v = max(v, uint32_t(dpp_i<0xB1>(int(v))));   // quad_perm [1,0,3,2]
    v = max(v, uint32_t(dpp_i<0x4E>(int(v))));   // quad_perm [2,3,0,1]
    v = max(v, uint32_t(dpp_i<0x141>(int(v))));  // row_half_mirror
    v = max(v, uint32_t(dpp_i<0x140>(int(v))));  // row_mirror
    const auto a = __builtin_amdgcn_permlane16_swap(int(v), int(v), false, false);
    v = max(uint32_t(a[0]), uint32_t(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(int(v), int(v), false, false);
    return __uint_as_float(max(uint32_t(b[0]), uint32_t(b[1])));
}

template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
    const long long u = __double_as_longlong(v);
    const int lo = dpp_i<CTRL>(int(u)), hi = dpp_i<CTRL>(int(u >> 32));
    return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned int>(lo));
}

__device__ __forceinline__ double join_d(int lo, int hi) {
    return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned int>(lo));
}

__device__ __forceinline__ double wave_sum(double v) {
    v = v + dpp_d<0xB1>(v);
    v = v + dpp_d<0x4E>(v);
    v = v + dpp_d<0x141>(v);
    v = v + dpp_d<0x140>(v);
    {
        const long long u = __double_as_longlong(v);
        const auto lo = __builtin_amdgcn_permlane16_swap(int(u), int(u), false, false);
        const auto hi = __builtin_amdgcn_permlane16_swap(int(u >> 32), int(u >> 32), false, false);
        v = join_d(lo[0], hi[0]) + join_d(lo[1], hi[1]);
    }
    {
        const long long u = __double_as_longlong(v);
        const auto lo = __builtin_amdgcn_permlane32_swap(int(u), int(u), false, false);
        const auto hi = __builtin_amdgcn_permlane32_swap(int(u >> 32), int(u >> 32), false, false);
        v = join_d(lo[0], hi[0]) + join_d(lo[1], hi[1]);
    }
    return v;
}

// One cross-lane butterfly stage.  The lower lane of each pair keeps lo + hi;
// the upper lane keeps lo - hi NEGATED, computed as own + (-1) * partner.  That
// makes the partner's value the multiplied operand of one v_fmac_f32 that reads
// it through DPP, one instruction per value where a DPP move and an fma took
// two.  The negation is exact and round-to-nearest is symmetric, so each stored
// value is the butterfly's value times a per-lane sign (the product of the
// stages' signs), bit for bit; the caller removes it with the final 1/sqrt(b)
// scaling.  Stages run with increasing distance, so a pair's two lanes always
// carry the same sign from the earlier stages.
//
// The compiler does not fold a DPP move into v_fmac_f32, so the stage is
// written out: blocks of 8 values, each opened with 5 wait states (a VALU
// write of a VGPR or of EXEC before a DPP read) and closed with 2 (a DPP read
// after the block).  Distances 4 and 8 take two lane permutations, the first
// as a plain DPP move into a temporary.
#define FQ_DPPM " row_mask:0xf bank_mask:0xf\n\t"
#define FQ_FMAC8(C)                                                                                        \
    "s_nop 4\n\t"                                                                                          \
    "v_fmac_f32_dpp %0, %0, %8 " C FQ_DPPM "v_fmac_f32_dpp %1, %1, %8 " C FQ_DPPM                           \
    "v_fmac_f32_dpp %2, %2, %8 " C FQ_DPPM "v_fmac_f32_dpp %3, %3, %8 " C FQ_DPPM                           \
    "v_fmac_f32_dpp %4, %4, %8 " C FQ_DPPM "v_fmac_f32_dpp %5, %5, %8 " C FQ_DPPM                           \
    "v_fmac_f32_dpp %6, %6, %8 " C FQ_DPPM "v_fmac_f32_dpp %7, %7, %8 " C FQ_DPPM "s_nop 1"
#define FQ_MOVFMAC8(P, C)                                                                                  \
    "s_nop 4\n\t"                                                                                          \
    "v_mov_b32_dpp %8, %0 " P FQ_DPPM "v_mov_b32_dpp %9, %1 " P FQ_DPPM                                     \
    "v_mov_b32_dpp %10, %2 " P FQ_DPPM "v_mov_b32_dpp %11, %3 " P FQ_DPPM                                   \
    "v_mov_b32_dpp %12, %4 " P FQ_DPPM "v_mov_b32_dpp %13, %5 " P FQ_DPPM                                   \
    "v_mov_b32_dpp %14, %6 " P FQ_DPPM "v_mov_b32_dpp %15, %7 " P FQ_DPPM "s_nop 1\n\t"                     \
    "v_fmac_f32_dpp %0, %8, %16 " C FQ_DPPM "v_fmac_f32_dpp %1, %9, %16 " C FQ_DPPM                         \
    "v_fmac_f32_dpp %2, %10, %16 " C FQ_DPPM "v_fmac_f32_dpp %3, %11, %16 " C FQ_DPPM                       \
    "v_fmac_f32_dpp %4, %12, %16 " C FQ_DPPM "v_fmac_f32_dpp %5, %13, %16 " C FQ_DPPM                       \
    "v_fmac_f32_dpp %6, %14, %16 " C FQ_DPPM "v_fmac_f32_dpp %7, %15, %16 " C FQ_DPPM "s_nop 1"

template <int D, int E>
__device__ __forceinline__ void cross_stage(float (&v)[E], int lane) {
    static_assert(E % 8 == 0, "cross-lane stages work on blocks of 8 values");
    const float sgn = (lane & D) ? -1.0f : 1.0f;
#pragma unroll
    for (int b = 0; b < E / 8; ++b) {
        float* const p = &v[8 * b];
        if constexpr (D == 1 || D == 2) {
            // D = 1: quad_perm [1,0,3,2]; D = 2: quad_perm [2,3,0,1]
            if constexpr (D == 1)
                asm volatile(FQ_FMAC8("quad_perm:[1,0,3,2]")
                             : "+v"(p[0]), "+v"(p[1]), "+v"(p[2]), "+v"(p[3]), "+v"(p[4]), "+v"(p[5]), "+v"(p[6]),
                               "+v"(p[7])
                             : "v"(sgn));
            else
                asm volatile(FQ_FMAC8("quad_perm:[2,3,0,1]")
                             : "+v"(p[0]), "+v"(p[1]), "+v"(p[2]), "+v"(p[3]), "+v"(p[4]), "+v"(p[5]), "+v"(p[6]),
                               "+v"(p[7])
                             : "v"(sgn));
        } else {
            // D = 4: row_half_mirror (xor 7 within 8 lanes), then quad_perm [3,2,1,0] (xor 3);
            // D = 8: row_mirror (xor 15 within 16 lanes), then row_half_mirror (xor 7)
            float t[8];
            if constexpr (D == 4)
                asm volatile(FQ_MOVFMAC8("row_half_mirror", "quad_perm:[3,2,1,0]")
                             : "+v"(p[0]), "+v"(p[1]), "+v"(p[2]), "+v"(p[3]), "+v"(p[4]), "+v"(p[5]), "+v"(p[6]),
                               "+v"(p[7]), "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3]), "=&v"(t[4]),
                               "=&v"(t[5]), "=&v"(t[6]), "=&v"(t[7])
                             : "v"(sgn));
            else
                asm volatile(FQ_MOVFMAC8("row_mirror", "row_half_mirror")
                             : "+v"(p[0]), "+v"(p[1]), "+v"(p[2]), "+v"(p[3]), "+v"(p[4]), "+v"(p[5]), "+v"(p[6]),
                               "+v"(p[7]), "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3]), "=&v"(t[4]),
                               "=&v"(t[5]), "=&v"(t[6]), "=&v"(t[7])
                             : "v"(sgn));
        }
    }
}
#undef FQ_MOVFMAC8
#undef FQ_FMAC8
#undef FQ_DPPM

__device__ __forceinline__ void unpack8(uint4 d, float* o) {
    o[0] = bf16_lo(d.x);
    o[1] = bf16_hi(d.x);
    o[2] = bf16_lo(d.y);
    o[3] = bf16_hi(d.y);
    o[4] = bf16_lo(d.z);
    o[5] = bf16_hi(d.z);
    o[6] = bf16_lo(d.w);
    o[7] = bf16_hi(d.w);
}

template <int E>
__device__ __forceinline__ void divide_by_vector(float (&v)[E], const float* __restrict__ a, int c, bool active) {
    if (active) {
#pragma unroll
        for (int q = 0; q < E / 4; ++q) {
            const float4 d = *reinterpret_cast<const float4*>(a + E * c + 4 * q);
            v[4 * q + 0] = v[4 * q + 0] / d.x;
            v[4 * q + 1] = v[4 * q + 1] / d.y;
            v[4 * q + 2] = v[4 * q + 2] / d.z;
            v[4 * q + 3] = v[4 * q + 3] / d.w;
        }
    }
}

// Sum / max of a lane's E values as a balanced tree (short dependency chain).
template <int E>
__device__ __forceinline__ double lane_sumsq(const float (&v)[E]) {
    // x*x is exact in float64, so fma(x, x, t) rounds exactly like x*x + t
    double t[E / 2];
#pragma unroll
    for (int i = 0; i < E / 2; ++i) {
        const double a = double(v[2 * i]), b = double(v[2 * i + 1]);
        t[i] = __builtin_fma(b, b, a * a);
    }
#pragma unroll
    for (int w = E / 4; w >= 1; w >>= 1)
#pragma unroll
        for (int i = 0; i < w; ++i) t[i] = t[i] + t[i + w];
    return t[0];
}

// max(|a|, |b|, c) in one v_max3_f32 with |.| source modifiers (fmaxf of
// fabsf compiled to an extra quieting max per value).  Like fmaxf it returns
// the other operands where one is a quiet NaN, so with c = 0 the result is
// never NaN.
__device__ __forceinline__ float max3_abs(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, |%1|, |%2|, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// max |v_i| over a lane's values, in two interleaved chains; >= 0, not NaN
template <int E>
__device__ __forceinline__ float lane_absmax(const float (&v)[E]) {
    static_assert(E % 4 == 0, "values in groups of four");
    float m0 = max3_abs(v[0], v[1], 0.0f), m1 = max3_abs(v[2], v[3], 0.0f);
#pragma unroll
    for (int i = 4; i < E; i += 4) {
        m0 = max3_abs(v[i], v[i + 1], m0);
        m1 = max3_abs(v[i + 2], v[i + 3], m1);
    }
    return __uint_as_float(max(__float_as_uint(m0), __float_as_uint(m1)));
}

// Adding 1.5 * 2^23 to |q| <= 2^22 rounds q to an integer, ties to even (the
// add itself rounds to nearest even at unit spacing), and leaves that integer
// in the low mantissa bits: the low byte of the sum is the two's complement code.
__device__ __forceinline__ uint32_t round_to_code_bits(float q) { return __float_as_uint(q + 0x1.8p23f); }

// A token's inputs as loaded: thread c's bf16 values [E c, E c + E) and, with
// the norm and E <= 32, its slice of the gain (zeros past K).  Loading and
// quantising are separate steps so that a caller can put other memory
// requests behind these loads.
template <int E, bool NORM>
struct TokenLoad {
    static constexpr bool kPreG = NORM && E <= 32;  // the gain comes with x while registers allow
    uint4 d[E / 8];
    float4 g[kPreG ? E / 4 : 1];
};

template <int E, bool NORM>
__device__ __forceinline__ TokenLoad<E, NORM> load_token(const uint16_t* __restrict__ xr, int K,
                                                         const float* __restrict__ gamma, int c) {
    TokenLoad<E, NORM> t;
#pragma unroll
    for (int q = 0; q < E / 8; ++q) t.d[q] = make_uint4(0, 0, 0, 0);
    if (c < K / E) {
#pragma unroll
        for (int q = 0; q < E / 8; ++q) t.d[q] = *reinterpret_cast<const uint4*>(xr + E * c + 8 * q);
        if constexpr (TokenLoad<E, NORM>::kPreG) {
#pragma unroll
            for (int q = 0; q < E / 4; ++q) t.g[q] = *reinterpret_cast<const float4*>(gamma + E * c + 4 * q);
        }
    }
    return t;
}

// The same loads with no condition: lanes past K load lane 0's values, which
// quantise_loaded leaves out of its sums and maxima.  With every load
// unconditional the compiler's memory-counter waits stay exact, so a caller
// that issues other loads after these waits only for these.
template <int E, bool NORM>
__device__ __forceinline__ TokenLoad<E, NORM> load_token_clamped(const uint16_t* __restrict__ xr, int K,
                                                                 const float* __restrict__ gamma, int c) {
    TokenLoad<E, NORM> t;
    const int cc = c < K / E ? c : 0;
#pragma unroll
    for (int q = 0; q < E / 8; ++q) t.d[q] = *reinterpret_cast<const uint4*>(xr + E * cc + 8 * q);
    if constexpr (TokenLoad<E, NORM>::kPreG) {
#pragma unroll
        for (int q = 0; q < E / 4; ++q) t.g[q] = *reinterpret_cast<const float4*>(gamma + E * cc + 4 * q);
    }
    return t;
}

// Quantise one loaded token: RMSNorm with the folded gain (NORM), the optional
// smoothing divide (AMODE 0 none, 1 before the rotation, 2 after it), the
// block Hadamard rotation of 2^LOG2B values and the per-token symmetric
// quantisation.  Called by every thread of a workgroup (c = thread index,
// nwaves = waves in the workgroup, all of which reach the same barriers);
// thread c owns values [E c, E c + E) of the token.  The codes go out through
// store(byte offset in the token's code row, uint4 | uint2 | uint32_t); the
// scale is returned (the same value in every thread).  red_d and red_f are
// nwaves-entry LDS scratch for the cross-wave reductions.
template <int E, int ABITS, bool NORM, int AMODE, int LOG2B, class Store>
__device__ __forceinline__ float quantise_loaded(const TokenLoad<E, NORM>& t, int K, const float* __restrict__ gamma,
                                                 float eps, const float* __restrict__ ascale, TokenConsts tc, int c,
                                                 int nwaves, double* red_d, float* red_f, Store store) {
    constexpr int hblock = 1 << LOG2B;
    static_assert(hblock <= 16 * E, "a Hadamard block spans at most 16 lanes (cross-lane distances 1 .. 8)");
    static_assert(ABITS != 6 || E >= 16, "E2M3 codes leave in groups of 16 values (12 bytes)");
    constexpr int qmax = ABITS == 8 ? 127 : 7;
    const int lane = c & 63;
    const int wave = c >> 6;
    const bool active = c < K / E;  // lanes past K only join the exchanges; their values are left out

    constexpr bool kPreG = TokenLoad<E, NORM>::kPreG;
    float v[E];
    const float4* const g = t.g;
#pragma unroll
    for (int q = 0; q < E / 8; ++q) unpack8(t.d[q], &v[8 * q]);

    // RMSNorm with the folded gain: the float32 squares are exact in float64
    if (NORM) {
        double ss = wave_sum(active ? lane_sumsq<E>(v) : 0.0);
        if (nwaves > 1) {
            if (lane == 0) red_d[wave] = ss;
            __syncthreads();
            ss = 0.0;
            for (int w = 0; w < nwaves; ++w) ss += red_d[w];
        }
        // ss / K correctly rounded in float64 without a divide: Markstein's
        // correction of ss * RN(1/K) (the remainder is exact in an fma)
        const double q0 = ss * tc.rk;
        const float ms = float(__builtin_fma(__builtin_fma(-q0, double(K), ss), tc.rk, q0));
        const float rinv = 1.0f / sqrtf(ms + eps);
        if (active) {
#pragma unroll
            for (int q = 0; q < E / 4; ++q) {
                const float4 gq = kPreG ? g[q < (kPreG ? E / 4 : 1) ? q : 0]
                                        : *reinterpret_cast<const float4*>(gamma + E * c + 4 * q);
                v[4 * q + 0] = (v[4 * q + 0] * rinv) * gq.x;
                v[4 * q + 1] = (v[4 * q + 1] * rinv) * gq.y;
                v[4 * q + 2] = (v[4 * q + 2] * rinv) * gq.z;
                v[4 * q + 3] = (v[4 * q + 3] * rinv) * gq.w;
            }
        }
    }

    if (AMODE == 1) divide_by_vector<E>(v, ascale, c, active);

    // block Hadamard butterfly: spans 1 .. E/2 inside the lane ...
#pragma unroll
    for (int span = 1; span < E; span <<= 1) {
        if (span < hblock) {  // compile-time
#pragma unroll
            for (int i = 0; i < E; ++i)
                if ((i & span) == 0) {
                    const float lo = v[i], hi = v[i + span];
                    v[i] = lo + hi;
                    v[i + span] = lo - hi;
                }
        }
    }
    // ... spans E .. b/2 across lanes (lane distance span / E)
    if constexpr (hblock > E) cross_stage<1, E>(v, lane);
    if constexpr (hblock > 2 * E) cross_stage<2, E>(v, lane);
    if constexpr (hblock > 4 * E) cross_stage<4, E>(v, lane);
    if constexpr (hblock > 8 * E) cross_stage<8, E>(v, lane);
    // the cross stages' sign: -1 for an odd number of set lane bits among those they used
    constexpr int kCrossBits = hblock > E ? hblock / E - 1 : 0;
    const float rs_lane = (__builtin_popcount(lane & kCrossBits) & 1) ? -tc.rs : tc.rs;
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] = v[i] * rs_lane;

    if (AMODE == 2) divide_by_vector<E>(v, ascale, c, active);

    // per-token amax (lanes past K hold zeros)
    float amax = wave_max_nonneg(active ? lane_absmax<E>(v) : 0.0f);
    if (nwaves > 1) {
        if (lane == 0) red_f[wave] = amax;
        __syncthreads();
        uint32_t m = 0;
        for (int w = 0; w < nwaves; ++w) m = max(m, __float_as_uint(red_f[w]));
        amax = __uint_as_float(m);
    }
    // s = amax / qmax, correctly rounded: Markstein's correction of
    // amax * RN(1/qmax) equals the IEEE quotient for every finite amax >= 0
    // (checked exhaustively for both qmax); a token outside the fast range,
    // or with a non-finite amax, divides below.  (fast is the same in every
    // lane; taken from lane 0 it is a scalar branch.)
    constexpr float rq = 1.0f / float(qmax);
    const float s0 = amax * rq;
    float s = __builtin_fmaf(__builtin_fmaf(-s0, float(qmax), amax), rq, s0);
    const bool fast = __builtin_amdgcn_readfirstlane(int(s >= 0x1p-100f && s <= 0x1p+100f)) != 0;

    float r = 0.0f;

    // Codes.  |h| <= amax and s is amax / qmax rounded, so |h / s| stays below
    // qmax + 1/2 and round-half-even never leaves [-qmax, qmax]: the clamp of
    // the definition is implied and not executed.
    // (one code path per divide form: as a per-element condition it cost a
    // branch around every element's fallback divide)
    auto quantise = [&](auto fast_tag) {
        constexpr bool kFast = decltype(fast_tag)::value;
        // codes per store: at most 16 bytes of them (E2M3: 16 or 32 values, 12 or 24 bytes)
        constexpr int G = ABITS == 8 ? (E < 16 ? E : 16) : (E < 32 ? E : 32);
#pragma unroll
        for (int grp = 0; grp < E / G; ++grp) {
            uint32_t t[G];
#pragma unroll
            for (int i = 0; i < G; ++i) {
                const float h = v[G * grp + i];
                float qf;
                if constexpr (kFast) {
                    const float q0 = h * r;
                    const float rem = __builtin_fmaf(-s, q0, h);
                    qf = __builtin_fmaf(rem, r, q0);
                } else {
                    qf = s > 0.0f ? h / s : 0.0f;
                }
                t[i] = round_to_code_bits(qf);
            }
            if constexpr (ABITS == 6) {
                // E2M3: the rounded codes are exact float integers in [-7, 7]; the
                // converter interleaves its two sources (field 2i from the first,
                // 2i + 1 from the second), so even values go first and odd second,
                // which puts value j of the group in bits 6j .. 6j+5
                v16f ev, od;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    ev[i] = 2 * i < G ? __uint_as_float(t[2 * i < G ? 2 * i : 0]) - 0x1.8p23f : 0.0f;
                    od[i] = 2 * i + 1 < G ? __uint_as_float(t[2 * i + 1 < G ? 2 * i + 1 : 0]) - 0x1.8p23f : 0.0f;
                }
                const v6i f = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(ev, od, 1.0f);
                const int off = (E * c + G * grp) / 4 * 3;
                if constexpr (G == 32) {
                    store(off, make_uint2(uint32_t(f[0]), uint32_t(f[1])));
                    store(off + 8, make_uint2(uint32_t(f[2]), uint32_t(f[3])));
                    store(off + 16, make_uint2(uint32_t(f[4]), uint32_t(f[5])));
                } else {
                    store(off, uint32_t(f[0]));
                    store(off + 4, uint32_t(f[1]));
                    store(off + 8, uint32_t(f[2]));
                }
            } else if (ABITS == 8) {
                uint32_t w[G / 4];
#pragma unroll
                for (int i = 0; i < G / 4; ++i) {
                    // byte 0 of t[4i .. 4i+3] -> one dword
                    const uint32_t lo = __builtin_amdgcn_perm(t[4 * i + 1], t[4 * i + 0], 0x0C0C0400u);
                    const uint32_t hi = __builtin_amdgcn_perm(t[4 * i + 3], t[4 * i + 2], 0x0C0C0400u);
                    w[i] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
                }
                if constexpr (G == 16)
                    store(E * c + G * grp, make_uint4(w[0], w[1], w[2], w[3]));
                else
                    store(E * c + G * grp, make_uint2(w[0], w[1]));
            } else {
                uint32_t w[G / 8];
#pragma unroll
                for (int i = 0; i < G / 8; ++i) {
                    uint32_t acc = 0;
#pragma unroll
                    for (int j = 0; j < 8; ++j) acc |= (t[8 * i + j] & 0xFu) << (4 * j);
                    w[i] = acc;
                }
                if constexpr (G == 32)
                    store((E / 2) * c + (G / 2) * grp, make_uint4(w[0], w[1], w[2], w[3]));
                else if constexpr (G == 16)
                    store((E / 2) * c + (G / 2) * grp, make_uint2(w[0], w[1]));
                else
                    store((E / 2) * c + (G / 2) * grp, w[0]);
            }
        }
    };
    if (fast) {
        r = 1.0f / s;
        if (active) quantise(std::true_type{});
    } else {
        s = amax / float(qmax);
        if (active) quantise(std::false_type{});
    }
    return s;
}

template <int E, int ABITS, bool NORM, int AMODE, int LOG2B, class Store>
__device__ __forceinline__ float quantise_token(const uint16_t* __restrict__ xr, int K,
                                                const float* __restrict__ gamma, float eps,
                                                const float* __restrict__ ascale, TokenConsts tc, int c, int nwaves,
                                                double* red_d, float* red_f, Store store) {
    return quantise_loaded<E, ABITS, NORM, AMODE, LOG2B>(load_token<E, NORM>(xr, K, gamma, c), K, gamma, eps,
                                                         ascale, tc, c, nwaves, red_d, red_f, store);
}

}  // namespace fq

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

// Whole-wave reductions on the VALU: DPP within rows of 16 lanes (xor 1,
// xor 2, half-row mirror, row mirror), then the gfx950 row swaps (lanes
// l <-> l ^ 16 and l <-> l ^ 32).  Each step combines two complete partial
// results, so every lane ends with the same value, in a fixed order.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}

__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, __int_as_float(dpp_i<0xB1>(__float_as_int(v))));   // quad_perm [1,0,3,2]
    v = fmaxf(v, __int_as_float(dpp_i<0x4E>(__float_as_int(v))));   // quad_perm [2,3,0,1]
    v = fmaxf(v, __int_as_float(dpp_i<0x141>(__float_as_int(v))));  // row_half_mirror
    v = fmaxf(v, __int_as_float(dpp_i<0x140>(__float_as_int(v))));  // row_mirror
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
    v = fmaxf(__int_as_float(a[0]), __int_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
    return fmaxf(__int_as_float(b[0]), __int_as_float(b[1]));
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

// value held by lane (lane ^ d) of the same wave, d in {1, 2, 4, 8}, via DPP
template <int D>
__device__ __forceinline__ float lane_xor(float v) {
    const int i = __float_as_int(v);
    if (D == 1) return __int_as_float(__builtin_amdgcn_mov_dpp(i, 0xB1, 0xF, 0xF, true));  // quad_perm [1,0,3,2]
    if (D == 2) return __int_as_float(__builtin_amdgcn_mov_dpp(i, 0x4E, 0xF, 0xF, true));  // quad_perm [2,3,0,1]
    if (D == 4) {
        // xor 4 = (xor 7 within 8 lanes: row_half_mirror) then (xor 3: quad_perm [3,2,1,0])
        const int m = __builtin_amdgcn_mov_dpp(i, 0x141, 0xF, 0xF, true);
        return __int_as_float(__builtin_amdgcn_mov_dpp(m, 0x1B, 0xF, 0xF, true));
    }
    // xor 8 = (xor 15 within 16 lanes: row_mirror) then (xor 7: row_half_mirror)
    const int m = __builtin_amdgcn_mov_dpp(i, 0x140, 0xF, 0xF, true);
    return __int_as_float(__builtin_amdgcn_mov_dpp(m, 0x141, 0xF, 0xF, true));
}

// one cross-lane butterfly stage: the lower lane of each pair keeps lo + hi,
// the upper lane lo - hi (sign * v is exact, so the fma rounds exactly once)
template <int D, int E>
__device__ __forceinline__ void cross_stage(float (&v)[E], int lane) {
    const float sgn = (lane & D) ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] = __builtin_fmaf(sgn, v[i], lane_xor<D>(v[i]));
}

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

template <int E>
__device__ __forceinline__ float lane_absmax(const float (&v)[E]) {
    float t[E / 2];
#pragma unroll
    for (int i = 0; i < E / 2; ++i) t[i] = fmaxf(fabsf(v[2 * i]), fabsf(v[2 * i + 1]));
#pragma unroll
    for (int w = E / 4; w >= 1; w >>= 1)
#pragma unroll
        for (int i = 0; i < w; ++i) t[i] = fmaxf(t[i], t[i + w]);
    return t[0];
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
                                                 float eps, const float* __restrict__ ascale, float rs, int c,
                                                 int nwaves, double* red_d, float* red_f, Store store) {
    constexpr int hblock = 1 << LOG2B;
    constexpr int qmax = ABITS == 8 ? 127 : 7;
    const int lane = c & 63;
    const int wave = c >> 6;
    const bool active = c < K / E;  // lanes past K hold zeros and only join the exchanges

    constexpr bool kPreG = TokenLoad<E, NORM>::kPreG;
    float v[E];
    const float4* const g = t.g;
#pragma unroll
    for (int q = 0; q < E / 8; ++q) unpack8(t.d[q], &v[8 * q]);

    // RMSNorm with the folded gain: the float32 squares are exact in float64
    if (NORM) {
        double ss = wave_sum(lane_sumsq<E>(v));
        if (nwaves > 1) {
            if (lane == 0) red_d[wave] = ss;
            __syncthreads();
            ss = 0.0;
            for (int w = 0; w < nwaves; ++w) ss += red_d[w];
        }
        const float ms = float(ss / double(K));
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
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] = v[i] * rs;

    if (AMODE == 2) divide_by_vector<E>(v, ascale, c, active);

    // per-token amax (lanes past K hold zeros)
    float amax = wave_max(lane_absmax<E>(v));
    if (nwaves > 1) {
        if (lane == 0) red_f[wave] = amax;
        __syncthreads();
        amax = 0.0f;
        for (int w = 0; w < nwaves; ++w) amax = fmaxf(amax, red_f[w]);
    }
    const float s = amax / float(qmax);
    const bool fast = s >= 0x1p-100f && s <= 0x1p+100f;
    const float r = fast ? 1.0f / s : 0.0f;

    // Codes.  |h| <= amax and s is amax / qmax rounded, so |h / s| stays below
    // qmax + 1/2 and round-half-even never leaves [-qmax, qmax]: the clamp of
    // the definition is implied and not executed.
    // (one code path per divide form: as a per-element condition it cost a
    // branch around every element's fallback divide)
    auto quantise = [&](auto fast_tag) {
        constexpr bool kFast = decltype(fast_tag)::value;
        constexpr int G = E < 16 ? E : 16;  // codes per store
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
            if (ABITS == 8) {
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
                if constexpr (G == 16)
                    store((E / 2) * c + (G / 2) * grp, make_uint2(w[0], w[1]));
                else
                    store((E / 2) * c + (G / 2) * grp, w[0]);
            }
        }
    };
    if (active) {
        if (fast)
            quantise(std::true_type{});
        else
            quantise(std::false_type{});
    }
    return s;
}

template <int E, int ABITS, bool NORM, int AMODE, int LOG2B, class Store>
__device__ __forceinline__ float quantise_token(const uint16_t* __restrict__ xr, int K,
                                                const float* __restrict__ gamma, float eps,
                                                const float* __restrict__ ascale, float rs, int c, int nwaves,
                                                double* red_d, float* red_f, Store store) {
    return quantise_loaded<E, ABITS, NORM, AMODE, LOG2B>(load_token<E, NORM>(xr, K, gamma, c), K, gamma, eps,
                                                         ascale, rs, c, nwaves, red_d, red_f, store);
}

}  // namespace fq

// Device helpers shared by the FoldQuant kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v6i __attribute__((ext_vector_type(6)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Streaming loads that bypass cache allocation for data read exactly once.
__device__ __forceinline__ uint4 load_stream16(const uint8_t* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint2 load_stream8(const uint8_t* p) {
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    return make_uint2(v[0], v[1]);
}

// Device-scope (sc1) stores: written through L2 as they are made, so that a
// kernel's output is not left dirty in L2 for the write-back at its end.  The
// compiler does not count these stores in its memory-counter waits; they only
// add to the count, so its waits for its own loads stay long enough.
__device__ __forceinline__ void store_dev16(void* p, uint4 v) {
    const u32x4 d = {v.x, v.y, v.z, v.w};
    asm volatile("global_store_dwordx4 %0, %1, off sc1" ::"v"(p), "v"(d) : "memory");
}
__device__ __forceinline__ void store_dev8(void* p, uint2 v) {
    const u32x2 d = {v.x, v.y};
    asm volatile("global_store_dwordx2 %0, %1, off sc1" ::"v"(p), "v"(d) : "memory");
}
__device__ __forceinline__ void store_dev4(void* p, uint32_t v) {
    asm volatile("global_store_dword %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two float32 -> bfloat16 conversions packed in one dword (lo in the low half),
// round to nearest, ties to even: gfx950's v_cvt_pk_bf16_f32 (NaN -> quiet NaN).
// (Written as one vector conversion: two scalar casts compile to two
// conversions plus a shift and an or.)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t v = __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t);
    return __builtin_bit_cast(uint32_t, v);
}

// Operand fragments for v_mfma_i32_16x16x64_i8.  The MFMA sums over its 64 k
// values in any order, so each operand only has to present the same k to the
// same byte slot as the other operand.
//
// 8-bit codes: 16 bytes = k0..k15 in natural order.
// 4-bit codes: 8 bytes = 16 nibbles (even k low).  Each nibble is moved into the
// high half of a byte, which makes the byte exactly 16x the signed code:
//   lo(d) = (d << 4) & 0xF0F0F0F0 -> 16*[k0, k2, k4, k6]
//   hi(d) =  d       & 0xF0F0F0F0 -> 16*[k1, k3, k5, k7]
// giving the k order [0,2,4,6, 1,3,5,7, 8,10,12,14, 9,11,13,15]; the product
// is then 16x (one 4-bit side) or 256x (two) the true one and the
// accumulator is shifted back exactly.  An 8-bit operand facing a 4-bit one is
// byte-permuted into that same order.
__device__ __forceinline__ v4i frag_from_nibbles(uint2 p) {
    v4i r;
    r[0] = int((p.x << 4) & 0xF0F0F0F0u);
    r[1] = int(p.x & 0xF0F0F0F0u);
    r[2] = int((p.y << 4) & 0xF0F0F0F0u);
    r[3] = int(p.y & 0xF0F0F0F0u);
    return r;
}

__device__ __forceinline__ v4i frag_from_bytes(uint4 p) {
    v4i r;
    r[0] = int(p.x);
    r[1] = int(p.y);
    r[2] = int(p.z);
    r[3] = int(p.w);
    return r;
}

// 16 natural-order bytes permuted into the nibble order above.
__device__ __forceinline__ v4i frag_from_bytes_nibble_order(uint4 p) {
    v4i r;
    // __builtin_amdgcn_perm(hi, lo, sel): byte i of the result = byte sel_i of {hi:lo}
    r[0] = int(__builtin_amdgcn_perm(p.y, p.x, 0x06040200u));  // k0 k2 k4 k6
    r[1] = int(__builtin_amdgcn_perm(p.y, p.x, 0x07050301u));  // k1 k3 k5 k7
    r[2] = int(__builtin_amdgcn_perm(p.w, p.z, 0x06040200u));  // k8 k10 k12 k14
    r[3] = int(__builtin_amdgcn_perm(p.w, p.z, 0x07050301u));  // k9 k11 k13 k15
    return r;
}

template <int BITS_SELF, int BITS_OTHER>
struct Frag;

template <>
struct Frag<8, 8> {
    static constexpr int kBytes = 16;
    __device__ __forceinline__ static v4i load(const uint8_t* p) {
        return frag_from_bytes(*reinterpret_cast<const uint4*>(p));
    }
};
template <>
struct Frag<8, 4> {
    static constexpr int kBytes = 16;
    __device__ __forceinline__ static v4i load(const uint8_t* p) {
        return frag_from_bytes_nibble_order(*reinterpret_cast<const uint4*>(p));
    }
};
template <int OTHER>
struct Frag4 {
    static constexpr int kBytes = 8;
    __device__ __forceinline__ static v4i load(const uint8_t* p) {
        return frag_from_nibbles(*reinterpret_cast<const uint2*>(p));
    }
};
template <>
struct Frag<4, 4> : Frag4<4> {};
template <>
struct Frag<4, 8> : Frag4<8> {};

// Shift that undoes the 16x per 4-bit operand.
template <int ABITS, int WBITS>
struct AccShift {
    static constexpr int value = (ABITS == 4 ? 4 : 0) + (WBITS == 4 ? 4 : 0);
};

__device__ __forceinline__ v4i mfma16x16x64(v4i a, v4i b, v4i c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// Epilogue for a wave's TN x TM accumulator tiles: tile (i, ii) holds output
// features n[i] + 4 (lane / 16) + r (r = 0..3, the four accumulator values) of
// token m[ii] + lane % 16, with n[i] and m[ii] already including the lane's part:
//   y[m][n] = bf16_rne(float(acc >> shift) * (s_m * s_n) [+ bias_n] [+ residual_mn])
// in float32, each step rounded (no contraction); acc_out, when given, receives
// the exact integer sums.  y is [M][ldy], or [N/head_dim][M][head_dim] when
// head_dim > 0.  Every operand is loaded before the first store: on
// gfx9 stores count in the same vector-memory counter as loads, so a load placed
// after a store would wait for that store to complete.
template <int TN, int TM>
__device__ __forceinline__ void store_tiles(const v4i (&acc)[TN][TM], int shift, const int (&m)[TM], const int (&n)[TN],
                                            int M, int N, const float* __restrict__ act_scale,
                                            const float* __restrict__ wscale, const float* __restrict__ bias,
                                            const uint16_t* __restrict__ residual, int64_t ldr,
                                            uint16_t* __restrict__ y, int64_t ldy, int32_t* __restrict__ acc_out,
                                            int head_dim) {
    float sa[TM];
#pragma unroll
    for (int ii = 0; ii < TM; ++ii) sa[ii] = m[ii] < M ? act_scale[m[ii]] : 0.0f;
    float4 sw[TN], bs[TN];
#pragma unroll
    for (int i = 0; i < TN; ++i) {
        const bool ok = n[i] < N;
        sw[i] = ok ? *reinterpret_cast<const float4*>(wscale + n[i]) : make_float4(0.f, 0.f, 0.f, 0.f);
        bs[i] = (bias && ok) ? *reinterpret_cast<const float4*>(bias + n[i]) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    uint2 rs[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int ii = 0; ii < TM; ++ii)
            rs[i][ii] = (residual && n[i] < N && m[ii] < M)
                            ? *reinterpret_cast<const uint2*>(residual + int64_t(m[ii]) * ldr + n[i])
                            : make_uint2(0, 0);
    // one wait for all of them, outside any branch, so that no wait is placed
    // behind a store below (vmcnt(0), other counters untouched)
    __builtin_amdgcn_s_waitcnt(0x0F70);
#pragma unroll
    for (int ii = 0; ii < TM; ++ii)
#pragma unroll
        for (int i = 0; i < TN; ++i) {
            if (m[ii] >= M || n[i] >= N) continue;
            const int a0 = acc[i][ii][0] >> shift, a1 = acc[i][ii][1] >> shift;
            const int a2 = acc[i][ii][2] >> shift, a3 = acc[i][ii][3] >> shift;
            float t0 = float(a0) * (sa[ii] * sw[i].x);
            float t1 = float(a1) * (sa[ii] * sw[i].y);
            float t2 = float(a2) * (sa[ii] * sw[i].z);
            float t3 = float(a3) * (sa[ii] * sw[i].w);
            if (bias) {
                t0 = t0 + bs[i].x;
                t1 = t1 + bs[i].y;
                t2 = t2 + bs[i].z;
                t3 = t3 + bs[i].w;
            }
            if (residual) {
                t0 = t0 + bf16_lo(rs[i][ii].x);
                t1 = t1 + bf16_hi(rs[i][ii].x);
                t2 = t2 + bf16_lo(rs[i][ii].y);
                t3 = t3 + bf16_hi(rs[i][ii].y);
            }
            uint2 o;
            o.x = pack_bf16x2(t0, t1);
            o.y = pack_bf16x2(t2, t3);
            uint16_t* yp = y + int64_t(m[ii]) * ldy + n[i];
            if (head_dim > 0) {  // [N/head_dim][M][head_dim]; 4 consecutive n stay in one head
                const int h = n[i] / head_dim;
                yp = y + (int64_t(h) * M + m[ii]) * head_dim + (n[i] - h * head_dim);
            }
            *reinterpret_cast<uint2*>(yp) = o;
            if (acc_out) *reinterpret_cast<int4*>(acc_out + int64_t(m[ii]) * N + n[i]) = make_int4(a0, a1, a2, a3);
        }
}

}  // namespace fq

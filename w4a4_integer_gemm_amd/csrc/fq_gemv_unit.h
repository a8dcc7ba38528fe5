// The unit of work of the decode GEMV kernels (gfx950, wave64), shared by the
// split-K and streaming kernels (fq_gemv.hip) and the one-token decode kernel
// (fq_decode1.hip).
//
// A unit is one 16-byte weight load per lane: 64 k of 8-bit or 128 k of 4-bit
// codes for the 16 rows of a v_mfma_i32_16x16x64_i8 A operand.  Lane l serves
// row l % 16 and the k quarter q = l / 16 of the unit; the B operand holds up
// to 16 tokens, token l % 16 in lane l.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fq_device.h"

namespace fq {

// k per unit and the bytes of one lane's activation codes per unit.
template <int ABITS, int WBITS>
struct Unit {
    static constexpr int K = WBITS == 8 ? 64 : 128;
    static constexpr int WROW = K * WBITS / 8;       // weight bytes per row per unit (64)
    static constexpr int AROW = K * ABITS / 8;       // activation bytes per token per unit
    static constexpr int ALANE = AROW / 4;           // 8, 16 or 32
    static constexpr int AREGS = ALANE > 16 ? 2 : 1; // 16-byte registers per lane
};

// One lane's activation codes of one unit (8, 16 or 32 bytes).
struct ActReg {
    uint4 v[2];
};

template <int ABITS, int WBITS>
__device__ __forceinline__ void load_act(ActReg& a, const uint8_t* p, bool ok) {
    using U = Unit<ABITS, WBITS>;
    a.v[0] = make_uint4(0, 0, 0, 0);
    a.v[1] = make_uint4(0, 0, 0, 0);
    if (ok) {
        if (U::ALANE == 8) {
            const uint2 t = *reinterpret_cast<const uint2*>(p);
            a.v[0] = make_uint4(t.x, t.y, 0, 0);
        } else {
            a.v[0] = *reinterpret_cast<const uint4*>(p);
            if (U::AREGS == 2) a.v[1] = *reinterpret_cast<const uint4*>(p + 16);
        }
    }
}

// acc += the unit's product; w = the lane's 16 weight bytes.
//  8-bit weights: one MFMA over k = 16 q + [0, 16) of the unit.
//  4-bit weights: the lane's 32 nibbles are k = 32 q + [0, 32); MFMA j takes
//  bytes 8 j .. 8 j + 7 of both operands, k = 32 q + 16 j + [0, 16).
template <int ABITS, int WBITS>
__device__ __forceinline__ v4i unit_mfma(const uint4 w, const ActReg& a, v4i acc) {
    if (WBITS == 8) {
        if (ABITS == 8) return mfma16x16x64(frag_from_bytes(w), frag_from_bytes(a.v[0]), acc);
        return mfma16x16x64(frag_from_bytes_nibble_order(w), frag_from_nibbles(make_uint2(a.v[0].x, a.v[0].y)),
                            acc);
    }
    const v4i w0 = frag_from_nibbles(make_uint2(w.x, w.y));
    const v4i w1 = frag_from_nibbles(make_uint2(w.z, w.w));
    if (ABITS == 4) {
        acc = mfma16x16x64(w0, frag_from_nibbles(make_uint2(a.v[0].x, a.v[0].y)), acc);
        return mfma16x16x64(w1, frag_from_nibbles(make_uint2(a.v[0].z, a.v[0].w)), acc);
    }
    acc = mfma16x16x64(w0, frag_from_bytes_nibble_order(a.v[0]), acc);
    return mfma16x16x64(w1, frag_from_bytes_nibble_order(a.v[1]), acc);
}

template <int ABITS, int WBITS>
__device__ __forceinline__ void lds_act(ActReg& a, const uint8_t* p) {
    using U = Unit<ABITS, WBITS>;
    a.v[1] = make_uint4(0, 0, 0, 0);
    if (U::ALANE == 8) {
        const uint2 t = *reinterpret_cast<const uint2*>(p);
        a.v[0] = make_uint4(t.x, t.y, 0, 0);
    } else {
        a.v[0] = *reinterpret_cast<const uint4*>(p);
        if (U::AREGS == 2) a.v[1] = *reinterpret_cast<const uint4*>(p + 16);
    }
}

}  // namespace fq

// FoldQuant activation prologue on gfx950 (the vla.cpp page's fused
// "RMSNorm + butterfly + quant" act node; its OpenVINO commit lists the steps:
// RMSNorm with the folded gain, the ascale divide, the block rotation, a
// per-token amax scale, round-half-even and a clamp).
//
// Layout: one workgroup per token.  Lane t of the workgroup owns 8 consecutive
// bf16 values (one 16-byte load) per pass; a token of K values takes K/8 lanes
// spread over P passes (P <= 8, so K <= 65536).  A Hadamard block of b values is
// b/8 consecutive lanes of one wavefront (b <= 256 -> at most 32 lanes), so
// the butterfly's first three stages (span 1, 2, 4) run inside a lane's
// registers and the later ones (span 8 .. b/2) exchange across lanes.  Every
// element goes through the same float32 operations in the same order as the
// definition (stage spans 1, 2, 4, ...), so the rotation is bit-reproducible.
// The whole token stays in registers between the two reductions (sum of
// squares, then amax), so x is read from HBM once and the codes written once.
#include <hip/hip_runtime.h>

#include <cmath>

#include "fq_device.h"
#include "fq_internal.h"

namespace fq {
namespace {

constexpr int kMaxThreads = 1024;
constexpr int kMaxWaves = kMaxThreads / 64;

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

template <int P, int ABITS>
__global__ __launch_bounds__(kMaxThreads) void prologue_kernel(
    const uint16_t* __restrict__ x, int K, int64_t ldx, const float* __restrict__ gamma, float eps,
    const float* __restrict__ ascale, int fold_after, int hblock, float rs, uint8_t* __restrict__ codes,
    float* __restrict__ act_scale) {
    constexpr int qmax = ABITS == 8 ? 127 : 7;
    __shared__ double red_d[kMaxWaves];
    __shared__ float red_f[kMaxWaves];

    const int m = blockIdx.x;
    const int T = blockDim.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int nwaves = T >> 6;
    const int nchunks = K >> 3;
    const uint16_t* xr = x + int64_t(m) * ldx;

    float v[P][8];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const int c = p * T + tid;
        uint4 d = make_uint4(0, 0, 0, 0);
        if (c < nchunks) d = *reinterpret_cast<const uint4*>(xr + 8 * c);
        v[p][0] = bf16_lo(d.x);
        v[p][1] = bf16_hi(d.x);
        v[p][2] = bf16_lo(d.y);
        v[p][3] = bf16_hi(d.y);
        v[p][4] = bf16_lo(d.z);
        v[p][5] = bf16_hi(d.z);
        v[p][6] = bf16_lo(d.w);
        v[p][7] = bf16_hi(d.w);
    }

    // RMSNorm with the folded gain: the float32 squares are exact in float64
    if (gamma) {
        double ss = 0.0;
#pragma unroll
        for (int p = 0; p < P; ++p)
#pragma unroll
            for (int i = 0; i < 8; ++i) ss += double(v[p][i]) * double(v[p][i]);
        ss = wave_sum(ss);
        if (lane == 0) red_d[wave] = ss;
        __syncthreads();
        double tot = 0.0;
        for (int w = 0; w < nwaves; ++w) tot += red_d[w];
        const float ms = float(tot / double(K));
        const float rinv = 1.0f / sqrtf(ms + eps);
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int c = p * T + tid;
            if (c < nchunks) {
                const float4 g0 = *reinterpret_cast<const float4*>(gamma + 8 * c);
                const float4 g1 = *reinterpret_cast<const float4*>(gamma + 8 * c + 4);
                const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
                for (int i = 0; i < 8; ++i) v[p][i] = (v[p][i] * rinv) * g[i];
            }
        }
    }

    // explicit smoothing divide before the rotation
    if (ascale && !fold_after) {
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int c = p * T + tid;
            if (c < nchunks) {
                const float4 a0 = *reinterpret_cast<const float4*>(ascale + 8 * c);
                const float4 a1 = *reinterpret_cast<const float4*>(ascale + 8 * c + 4);
                const float a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
                for (int i = 0; i < 8; ++i) v[p][i] = v[p][i] / a[i];
            }
        }
    }

    // block Hadamard butterfly: spans 1, 2, 4 inside the lane ...
#pragma unroll
    for (int span = 1; span < 8; span <<= 1) {
        if (span < hblock) {
#pragma unroll
            for (int p = 0; p < P; ++p)
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    if ((i & span) == 0) {
                        const float lo = v[p][i], hi = v[p][i + span];
                        v[p][i] = lo + hi;
                        v[p][i + span] = lo - hi;
                    }
        }
    }
    // ... spans 8 .. b/2 across lanes (lane distance span/8)
    for (int d = 1; 8 * d < hblock; d <<= 1) {
        const bool upper = (lane & d) != 0;
#pragma unroll
        for (int p = 0; p < P; ++p)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float other = __shfl_xor(v[p][i], d);
                // lower lane holds the first operand: lo + hi; upper lane: lo - hi
                v[p][i] = upper ? (other - v[p][i]) : (v[p][i] + other);
            }
    }
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
        for (int i = 0; i < 8; ++i) v[p][i] = v[p][i] * rs;

    // explicit smoothing divide after the rotation
    if (ascale && fold_after) {
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int c = p * T + tid;
            if (c < nchunks) {
                const float4 a0 = *reinterpret_cast<const float4*>(ascale + 8 * c);
                const float4 a1 = *reinterpret_cast<const float4*>(ascale + 8 * c + 4);
                const float a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
                for (int i = 0; i < 8; ++i) v[p][i] = v[p][i] / a[i];
            }
        }
    }

    // per-token amax (lanes past K hold zeros)
    float amax = 0.0f;
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[p][i]));
    amax = wave_max(amax);
    if (lane == 0) red_f[wave] = amax;
    __syncthreads();
    amax = 0.0f;
    for (int w = 0; w < nwaves; ++w) amax = fmaxf(amax, red_f[w]);
    const float s = amax / float(qmax);

    constexpr int row_div = ABITS == 8 ? 1 : 2;
    uint8_t* cr = codes + int64_t(m) * (K / row_div);
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const int c = p * T + tid;
        if (c < nchunks) {
            int q[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float r = s > 0.0f ? rintf(v[p][i] / s) : 0.0f;
                r = fminf(fmaxf(r, float(-qmax)), float(qmax));
                q[i] = int(r);
            }
            if (ABITS == 8) {
                uint2 o;
                o.x = (uint32_t(q[0]) & 0xFF) | ((uint32_t(q[1]) & 0xFF) << 8) | ((uint32_t(q[2]) & 0xFF) << 16) |
                      (uint32_t(q[3]) << 24);
                o.y = (uint32_t(q[4]) & 0xFF) | ((uint32_t(q[5]) & 0xFF) << 8) | ((uint32_t(q[6]) & 0xFF) << 16) |
                      (uint32_t(q[7]) << 24);
                *reinterpret_cast<uint2*>(cr + 8 * c) = o;
            } else {
                uint32_t o = 0;
#pragma unroll
                for (int i = 0; i < 8; ++i) o |= (uint32_t(q[i]) & 0xF) << (4 * i);
                *reinterpret_cast<uint32_t*>(cr + 4 * c) = o;
            }
        }
    }
    if (tid == 0) act_scale[m] = s;
}

template <int ABITS>
hipError_t launch_p(int P, dim3 grid, dim3 block, hipStream_t st, const PrologueArgs& a, float rs) {
#define FQ_PRO_CASE(PP)                                                                                     \
    case PP:                                                                                                \
        hipLaunchKernelGGL((prologue_kernel<PP, ABITS>), grid, block, 0, st, a.x, a.K, a.ldx, a.gamma, a.eps, \
                           a.ascale, a.fold_after, a.hblock, rs, a.codes, a.act_scale);                     \
        break;
    switch (P) {
        FQ_PRO_CASE(1)
        FQ_PRO_CASE(2)
        FQ_PRO_CASE(3)
        FQ_PRO_CASE(4)
        FQ_PRO_CASE(5)
        FQ_PRO_CASE(6)
        FQ_PRO_CASE(7)
        FQ_PRO_CASE(8)
        default:
            return hipErrorInvalidValue;
    }
#undef FQ_PRO_CASE
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prologue(const PrologueArgs& a, hipStream_t stream) {
    const int nchunks = a.K / 8;
    const int P = (nchunks + kMaxThreads - 1) / kMaxThreads;
    int T = (nchunks + P - 1) / P;
    T = (T + 63) / 64 * 64;
    const float rs = float(1.0 / std::sqrt(double(a.hblock)));
    dim3 grid(a.M), block(T);
    return a.abits == 8 ? launch_p<8>(P, grid, block, stream, a, rs) : launch_p<4>(P, grid, block, stream, a, rs);
}

}  // namespace fq

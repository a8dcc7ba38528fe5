// FoldQuant decode path (M <= 32 tokens) on gfx950: a weight-streaming GEMV.
//
// For decode-sized M the layer is bound by reading the weight codes once from
// HBM (the SYCL commit of the vla.cpp FoldQuant page also switches to a GEMV
// for M <= 32).  Each wave owns 16 weight rows and walks the whole K: per
// 64-deep step a lane loads 16 bytes (8 for 4-bit) of one row, and the
// v_mfma_i32_16x16x64_i8 consumes them against the tokens' codes (tokens as
// the 16-wide B operand; M > 16 takes a second MFMA).  U steps are loaded
// before any is consumed so that each wave keeps U loads in flight.
#include <hip/hip_runtime.h>

#include "fq_device.h"
#include "fq_internal.h"

namespace fq {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kUnroll = 8;

template <int ABITS, int WBITS, int MT>
__global__ __launch_bounds__(kThreads) void gemv_kernel(GemmArgs g) {
    constexpr int wlane = WBITS == 8 ? 16 : 8;  // bytes per lane per step
    constexpr int alane = ABITS == 8 ? 16 : 8;
    constexpr int wrow = WBITS == 8 ? 64 : 32;  // bytes per row per step
    constexpr int arow = ABITS == 8 ? 64 : 32;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n0 = (blockIdx.x * kWaves + wave) * 16;
    if (n0 >= g.N) return;  // whole wave
    const int64_t ldw = WBITS == 8 ? g.K : g.K / 2;
    const int64_t lda = ABITS == 8 ? g.K : g.K / 2;
    const int nk = g.K / 64;
    const int row = n0 + (lane & 15);
    const bool row_ok = row < g.N;
    const uint8_t* wp = g.w + int64_t(row_ok ? row : 0) * ldw + (lane >> 4) * wlane;
    const uint8_t* ap[MT];
    bool tok_ok[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        const int tok = t * 16 + (lane & 15);
        tok_ok[t] = tok < g.M;
        ap[t] = g.act + int64_t(tok_ok[t] ? tok : 0) * lda + (lane >> 4) * alane;
    }

    v4i acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = v4i{0, 0, 0, 0};

    for (int k0 = 0; k0 < nk; k0 += kUnroll) {
        uint4 wv[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            wv[u] = make_uint4(0, 0, 0, 0);
            if (k0 + u < nk && row_ok) {
                const uint8_t* p = wp + int64_t(k0 + u) * wrow;
                if (WBITS == 8) {
                    wv[u] = load_stream16(p);
                } else {
                    const uint2 v = load_stream8(p);
                    wv[u].x = v.x;
                    wv[u].y = v.y;
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (k0 + u < nk) {
                v4i fw;
                if (WBITS == 8) {
                    fw = ABITS == 8 ? frag_from_bytes(wv[u]) : frag_from_bytes_nibble_order(wv[u]);
                } else {
                    fw = frag_from_nibbles(make_uint2(wv[u].x, wv[u].y));
                }
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    v4i fa = v4i{0, 0, 0, 0};
                    if (tok_ok[t]) fa = Frag<ABITS, WBITS>::load(ap[t] + int64_t(k0 + u) * arow);
                    acc[t] = mfma16x16x64(fw, fa, acc[t]);
                }
            }
        }
    }

    constexpr int shift = AccShift<ABITS, WBITS>::value;
    const int n = n0 + (lane >> 4) * 4;
    if (n >= g.N) return;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        const int m = t * 16 + (lane & 15);
        if (m < g.M)
            store_out4(acc[t], shift, m, n, g.act_scale[m], g.wscale, g.bias, g.residual, g.ldr, g.y, g.ldy, g.acc,
                       g.N);
    }
}

template <int ABITS, int WBITS>
void launch_bits(const GemmArgs& g, hipStream_t st) {
    dim3 grid((g.N + kWaves * 16 - 1) / (kWaves * 16)), block(kThreads);
    if (g.M <= 16)
        hipLaunchKernelGGL((gemv_kernel<ABITS, WBITS, 1>), grid, block, 0, st, g);
    else
        hipLaunchKernelGGL((gemv_kernel<ABITS, WBITS, 2>), grid, block, 0, st, g);
}

}  // namespace

hipError_t launch_gemv(const GemmArgs& g, hipStream_t stream) {
    if (g.M > kGemvMaxM) return hipErrorInvalidValue;
    if (g.abits == 8 && g.wbits == 8)
        launch_bits<8, 8>(g, stream);
    else if (g.abits == 4 && g.wbits == 4)
        launch_bits<4, 4>(g, stream);
    else if (g.abits == 8 && g.wbits == 4)
        launch_bits<8, 4>(g, stream);
    else
        launch_bits<4, 8>(g, stream);
    return hipGetLastError();
}

}  // namespace fq

// GeGLU between the two sites of a chained MLP block (gate+up site -> GeGLU ->
// down site with the residual), the block of the Gemma-style backbones the
// vla.cpp FoldQuant page runs W4A4:
//   h[m][j] = bf16_rne(gelu_tanh(gate[m][j]) * up[m][j]),
//   gelu_tanh(g) = g/2 * (1 + tanh(sqrt(2/pi) * (g + 0.044715 g^3))),
// gate and up the two halves of the gate+up site's bf16 output row.  float32
// with no contraction; tanh from the device math library.  Bandwidth-bound:
// each thread reads 16 bytes of gate and of up and writes 16 bytes of h.
#include <hip/hip_runtime.h>

#include "fq_device.h"
#include "fq_internal.h"

namespace fq {
namespace {

__device__ __forceinline__ float gelu_tanh(float g) {
    const float c = 0.7978845608028654f;  // sqrt(2 / pi)
    const float g3 = (g * g) * g;
    const float inner = c * (g + 0.044715f * g3);
    return (0.5f * g) * (1.0f + tanhf(inner));
}

__global__ __launch_bounds__(256) void geglu_kernel(const uint16_t* __restrict__ gu, int32_t M, int32_t F,
                                                    int64_t ld_in, uint16_t* __restrict__ h, int64_t ld_out) {
    const int32_t per_row = F / 8;
    const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (idx >= int64_t(M) * per_row) return;
    const int32_t m = int32_t(idx / per_row);
    const int32_t j = int32_t(idx % per_row) * 8;
    const uint4 g = *reinterpret_cast<const uint4*>(gu + int64_t(m) * ld_in + j);
    const uint4 u = *reinterpret_cast<const uint4*>(gu + int64_t(m) * ld_in + F + j);
    const uint32_t gw[4] = {g.x, g.y, g.z, g.w}, uw[4] = {u.x, u.y, u.z, u.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float lo = gelu_tanh(bf16_lo(gw[i])) * bf16_lo(uw[i]);
        const float hi = gelu_tanh(bf16_hi(gw[i])) * bf16_hi(uw[i]);
        o[i] = pack_bf16x2(lo, hi);
    }
    *reinterpret_cast<uint4*>(h + int64_t(m) * ld_out + j) = make_uint4(o[0], o[1], o[2], o[3]);
}

}  // namespace

hipError_t launch_geglu(const uint16_t* gu, int32_t M, int32_t F, int64_t ld_in, uint16_t* h, int64_t ld_out,
                        hipStream_t stream) {
    const int64_t threads = int64_t(M) * (F / 8);
    const int64_t blocks = (threads + 255) / 256;
    hipLaunchKernelGGL(geglu_kernel, dim3(uint32_t(blocks)), dim3(256), 0, stream, gu, M, F, ld_in, h, ld_out);
    return hipGetLastError();
}

}  // namespace fq

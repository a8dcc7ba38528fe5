// Ceiling probes of the benchmark: the rates this MI355X sustains for the two
// things the FoldQuant layer is bound by, measured next to the layer so that
// its roofline fractions can be stated against measured ceilings as well as
// against the datasheet.  Not part of the layer's C ABI (include/fq.h): a
// separate library, libfq_ceiling.so, loaded by the benchmark only.
//
//   fqc_mfma_i8:   back-to-back v_mfma_i32_16x16x64_i8 (the GEMM's and the
//                  GEMV's instruction) on operands read from a caller buffer:
//                  random bytes give the rate under the power draw of random
//                  codes, zero bytes the rate with quiet operands.
//   fqc_stream_read: every 16-byte piece of a buffer read once (grid-stride,
//                  U loads in flight per lane), the HBM read rate a
//                  weight-streaming kernel can reach.
//
// Both are asynchronous on the caller's stream; the caller times them.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kOps = 8;        // operand registers per lane (A and B each)
constexpr int kAcc = 8;        // independent accumulators
constexpr int kThreads = 256;  // 4 waves

// Each lane takes its 2 kOps operand registers from src (16 bytes each, lane
// l reading pieces 2 kOps l .. 2 kOps l + 2 kOps - 1), then runs `iters` rounds of kOps MFMAs; round
// r pairs A[j] with B[(j + 3) % kOps], so consecutive instructions never
// repeat an operand.  The accumulators are folded into one word per lane and
// written only if it equals a value no sum of these codes reaches in practice
// (so the MFMAs cannot be removed, and out is written almost never).
__global__ __launch_bounds__(kThreads) void mfma_rate_kernel(const uint4* __restrict__ src, int iters,
                                                            int32_t* __restrict__ out) {
    const int64_t lane_id = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    v4i a[kOps], b[kOps];
#pragma unroll
    for (int j = 0; j < kOps; ++j) {
        const uint4 ua = src[lane_id * 2 * kOps + j];
        const uint4 ub = src[lane_id * 2 * kOps + kOps + j];
        a[j] = v4i{int(ua.x), int(ua.y), int(ua.z), int(ua.w)};
        b[j] = v4i{int(ub.x), int(ub.y), int(ub.z), int(ub.w)};
    }
    v4i acc[kAcc];
#pragma unroll
    for (int j = 0; j < kAcc; ++j) acc[j] = v4i{0, 0, 0, 0};
    for (int r = 0; r < iters; ++r) {
#pragma unroll
        for (int j = 0; j < kOps; ++j)
            acc[j % kAcc] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[j], b[(j + 3) % kOps], acc[j % kAcc], 0, 0, 0);
    }
    int s = 0;
#pragma unroll
    for (int j = 0; j < kAcc; ++j) s ^= acc[j][0] ^ acc[j][1] ^ acc[j][2] ^ acc[j][3];
    if (s == 0x7F3A5C19) out[0] = s;
}

template <int U>
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4* __restrict__ p, int64_t n16,
                                                               uint32_t* __restrict__ out) {
    const int64_t stride = int64_t(gridDim.x) * kThreads;
    int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    uint32_t x = 0;
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = p[i + u * stride];
#pragma unroll
        for (int u = 0; u < U; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const uint4 v = p[i];
        x ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (x == 0x9E3779B9u) out[0] = x;
}

}  // namespace

extern "C" {

// Operations one fqc_mfma_i8 launch performs (2 * 16 * 16 * 64 per MFMA).
int64_t fqc_mfma_i8_ops(int32_t blocks, int32_t iters) {
    return int64_t(blocks) * (kThreads / 64) * int64_t(iters) * kOps * 2 * 16 * 16 * 64;
}

// blocks workgroups of 4 waves; src: device buffer of n16 16-byte pieces, at
// least 2 kOps per lane (blocks * 256 * 16); out: one device int32.  Returns 0,
// or a hipError_t.
int fqc_mfma_i8(const void* src, int64_t n16, int32_t blocks, int32_t iters, void* out, void* stream) {
    if (!src || !out || blocks < 1 || iters < 1) return int(hipErrorInvalidValue);
    if (n16 < int64_t(blocks) * kThreads * 2 * kOps) return int(hipErrorInvalidValue);
    hipLaunchKernelGGL(mfma_rate_kernel, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint4*>(src), iters, static_cast<int32_t*>(out));
    return int(hipGetLastError());
}

// Reads n16 16-byte pieces of buf with `blocks` workgroups of 256 lanes and
// u in {1, 2, 4, 8, 16} loads in flight per lane; out: one device uint32.
int fqc_stream_read(const void* buf, int64_t n16, int32_t blocks, int32_t u, void* out, void* stream) {
    if (!buf || !out || n16 < 1 || blocks < 1) return int(hipErrorInvalidValue);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const uint4* p = static_cast<const uint4*>(buf);
    uint32_t* o = static_cast<uint32_t*>(out);
    switch (u) {
        case 1: hipLaunchKernelGGL(stream_read_kernel<1>, dim3(blocks), dim3(kThreads), 0, st, p, n16, o); break;
        case 2: hipLaunchKernelGGL(stream_read_kernel<2>, dim3(blocks), dim3(kThreads), 0, st, p, n16, o); break;
        case 4: hipLaunchKernelGGL(stream_read_kernel<4>, dim3(blocks), dim3(kThreads), 0, st, p, n16, o); break;
        case 8: hipLaunchKernelGGL(stream_read_kernel<8>, dim3(blocks), dim3(kThreads), 0, st, p, n16, o); break;
        case 16: hipLaunchKernelGGL(stream_read_kernel<16>, dim3(blocks), dim3(kThreads), 0, st, p, n16, o); break;
        default: return int(hipErrorInvalidValue);
    }
    return int(hipGetLastError());
}

}  // extern "C"

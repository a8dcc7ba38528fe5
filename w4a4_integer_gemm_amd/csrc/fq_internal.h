// Internal interfaces between the C ABI layer (fq_api.cpp) and the kernel
// translation units.  Not installed; the public surface is include/fq.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

namespace fq {

// Thread-local error message shared by every entry point.
void set_error(const std::string& msg);
void clear_error();

struct PrologueArgs {
    const uint16_t* x;
    int32_t M, K;
    int64_t ldx;
    const float* gamma;   // nullptr: no RMSNorm
    float eps;
    const float* ascale;  // nullptr: no explicit smoothing
    int32_t fold_after;
    int32_t hblock;
    int32_t abits;
    uint8_t* codes;
    float* act_scale;
};

struct GemmArgs {
    const uint8_t* act;   // [M][K*abits/8]
    const float* act_scale;
    int32_t M, abits;
    const uint8_t* w;     // [N][K*wbits/8]
    const float* wscale;
    int32_t N, K, wbits;
    const float* bias;        // nullptr: none
    const uint16_t* residual; // nullptr: none
    int64_t ldr;
    uint16_t* y;
    int64_t ldy;
    int32_t* acc;             // nullptr: not written
    int32_t head_dim;         // 0: y is [M][ldy]; else y is [N/head_dim][M][head_dim]
};

// Address of output (m, n) (n a multiple of 4 inside one head when head_dim > 0).
__host__ __device__ inline uint16_t* out_ptr(const GemmArgs& g, int m, int n) {
    if (g.head_dim > 0) {
        const int h = n / g.head_dim;
        return g.y + (int64_t(h) * g.M + m) * g.head_dim + (n - h * g.head_dim);
    }
    return g.y + int64_t(m) * g.ldy + n;
}

// Enqueue the kernels; they return hipGetLastError() of the launch.
hipError_t launch_prologue(const PrologueArgs& a, hipStream_t stream);
hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream);
hipError_t launch_gemv(const GemmArgs& a, hipStream_t stream);
hipError_t launch_geglu(const uint16_t* gu, int32_t M, int32_t F, int64_t ld_in, uint16_t* h, int64_t ld_out,
                        hipStream_t stream);

// Largest M that the GEMV kernel takes.
constexpr int32_t kGemvMaxM = 32;

}  // namespace fq

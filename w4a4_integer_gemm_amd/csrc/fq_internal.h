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
};

// Enqueue the kernels; they return hipGetLastError() of the launch.
hipError_t launch_prologue(const PrologueArgs& a, hipStream_t stream);
hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream);
hipError_t launch_gemv(const GemmArgs& a, hipStream_t stream);

// Largest M that the GEMV kernel takes.
constexpr int32_t kGemvMaxM = 32;

}  // namespace fq

// Internal interfaces between the C ABI layer (fq_api.cpp) and the kernel
// translation units.  Not installed; the public surface is include/fq.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
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

// Forced kernel choices for the tests (fq_test_hook, or the FQ_TEST_HOOK
// environment variable read once, at the first use).  The launch paths read
// these with relaxed atomic loads; nothing on them calls getenv.
struct Hooks {
    std::atomic<int> gemm_tile{-1};  // -1: the cost model picks; else a tile id of fq_gemm.hip
    std::atomic<int> gemm_mfma{16};  // 16: v_mfma_i32_16x16x64_i8 where it applies; 32: 32x32x32 only
    std::atomic<int> gemv_split{0};  // 1: decode-sized M always takes the split-K GEMV
    std::atomic<int> decode1_off{0}; // 1: one-token fq_linear as two launches, never the fused kernel
};
Hooks& hooks();
// Tile id of a tile name ("128x144", ...), or -1 (fq_gemm.hip).
int gemm_tile_id(const char* name);

// What a device's launches need to know, gathered once per device and process
// by prepare_device (fq_api.cpp): the compute-unit count, the LDS of a CU and,
// per streaming-GEMV kernel (bit mix x token tiles), how many of its
// workgroups the register file lets a CU hold.  The same set-up raises those
// kernels' dynamic-LDS limit, so no launch makes a HIP call other than the
// launch itself.
constexpr int kMaxDevices = 64;
struct DeviceInfo {
    int device;
    int cus;
    int lds_per_cu;
    int stream_regs_wg[4][2];  // [bit mix: 8/8, 4/4, 8/4, 4/8][token tiles - 1]
    void* scratch;             // this device's copy of the allocation-free workspace
};

// Size of the device array that fq_linear_noalloc uses as its workspace (the
// activation codes and scales, laid out as fq_linear's workspace).
constexpr size_t kNoallocScratchBytes = size_t(24) << 20;
// Set-up of the current device (once); *info points at its record.
hipError_t prepare_device(const DeviceInfo** info);
// The streaming GEMV's part of that set-up (fq_gemv.hip).
hipError_t init_gemv_device(DeviceInfo& d);
// The address of this device's scratch array (fq_noalloc.hip).
hipError_t init_scratch_device(DeviceInfo& d);

// Enqueue the kernels; they return hipGetLastError() of the launch.  Shapes
// are validated by the caller; a launch makes no other HIP call.
hipError_t launch_prologue(const PrologueArgs& a, hipStream_t stream);
hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream);
// The FP6 kernel for E2M3 codes (abits = wbits = 6), every M.
hipError_t launch_gemm_e2m3(const GemmArgs& g, hipStream_t stream);
hipError_t launch_gemv(const GemmArgs& a, const DeviceInfo& dev, hipStream_t stream);
// One-token fq_linear in one launch (fq_decode1.hip): whether the shape takes
// it, and the launch (prologue arguments and GEMM arguments of the same call).
bool decode1_eligible(const PrologueArgs& p, const GemmArgs& g);
hipError_t launch_decode1(const PrologueArgs& p, const GemmArgs& g, hipStream_t stream);
hipError_t launch_geglu(const uint16_t* gu, int32_t M, int32_t F, int64_t ld_in, uint16_t* h, int64_t ld_out,
                        hipStream_t stream);

// Largest M that the GEMV kernel takes.
constexpr int32_t kGemvMaxM = 32;

}  // namespace fq

// One-token decode in one launch (fq_linear with M = 1): the prologue and the
// weight-streaming GEMV of the vla.cpp FoldQuant page's decode path (its SYCL
// commit switches to a GEMV for M <= 32) fused, so that the token's
// quantisation overlaps the weight stream instead of preceding it.
//
// Every workgroup quantises the token itself, with fq_token.h (the prologue's
// own per-token code, so the codes and scale are the prologue's bit for bit),
// while its weight loads are already in flight: the token's loads are issued
// first and the weight loads right after them, all unconditional, so the wait
// for the token leaves the weights in flight.  The codes go to LDS; workgroup
// 0 also writes them and the scale to the caller's workspace, which then holds
// what the two-launch path would have written.  The workgroup then runs the
// split-K GEMV on R = 2 groups of 16 weight rows: 8 waves split K, each with
// its units of both row groups in registers (PER units per wave, the last
// unit requested again where its share is smaller), the partial tiles meet in
// LDS and two waves run the shared epilogue.
//
// The token is redone by every workgroup: N / 32 times in all, about 2.3 us
// of VALU per SIMD at the 37888-row decode layer, spread over a launch that
// streams 136 MB and leaves the VALU otherwise idle.  Measured (M = 1, K =
// 3584, N = 37888, W8A8, weights rotated over 5 copies, one box): 27.0 us
// against 28.3 us for the prologue and the split-K GEMV as two launches; one
// row group per workgroup 27.5 us, three 29.3 us, four 32.7 us (the register
// file then holds fewer workgroups).
//
// Taken when M = 1, K <= 4096 (8 values per lane over 512 lanes), the codes
// are 4- or 8-bit and the Hadamard block is 32, 64 or 128 (a block spans at
// most 16 lanes); other one-token calls take the two launches.
#include <hip/hip_runtime.h>

#include <cmath>

#include "fq_device.h"
#include "fq_gemv_unit.h"
#include "fq_internal.h"
#include "fq_token.h"

namespace fq {
namespace {

constexpr int kWaves = 8;
constexpr int kE = 8;     // token values per lane
constexpr int kRows = 2;  // groups of 16 weight rows per workgroup
constexpr int kMaxK = kWaves * 64 * kE;

template <int ABITS, int WBITS, bool NORM, int AMODE, int LOG2B, int PER>
__global__ __launch_bounds__(64 * kWaves) void decode1_kernel(PrologueArgs p, GemmArgs g, TokenConsts tc) {
    using U = Unit<ABITS, WBITS>;
    __shared__ double red_d[kWaves];
    __shared__ float red_f[kWaves];
    __shared__ __attribute__((aligned(16))) uint8_t act_lds[kMaxK * ABITS / 8];
    __shared__ float s_scale;
    __shared__ v4i red[kWaves][kRows][64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, q = lane >> 4;
    const int K = g.K;

    // the token's loads first ...
    const TokenLoad<kE, NORM> t = load_token_clamped<kE, NORM>(p.x, K, p.gamma, tid);
    __builtin_amdgcn_sched_barrier(0);  // (the scheduler would otherwise sink the gain's loads below the weights')
    // ... then every weight unit of this wave, requested at once
    const int nu = K / U::K;
    const int per = (nu + kWaves - 1) / kWaves;
    const int u0 = wave * per;
    const int n0 = blockIdx.x * 16 * kRows;
    const int64_t ldw = int64_t(K) * WBITS / 8;
    uint4 wv[PER][kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
        int row = n0 + 16 * r + (lane & 15);
        row = row < g.N ? row : g.N - 1;  // rows past N load a valid row; their outputs are not stored
        const uint8_t* wp = g.w + int64_t(row) * ldw + q * 16;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            int u = u0 + (i < per ? i : per - 1);
            u = u < nu ? u : nu - 1;  // repeated units are loaded but not used
            wv[i][r] = *reinterpret_cast<const uint4*>(wp + int64_t(u) * U::WROW);
        }
    }

    // the token's codes into LDS (and, from workgroup 0, into the workspace)
    uint8_t* const ws_codes = p.codes;
    const bool first = blockIdx.x == 0;
    const float s = quantise_loaded<kE, ABITS, NORM, AMODE, LOG2B>(
        t, K, p.gamma, p.eps, p.ascale, tc, tid, kWaves, red_d, red_f, [&](int off, auto v) {
            *reinterpret_cast<decltype(v)*>(act_lds + off) = v;
            if (first) *reinterpret_cast<decltype(v)*>(ws_codes + off) = v;
        });
    if (tid == 0) {
        s_scale = s;
        if (first) p.act_scale[0] = s;
    }
    __syncthreads();

    // the products: the token is column 0 of the B operand (lane 16 q of each
    // k quarter); the other 15 columns are zero
    v4i acc[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) acc[r] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int u = u0 + i;
        if (i < per && u < nu) {  // wave-uniform
            ActReg a;
            a.v[0] = make_uint4(0, 0, 0, 0);
            a.v[1] = make_uint4(0, 0, 0, 0);
            if ((lane & 15) == 0) lds_act<ABITS, WBITS>(a, act_lds + u * U::AROW + q * U::ALANE);
#pragma unroll
            for (int r = 0; r < kRows; ++r) acc[r] = unit_mfma<ABITS, WBITS>(wv[i][r], a, acc[r]);
        }
    }

    // the waves' partial tiles meet in LDS; wave r stores row group r
#pragma unroll
    for (int r = 0; r < kRows; ++r) red[wave][r][lane] = acc[r];
    __syncthreads();
    if (wave >= kRows) return;
    v4i sum[1][1] = {{red[0][wave][lane]}};
#pragma unroll
    for (int w = 1; w < kWaves; ++w) sum[0][0] += red[w][wave][lane];
    const int mm[1] = {lane & 15};
    const int nn[1] = {n0 + 16 * wave + q * 4};
    constexpr int shift = AccShift<ABITS, WBITS>::value;
    store_tiles<1, 1>(sum, shift, mm, nn, 1, g.N, &s_scale, g.wscale, g.bias, g.residual, g.ldr, g.y, g.ldy, g.acc,
                      g.head_dim);
}

template <int ABITS, int WBITS, bool NORM, int AMODE, int LOG2B>
hipError_t launch_per(const PrologueArgs& p, const GemmArgs& g, int per, hipStream_t st) {
    const TokenConsts tc{float(1.0 / std::sqrt(double(p.hblock))), 1.0 / double(p.K)};
    const dim3 grid((g.N + 16 * kRows - 1) / (16 * kRows)), block(64 * kWaves);
    // PER: units per wave in registers, rounded up to 4 or 8, with 7 exact for
    // 8-bit codes (the 3584-wide layers: 56 units over 8 waves; one unit
    // repeated there measured 27.3 against 27.0 us)
    if (per <= 4) {
        hipLaunchKernelGGL((decode1_kernel<ABITS, WBITS, NORM, AMODE, LOG2B, 4>), grid, block, 0, st, p, g, tc);
        return hipGetLastError();
    }
    if constexpr (ABITS == 8 && WBITS == 8) {
        if (per == 7) {
            hipLaunchKernelGGL((decode1_kernel<ABITS, WBITS, NORM, AMODE, LOG2B, 7>), grid, block, 0, st, p, g,
                               tc);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((decode1_kernel<ABITS, WBITS, NORM, AMODE, LOG2B, 8>), grid, block, 0, st, p, g, tc);
    return hipGetLastError();
}

template <int ABITS, int WBITS, bool NORM, int AMODE>
hipError_t launch_block(const PrologueArgs& p, const GemmArgs& g, int per, hipStream_t st) {
    switch (p.hblock) {
        case 32: return launch_per<ABITS, WBITS, NORM, AMODE, 5>(p, g, per, st);
        case 64: return launch_per<ABITS, WBITS, NORM, AMODE, 6>(p, g, per, st);
        case 128: return launch_per<ABITS, WBITS, NORM, AMODE, 7>(p, g, per, st);
        default: return hipErrorInvalidValue;  // not eligible (decode1_eligible)
    }
}

template <int ABITS, int WBITS>
hipError_t launch_bits(const PrologueArgs& p, const GemmArgs& g, int per, hipStream_t st) {
    const int amode = p.ascale ? (p.fold_after ? 2 : 1) : 0;
    if (p.gamma) {
        if (amode == 0) return launch_block<ABITS, WBITS, true, 0>(p, g, per, st);
        if (amode == 1) return launch_block<ABITS, WBITS, true, 1>(p, g, per, st);
        return launch_block<ABITS, WBITS, true, 2>(p, g, per, st);
    }
    if (amode == 0) return launch_block<ABITS, WBITS, false, 0>(p, g, per, st);
    if (amode == 1) return launch_block<ABITS, WBITS, false, 1>(p, g, per, st);
    return launch_block<ABITS, WBITS, false, 2>(p, g, per, st);
}

}  // namespace

bool decode1_eligible(const PrologueArgs& p, const GemmArgs& g) {
    if (hooks().decode1_off.load(std::memory_order_relaxed)) return false;
    return g.M == 1 && p.M == 1 && g.abits != 6 && g.K <= kMaxK &&
           (p.hblock == 32 || p.hblock == 64 || p.hblock == 128);
}

hipError_t launch_decode1(const PrologueArgs& p, const GemmArgs& g, hipStream_t stream) {
    if (!decode1_eligible(p, g)) return hipErrorInvalidValue;
    const int unit_k = g.wbits == 8 ? 64 : 128;
    const int nu = g.K / unit_k;
    const int per = (nu + kWaves - 1) / kWaves;  // <= 8 for K <= 4096
    if (g.abits == 8 && g.wbits == 8) return launch_bits<8, 8>(p, g, per, stream);
    if (g.abits == 4 && g.wbits == 4) return launch_bits<4, 4>(p, g, per, stream);
    if (g.abits == 8 && g.wbits == 4) return launch_bits<8, 4>(p, g, per, stream);
    return launch_bits<4, 8>(p, g, per, stream);
}

}  // namespace fq

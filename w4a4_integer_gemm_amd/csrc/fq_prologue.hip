// FoldQuant activation prologue on gfx950 (the vla.cpp page's fused
// "RMSNorm + butterfly + quant" act node; its OpenVINO commit lists the steps:
// RMSNorm with the folded gain, the ascale divide, the block rotation, a
// per-token amax scale, round-half-even and a clamp).
//
// Layout: one workgroup per token.  Lane t owns E = 8 (at most 32 tokens of
// at most 2048 values), 16 (K <= 8192), 32 (K <= 32768) or 64 consecutive
// bf16 values (E/8 16-byte loads), so a token of up to 65536 values is one
// pass of at most 1024 lanes.  The butterfly's
// first log2(E) stages (span 1 .. E/2) run inside a lane's registers; a
// Hadamard block of b > E values spans b/E (at most 16) consecutive lanes,
// whose stages (span E .. b/2) exchange values with DPP lane permutations
// (xor 1, xor 2, and xor 4 and xor 8 composed from two permutations), one
// multiply-add per value that reads the partner through DPP; the upper lane
// of each pair keeps its result negated, and the final 1/sqrt(b) scaling
// removes that sign (exact, so the values are unchanged bit for bit).  Every element goes
// through the same float32 operations in the same order as the definition
// (stage spans 1, 2, 4, ...), so the rotation is bit-reproducible.  The token
// stays in registers between the two reductions (sum of squares, amax): x is
// read from HBM once and the codes written once.
//
// Quantisation divides by the per-token scale s.  The quotient is computed as
// q0 = h * r, rem = fma(-s, q0, h), q = fma(rem, r, q0) with r = 1/s (one IEEE
// divide per token): with r correctly rounded and no underflow in the
// remainder this is the correctly rounded h / s (Markstein's theorem), so it
// equals the IEEE quotient bit for bit.  The fast form is used when
// 2^-100 <= s <= 2^100 (r stays normal and the remainder cannot underflow for
// any |h| whose quotient could round away from zero); other scales divide per
// element.
#include <hip/hip_runtime.h>

#include <cmath>
#include <type_traits>

#include "fq_device.h"
#include "fq_internal.h"
#include "fq_token.h"

namespace fq {
namespace {

constexpr int kMaxThreads = 1024;
// Few tokens of at most 2048 values take 8 values per lane: no two
// workgroups then share a SIMD's issue, and the shorter per-lane chain wins
// while the cross-wave reductions stay within 4 waves (graph-replayed, one
// launch: 16 x 256 2.84 -> 2.59 us, 16 x 2048 3.30 -> 3.19 us; at K = 3584,
// 7 waves, 3.24 -> 3.39 us, so 16 values there).
constexpr int kFewTokens = 32;
constexpr int kFewTokensMaxK = 2048;
constexpr int kMaxWaves = kMaxThreads / 64;

// One workgroup per token; lane t owns values [E t, E t + E) of the token.
// NORM: RMSNorm with the gain (loaded together with x); AMODE: explicit
// smoothing divide 0 none, 1 before the rotation, 2 after it; the Hadamard
// block is 2^LOG2B (compile time, so skipped stages cost no code).
template <int E, int ABITS, bool NORM, int AMODE, int LOG2B>
__global__ __launch_bounds__(kMaxThreads) void prologue_kernel(const uint16_t* __restrict__ x, int K, int64_t ldx,
                                                                const float* __restrict__ gamma, float eps,
                                                                const float* __restrict__ ascale, TokenConsts tc,
                                                                uint8_t* __restrict__ codes,
                                                                float* __restrict__ act_scale) {
    // A lane's codes (E * ABITS / 8 bytes) leave in one store when they are at
    // most 16 bytes, so that a wave's store covers whole lines; those stores
    // are written through at device scope, and the codes reach memory while
    // the kernel runs instead of in the write-back at its end.  Wider shares
    // leave in strided 16-byte pieces, which cost less merged in L2 first
    // (1024 tokens x 18944 8-bit codes: 13.7 us that way, 15.3 us written
    // through; 1024 and 4096 tokens x 3584 gained 0.4 and 1.3 us written
    // through).
    constexpr bool kWriteThrough = E * ABITS / 8 <= 16;
    __shared__ double red_d[kMaxWaves];
    __shared__ float red_f[kMaxWaves];
    const int m = blockIdx.x;
    const int c = threadIdx.x;
    uint8_t* const row = codes + int64_t(m) * (ABITS == 8 ? K : ABITS == 6 ? K / 4 * 3 : K / 2);
    const float s = quantise_token<E, ABITS, NORM, AMODE, LOG2B>(
        x + int64_t(m) * ldx, K, gamma, eps, ascale, tc, c, int(blockDim.x) >> 6, red_d, red_f,
        [&](int off, auto v) {
            if constexpr (kWriteThrough) {
                if constexpr (sizeof(v) == 16)
                    store_dev16(row + off, v);
                else if constexpr (sizeof(v) == 8)
                    store_dev8(row + off, v);
                else
                    store_dev4(row + off, v);
            } else {
                *reinterpret_cast<decltype(v)*>(row + off) = v;
            }
        });
    if (c == 0) act_scale[m] = s;
}

template <int E, int ABITS, bool NORM, int AMODE, int LOG2B>
hipError_t launch_e(dim3 grid, dim3 block, hipStream_t st, const PrologueArgs& a, TokenConsts tc) {
    if constexpr ((1 << LOG2B) > 16 * E || (ABITS == 6 && E < 16)) {
        return hipErrorInvalidValue;  // not chosen by launch_prologue
    } else {
        hipLaunchKernelGGL((prologue_kernel<E, ABITS, NORM, AMODE, LOG2B>), grid, block, 0, st, a.x, a.K, a.ldx,
                           a.gamma, a.eps, a.ascale, tc, a.codes, a.act_scale);
        return hipGetLastError();
    }
}

template <int E, int ABITS, bool NORM, int AMODE>
hipError_t launch_b(int log2b, dim3 grid, dim3 block, hipStream_t st, const PrologueArgs& a, TokenConsts tc) {
    switch (log2b) {
        case 0: return launch_e<E, ABITS, NORM, AMODE, 0>(grid, block, st, a, tc);
        case 1: return launch_e<E, ABITS, NORM, AMODE, 1>(grid, block, st, a, tc);
        case 2: return launch_e<E, ABITS, NORM, AMODE, 2>(grid, block, st, a, tc);
        case 3: return launch_e<E, ABITS, NORM, AMODE, 3>(grid, block, st, a, tc);
        case 4: return launch_e<E, ABITS, NORM, AMODE, 4>(grid, block, st, a, tc);
        case 5: return launch_e<E, ABITS, NORM, AMODE, 5>(grid, block, st, a, tc);
        case 6: return launch_e<E, ABITS, NORM, AMODE, 6>(grid, block, st, a, tc);
        case 7: return launch_e<E, ABITS, NORM, AMODE, 7>(grid, block, st, a, tc);
        case 8: return launch_e<E, ABITS, NORM, AMODE, 8>(grid, block, st, a, tc);
        default: return hipErrorInvalidValue;
    }
}

template <int E, int ABITS>
hipError_t launch_modes(dim3 grid, dim3 block, hipStream_t st, const PrologueArgs& a, TokenConsts tc) {
    int log2b = 0;
    while ((1 << log2b) < a.hblock) ++log2b;
    const int amode = a.ascale ? (a.fold_after ? 2 : 1) : 0;
    if (a.gamma) {
        if (amode == 0) return launch_b<E, ABITS, true, 0>(log2b, grid, block, st, a, tc);
        if (amode == 1) return launch_b<E, ABITS, true, 1>(log2b, grid, block, st, a, tc);
        return launch_b<E, ABITS, true, 2>(log2b, grid, block, st, a, tc);
    }
    if (amode == 0) return launch_b<E, ABITS, false, 0>(log2b, grid, block, st, a, tc);
    if (amode == 1) return launch_b<E, ABITS, false, 1>(log2b, grid, block, st, a, tc);
    return launch_b<E, ABITS, false, 2>(log2b, grid, block, st, a, tc);
}

}  // namespace

// Values per lane: 8 for a few short tokens (above), else 16 up to K = 8192:
// each token is a chain of dependent
// steps, and halving a lane's share shortens it (measured on the qkv prologue,
// K = 3584: 7.0 -> 6.0 us for 1024 tokens, 4.0 -> 3.4 us for one; 8 per lane
// gained nothing more); 32 up to K = 32768 (one pass of at most 1024 lanes),
// 64 beyond.  E2M3 codes take at least 16 (they leave in 12-byte groups).
hipError_t launch_prologue(const PrologueArgs& a, hipStream_t stream) {
    // (a Hadamard block spans at most 16 lanes: 8 values per lane only for b <= 128)
    const int E = a.M <= kFewTokens && a.K <= kFewTokensMaxK && a.hblock <= 128 && a.abits != 6 ? 8
                  : a.K <= 8192                                                         ? 16
                  : a.K > 32768                                                         ? 64
                                                                                        : 32;
    const int nlanes = a.K / E;
    const int T = (nlanes + 63) / 64 * 64;
    if (T > kMaxThreads) return hipErrorInvalidValue;
    const TokenConsts tc{float(1.0 / std::sqrt(double(a.hblock))), 1.0 / double(a.K)};
    dim3 grid(a.M), block(T);
    if (E == 8)
        return a.abits == 8 ? launch_modes<8, 8>(grid, block, stream, a, tc) : launch_modes<8, 4>(grid, block, stream, a, tc);
    if (E == 16)
        return a.abits == 8   ? launch_modes<16, 8>(grid, block, stream, a, tc)
               : a.abits == 6 ? launch_modes<16, 6>(grid, block, stream, a, tc)
                              : launch_modes<16, 4>(grid, block, stream, a, tc);
    if (E == 32)
        return a.abits == 8   ? launch_modes<32, 8>(grid, block, stream, a, tc)
               : a.abits == 6 ? launch_modes<32, 6>(grid, block, stream, a, tc)
                              : launch_modes<32, 4>(grid, block, stream, a, tc);
    return a.abits == 8   ? launch_modes<64, 8>(grid, block, stream, a, tc)
           : a.abits == 6 ? launch_modes<64, 6>(grid, block, stream, a, tc)
                          : launch_modes<64, 4>(grid, block, stream, a, tc);
}

}  // namespace fq

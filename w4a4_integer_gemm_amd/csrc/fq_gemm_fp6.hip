// W4A4 GEMM on gfx950's FP6 matrix instruction, for 4-bit codes stored as
// E2M3 (code width 6; the vla.cpp FoldQuant page's W4A4 integer GEMM, its
// "gemm" node, computed on another unit of the same chip).
//
// Every 4-bit code (an integer in [-7, 7]) is an exact E2M3 number, and
// v_mfma_scale_f32_16x16x128_f8f6f4 with both operands in E2M3 (format 2) and
// unit block scales multiplies them exactly and adds in float32.  A sum of K
// products of at most 49 stays below 2^24 for every K this library takes, so
// every partial sum is an exact integer: the float32 accumulators hold the
// int32 sums of the integer kernel, converted without rounding for the shared
// epilogue.  The instruction runs 16 x 16 x 128 in the time the int8 one runs
// 16 x 16 x 64, and the operands need no unpacking in registers.
//
// Tile BM tokens x BN weight rows, one k stage = 128 codes = 96 bytes of each
// row.  Four load waves copy a stage into an LDS ring slot with
// global_load_lds_dwordx4 (1 KB per wave instruction): a row takes 7 slots of
// 16 bytes, its 6 data chunks and one pad (a repeat of chunk 5), so that rows
// sit 112 bytes apart and the 16 rows of a fragment read from 16 distinct bank
// pairs.  Four MFMA waves split the tile 2 x 2 (wave tile BM/2 x BN/2) and run
// every stage: lane l takes row l % 16 of a fragment and the 24 bytes of k
// quarter l / 16 (32 codes), read as three 8-byte LDS reads.  A wave reads
// stage s + 1 into its second register set while the MFMAs of stage s run.
//
// Ring protocol (barrier B(s) ends MFMA iteration s; B(-1) precedes it):
//   - an MFMA wave reads stage 0 after B(-1) and stage s + 1 during iteration
//     s, and waits for those reads before B(s): after B(s) the slots of
//     stages <= s + 1 are free;
//   - the load waves first fill the slots of stages 0 .. NS-2; at iteration s
//     a load wave refills slot (s - 1) mod NS (stage s - 1's, free since
//     B(s - 1); at s = 0 the slot still empty) with stage s + NS - 1, waits
//     until stage s + 2 has landed, and reaches B(s), which publishes it for
//     iteration s + 1's reads.  NS - 3 stages stay in flight.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "fq_device.h"
#include "fq_internal.h"
#include "fq_ring.h"

namespace fq {
namespace {

constexpr int kThreads = 512;   // 4 load waves + 4 MFMA waves
constexpr int kRowBytes = 96;   // one row's 128 codes in a stage
constexpr int kChunks = 7;      // 16-byte LDS slots per row: 6 data + 1 pad
constexpr int kPitch = 16 * kChunks;
constexpr int kLdsMax = 160 * 1024;

template <int BM_, int BN_>
struct Fp6Cfg {
    static constexpr int BM = BM_, BN = BN_;
    static constexpr int ROWS = BM + BN;
    static constexpr int COPIES = (ROWS * kChunks + 63) / 64;  // 1 KB copies per stage
    static constexpr int STAGE = COPIES * 1024;               // (the last copy's spare lanes land in the pad)
    static constexpr int NHI = (COPIES + 3) / 4;               // copies per load wave (uniform)
    static constexpr int NS = kLdsMax / STAGE > 8 ? 8 : kLdsMax / STAGE;
    static constexpr int LDS = NS * STAGE;
    static constexpr int TF = BM / 32;  // token fragments per MFMA wave
    static constexpr int TW = BN / 32;  // weight fragments per MFMA wave
    static_assert(BM % 64 == 0 && BN % 32 == 0, "whole fragments per wave; no copy spans both operands");
    static_assert(NS >= 4, "the ring needs four stages");
    static_assert((NS - 2) * NHI < 64, "vmcnt range");
};

// One lane's 32 codes of a fragment: 24 bytes (the upper two dwords of the
// operand are not read by the FP6 form).
typedef int v2i __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) const v2i lds_v2i;
typedef v4i v4i_a8 __attribute__((aligned(8)));
typedef __attribute__((address_space(3))) const v4i_a8 lds_v4i_a8;
// 16 + 8 bytes at an 8-byte aligned LDS address (gfx950 reads 16 bytes at
// 8-byte alignment in one instruction)
__device__ __forceinline__ v8i read_frag(uint32_t addr) {
    const v4i a = *reinterpret_cast<lds_v4i_a8*>(uintptr_t(addr));
    const v2i b = *reinterpret_cast<lds_v2i*>(uintptr_t(addr + 16));
    const v4i bb = __builtin_shufflevector(b, b, 0, 1, -1, -1);
    return __builtin_shufflevector(a, bb, 0, 1, 2, 3, 4, 5, -1, -1);
}

__device__ __forceinline__ v4f mfma_e2m3(const v8i& w, const v8i& a, const v4f& c) {
    // formats 2/2: E2M3 x E2M3; scale exponents 127 = 2^0 for both operands
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, a, c, 2, 2, 0, 127, 0, 127);
}

template <class CF>
__global__ __launch_bounds__(kThreads) void gemm_e2m3_kernel(GemmArgs g, int tiles_m, int tiles_n) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[CF::LDS];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // XCD-aware tile order, as in the int8 kernel: dispatch b runs on XCD b % 8,
    // which takes the tile range [x per, (x + 1) per), m fastest
    const int ntiles = tiles_m * tiles_n;
    int t = blockIdx.x;
    if (ntiles % 8 == 0) {
        const int per = ntiles / 8;
        t = (blockIdx.x % 8) * per + blockIdx.x / 8;
    }
    const int tm = t % tiles_m, tn = t / tiles_m;
    const int m0 = tm * CF::BM, n0 = tn * CF::BN;
    const int64_t ld = int64_t(g.K) / 4 * 3;  // bytes per row of either operand
    const int nk = g.K / 128;

    if (wave >= 4) {
        // ---------------------------------------------------------- load waves
        // copy q = p + 4 i of a stage: lane l fills LDS slot sigma = 64 q + l of
        // the stage = row sigma / 7, chunk sigma % 7 (chunk 6: the pad, which
        // repeats chunk 5; slots past the rows repeat the first weight row's
        // chunk 0).  A wave with fewer copies repeats its last one (same bytes to
        // the same place).
        const int p = wave - 4;
        uint32_t voff[CF::NHI];
        bool is_act[CF::NHI];
        int ldsoff[CF::NHI];
#pragma unroll
        for (int i = 0; i < CF::NHI; ++i) {
            int q = p + 4 * i;
            q = q < CF::COPIES ? q : CF::COPIES - 1;
            ldsoff[i] = q * 1024;
            const int sigma = 64 * q + lane;
            int rho = sigma / kChunks, c = sigma % kChunks;
            // a copy is all token rows or all weight rows (BM * 7 is a multiple of
            // 64), so the operand is wave uniform
            is_act[i] = 64 * q < CF::BM * kChunks;
            if (rho >= CF::ROWS) rho = CF::BM, c = 0;
            if (c == kChunks - 1) c = kChunks - 2;
            int row, base_row;
            if (is_act[i]) {
                row = m0 + rho;
                row = row < g.M ? row : g.M - 1;
                base_row = m0;
            } else {
                row = n0 + rho - CF::BM;
                row = row < g.N ? row : g.N - 1;
                base_row = n0;
            }
            voff[i] = uint32_t(int64_t(row - base_row) * ld + 16 * c);
        }
        const uint8_t* const abase = g.act + int64_t(m0) * ld;
        const uint8_t* const wbase = g.w + int64_t(n0) * ld;
        const uint32_t lds0 = lds_address(lds);
        auto load_stage = [&](int j) {
            const int src = j < nk ? j : nk - 1;  // stages past K repeat the last one (never read)
            const uint32_t dst = lds0 + uint32_t((j % CF::NS) * CF::STAGE);
#pragma unroll
            for (int i = 0; i < CF::NHI; ++i)
                copy16_to_lds((is_act[i] ? abase : wbase) + int64_t(src) * kRowBytes, voff[i], dst + ldsoff[i]);
        };
        for (int j = 0; j < CF::NS - 1; ++j) load_stage(j);
        int issued = CF::NS - 1;
        wait_vmcnt<(CF::NS - 3) * CF::NHI>();  // stages 0 and 1 landed
        barrier_nofence();                      // B(-1)
        for (int s = 0; s < nk; ++s) {
            if (s + CF::NS - 1 < nk) {
                load_stage(s + CF::NS - 1);
                ++issued;
            }
            const int younger = issued - (s + 3);  // copies issued after stage s + 2
            wait_stages_in_flight<CF::NHI>(younger > 0 ? younger : 0);
            barrier_nofence();  // B(s)
        }
        return;
    }

    // ------------------------------------------------------------ MFMA waves
    constexpr int TF = CF::TF, TW = CF::TW;
    const int wm = wave & 1, wn = wave >> 1;
    const int q = lane >> 4;
    const int offa = (wm * (CF::BM / 2) + (lane & 15)) * kPitch + 24 * q;
    const int offw = (CF::BM + wn * (CF::BN / 2) + (lane & 15)) * kPitch + 24 * q;
    v4f acc[TW][TF];
#pragma unroll
    for (int n = 0; n < TW; ++n)
#pragma unroll
        for (int f = 0; f < TF; ++f) acc[n][f] = v4f{0.f, 0.f, 0.f, 0.f};
    v8i fa[2][TF], fw[2][TW];
    const uint32_t lds0 = lds_address(lds);
    // each fragment's offset goes through an empty asm once, so that the
    // compiler cannot pair one fragment's reads with another's into one
    // ds_read2 (which then cost register moves and waits in the loop)
    uint32_t oa[TF], ow[TW];
#pragma unroll
    for (int f = 0; f < TF; ++f) {
        oa[f] = uint32_t(offa + f * 16 * kPitch);
        asm volatile("" : "+v"(oa[f]));
    }
#pragma unroll
    for (int n = 0; n < TW; ++n) {
        ow[n] = uint32_t(offw + n * 16 * kPitch);
        asm volatile("" : "+v"(ow[n]));
    }
    auto read_stage = [&](int s, int b) {
        const uint32_t base = lds0 + uint32_t((s % CF::NS) * CF::STAGE);
#pragma unroll
        for (int f = 0; f < TF; ++f) fa[b][f] = read_frag(base + oa[f]);
#pragma unroll
        for (int n = 0; n < TW; ++n) fw[b][n] = read_frag(base + ow[n]);
    };
    auto iteration = [&](int s, auto b_tag) {
        constexpr int B = decltype(b_tag)::value;
        read_stage(s + 1, B ^ 1);  // (past K: a slot's stale bytes, never used)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int n = 0; n < TW; ++n)
#pragma unroll
            for (int f = 0; f < TF; ++f) acc[n][f] = mfma_e2m3(fw[B][n], fa[B][f], acc[n][f]);
        // (the MFMAs stay ahead of the wait: left alone the compiler moved them
        // behind the barrier, where the read latency was no longer hidden)
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): stage s + 1 is in registers
        barrier_nofence();                   // B(s)
    };
    barrier_nofence();  // B(-1): stages 0 and 1 published
    read_stage(0, 0);
    // stage 0 in registers before the loop, so that no wait carried in from
    // here makes the compiler wait for every read at the top of each iteration
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_sched_barrier(0);
    int s = 0;
    for (; s + 1 < nk; s += 2) {  // stages in pairs, so that the register set of each is fixed
        iteration(s, std::integral_constant<int, 0>{});
        iteration(s + 1, std::integral_constant<int, 1>{});
    }
    if (s < nk) iteration(s, std::integral_constant<int, 0>{});

    // epilogue straight from the registers: lane holds D[n = 16 fragment + 4 q + i][m = lane % 16]
    v4i sum[TW][TF];
#pragma unroll
    for (int n = 0; n < TW; ++n)
#pragma unroll
        for (int f = 0; f < TF; ++f)
#pragma unroll
            for (int i = 0; i < 4; ++i) sum[n][f][i] = int(acc[n][f][i]);  // exact: integers below 2^24
    int mm[TF], nn[TW];
#pragma unroll
    for (int f = 0; f < TF; ++f) mm[f] = m0 + wm * (CF::BM / 2) + 16 * f + (lane & 15);
#pragma unroll
    for (int n = 0; n < TW; ++n) nn[n] = n0 + wn * (CF::BN / 2) + 16 * n + 4 * q;
    store_tiles<TW, TF>(sum, 0, mm, nn, g.M, g.N, g.act_scale, g.wscale, g.bias, g.residual, g.ldr, g.y, g.ldy,
                        g.acc, g.head_dim);
}

template <class CF>
hipError_t launch_cfg(const GemmArgs& g, hipStream_t st) {
    const int tiles_m = (g.M + CF::BM - 1) / CF::BM;
    const int tiles_n = (g.N + CF::BN - 1) / CF::BN;
    hipLaunchKernelGGL((gemm_e2m3_kernel<CF>), dim3(tiles_m * tiles_n), dim3(kThreads), 0, st, g, tiles_m, tiles_n);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_e2m3(const GemmArgs& g, hipStream_t stream) {
    if (g.abits != 6 || g.wbits != 6 || g.K % 128) return hipErrorInvalidValue;
    return launch_cfg<Fp6Cfg<128, 128>>(g, stream);
}

}  // namespace fq

// FoldQuant integer GEMM with the fused dequant/residual epilogue on gfx950.
//
// acc[m][n] = sum_k qa[m][k] * qw[n][k] on v_mfma_i32_16x16x64_i8 (the vla.cpp
// FoldQuant page's "gemm" node: integer GEMM against per-row scaled INT8/INT4
// weight codes with per-shape tiling and the residual add in the epilogue).
// Integer sums are exact in any order, so tile shape and k order are free.
//
// Structure (one 256-thread workgroup = 4 waves per BM x BN output tile):
//   - k advances in stages of 128.  A stage of the two operand tiles is copied
//     global -> LDS with global_load_lds_dwordx4 (no VGPR staging); NS stages
//     live in an LDS ring so NS-1 stages of loads are in flight while the MFMAs
//     consume the oldest one.  One s_barrier per stage; the waits count each
//     wave's own outstanding loads (vmcnt), so no wave waits for loads that a
//     later stage issued.
//   - Each 1 KB chunk of a stage is one wave-wide load: lane l fetches 16 bytes
//     of row (l % 16).  The chunk is therefore already in MFMA operand order
//     (lane l reads bytes 16*l .. 16*l+15), so operand reads are conflict-free
//     ds_read_b128.
//   - The MFMA's A operand is a 16-row weight fragment and its B operand a
//     16-token activation fragment, so each lane ends with four consecutive
//     output features of one token: one 8-byte bf16 store in the epilogue.
//   - Rows past M or N are clamped to the last row when loading (their results
//     are never stored), so no load is ever masked or out of bounds.
//   - The workgroup -> tile map is XCD aware: consecutive dispatch ids land on
//     different XCDs, so tiles are renumbered to give each XCD a compact block
//     of the output that shares operand rows in its own L2.
//
// k order inside a 128-k stage (lane l, MFMA sub-step j in {0, 1}):
//   both operands 8-bit: k = 64 j + 16 (l / 16) + [0, 16)
//   otherwise:           k = 32 (l / 16) + 16 j + [0, 16)  (4-bit codes: the
//     16 packed bytes of a lane hold both sub-steps; an 8-bit partner loads
//     the same k and permutes its bytes into the nibble order of fq_device.h)
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "fq_device.h"
#include "fq_internal.h"

namespace fq {
namespace {

constexpr int kThreads = 256;

// 16-byte-per-lane global -> LDS copy (global_load_lds_dwordx4): lane l's 16
// bytes land at lds_dst + 16 l; lds_dst must be wave uniform (it goes to M0).
// Written as inline asm so that the compiler does not wait for every
// outstanding copy before each LDS read; completion is tracked explicitly
// with wait_vmcnt and the stage barrier.  M0 is restored afterwards.  The
// instruction has no VGPR result, only the address operand, which the
// hardware consumes at issue.
__device__ __forceinline__ void copy16_to_lds(const uint8_t* gsrc, uint8_t* lds_dst) {
    typedef __attribute__((address_space(3))) uint8_t lds_byte;
    uint32_t a = uint32_t(reinterpret_cast<uintptr_t>((lds_byte*)lds_dst));
    a = __builtin_amdgcn_readfirstlane(a);
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(gsrc), "s"(a)
        : "memory");
}

// s_waitcnt vmcnt(n) leaving the other counters untouched (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | 0x70 | 0xF00 | ((N >> 4) << 14));
}

// Workgroup barrier without a memory fence (the LDS-DMA waits are explicit);
// the empty asm statements keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void barrier_nofence() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int ABITS, int WBITS, int BM_, int BN_, int WGM_, int WGN_, int NS_>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_, NS = NS_;
    static constexpr bool MIXED = ABITS != WBITS;
    static constexpr int KS = (ABITS == 4 || WBITS == 4) ? 256 : 128;  // k per stage
    static constexpr int NSUB = KS / 64;                                // MFMA steps per stage
    static constexpr int RA = KS * ABITS / 8, RW = KS * WBITS / 8;      // bytes per row per stage
    static constexpr int FA = BM / 16, FW = BN / 16;                    // 16-row fragments
    static constexpr int IA = 16 * RA / 1024, IW = 16 * RW / 1024;      // 1 KB loads per fragment
    static constexpr int CA = FA * IA, CW = FW * IW, C = CA + CW;       // 1 KB loads per stage
    static constexpr int STAGE = C * 1024;
    static constexpr int LDS = NS * STAGE;
    static constexpr int WTM = BM / WGM, WTN = BN / WGN;
    static constexpr int TM = WTM / 16, TN = WTN / 16;
    static constexpr int NLO = C / 4, NHI = (C + 3) / 4;
    static_assert(WGM * WGN == 4, "four waves");
    static_assert(BM % (16 * WGM) == 0 && BN % (16 * WGN) == 0, "wave tiles of whole fragments");
    static_assert(LDS <= 163840, "LDS ring exceeds 160 KiB");
    static_assert(NS >= 3, "the ring needs a slot being filled, one ready and one being read");
    static_assert((NS - 2) * NHI < 64, "vmcnt range");
};

// LDS layout of one 16-row fragment of an operand whose rows hold R bytes per
// stage: 16-byte slot (rho, kc) sits at KC*rho + (kc ^ g(rho)), KC = R/16.  A
// 1 KB load instruction covers whole rows (8 rows of 128 B or 4 of 256 B), so
// every row segment it fetches is whole 128-byte lines; the xor keeps the 16
// lanes of an MFMA operand read (16 rows, one kc) on 16 distinct slot columns.
template <int R>
__device__ __forceinline__ int slot_of(int rho, int kc) {
    constexpr int KC = R / 16;
    const int gx = KC == 8 ? ((rho >> 1) & 7) : (rho & 15);
    return KC * rho + (kc ^ gx);
}

// LDS byte offset (inside a fragment) of lane `lane`'s operand for MFMA step j:
// step j covers k = 64 j + 16 (lane / 16) + [0, 16) of the stage
template <int BITS, int R>
__device__ __forceinline__ int operand_offset(int lane, int j) {
    const int rho = lane & 15;
    if (BITS == 8) return 16 * slot_of<R>(rho, 4 * j + (lane >> 4));             // 16 k = 16 bytes
    return 16 * slot_of<R>(rho, 2 * j + (lane >> 5)) + 8 * ((lane >> 4) & 1);  // 16 k = 8 bytes
}

template <int BITS, int PARTNER>
__device__ __forceinline__ v4i operand_from_lds(const uint8_t* p) {
    if (BITS == 4) return frag_from_nibbles(*reinterpret_cast<const uint2*>(p));
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    return PARTNER == 4 ? frag_from_bytes_nibble_order(v) : frag_from_bytes(v);
}

// global source of load instruction q (of a fragment) for `lane`: row rho of the
// fragment and 16-byte column kc, inverse of slot_of
template <int R>
__device__ __forceinline__ void slot_source(int q, int lane, int& rho, int& kc) {
    constexpr int KC = R / 16;
    const int sigma = 64 * q + lane;
    rho = sigma / KC;
    kc = (sigma % KC) ^ (KC == 8 ? ((rho >> 1) & 7) : (rho & 15));
}

template <int ABITS, int WBITS, class CF>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs g, int tiles_m, int tiles_n) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[CF::LDS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // XCD-aware tile order: dispatch id b runs on XCD b % 8; give XCD x the tile
    // range [x * per, (x + 1) * per) and walk it m-fastest.
    const int ntiles = tiles_m * tiles_n;
    int t = blockIdx.x;
    if (ntiles % 8 == 0) {
        const int per = ntiles / 8;
        t = (blockIdx.x % 8) * per + blockIdx.x / 8;
    }
    const int tm = t % tiles_m, tn = t / tiles_m;
    const int m0 = tm * CF::BM, n0 = tn * CF::BN;
    const int64_t lda = ABITS == 8 ? g.K : g.K / 2;
    const int64_t ldw = WBITS == 8 ? g.K : g.K / 2;
    // K is a multiple of 128; with a 4-bit operand a stage is 256 deep and the
    // last stage may be half (128) deep
    const int nk = (g.K + CF::KS - 1) / CF::KS;
    const bool half_last = (g.K % CF::KS) != 0;

    // This wave's load instructions: c = wave + 4 i.  Waves with one fewer
    // instruction repeat their last one (same source, same LDS bytes), so every
    // wave issues NHI loads per stage and the waits below are uniform.  A lane
    // whose column would run past the end of a row (only in a half-deep last
    // stage) re-reads bytes of its row's first 64; that LDS slot is never used.
    const uint8_t* gp[CF::NHI];
    int col[CF::NHI], gstep[CF::NHI], rowlen[CF::NHI], ldsoff[CF::NHI];
#pragma unroll
    for (int i = 0; i < CF::NHI; ++i) {
        int c = wave + 4 * i;
        if (c >= CF::C) c -= 4;
        ldsoff[i] = c * 1024;
        int rho, kc;
        if (c < CF::CA) {
            slot_source<CF::RA>(c % CF::IA, lane, rho, kc);
            int row = m0 + (c / CF::IA) * 16 + rho;
            row = row < g.M ? row : g.M - 1;
            gp[i] = g.act + int64_t(row) * lda;
            gstep[i] = CF::RA;
            rowlen[i] = int(lda);
        } else {
            const int cw = c - CF::CA;
            slot_source<CF::RW>(cw % CF::IW, lane, rho, kc);
            int row = n0 + (cw / CF::IW) * 16 + rho;
            row = row < g.N ? row : g.N - 1;
            gp[i] = g.w + int64_t(row) * ldw;
            gstep[i] = CF::RW;
            rowlen[i] = int(ldw);
        }
        col[i] = 16 * kc;
    }
    auto dma = [&](int stage_idx, int slot, int i) {
        int off = stage_idx * gstep[i] + col[i];
        off = off < rowlen[i] ? off : (col[i] & 63);  // rows are at least 64 bytes
        copy16_to_lds(gp[i] + off, lds + slot * CF::STAGE + ldsoff[i]);
    };

    const int wm = wave % CF::WGM;  // wave's token block
    const int wn = wave / CF::WGM;  // wave's weight-row block
    int offa[CF::NSUB], offw[CF::NSUB];
#pragma unroll
    for (int j = 0; j < CF::NSUB; ++j) {
        offa[j] = operand_offset<ABITS, CF::RA>(lane, j) + wm * CF::TM * 16 * CF::RA;
        offw[j] = operand_offset<WBITS, CF::RW>(lane, j) + CF::CA * 1024 + wn * CF::TN * 16 * CF::RW;
    }

    v4i acc[CF::TN][CF::TM];
#pragma unroll
    for (int i = 0; i < CF::TN; ++i)
#pragma unroll
        for (int j = 0; j < CF::TM; ++j) acc[i][j] = v4i{0, 0, 0, 0};

    v4i fa[2][CF::TM], fw[2][CF::TN];
    auto read_frags = [&](int s, int j, int buf) {
        const uint8_t* base = lds + (s % CF::NS) * CF::STAGE;
#pragma unroll
        for (int i = 0; i < CF::TM; ++i)
            fa[buf][i] = operand_from_lds<ABITS, WBITS>(base + offa[j] + i * 16 * CF::RA);
#pragma unroll
        for (int i = 0; i < CF::TN; ++i)
            fw[buf][i] = operand_from_lds<WBITS, ABITS>(base + offw[j] + i * 16 * CF::RW);
    };

    // prologue: stages 0 .. NS-2 (clamped to the last stage when K is short)
    for (int s = 0; s < CF::NS - 1; ++s)
#pragma unroll
        for (int i = 0; i < CF::NHI; ++i) dma(s < nk ? s : nk - 1, s, i);
    wait_vmcnt<(CF::NS - 2) * CF::NHI>();
    barrier_nofence();
    read_frags(0, 0, 0);

    // this wave's loads of stage s + NS - 1 are spread over the MFMAs that follow
    // the operand reads in steps 0 .. NSUB-2 (TM * (TN - 1) per step); whatever
    // does not fit goes out at the start of the last step
    constexpr int kSlotsPerStep = CF::TM * (CF::TN - 1);
    constexpr int kDmaSlots = kSlotsPerStep * (CF::NSUB - 1);
    constexpr int kDmaEvery = kDmaSlots / CF::NHI > 0 ? kDmaSlots / CF::NHI : 1;
    constexpr int kDmaInLoop = kDmaSlots / kDmaEvery < CF::NHI ? kDmaSlots / kDmaEvery : CF::NHI;

    // One k stage.  In each MFMA step the first TM MFMAs run on operands that
    // were read one step earlier; then the next step's operands are read from
    // LDS (their latency hides behind the remaining MFMAs).  Before the last
    // step the next stage is waited for and published with the barrier.  A
    // full stage has no data-dependent branches: past the end of K the refill
    // loads re-read the last stage into the slot that was just freed (never
    // read again), and the last stage reads operands once more without using
    // them.  A half-deep last stage (FULL = false) runs its first NSUB/2 steps
    // and neither loads nor waits.
    auto stage = [&](int s, auto full_tag) {
        constexpr bool kFull = decltype(full_tag)::value;
        constexpr int kSteps = kFull ? CF::NSUB : CF::NSUB / 2;
        const int refill = s + CF::NS - 1 < nk ? s + CF::NS - 1 : nk - 1;
        const int refill_slot = (s + CF::NS - 1) % CF::NS;
        const int next = s + 1 < nk ? s + 1 : nk - 1;
#pragma unroll
        for (int j = 0; j < kSteps; ++j) {
            const int cur = j & 1;
#pragma unroll
            for (int ii = 0; ii < CF::TM; ++ii) acc[0][ii] = mfma16x16x64(fw[cur][0], fa[cur][ii], acc[0][ii]);
            __builtin_amdgcn_sched_barrier(0);
            if (j + 1 < kSteps) {
                read_frags(s, j + 1, cur ^ 1);
            } else if (kFull) {
#pragma unroll
                for (int i = kDmaInLoop; i < CF::NHI; ++i) dma(refill, refill_slot, i);
                // stage s+1 must have landed for every wave, and every wave must be
                // done reading stage s-1's slot before anyone refills it
                wait_vmcnt<(CF::NS - 2) * CF::NHI>();
                __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
                barrier_nofence();
                read_frags(next, 0, cur ^ 1);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 1; i < CF::TN; ++i)
#pragma unroll
                for (int ii = 0; ii < CF::TM; ++ii) {
                    acc[i][ii] = mfma16x16x64(fw[cur][i], fa[cur][ii], acc[i][ii]);
                    if (kFull && j + 1 < CF::NSUB) {
                        const int slot = j * kSlotsPerStep + (i - 1) * CF::TM + ii;
                        if (slot % kDmaEvery == 0 && slot / kDmaEvery < kDmaInLoop) {
                            __builtin_amdgcn_sched_barrier(0);
                            dma(refill, refill_slot, slot / kDmaEvery);
                            __builtin_amdgcn_sched_barrier(0);
                        }
                    }
                }
        }
    };

    const int nfull = nk - (half_last ? 1 : 0);
    for (int s = 0; s < nfull; ++s) stage(s, std::true_type{});
    if (half_last) stage(nk - 1, std::false_type{});
    wait_vmcnt<0>();  // no load may still be writing LDS when the workgroup retires

    // epilogue: lane holds D[n][m] for n = nb + 4 (lane / 16) + r, m = mb + lane % 16
    constexpr int shift = AccShift<ABITS, WBITS>::value;
#pragma unroll
    for (int ii = 0; ii < CF::TM; ++ii) {
        const int m = m0 + (wm * CF::TM + ii) * 16 + (lane & 15);
        if (m >= g.M) continue;
        const float sam = g.act_scale[m];
#pragma unroll
        for (int i = 0; i < CF::TN; ++i) {
            const int n = n0 + (wn * CF::TN + i) * 16 + (lane >> 4) * 4;
            if (n >= g.N) continue;
            store_out4(acc[i][ii], shift, m, n, sam, g.wscale, g.bias, g.residual, g.ldr, g.y, g.ldy, g.acc, g.N);
        }
    }
}

template <int ABITS, int WBITS, class CF>
hipError_t launch_cfg(const GemmArgs& g, hipStream_t st) {
    const int tiles_m = (g.M + CF::BM - 1) / CF::BM;
    const int tiles_n = (g.N + CF::BN - 1) / CF::BN;
    hipLaunchKernelGGL((gemm_kernel<ABITS, WBITS, CF>), dim3(tiles_m * tiles_n), dim3(kThreads), 0, st, g, tiles_m,
                       tiles_n);
    return hipGetLastError();
}

// Tile shapes (tokens x weight rows, wave grid, pipeline depth).
enum TileId { T128x128 = 0, T128x144, T128x112, T256x128, T128x256, T64x128, kNumTiles };

const char* const kTileNames[kNumTiles] = {"128x128", "128x144", "128x112", "256x128", "128x256", "64x128"};

// Pipeline depth: as many stages as fit in 160 KiB of LDS, at most 5.
template <int ABITS, int WBITS, int BM, int BN>
constexpr int ring_depth() {
    constexpr int ks = (ABITS == 4 || WBITS == 4) ? 256 : 128;
    constexpr int stage = (BM * ks * ABITS / 8) + (BN * ks * WBITS / 8);
    constexpr int n = 163840 / stage;
    return n > 5 ? 5 : n;
}

template <int ABITS, int WBITS, int BM, int BN, int WGM, int WGN>
hipError_t launch_shape(const GemmArgs& g, hipStream_t st) {
    constexpr int ns = ring_depth<ABITS, WBITS, BM, BN>();
    if constexpr (ns >= 3) {
        return launch_cfg<ABITS, WBITS, Cfg<ABITS, WBITS, BM, BN, WGM, WGN, ns>>(g, st);
    } else {
        // this operand mix does not fit three stages of this tile: use 128 x 128
        return launch_cfg<ABITS, WBITS, Cfg<ABITS, WBITS, 128, 128, 2, 2, ring_depth<ABITS, WBITS, 128, 128>()>>(g, st);
    }
}

template <int ABITS, int WBITS>
hipError_t launch_tile(int tile, const GemmArgs& g, hipStream_t st) {
    switch (tile) {
        case T128x144:
            return launch_shape<ABITS, WBITS, 128, 144, 4, 1>(g, st);
        case T128x112:
            return launch_shape<ABITS, WBITS, 128, 112, 4, 1>(g, st);
        case T256x128:
            return launch_shape<ABITS, WBITS, 256, 128, 2, 2>(g, st);
        case T128x256:
            return launch_shape<ABITS, WBITS, 128, 256, 2, 2>(g, st);
        case T64x128:
            return launch_shape<ABITS, WBITS, 64, 128, 1, 4>(g, st);
        case T128x128:
        default:
            return launch_shape<ABITS, WBITS, 128, 128, 2, 2>(g, st);
    }
}

// Pick the tile that minimises (waves of 256 workgroups) x (tile area): the
// shapes of interest fill the 256 CUs in one wave with 128 x 144 (QKV, N = 4608)
// or 128 x 112 (down projection, N = 3584).
int choose_tile(int M, int N) {
    const int cand[] = {T128x128, T128x144, T128x112, T256x128, T128x256, T64x128};
    const int bm[] = {128, 128, 128, 256, 128, 64};
    const int bn[] = {128, 144, 112, 128, 256, 128};
    // relative per-tile throughput (bigger tiles reuse operands better)
    const double eff[] = {1.0, 1.03, 0.95, 1.15, 1.15, 0.8};
    int best = T128x128;
    double best_cost = 1e300;
    for (int c : cand) {
        const long tiles = long((M + bm[c] - 1) / bm[c]) * long((N + bn[c] - 1) / bn[c]);
        const long waves = (tiles + 255) / 256;
        const double cost = double(waves) * bm[c] * bn[c] / eff[c];
        if (cost < best_cost * 0.999) {
            best_cost = cost;
            best = c;
        }
    }
    return best;
}

// Test hook: FQ_GEMM_TILE=<name> forces one tile shape (read at every launch).
int tile_override() {
    const char* e = std::getenv("FQ_GEMM_TILE");
    if (!e) return -1;
    for (int i = 0; i < kNumTiles; ++i)
        if (std::strcmp(e, kTileNames[i]) == 0) return i;
    return -1;
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& g, hipStream_t stream) {
    int tile = tile_override();
    if (tile < 0) tile = choose_tile(g.M, g.N);
    if (g.abits == 8 && g.wbits == 8) return launch_tile<8, 8>(tile, g, stream);
    if (g.abits == 4 && g.wbits == 4) return launch_tile<4, 4>(tile, g, stream);
    if (g.abits == 8 && g.wbits == 4) return launch_tile<8, 4>(tile, g, stream);
    return launch_tile<4, 8>(tile, g, stream);
}

}  // namespace fq

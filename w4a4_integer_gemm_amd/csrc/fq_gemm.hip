// FoldQuant integer GEMM with the fused dequant/residual epilogue on gfx950.
//
// acc[m][n] = sum_k qa[m][k] * qw[n][k] on v_mfma_i32_32x32x32_i8 (the vla.cpp
// FoldQuant page's "gemm" node: integer GEMM against per-row scaled INT8/INT4
// weight codes with per-shape tiling and the residual add in the epilogue).
// Integer sums are exact in any order, so tile shape and k order are free.
//
// Structure (one 512-thread workgroup = 4 MFMA waves + 4 load waves per
// BM x BNS output tile):
//   - MFMA: v_mfma_i32_32x32x32_i8 with the weight fragment (32 rows n) as the
//     A operand and the token fragment (32 tokens m) as B; lane l holds token
//     l % 32 of the result and rows n = 8 g + 4 (l / 32) + i in register 4 g + i.
//     By default v_mfma_i32_16x16x64_i8 is used instead (the MF16 form: 16-row
//     fragments, so no padded rows for a 144-row tile, and a higher sustained
//     rate under the power limit); lane l then holds token l % 16 and rows
//     n = 4 (l / 16) + i.
//   - k advances in stages of 128 (256 with a 4-bit operand).  A stage of the
//     two operand tiles is copied global -> LDS with global_load_lds_dwordx4 (no
//     VGPR staging); NS stages live in an LDS ring, so NS-1 stages of loads are
//     in flight while the MFMAs consume the oldest one.  One s_barrier per
//     stage; the waits count each wave's own outstanding loads (vmcnt).
//   - Waves 0/1 take tokens 0 .. BM/2-1 / BM/2 .. BM-1 and waves 0,1 / 2,3 take
//     alternate 32-deep k steps of every stage (split k inside the workgroup),
//     so each wave reads half the weight fragments a token-only split would.
//     At the end the two k halves of a token block add up through LDS.  On
//     64-token tiles with a 4-bit operand waves 0/1 take the two halves of
//     the rows instead, so that every unpacked fragment feeds two MFMAs.
//   - A tile computes BNC rows (BNS rounded up to 32); rows past BNS belong to
//     the next tile and are not stored.
//   - Rows past M or N are clamped to the last row when loading (their results
//     are never stored), so no load is ever masked or out of bounds.
//   - The workgroup -> tile map is XCD aware: consecutive dispatch ids land on
//     different XCDs, so tiles are renumbered to give each XCD a compact block
//     of the output that shares operand rows in its own L2.
//
// k order inside a stage (lane l, MFMA k step j): k = 32 j + 16 (l / 32) + [0, 16)
// with 8-bit codes; with a 4-bit operand the steps go in pairs, step 2 p + e
// taking k = 64 p + 32 (l / 32) + 16 e + [0, 16) (pair_offset below).  A 4-bit
// operand's 16 codes are 8 bytes, unpacked to bytes in registers; an 8-bit
// partner permutes its bytes into the nibble order of fq_device.h.
#include <hip/hip_runtime.h>

#include <cstring>
#include <type_traits>

#include "fq_device.h"
#include "fq_internal.h"
#include "fq_ring.h"

namespace fq {
namespace {

constexpr int kThreads = 512;  // 4 MFMA waves + 4 load waves

template <int ABITS, int WBITS, int BM_, int BNS_, int BNC_, int NS_, int KS8 = 128, bool MF16_ = false,
          bool TWO_ = false>
struct Cfg {
    // TWO: two workgroups share a CU (at most 80 KiB of LDS and 128 VGPRs
    // each), so that one's fill and epilogue overlap the other's k loop
    static constexpr bool TWO = TWO_;
    // BM tokens x BNS stored weight rows per tile; BNC >= BNS rows are computed
    // (a multiple of 32: the MFMA's row count); rows past BNS belong to the next
    // tile and are discarded.
    static constexpr int BM = BM_, BNS = BNS_, BNC = BNC_, NS = NS_;
    static constexpr int KS = (ABITS == 4 || WBITS == 4) ? 256 : KS8;  // k per stage
    static constexpr int NK32 = KS / 32;                                // MFMA k steps per stage
    static constexpr int NSTEP = NK32 / 2;                              // per wave (k split over pairs)
    static constexpr int RA = KS * ABITS / 8, RW = KS * WBITS / 8;      // bytes per row per stage
    static constexpr int CA = BM * RA / 1024, CW = BNC * RW / 1024;     // 1 KB loads per stage
    static constexpr int C = CA + CW;
    static constexpr int STAGE = C * 1024;
    static constexpr int LDS = NS * STAGE;
    // 32x32x32 form: the two wave pairs split the tokens (TMF fragments of 32
    // per wave, all BNC rows); with a 4-bit operand on a 64-token tile they
    // split the rows instead (RSPLIT: all tokens, BNC / 2 rows per wave), so
    // that each unpacked weight fragment feeds two MFMAs
    static constexpr bool RSPLIT = !MF16_ && KS == 256 && BM_ == 64 && BNC_ % 64 == 0;
    static constexpr int TMF = RSPLIT ? BM / 32 : BM / 64;  // 32-token fragments per wave
    static constexpr int TN = RSPLIT ? BNC / 64 : BNC / 32;  // 32-row weight fragments per wave
    static constexpr int TN0 = (TN + 1) / 2;  // output fragments stored by the k-half 0 wave
    static constexpr int NLO = C / 4, NHI = (C + 3) / 4;
    // MF16: v_mfma_i32_16x16x64_i8 instead of 32x32x32: rows in fragments of
    // 16, NSW16 64-deep k steps per wave per stage, TF16 token and TW16 row
    // fragments per wave, weight fragments read D16 - 1 ahead through a ring
    // of D16 registers (D16 divides TW16, so every step starts at ring slot 0;
    // at least 3, or 5 when a fragment feeds only two MFMAs)
    static constexpr bool MF16 = MF16_;
    static constexpr int TF16 = BM / 32;
    static constexpr int TW16 = BNC / 16;
    static constexpr int ring16() {
        const int need = TF16 >= 4 ? 3 : 5;
        for (int d = need; d < TW16; ++d)
            if (TW16 % d == 0) return d;
        return TW16;
    }
    static constexpr int D16 = ring16();
    static_assert(BM == 64 || BM == 128, "two waves of 32 or 64 tokens");
    static_assert(BNC % (MF16 ? 16 : 32) == 0 && BNC >= BNS, "computed rows in whole MFMA fragments");
    static constexpr int NSW16 = KS / 128;  // 64-deep steps per wave per stage (the k halves alternate)
    static_assert((BM * RA) % 1024 == 0 && (BNC * RW) % 1024 == 0, "whole 1 KB loads");
    static_assert(LDS <= (TWO ? 81920 : 163840), "LDS ring exceeds the workgroup's share of the CU");
    static_assert(NS >= 3, "the ring needs a slot being filled, one ready and one being read");
    static_assert((NS - 2) * NHI < 64, "vmcnt range");
    static_assert(MF16 || LDS >= 2 * TMF * TN * 4096, "the split-k exchange reuses the ring");
};

typedef int v16i __attribute__((ext_vector_type(16)));

__device__ __forceinline__ v16i mfma32x32x32(v4i a, v4i b, v16i c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

// LDS layout of an operand tile whose rows hold R bytes per stage: 16-byte slot
// (rho, kc) sits at KC*rho + (kc ^ g(rho)), KC = R/16.  A 1 KB load covers
// whole rows (16 rows of 64 B, 8 of 128 B or 4 of 256 B); the
// xor keeps the 16 lanes that one ds_read_b128 phase serves (16 consecutive
// rows, one kc) on 16 distinct groups of four banks.
template <int R>
__device__ __forceinline__ int slot_swizzle(int rho) {
    constexpr int KC = R / 16;
    static_assert(KC == 4 || KC == 8 || KC == 16, "rows of 64, 128 or 256 bytes");
    return KC == 4 ? ((rho >> 2) & 3) : KC == 8 ? ((rho >> 1) & 7) : (rho & 15);
}
template <int R>
__device__ __forceinline__ int slot_of(int rho, int kc) {
    return (R / 16) * rho + (kc ^ slot_swizzle<R>(rho));
}

// LDS byte offset of lane `lane`'s 16-k operand chunk for MFMA k step j of a
// stage, in the operand tile's first 32 rows (row 32 f + r is R * 32 f further:
// the swizzle only uses the low 4 bits of the row).  Lane l serves row l % 32
// and the k half h = l / 32: k = 32 j + 16 h + [0, 16).
template <int BITS, int R>
__device__ __forceinline__ int operand_offset(int lane, int j) {
    const int rho = lane & 31, h = lane >> 5;
    if (BITS == 8) return 16 * slot_of<R>(rho, 2 * j + h);  // 16 k = 16 bytes
    return 16 * slot_of<R>(rho, j) + 8 * h;                 // 16 k = 8 bytes
}

// The same for v_mfma_i32_16x16x64_i8: lane l serves row l % 16 of the
// fragment and k = 64 s + 16 (l / 16) + [0, 16) of 64-deep step s.
template <int BITS, int R>
__device__ __forceinline__ int operand_offset16(int lane, int s) {
    const int rho = lane & 15, q = lane >> 4;
    if (BITS == 8) return 16 * slot_of<R>(rho, 4 * s + q);             // 16 k = 16 bytes
    return 16 * slot_of<R>(rho, 2 * s + (q >> 1)) + 8 * (q & 1);        // 16 k = 8 bytes
}

// One lane's operand chunk as read from LDS (`raw`: 8 bytes of nibbles or 16
// code bytes) and as the MFMA takes it (`expand`).  The MFMA waves read raw
// chunks ahead and expand them only where they are used: expanding next to the
// read would make the wave wait for the read there.  8-bit codes facing 8-bit
// codes need no expansion (kIdentity).
template <int BITS, int PARTNER>
struct LdsOperand;
template <int PARTNER>
struct LdsOperand<4, PARTNER> {
    typedef uint2 raw;
    static constexpr bool kIdentity = false;
    __device__ __forceinline__ static raw load(const uint8_t* p) { return *reinterpret_cast<const uint2*>(p); }
    __device__ __forceinline__ static v4i expand(raw r) { return frag_from_nibbles(r); }
};
template <>
struct LdsOperand<8, 4> {
    typedef uint4 raw;
    static constexpr bool kIdentity = false;
    __device__ __forceinline__ static raw load(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }
    __device__ __forceinline__ static v4i expand(raw r) { return frag_from_bytes_nibble_order(r); }
};
template <>
struct LdsOperand<8, 8> {
    typedef v4i raw;
    static constexpr bool kIdentity = true;
    __device__ __forceinline__ static raw load(const uint8_t* p) { return *reinterpret_cast<const v4i*>(p); }
    __device__ __forceinline__ static v4i expand(raw r) { return r; }
};

// 32x32x32 form with a 4-bit operand (stages of 256 k): the MFMA k steps go
// in pairs.  Lane half h of pair p takes k = 64 p + 32 h + 16 e + [0, 16) in
// step 2 p + e (any order of k serves, as long as both operands use it), so a
// lane's 4-bit chunk of the pair is one whole 16-byte slot (e = 0 in its low
// 8 bytes) and an 8-bit partner's chunk of each step is the slot after the
// previous one.  Every LDS read of these stages is then a ds_read_b128, which
// the slot swizzle keeps conflict-free; 8-byte reads of one k half put two
// rows on every bank pair.
template <int BITS, int R>
__device__ __forceinline__ int pair_offset(int lane, int p, int e) {
    const int rho = lane & 31, h = lane >> 5;
    if (BITS == 4) return 16 * slot_of<R>(rho, 2 * p + h);
    return 16 * slot_of<R>(rho, 4 * p + 2 * h + e);
}

// One lane's operand chunk of a step pair as read (`raw`) and one step of it as
// the MFMA takes it (`expand`).
template <int BITS, int PARTNER>
struct PairOperand;
template <int PARTNER>
struct PairOperand<4, PARTNER> {
    typedef uint4 raw;
    __device__ __forceinline__ static raw load(const uint8_t* base, const int (&off)[2]) {
        return *reinterpret_cast<const uint4*>(base + off[0]);
    }
    __device__ __forceinline__ static v4i expand(const raw& r, int e) {
        return frag_from_nibbles(e ? make_uint2(r.z, r.w) : make_uint2(r.x, r.y));
    }
};
template <>
struct PairOperand<8, 4> {
    struct raw {
        uint4 lo, hi;
    };
    __device__ __forceinline__ static raw load(const uint8_t* base, const int (&off)[2]) {
        return raw{*reinterpret_cast<const uint4*>(base + off[0]), *reinterpret_cast<const uint4*>(base + off[1])};
    }
    __device__ __forceinline__ static v4i expand(const raw& r, int e) {
        return frag_from_bytes_nibble_order(e ? r.hi : r.lo);
    }
};

// global source of 1 KB load q of an operand tile for `lane`: row rho of the
// tile and 16-byte column kc, the inverse of slot_of
template <int R>
__device__ __forceinline__ void slot_source(int q, int lane, int& rho, int& kc) {
    constexpr int KC = R / 16;
    const int sigma = 64 * q + lane;
    rho = sigma / KC;
    kc = (sigma % KC) ^ slot_swizzle<R>(rho);
}

// Row stride (int32 elements) of the accumulator tile staged in LDS for the
// epilogue: BNC + 4 keeps a b128 write phase (16 consecutive tokens) on 16
// distinct groups of four banks.
template <class CF>
constexpr int acc_stride() {
    return CF::BNC + 4;
}

template <int ABITS, int WBITS, class CF>
__device__ __forceinline__ void gemm_body(const GemmArgs& g, int tiles_m, int tiles_n) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[CF::LDS];
    static_assert(CF::BM * acc_stride<CF>() * 4 <= CF::LDS, "the epilogue tile reuses the ring");

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
    const int m0 = tm * CF::BM, n0 = tn * CF::BNS;
    const int64_t lda = ABITS == 8 ? g.K : g.K / 2;
    const int64_t ldw = WBITS == 8 ? g.K : g.K / 2;
    // K is a multiple of 128; with a 4-bit operand a stage is 256 deep and the
    // last stage may be half (128) deep
    const int nk = (g.K + CF::KS - 1) / CF::KS;
    const bool half_last = (g.K % CF::KS) != 0;
    const int nfull = nk - (half_last ? 1 : 0);

    // Epilogue operands.  All eight waves store: wave w takes tile rows
    // w BM/8 .. + BM/8; a lane takes 8 consecutive outputs n .. n + 7 of one
    // token (one 16-byte bf16 store; in the head layout the 8 stay inside one
    // head since head_dim % 8 == 0).  Each wave issues these loads as soon as
    // its part of the main loop is done, so that their latency hides behind
    // the exchange of the two k halves.
    constexpr int LPR = CF::BNS / 8;   // lanes per token row
    constexpr int RPI = 64 / LPR;      // token rows per pass
    constexpr int ROWS = CF::BM / 8;   // token rows per wave
    constexpr int NIT = (ROWS + RPI - 1) / RPI;
    const int lr = lane / LPR, lc = lane % LPR;
    const int n_epi = n0 + 8 * lc;
    const bool col_ok = lr < RPI && n_epi < g.N;
    float4 sw0 = make_float4(0.f, 0.f, 0.f, 0.f), sw1 = sw0, b0 = sw0, b1 = sw0;
    bool ok[NIT];
    int rr[NIT];
    float sa[NIT];
    uint4 rs[NIT];
    auto load_epilogue_operands = [&]() {
        if (col_ok) {
            sw0 = *reinterpret_cast<const float4*>(g.wscale + n_epi);
            sw1 = *reinterpret_cast<const float4*>(g.wscale + n_epi + 4);
            if (g.bias) {
                b0 = *reinterpret_cast<const float4*>(g.bias + n_epi);
                b1 = *reinterpret_cast<const float4*>(g.bias + n_epi + 4);
            }
        }
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            rr[it] = wave * ROWS + it * RPI + lr;
            const int m = m0 + rr[it];
            ok[it] = col_ok && it * RPI + lr < ROWS && m < g.M;
            sa[it] = ok[it] ? g.act_scale[m] : 0.0f;
            rs[it] = (ok[it] && g.residual)
                         ? *reinterpret_cast<const uint4*>(g.residual + int64_t(m) * g.ldr + n_epi)
                         : make_uint4(0, 0, 0, 0);
        }
    };

    if (wave >= 4) {
        // ---------------------------------------------------------- load waves
        // Load wave p issues the stage's 1 KB copies c = p + 4 i; a wave with one
        // fewer copy repeats its last one (same source, same LDS bytes), so all
        // issue NHI per stage and the waits are uniform.  Each copy reads a
        // row-block base (scalar, advanced per stage) + a fixed per-lane offset.
        // In a half-deep last stage a lane whose column would run past the end
        // of its row reads bytes of the stage's first 64 instead; that LDS slot
        // is never read.
        const int p = wave - 4;
        const uint8_t* abase = g.act + int64_t(m0) * lda;
        const uint8_t* wbase = g.w + int64_t(n0) * ldw;
        uint32_t voff[CF::NHI], dlast[CF::NHI];
        int ldsoff[CF::NHI];
        bool is_act[CF::NHI];
#pragma unroll
        for (int i = 0; i < CF::NHI; ++i) {
            int c = p + 4 * i;
            if (c >= CF::C) c -= 4;
            ldsoff[i] = c * 1024;
            int rho, kc, rowoff, half;
            is_act[i] = c < CF::CA;
            if (c < CF::CA) {
                slot_source<CF::RA>(c, lane, rho, kc);
                int row = m0 + rho;
                row = row < g.M ? row : g.M - 1;
                rowoff = (row - m0) * int(lda);
                half = CF::RA / 2;
            } else {
                slot_source<CF::RW>(c - CF::CA, lane, rho, kc);
                int row = n0 + rho;
                row = row < g.N ? row : g.N - 1;
                rowoff = (row - n0) * int(ldw);
                half = CF::RW / 2;
            }
            const int col = 16 * kc;
            voff[i] = uint32_t(rowoff + col);
            dlast[i] = uint32_t((col < half ? col : (col & 63)) - col);  // rows are at least 64 bytes
        }
        const uint32_t lds0 = lds_address(lds);
        auto load_stage = [&](int stage_idx, int slot) {
#pragma unroll
            for (int i = 0; i < CF::NHI; ++i) {
                const uint8_t* base =
                    is_act[i] ? abase + int64_t(stage_idx) * CF::RA : wbase + int64_t(stage_idx) * CF::RW;
                const uint32_t off = voff[i] + ((half_last && stage_idx == nk - 1) ? dlast[i] : 0u);
                copy16_to_lds(base, off, lds0 + uint32_t(slot * CF::STAGE + ldsoff[i]));
            }
        };
        // stage 0 alone, published as soon as it lands, then stages 1 .. NS-2
        // (clamped to the last stage when K is short): at launch every CU's
        // first stage then queues ahead of the others' prefetch (qkv 19.50 ->
        // 19.30 us, down 64.09 -> 63.64 us against issuing all NS - 1 first)
        load_stage(0, 0);
        wait_vmcnt<0>();
        barrier_nofence();
        for (int s = 1; s < CF::NS - 1; ++s) load_stage(s < nk ? s : nk - 1, s);
        // After barrier s-1 every MFMA wave is done with stage s-1, whose slot
        // takes stage s + NS - 1 while that is a stage of K.  Barrier s
        // publishes stage s + 1: the wait lets the stages issued after it stay
        // in flight (NS - 2 of them, fewer in the last iterations, which issue
        // nothing; the epilogue's loads then do not queue behind copies).
        int issued = CF::NS - 1;  // stage copies issued so far
        for (int s = 0; s < nfull; ++s) {
            if (s + CF::NS - 1 < nk) {
                load_stage(s + CF::NS - 1, (s + CF::NS - 1) % CF::NS);
                ++issued;
                wait_vmcnt<(CF::NS - 2) * CF::NHI>();
            } else {
                wait_stages_in_flight<CF::NHI>(issued - (s + 2));
            }
            barrier_nofence();
        }
        wait_vmcnt<0>();      // every ring load has landed
        load_epilogue_operands();
        barrier_nofence();    // E1: the ring is idle
        barrier_nofence();    // E2: k-half 1 partial sums staged
        barrier_nofence();    // E3: tile complete
    } else if constexpr (CF::MF16) {
        // ------------------------------------------- MFMA waves, 16x16x64 form
        // wave roles: tokens wm * BM/2 .. + BM/2 (TF16 fragments of 16), all BNC
        // weight rows (TW16 fragments of 16), the 64-deep k steps 2 i + kh of
        // every stage.  The (step, weight fragment) units of a stage run in
        // order; the unit D - 1 ahead is read while the current one's MFMAs
        // run, and a step's token fragments are read with its first weight
        // fragment.  The reads that would start the next stage first wait for
        // this wave's reads of the stage and for the barrier that publishes it.
        // A half-deep last stage (4-bit operands, K % 256 = 128) has one step
        // per wave and no barrier.  The last stage reads "next stage" operands
        // from slot (s + 1) % NS too and never uses them: with no condition on
        // those reads the loop is straight-line code, whose LDS waits the
        // compiler counts exactly (a conditional read made it wait for every
        // read in flight, the one just issued included, at each stage start).
        constexpr int TF = CF::TF16, TW = CF::TW16, D = CF::D16, NSW = CF::NSW16;
        const int wm = wave & 1;
        const int kh = wave >> 1;
        int offa[NSW], offw[NSW];
#pragma unroll
        for (int i = 0; i < NSW; ++i) {
            offa[i] = operand_offset16<ABITS, CF::RA>(lane, 2 * i + kh) + wm * (CF::BM / 2) * CF::RA;
            offw[i] = operand_offset16<WBITS, CF::RW>(lane, 2 * i + kh) + CF::CA * 1024;
        }
        v4i acc[TW][TF];
#pragma unroll
        for (int n = 0; n < TW; ++n)
#pragma unroll
            for (int f = 0; f < TF; ++f) acc[n][f] = v4i{0, 0, 0, 0};
        typedef LdsOperand<ABITS, WBITS> OpA;
        typedef LdsOperand<WBITS, ABITS> OpW;
        typename OpA::raw fa_raw[2][TF];  // token fragments of two steps, as read
        typename OpW::raw ring[D];         // weight fragments, as read
        v4i fa[TF];                        // the current step's token fragments, expanded
        auto read_a = [&](int s, int i, int b) {
            const uint8_t* base = lds + (s % CF::NS) * CF::STAGE + offa[i];
#pragma unroll
            for (int f = 0; f < TF; ++f) fa_raw[b][f] = OpA::load(base + f * 16 * CF::RA);
        };
        auto read_w = [&](int s, int i, int n) {
            return OpW::load(lds + (s % CF::NS) * CF::STAGE + offw[i] + n * 16 * CF::RW);
        };
        barrier_nofence();  // stage 0 published
        read_a(0, 0, 0);
#pragma unroll
        for (int q = 0; q < D - 1; ++q) ring[q] = read_w(0, 0, q);
        // with nothing in flight on entry, the compiler's LDS wait at the top of
        // the stage loop counts the reads of the loop's back edge alone (a read
        // still in flight from here made it wait for all of them)
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_sched_barrier(0);
        // stage s; SP = the stage's parity (token-fragment buffer of step i is
        // (SP * NSW + i) & 1); HALF: a half-deep last stage
        auto stage16 = [&](int s, auto sp_tag, auto half_tag) {
            constexpr int SP = decltype(sp_tag)::value;
            constexpr bool kHalf = decltype(half_tag)::value;
            constexpr int steps = kHalf ? 1 : NSW;
            constexpr int units = steps * TW;
#pragma unroll
            for (int t = 0; t < units; ++t) {
                const int i = t / TW, n = t % TW;
                const int q = t + D - 1;  // the unit read in this iteration
                const int b = (SP * NSW + i) & 1;
                auto mfmas = [&]() {
                    if constexpr (!OpA::kIdentity) {
                        if (n == 0) {  // a step's first unit expands its token fragments
#pragma unroll
                            for (int f = 0; f < TF; ++f) fa[f] = OpA::expand(fa_raw[b][f]);
                        }
                    }
                    const v4i w = OpW::expand(ring[n % D]);
#pragma unroll
                    for (int f = 0; f < TF; ++f)
                        acc[n][f] = mfma16x16x64(w, OpA::kIdentity ? OpA::expand(fa_raw[b][f]) : fa[f], acc[n][f]);
                };
                // the scheduling barriers keep this order: left to itself the
                // compiler moved reads next to their first use
                if (q < units) {
                    if (q % TW == 0) read_a(s, q / TW, (SP * NSW + q / TW) & 1);
                    ring[q % D] = read_w(s, q / TW, q % TW);
                    __builtin_amdgcn_sched_barrier(0);
                    mfmas();
                } else if (!kHalf) {
                    if (q == units) {
                        // the unit's MFMAs go first so that the wait below finds
                        // the stage's last read landed
                        mfmas();
                        __builtin_amdgcn_sched_barrier(0);
                        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave is done with stage s
                        barrier_nofence();
                        read_a(s + 1, 0, ((SP + 1) * NSW) & 1);
                        ring[q % D] = read_w(s + 1, 0, 0);
                    } else {
                        ring[q % D] = read_w(s + 1, 0, q - units);
                        __builtin_amdgcn_sched_barrier(0);
                        mfmas();
                    }
                } else {
                    mfmas();
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        // stages in unconditional pairs (a conditional second stage inside the
        // loop made the compiler copy the accumulators at every iteration to
        // reconcile the two paths), then an odd last full stage, then the
        // half-deep stage of 4-bit operands
        int s = 0;
        for (; s + 1 < nfull; s += 2) {
            stage16(s, std::integral_constant<int, 0>{}, std::false_type{});
            stage16(s + 1, std::integral_constant<int, 1>{}, std::false_type{});
        }
        const bool odd = s < nfull;
        if (odd) stage16(s, std::integral_constant<int, 0>{}, std::false_type{});
        if constexpr (NSW > 1) {  // only 4-bit operands have half-deep stages
            if (half_last) {
                if (odd)
                    stage16(nfull, std::integral_constant<int, 1>{}, std::true_type{});
                else
                    stage16(nfull, std::integral_constant<int, 0>{}, std::true_type{});
            }
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's ring reads are done
        load_epilogue_operands();
        barrier_nofence();                   // E1: the ring is idle

        // The two k halves meet in X: the k-half 0 wave finishes row fragments
        // n < TWH and the k-half 1 wave the rest.  Each first stores the
        // fragments the other finishes, then adds the other's partial sums to
        // its own and stores the total (half the serial LDS work of one wave
        // doing all the adds).  Lane l holds token wm BM/2 + 16 f + l % 16 and
        // rows 16 n + 4 (l / 16) + [0, 4).
        int32_t* X = reinterpret_cast<int32_t*>(lds);
        constexpr int XS = acc_stride<CF>();
        constexpr int TWH = (TW + 1) / 2;
        auto xrow = [&](int f, int n) {
            const int m = wm * (CF::BM / 2) + 16 * f + (lane & 15);
            return reinterpret_cast<v4i*>(X + m * XS + 16 * n + 4 * (lane >> 4));
        };
        // (one code path per k half, so that which fragments a wave owns is
        // known at compile time)
        auto exchange = [&](auto kh_tag) {
            constexpr int KH = decltype(kh_tag)::value;
            constexpr int own_lo = KH == 0 ? 0 : TWH, own_hi = KH == 0 ? TWH : TW;
#pragma unroll
            for (int n = 0; n < TW; ++n)
                if (n < own_lo || n >= own_hi) {
#pragma unroll
                    for (int f = 0; f < TF; ++f) *xrow(f, n) = acc[n][f];
                }
            barrier_lds();  // E2
#pragma unroll
            for (int n = own_lo; n < own_hi; ++n)
#pragma unroll
                for (int f = 0; f < TF; ++f) {
                    v4i* p = xrow(f, n);
                    *p = acc[n][f] + *p;
                }
        };
        if (kh == 0)
            exchange(std::integral_constant<int, 0>{});
        else
            exchange(std::integral_constant<int, 1>{});
        barrier_lds();  // E3
    } else {
        // ---------------------------------------------------------- MFMA waves
        // wave roles: tokens wm * BM/2 .. + BM/2 (TMF fragments of 32), all BNC
        // weight rows (TN fragments), and the MFMA k steps j = 2 i + kh of every
        // stage; with RSPLIT all tokens and rows wm * BNC/2 .. + BNC/2
        const int wm = wave & 1;
        const int kh = wave >> 1;
        int offa[CF::NSTEP], offw[CF::NSTEP];
#pragma unroll
        for (int i = 0; i < CF::NSTEP; ++i) {
            offa[i] = operand_offset<ABITS, CF::RA>(lane, 2 * i + kh) + wm * CF::TMF * 32 * CF::RA;
            offw[i] = operand_offset<WBITS, CF::RW>(lane, 2 * i + kh) + CF::CA * 1024;
        }

        v16i acc[CF::TN][CF::TMF];
#pragma unroll
        for (int i = 0; i < CF::TN; ++i)
#pragma unroll
            for (int f = 0; f < CF::TMF; ++f) acc[i][f] = v16i{};

        if constexpr (CF::KS == 256) {
            // A 4-bit operand: the paired k order above.  Local pair t of a
            // stage is pair p = 2 t + kh (the k halves alternate by pair).  At
            // a pair's start its token fragments are expanded for both steps,
            // which frees their registers for the next pair's read; in its
            // second step each weight fragment's registers take the next pair's
            // chunk as soon as they are expanded.  The stage's last pair waits
            // for this wave's reads after its first step and passes the barrier
            // that frees the stage's slot and publishes the next stage, whose
            // first pair it then reads.  A half-deep last stage is one pair per
            // wave and has no barrier.
            constexpr int NP = CF::NSTEP / 2;  // pairs per wave in a full stage
            typedef PairOperand<ABITS, WBITS> PA;
            typedef PairOperand<WBITS, ABITS> PW;
            int pa[NP][2], pw[NP][2];
#pragma unroll
            for (int t = 0; t < NP; ++t)
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    pa[t][e] = pair_offset<ABITS, CF::RA>(lane, 2 * t + kh, e) +
                               (CF::RSPLIT ? 0 : wm * CF::TMF * 32 * CF::RA);
                    pw[t][e] = pair_offset<WBITS, CF::RW>(lane, 2 * t + kh, e) + CF::CA * 1024 +
                               (CF::RSPLIT ? wm * CF::TN * 32 * CF::RW : 0);
                }
            typename PA::raw ra[CF::TMF];
            typename PW::raw rw[CF::TN];
            auto read_a = [&](int s, int t) {
                const uint8_t* base = lds + (s % CF::NS) * CF::STAGE;
#pragma unroll
                for (int f = 0; f < CF::TMF; ++f) ra[f] = PA::load(base + f * 32 * CF::RA, pa[t]);
            };
            auto read_w = [&](int s, int t, int n) {
                rw[n] = PW::load(lds + (s % CF::NS) * CF::STAGE + n * 32 * CF::RW, pw[t]);
            };
            barrier_nofence();  // stage 0 published
            read_a(0, 0);
#pragma unroll
            for (int n = 0; n < CF::TN; ++n) read_w(0, 0, n);
            auto stage = [&](int s, auto full_tag) {
                constexpr bool kFull = decltype(full_tag)::value;
                constexpr int kPairs = kFull ? NP : NP / 2;
                const int next = s + 1 < nk ? s + 1 : nk - 1;
#pragma unroll
                for (int t = 0; t < kPairs; ++t) {
                    const bool last = t + 1 == kPairs;
                    v4i xa[2][CF::TMF];
#pragma unroll
                    for (int f = 0; f < CF::TMF; ++f) {
                        xa[0][f] = PA::expand(ra[f], 0);
                        xa[1][f] = PA::expand(ra[f], 1);
                    }
                    if (!last) read_a(s, t + 1);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int n = 0; n < CF::TN; ++n) {
                        const v4i w = PW::expand(rw[n], 0);
#pragma unroll
                        for (int f = 0; f < CF::TMF; ++f) acc[n][f] = mfma32x32x32(w, xa[0][f], acc[n][f]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    if (last && kFull) {
                        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave is done with stage s
                        barrier_nofence();
                        read_a(next, 0);
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int n = 0; n < CF::TN; ++n) {
                        const v4i w = PW::expand(rw[n], 1);
                        if (!last)
                            read_w(s, t + 1, n);
                        else if (kFull)
                            read_w(next, 0, n);
#pragma unroll
                        for (int f = 0; f < CF::TMF; ++f) acc[n][f] = mfma32x32x32(w, xa[1][f], acc[n][f]);
                        // (each read goes out with its fragment's step: grouped at
                        // the step's end they left the next pair waiting for them)
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            };
            for (int s = 0; s < nfull; ++s) stage(s, std::true_type{});
            if (half_last) stage(nk - 1, std::false_type{});
        } else {
            typedef LdsOperand<ABITS, WBITS> OpA;
            typedef LdsOperand<WBITS, ABITS> OpW;
            typename OpA::raw fa[2][CF::TMF];  // two steps' operands, as read
            typename OpW::raw fw[2][CF::TN];
            auto read_frags = [&](int s, int i, int buf) {
                const uint8_t* base = lds + (s % CF::NS) * CF::STAGE;
    #pragma unroll
                for (int f = 0; f < CF::TMF; ++f) fa[buf][f] = OpA::load(base + offa[i] + f * 32 * CF::RA);
    #pragma unroll
                for (int n = 0; n < CF::TN; ++n) fw[buf][n] = OpW::load(base + offw[i] + n * 32 * CF::RW);
            };

            barrier_nofence();  // stage 0 published
            read_frags(0, 0, 0);

            // One k stage.  In each step the first TMF MFMAs run on operands read
            // one step earlier (expanded at the step's start); then the next step's
            // operands are read from LDS (their latency hides behind the remaining
            // MFMAs).  Before the last
            // step this wave's reads of the stage are waited for and the barrier
            // both frees the stage's slot and publishes the next stage.  A
            // half-deep last stage (FULL = false) runs its first NSTEP/2 steps and
            // has no barrier.
            auto stage = [&](int s, auto full_tag) {
                constexpr bool kFull = decltype(full_tag)::value;
                constexpr int kSteps = kFull ? CF::NSTEP : CF::NSTEP / 2;
                const int next = s + 1 < nk ? s + 1 : nk - 1;
    #pragma unroll
                for (int j = 0; j < kSteps; ++j) {
                    const int cur = j & 1;
                    v4i xa[CF::TMF];  // this step's token fragments, expanded
    #pragma unroll
                    for (int f = 0; f < CF::TMF; ++f) xa[f] = OpA::expand(fa[cur][f]);
                    const v4i w0 = OpW::expand(fw[cur][0]);
    #pragma unroll
                    for (int f = 0; f < CF::TMF; ++f) acc[0][f] = mfma32x32x32(w0, xa[f], acc[0][f]);
                    __builtin_amdgcn_sched_barrier(0);
                    if (j + 1 < kSteps) {
                        read_frags(s, j + 1, cur ^ 1);
                    } else if (kFull) {
                        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
                        barrier_nofence();
                        read_frags(next, 0, cur ^ 1);
                    }
                    __builtin_amdgcn_sched_barrier(0);
    #pragma unroll
                    for (int n = 1; n < CF::TN; ++n) {
                        const v4i w = OpW::expand(fw[cur][n]);
    #pragma unroll
                        for (int f = 0; f < CF::TMF; ++f) acc[n][f] = mfma32x32x32(w, xa[f], acc[n][f]);
                    }
                }
            };
            for (int s = 0; s < nfull; ++s) stage(s, std::true_type{});
            if (half_last) stage(nk - 1, std::false_type{});
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's ring reads are done
        load_epilogue_operands();
        barrier_nofence();                   // E1: the ring is idle

        // Stage the accumulator tile X[BM][BNC] (int32, row stride XS) in the
        // ring: the k-half 1 waves write their partial sums, then the k-half 0
        // waves add theirs.  Lane l holds token wm BM/2 + 32 f + l % 32 and rows
        // 32 n + 8 q + 4 (l / 32) + [0, 4) of fragment (n, f) in registers 4 q ...
        // (with RSPLIT token 32 f + l % 32 and rows wm BNC/2 + 32 n + ...)
        int32_t* X = reinterpret_cast<int32_t*>(lds);
        constexpr int XS = acc_stride<CF>();
        auto xrow = [&](int f, int n, int q) {
            const int m = (CF::RSPLIT ? 0 : wm * (CF::BM / 2)) + 32 * f + (lane & 31);
            const int col = (CF::RSPLIT ? wm * CF::TN * 32 : 0) + 32 * n + 8 * q + 4 * (lane >> 5);
            return reinterpret_cast<v4i*>(X + m * XS + col);
        };
        if (kh == 1) {
#pragma unroll
            for (int n = 0; n < CF::TN; ++n)
#pragma unroll
                for (int f = 0; f < CF::TMF; ++f)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        *xrow(f, n, q) = v4i{acc[n][f][4 * q], acc[n][f][4 * q + 1], acc[n][f][4 * q + 2],
                                             acc[n][f][4 * q + 3]};
        }
        barrier_lds();  // E2
        if (kh == 0) {
#pragma unroll
            for (int n = 0; n < CF::TN; ++n)
#pragma unroll
                for (int f = 0; f < CF::TMF; ++f)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        v4i* p = xrow(f, n, q);
                        const v4i v = *p;
                        *p = v4i{acc[n][f][4 * q] + v[0], acc[n][f][4 * q + 1] + v[1], acc[n][f][4 * q + 2] + v[2],
                                 acc[n][f][4 * q + 3] + v[3]};
                    }
        }
        barrier_lds();  // E3
    }

    // ---------------------------------------------------------------- epilogue
    //   y[m][n] = bf16_rne(float(acc >> shift) * (s_m * s_n) [+ bias_n] [+ residual_mn])
    // in float32, one rounding per step.  Every operand was loaded before the
    // first store (a load queued behind a store would wait for it).
    {
        const int32_t* X = reinterpret_cast<const int32_t*>(lds);
        constexpr int XS = acc_stride<CF>();
        constexpr int shift = AccShift<ABITS, WBITS>::value;
        const int n = n_epi;
        // output addresses: this lane's column n (head layout: its head's
        // [M][head_dim] block) plus token row times the row stride, computed
        // once and stepped by RPI rows per iteration
        const int64_t ystride = g.head_dim > 0 ? g.head_dim : g.ldy;
        int64_t ycol = n;
        if (g.head_dim > 0) {
            const int h = n / g.head_dim;
            ycol = int64_t(h) * g.M * g.head_dim + (n - h * g.head_dim);
        }
        uint16_t* const yp0 = g.y + ycol + int64_t(m0 + rr[0]) * ystride;
        int32_t* const ap0 = g.acc ? g.acc + n + int64_t(m0 + rr[0]) * g.N : nullptr;
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        // (one code path per bias/residual combination: as run-time
        // conditions they became two selects per output)
        auto run = [&](auto bias_tag, auto res_tag) {
            constexpr bool kBias = decltype(bias_tag)::value;
            constexpr bool kRes = decltype(res_tag)::value;
#pragma unroll
            for (int it = 0; it < NIT; ++it) {
                if (!ok[it]) continue;
                const v4i x0 = *reinterpret_cast<const v4i*>(X + rr[it] * XS + 8 * lc);
                const v4i x1 = *reinterpret_cast<const v4i*>(X + rr[it] * XS + 8 * lc + 4);
                const int a[8] = {x0[0] >> shift, x0[1] >> shift, x0[2] >> shift, x0[3] >> shift,
                                  x1[0] >> shift, x1[1] >> shift, x1[2] >> shift, x1[3] >> shift};
                const float sw[8] = {sw0.x, sw0.y, sw0.z, sw0.w, sw1.x, sw1.y, sw1.z, sw1.w};
                const float bb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
                const uint32_t rw[4] = {rs[it].x, rs[it].y, rs[it].z, rs[it].w};
                uint32_t o[4];
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    float t0 = float(a[e]) * (sa[it] * sw[e]);
                    float t1 = float(a[e + 1]) * (sa[it] * sw[e + 1]);
                    if constexpr (kBias) {
                        t0 = t0 + bb[e];
                        t1 = t1 + bb[e + 1];
                    }
                    if constexpr (kRes) {
                        t0 = t0 + bf16_lo(rw[e / 2]);
                        t1 = t1 + bf16_hi(rw[e / 2]);
                    }
                    o[e / 2] = pack_bf16x2(t0, t1);
                }
                store_dev16(yp0 + int64_t(it * RPI) * ystride, make_uint4(o[0], o[1], o[2], o[3]));
                if (ap0) {
                    int32_t* ap = ap0 + int64_t(it * RPI) * g.N;
                    *reinterpret_cast<int4*>(ap) = make_int4(a[0], a[1], a[2], a[3]);
                    *reinterpret_cast<int4*>(ap + 4) = make_int4(a[4], a[5], a[6], a[7]);
                }
            }
        };
        if (g.bias) {
            if (g.residual)
                run(std::true_type{}, std::true_type{});
            else
                run(std::true_type{}, std::false_type{});
        } else {
            if (g.residual)
                run(std::false_type{}, std::true_type{});
            else
                run(std::false_type{}, std::false_type{});
        }
    }
}

template <int ABITS, int WBITS, class CF>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs g, int tiles_m, int tiles_n) {
    gemm_body<ABITS, WBITS, CF>(g, tiles_m, tiles_n);
}

// The same kernel held to 128 VGPRs per wave, so that two workgroups fit a CU.
template <int ABITS, int WBITS, class CF>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void gemm_kernel_x2(GemmArgs g,
                                                                                                  int tiles_m,
                                                                                                  int tiles_n) {
    gemm_body<ABITS, WBITS, CF>(g, tiles_m, tiles_n);
}

template <int ABITS, int WBITS, class CF>
hipError_t launch_cfg(const GemmArgs& g, hipStream_t st) {
    const int tiles_m = (g.M + CF::BM - 1) / CF::BM;
    const int tiles_n = (g.N + CF::BNS - 1) / CF::BNS;
    if constexpr (CF::TWO)
        hipLaunchKernelGGL((gemm_kernel_x2<ABITS, WBITS, CF>), dim3(tiles_m * tiles_n), dim3(kThreads), 0, st, g,
                           tiles_m, tiles_n);
    else
        hipLaunchKernelGGL((gemm_kernel<ABITS, WBITS, CF>), dim3(tiles_m * tiles_n), dim3(kThreads), 0, st, g,
                           tiles_m, tiles_n);
    return hipGetLastError();
}

// Tile shapes: tokens x stored weight rows (computed rows rounded up to 32).
// 64x128x2: the 64 x 128 tile with a 3-stage ring, two workgroups per CU.
enum TileId { T128x128 = 0, T128x144, T128x112, T128x96, T64x128, T64x224, T64x256, T64x288, T64x128x2, kNumTiles };

const char* const kTileNames[kNumTiles] = {"128x128", "128x144", "128x112", "128x96",  "64x128",
                                           "64x224",  "64x256",  "64x288",  "64x128x2"};
const int kTileBM[kNumTiles] = {128, 128, 128, 128, 64, 64, 64, 64, 64};
const int kTileBN[kNumTiles] = {128, 144, 112, 96, 128, 224, 256, 288, 128};

// Pipeline depth: as many stages as fit in 160 KiB of LDS, at most 8.
template <int ABITS, int WBITS, int BM, int BNC, int KS8 = 128>
constexpr int ring_depth() {
    constexpr int ks = (ABITS == 4 || WBITS == 4) ? 256 : KS8;
    constexpr int stage = (BM * ks * ABITS / 8) + (BNC * ks * WBITS / 8);
    constexpr int n = 163840 / stage;
    return n > 8 ? 8 : n;
}

// MFMA form: v_mfma_i32_16x16x64_i8 (rows in fragments of 16, so a 144-row
// tile computes no padding rows) unless the test hook gemm_mfma=32 asks for
// v_mfma_i32_32x32x32_i8.  The 16x16x64 form measured 6-7 % faster on the
// W8A8 qkv and down layers (22.8 against 24.6 us, 73.9 against 79.1 us), also
// where no rows are padded: with random operands it sustains a higher rate
// under the power limit (3.4-3.6 against 3.2-3.3 POP/s).
int mfma_form() { return hooks().gemm_mfma.load(std::memory_order_relaxed); }

template <int ABITS, int WBITS, int BM, int BNS, bool TWO = false>
hipError_t launch_shape(const GemmArgs& g, hipStream_t st) {
    constexpr int bnc = (BNS + 31) / 32 * 32;
    constexpr int ns = TWO ? 3 : ring_depth<ABITS, WBITS, BM, bnc>();
    constexpr int bnc16 = (BNS + 15) / 16 * 16;
    constexpr int ns16 = TWO ? 3 : ring_depth<ABITS, WBITS, BM, bnc16>();
    // With a 4-bit operand the 16x16x64 form runs two steps per stage and
    // unpacks the nibbles of every weight fragment.  It pays only where each
    // unpacked fragment feeds four MFMAs (128-token tiles) and the 24
    // accumulator fragments still fit without spilling: of the eight tiles
    // that is 128 x 96 (W4A4 down projection 57.1 against 61.8 us, gate+up
    // 108.7 against 120.4); with 64-token tiles it was slower (58.9 against
    // 49.7 us), so the other tiles keep the 32x32x32 form for 4-bit codes.
    constexpr bool mf16 = ns16 >= 3 && ((ABITS == 8 && WBITS == 8) || (BM == 128 && (bnc16 / 16) * 4 <= 24));
    if constexpr (mf16) {
        if (mfma_form() == 16)
            return launch_cfg<ABITS, WBITS, Cfg<ABITS, WBITS, BM, BNS, bnc16, ns16, 128, true, TWO>>(g, st);
    }
    if constexpr (ns >= 3) {
        return launch_cfg<ABITS, WBITS, Cfg<ABITS, WBITS, BM, BNS, bnc, ns, 128, false, TWO>>(g, st);
    } else {
        // this operand mix does not fit three stages of this tile: use 128 x 128
        return launch_cfg<ABITS, WBITS, Cfg<ABITS, WBITS, 128, 128, 128, ring_depth<ABITS, WBITS, 128, 128>()>>(g,
                                                                                                             st);
    }
}

template <int ABITS, int WBITS>
hipError_t launch_tile(int tile, const GemmArgs& g, hipStream_t st) {
    switch (tile) {
        case T128x144:
            return launch_shape<ABITS, WBITS, 128, 144>(g, st);
        case T128x112:
            return launch_shape<ABITS, WBITS, 128, 112>(g, st);
        case T128x96:
            return launch_shape<ABITS, WBITS, 128, 96>(g, st);
        case T64x128:
            return launch_shape<ABITS, WBITS, 64, 128>(g, st);
        case T64x224:
            return launch_shape<ABITS, WBITS, 64, 224>(g, st);
        case T64x256:
            return launch_shape<ABITS, WBITS, 64, 256>(g, st);
        case T64x288:
            return launch_shape<ABITS, WBITS, 64, 288>(g, st);
        case T64x128x2:  // (mixed 8-bit/4-bit codes: three stages do not fit in 80 KiB)
            if constexpr (ABITS == WBITS)
                return launch_shape<ABITS, WBITS, 64, 128, true>(g, st);
            else
                return launch_shape<ABITS, WBITS, 64, 128>(g, st);
        case T128x128:
        default:
            return launch_shape<ABITS, WBITS, 128, 128>(g, st);
    }
}

// Pick the tile that minimises (waves of 256 workgroups) x (computed tile area
// / relative efficiency); computed rows are the stored ones rounded up to the
// MFMA's fragment (16 rows for the 8-bit 16x16x64 form, 32 otherwise).
// 64-token tiles reuse each weight fragment half as often: measured over all
// eight shapes they run at 0.86-0.93 of the 128-token rate per unit of area.
// With 0.9 the model picks the fastest measured tile on each 1024- and
// 816-token prefill layer: 128 x 144 for QKV (N = 4608, 256 tiles; 22.3 us
// against 23.5 for 64 x 288), 128 x 112 for the W8A8 down projection (N =
// 3584, 256 tiles; 69.2 us against 70.7 for 64 x 224 and 78.0 for 128 x 128,
// which leaves 32 CUs idle) and 64 x 128 for the W4A4 down projection (N =
// 2048, 208 tiles).  The two-per-CU 64 x 128 tile takes 512 workgroups per
// wave; where there are more tiles than CUs it hides one workgroup's fill and
// epilogue behind the other's k loop.  With 4-bit codes that made it the
// fastest tile for the W4A4 gate+up (N = 32768, 3328 tiles: 70 us against 91
// for 128 x 128) and for M = N = K = 4096 (78 against 84), hence 1.15; with
// 8-bit codes it only matched the 128-token tiles (0.95).
int choose_tile(int M, int N, int frag_rows, bool four_bit, bool two_per_cu) {
    int best = T128x128;
    double best_cost = 1e300;
    for (int c = 0; c < kNumTiles; ++c) {
        if (c == T64x128x2 && !two_per_cu) continue;
        const int bm = kTileBM[c], bn = kTileBN[c], bnc = (bn + frag_rows - 1) / frag_rows * frag_rows;
        const long tiles = long((M + bm - 1) / bm) * long((N + bn - 1) / bn);
        const int per_wave = c == T64x128x2 ? 512 : 256;
        const long waves = (tiles + per_wave - 1) / per_wave;
        const double eff = c == T64x128x2 ? (four_bit ? 1.15 : 0.95) : bm == 128 ? 1.0 : 0.9;
        const double cost = double(waves) * (per_wave / 256) * bm * bnc / eff;
        if (cost < best_cost * 0.999) {
            best_cost = cost;
            best = c;
        }
    }
    return best;
}

}  // namespace

int gemm_tile_id(const char* name) {
    for (int i = 0; i < kNumTiles; ++i)
        if (std::strcmp(name, kTileNames[i]) == 0) return i;
    return -1;
}

hipError_t launch_gemm(const GemmArgs& g, hipStream_t stream) {
    // test hook gemm_tile=<name> forces one tile shape
    int tile = hooks().gemm_tile.load(std::memory_order_relaxed);
    if (tile < 0)
        tile = choose_tile(g.M, g.N, g.abits == 8 && g.wbits == 8 && mfma_form() == 16 ? 16 : 32,
                           g.abits == 4 || g.wbits == 4, g.abits == g.wbits);
    if (g.abits == 8 && g.wbits == 8) return launch_tile<8, 8>(tile, g, stream);
    if (g.abits == 4 && g.wbits == 4) return launch_tile<4, 4>(tile, g, stream);
    if (g.abits == 8 && g.wbits == 4) return launch_tile<8, 4>(tile, g, stream);
    return launch_tile<4, 8>(tile, g, stream);
}

}  // namespace fq

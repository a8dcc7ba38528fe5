// FoldQuant integer GEMM with the fused dequant/residual epilogue on gfx950.
//
// acc[m][n] = sum_k qa[m][k] * qw[n][k] on v_mfma_i32_16x16x64_i8 (the page's
// "gemm" node: integer GEMM against per-row scaled INT8/INT4 weight codes,
// residual add in the epilogue).  Integer sums are exact in any order, so the
// tile shape and k order are free.
//
// Tiling: a 256-thread workgroup owns a BM (tokens) x BN (weight rows) output
// tile; its four waves split it 2 x 2.  Per 64-deep k step each wave holds
// 4 x 4 MFMA tiles.  The MFMA's A operand is the weight fragment and its B
// operand the activation fragment, so each lane ends with four consecutive
// output features of one token (one 8-byte bf16 store).
//
// Shared memory keeps every 16-row x 64-k fragment in MFMA lane order (lane l
// at byte 16*l, or 8*l for packed 4-bit codes), so the MFMA operand reads are
// contiguous and conflict free; tiles are double buffered through registers.
#include <hip/hip_runtime.h>

#include "fq_device.h"
#include "fq_internal.h"

namespace fq {
namespace {

constexpr int BM = 128;      // tokens per tile
constexpr int BN = 128;      // weight rows per tile
constexpr int BK = 64;       // k per step (one MFMA depth)
constexpr int kThreads = 256;

template <int BITS>
struct TileBytes {
    static constexpr int frag = BITS == 8 ? 1024 : 512;     // 16 rows x 64 k
    static constexpr int lane = BITS == 8 ? 16 : 8;         // bytes per lane per fragment
    static constexpr int row = BITS == 8 ? BK : BK / 2;     // bytes per row per step
};

// Global -> registers: wave w loads fragments 2w and 2w+1 of a 128-row tile.
template <int BITS>
struct Stage {
    uint4 r[2];
    __device__ __forceinline__ void load(const uint8_t* __restrict__ base, int64_t ld, int row0, int rows,
                                         int kbyte, int wave, int lane) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int f = wave * 2 + j;
            const int row = row0 + f * 16 + (lane & 15);
            r[j] = make_uint4(0, 0, 0, 0);
            if (row < rows) {
                const uint8_t* p = base + int64_t(row) * ld + kbyte + (lane >> 4) * TileBytes<BITS>::lane;
                if (BITS == 8) {
                    r[j] = *reinterpret_cast<const uint4*>(p);
                } else {
                    const uint2 v = *reinterpret_cast<const uint2*>(p);
                    r[j].x = v.x;
                    r[j].y = v.y;
                }
            }
        }
    }
    __device__ __forceinline__ void store(uint8_t* lds, int wave, int lane) const {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int f = wave * 2 + j;
            uint8_t* p = lds + f * TileBytes<BITS>::frag + lane * TileBytes<BITS>::lane;
            if (BITS == 8) {
                *reinterpret_cast<uint4*>(p) = r[j];
            } else {
                *reinterpret_cast<uint2*>(p) = make_uint2(r[j].x, r[j].y);
            }
        }
    }
};

template <int ABITS, int WBITS>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs g) {
    constexpr int kActTile = 8 * TileBytes<ABITS>::frag;
    constexpr int kWTile = 8 * TileBytes<WBITS>::frag;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][kActTile + kWTile];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int n0 = blockIdx.x * BN;
    const int m0 = blockIdx.y * BM;
    const int wn = wave & 1;   // wave's 64 weight rows
    const int wm = wave >> 1;  // wave's 64 tokens
    const int64_t lda = ABITS == 8 ? g.K : g.K / 2;
    const int64_t ldw = WBITS == 8 ? g.K : g.K / 2;
    const int nk = g.K / BK;

    Stage<ABITS> sa;
    Stage<WBITS> sw;
    sa.load(g.act, lda, m0, g.M, 0, wave, lane);
    sw.load(g.w, ldw, n0, g.N, 0, wave, lane);
    sa.store(lds[0], wave, lane);
    sw.store(lds[0] + kActTile, wave, lane);
    __syncthreads();

    v4i acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4i{0, 0, 0, 0};

    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) {
            sa.load(g.act, lda, m0, g.M, (kt + 1) * TileBytes<ABITS>::row, wave, lane);
            sw.load(g.w, ldw, n0, g.N, (kt + 1) * TileBytes<WBITS>::row, wave, lane);
        }
        const uint8_t* la = lds[cur];
        const uint8_t* lw = lds[cur] + kActTile;
        v4i fw[4], fa[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            fw[i] = Frag<WBITS, ABITS>::load(lw + (wn * 4 + i) * TileBytes<WBITS>::frag + lane * TileBytes<WBITS>::lane);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            fa[j] = Frag<ABITS, WBITS>::load(la + (wm * 4 + j) * TileBytes<ABITS>::frag + lane * TileBytes<ABITS>::lane);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x64(fw[i], fa[j], acc[i][j]);
        if (kt + 1 < nk) {
            sa.store(lds[cur ^ 1], wave, lane);
            sw.store(lds[cur ^ 1] + kActTile, wave, lane);
        }
        __syncthreads();
    }

    // epilogue: lane holds D[n][m] for n = nb + 4*(lane/16) + r, m = mb + lane%16
    constexpr int shift = AccShift<ABITS, WBITS>::value;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int m = m0 + wm * 64 + j * 16 + (lane & 15);
        if (m >= g.M) continue;
        const float sam = g.act_scale[m];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int n = n0 + wn * 64 + i * 16 + (lane >> 4) * 4;
            if (n >= g.N) continue;
            store_out4(acc[i][j], shift, m, n, sam, g.wscale, g.bias, g.residual, g.ldr, g.y, g.ldy, g.acc, g.N);
        }
    }
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& g, hipStream_t stream) {
    dim3 grid((g.N + BN - 1) / BN, (g.M + BM - 1) / BM);
    dim3 block(kThreads);
    if (g.abits == 8 && g.wbits == 8)
        hipLaunchKernelGGL((gemm_kernel<8, 8>), grid, block, 0, stream, g);
    else if (g.abits == 4 && g.wbits == 4)
        hipLaunchKernelGGL((gemm_kernel<4, 4>), grid, block, 0, stream, g);
    else if (g.abits == 8 && g.wbits == 4)
        hipLaunchKernelGGL((gemm_kernel<8, 4>), grid, block, 0, stream, g);
    else
        hipLaunchKernelGGL((gemm_kernel<4, 8>), grid, block, 0, stream, g);
    return hipGetLastError();
}

}  // namespace fq

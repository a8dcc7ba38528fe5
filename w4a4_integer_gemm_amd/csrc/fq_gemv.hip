// FoldQuant decode path (M <= 32 tokens) on gfx950: a weight-streaming GEMV.
//
// For decode-sized M the layer is bound by reading the weight codes once from
// HBM (the SYCL commit of the vla.cpp FoldQuant page also switches to a GEMV
// for M <= 32).  A workgroup owns R groups of 16 weight rows and splits K
// across its S waves; v_mfma_i32_16x16x64_i8 takes 16 rows as its A operand
// and up to 16 tokens as B (M > 16 takes a second MFMA per step).
//
// Unit of work: one 16-byte weight load per lane, i.e. 64 k of 8-bit codes or
// 128 k of 4-bit codes.  Lane l serves row l % 16 and the k quarter q = l / 16
// of the unit.  A wave issues the loads of up to C units back to back (with
// each unit's activation codes, which L2 serves) and only then consumes them,
// so a wave has its whole share of the row group in flight at once: with only
// N / 16 row groups in a decode layer, per-wave depth is what keeps HBM busy.
// The S partial sums of each 16 x 16 output tile meet in LDS, and one wave
// per tile runs the epilogue.
#include <hip/hip_runtime.h>

#include "fq_device.h"
#include "fq_gemv_unit.h"
#include "fq_internal.h"

namespace fq {
namespace {

constexpr int kMaxWaves = 8;

// grid: one workgroup per R groups of 16 rows; block: S waves; `per` units per wave.
// Each wave loads a unit's activation codes once and uses them for its R row
// groups, which keeps the activation re-reads (from L2) at M / (16 R) of the
// weight bytes.
template <int ABITS, int WBITS, int R, int MT, int C>
__global__ __launch_bounds__(64 * kMaxWaves) void gemv_kernel(GemmArgs g, int per) {
    using U = Unit<ABITS, WBITS>;
    constexpr int kTiles = R * MT;
    __shared__ v4i red[kMaxWaves][kTiles][64];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int S = blockDim.x >> 6;
    const int q = lane >> 4;
    const int n0 = blockIdx.x * 16 * R;
    const int nu = g.K / U::K;
    const int u_begin = wave * per;
    const int u_end = u_begin + per < nu ? u_begin + per : nu;

    const int64_t ldw = int64_t(g.K) * WBITS / 8;
    const uint8_t* wp[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        int row = n0 + 16 * r + (lane & 15);
        row = row < g.N ? row : g.N - 1;  // rows past N load a valid row; their outputs are not stored
        wp[r] = g.w + int64_t(row) * ldw + q * 16;
    }
    const int64_t lda = int64_t(g.K) * ABITS / 8;
    const uint8_t* ap[MT];
    bool tok_ok[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        const int tok = t * 16 + (lane & 15);
        tok_ok[t] = tok < g.M;
        ap[t] = g.act + int64_t(tok_ok[t] ? tok : 0) * lda + q * U::ALANE;
    }

    v4i acc[R][MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[r][t] = v4i{0, 0, 0, 0};

    for (int u0 = u_begin; u0 < u_end; u0 += C) {
        uint4 wv[C][R];
        ActReg av[C][MT];
#pragma unroll
        for (int c = 0; c < C; ++c) {
            if (u0 + c < u_end) {  // wave-uniform
#pragma unroll
                for (int r = 0; r < R; ++r)
                    wv[c][r] = *reinterpret_cast<const uint4*>(wp[r] + int64_t(u0 + c) * U::WROW);
#pragma unroll
                for (int t = 0; t < MT; ++t)
                    load_act<ABITS, WBITS>(av[c][t], ap[t] + int64_t(u0 + c) * U::AROW, tok_ok[t]);
            }
        }
#pragma unroll
        for (int c = 0; c < C; ++c) {
            if (u0 + c < u_end) {
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int t = 0; t < MT; ++t) acc[r][t] = unit_mfma<ABITS, WBITS>(wv[c][r], av[c][t], acc[r][t]);
            }
        }
    }

    // lane holds D[n = n0 + 16 r + 4 q + i][m = 16 t + lane % 16] of tile (r, t)
    constexpr int shift = AccShift<ABITS, WBITS>::value;
    if (S == 1) {  // block-uniform
        int mm[MT], nn[R];
#pragma unroll
        for (int t = 0; t < MT; ++t) mm[t] = t * 16 + (lane & 15);
#pragma unroll
        for (int r = 0; r < R; ++r) nn[r] = n0 + 16 * r + q * 4;
        store_tiles<R, MT>(acc, shift, mm, nn, g.M, g.N, g.act_scale, g.wscale, g.bias, g.residual, g.ldr, g.y, g.ldy,
                           g.acc, g.head_dim);
        return;
    }
    // tile i = (r, t) = (i / MT, i % MT): wave i sums the S partials of tile i and stores it
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t) red[wave][r * MT + t][lane] = acc[r][t];
    __syncthreads();
    if (wave >= kTiles) return;
    v4i sum[1][1] = {{red[0][wave][lane]}};
    for (int w = 1; w < S; ++w) sum[0][0] += red[w][wave][lane];
    const int mm[1] = {(wave % MT) * 16 + (lane & 15)};
    const int nn[1] = {n0 + 16 * (wave / MT) + q * 4};
    store_tiles<1, 1>(sum, shift, mm, nn, g.M, g.N, g.act_scale, g.wscale, g.bias, g.residual, g.ldr, g.y, g.ldy,
                      g.acc, g.head_dim);
}

// Waves per workgroup: enough that a wave's share fits one batch of C units,
// more while the layer has few workgroups and each wave keeps >= 4 units.
// At least R * MT waves so that every output tile has a wave to store it.
int split_waves(int nu, int groups, int C, int tiles) {
    int S = 1;
    while (S < kMaxWaves && (nu + S - 1) / S > C) S *= 2;
    while (S < kMaxWaves && int64_t(groups) * S < 4096 && (nu + 2 * S - 1) / (2 * S) >= 4) S *= 2;
    while (S < tiles && S > 1) S *= 2;
    return S;
}

template <int ABITS, int WBITS, int R, int MT, int C>
void launch_cfg(const GemmArgs& g, hipStream_t st) {
    const int nu = g.K / Unit<ABITS, WBITS>::K;
    const int groups = (g.N + 16 * R - 1) / (16 * R);
    const int S = split_waves(nu, groups, C, R * MT);
    const int per = (nu + S - 1) / S;
    hipLaunchKernelGGL((gemv_kernel<ABITS, WBITS, R, MT, C>), dim3(groups), dim3(64 * S), 0, st, g, per);
}

// Row groups per wave grow with M so that the activation re-reads stay a
// small fraction of the weight stream.
template <int ABITS, int WBITS>
void launch_bits(const GemmArgs& g, hipStream_t st) {
    if (g.M <= 4)
        launch_cfg<ABITS, WBITS, 1, 1, 16>(g, st);
    else if (g.M <= 16)
        launch_cfg<ABITS, WBITS, 2, 1, 8>(g, st);
    else
        launch_cfg<ABITS, WBITS, 2, 2, 8>(g, st);
}


// ---------------------------------------------------------------------------
// Persistent streaming GEMV: the decode path for 5 <= M <= 32 whenever the
// tokens' codes fit in LDS.
//
// The split-K kernel above reads each activation unit from L2 once per row
// group; from M = 8 on those reads cost more than they save (at M = 16 they
// are half as large as the weight stream itself).  Here each workgroup copies
// the M tokens' codes into LDS once and then walks the 16-row groups
// base, base + gridDim, ... (so that at any time the workgroups stream one
// contiguous band of the weights; contiguous ranges per workgroup measured
// 5 % slower; base is blockIdx permuted so that neighbouring groups share an
// XCD).  Seven waves split K: a wave streams its share of a group in
// chunks of CH 16-byte loads (8, or 4 with two token tiles, which need twice
// the activation registers) and keeps the next chunk (of the same or the
// next group) in flight while it consumes one, and it touches no other global
// memory, so nothing else waits behind its loads.  At the end of a group the
// seven partial tiles meet in LDS (double-buffered: one barrier per group)
// and the eighth wave runs the epilogue (scales, bias, residual, stores)
// while the others stream on.  A launch has as many workgroups as are
// resident at once, so the codes are copied a few hundred times in all.
constexpr int kStreamWaves = 8;  // waves per workgroup
constexpr int kLoadWaves = 7;    // waves that stream the weights; the last one stores
constexpr int kMaxLds = 160 * 1024;
constexpr int kStreamMinM = 5;   // below, the split-K kernel streams faster (its act reads are tiny)

// LDS row pitch of the codes: >= kb and 16 more than a multiple of 256, so the
// 16 token rows of a fragment start 4 banks apart.
__host__ __device__ inline int act_pitch(int kb) { return (kb + 239) / 256 * 256 + 16; }

// codes [16 MT][pitch] | partial tiles [2][7][MT][64] v4i | the tokens' scales [32]
__host__ __device__ inline size_t stream_lds_bytes(int mt, int pitch) {
    return size_t(16 * mt) * size_t(pitch) + size_t(2 * kLoadWaves * mt) * 64 * 16 + 128;
}


// grid: resident workgroups, each taking every gridDim-th of the `groups`
// 16-row groups; block: 8 waves (at most 128 VGPRs: two workgroups per CU
// when LDS allows).
template <int ABITS, int WBITS, int MT>
__global__ __launch_bounds__(64 * kStreamWaves) __attribute__((amdgpu_waves_per_eu(4))) void stream_kernel(
    GemmArgs g, int pitch, int groups) {
    using U = Unit<ABITS, WBITS>;
    constexpr int CH = MT == 1 ? 8 : 4;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint8_t* const act_lds = smem;
    v4i* const red = reinterpret_cast<v4i*>(smem + 16 * MT * pitch);
    float* const scale_lds = reinterpret_cast<float*>(smem + 16 * MT * pitch + 2 * kLoadWaves * MT * 64 * 16);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = lane >> 4;
    const bool loader = wave < kLoadWaves;
    const int nu = g.K / U::K;
    const int per = (nu + kLoadWaves - 1) / kLoadWaves;
    const int u_begin = loader && wave * per < nu ? wave * per : nu;
    const int u_end = u_begin + per < nu ? u_begin + per : nu;  // >= 1
    const int nb = (per + CH - 1) / CH;                 // chunks per group
    // group i of this workgroup is base + i gridDim (gridDim <= groups).  The
    // bases put four consecutive groups on one XCD (dispatch id b runs on XCD
    // b % 8): the 32-byte pieces that a group writes into each token's output
    // row then meet in that XCD's L2 as whole 128-byte lines instead of being
    // written back from four L2s (M = 8 / 16: 28.6 -> 27.7 / 29.8 -> 29.2 us).
    int base = int(blockIdx.x);
    if (gridDim.x % 32 == 0) {
        const int x = int(blockIdx.x) & 7, j = int(blockIdx.x) >> 3;
        base = 32 * (j >> 2) + 4 * x + (j & 3);  // a permutation of [0, gridDim)
    }
    const int gcount = (groups - base + int(gridDim.x) - 1) / int(gridDim.x);
    const int J = gcount * nb;
    auto group_of = [&](int i) { return base + i * int(gridDim.x); };
    const int64_t ldw = int64_t(g.K) * WBITS / 8;

    // chunk j = (group j / nb of this workgroup, units u_begin + CH (j % nb) + [0, CH));
    // units past the wave's share reload its last unit and are not used, so
    // every chunk is exactly CH loads
    auto issue = [&](uint4 (&w)[CH], int j) {
        const int jg = j / nb;
        const int b = j - jg * nb;
        int row = group_of(jg) * 16 + (lane & 15);
        row = row < g.N ? row : g.N - 1;  // rows past N load a valid row; their outputs are not stored
        const uint8_t* p = g.w + int64_t(row) * ldw + q * 16;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            int u = u_begin + b * CH + c;
            u = u < u_end ? u : u_end - 1;
            w[c] = *reinterpret_cast<const uint4*>(p + int64_t(u) * U::WROW);
        }
    };

    // chunk j lives in buffer j % 2; a step issues chunk j + 1 (the last chunk
    // again at the end: unused) and then consumes chunk j
    uint4 wa[CH], wb[CH];
    const int last = J - 1;
    if (loader && J > 0) issue(wa, 0);

    // the tokens' codes and scales into LDS; rows M .. 16 MT - 1 are zero.
    // A thread's pieces are requested kBatch at a time before any is written,
    // so the copy waits for one load latency per batch, not one per piece.
    {
        const float sc = tid < g.M ? g.act_scale[tid] : 0.0f;
        const int kb = g.K * ABITS / 8;
        const int pieces = kb >> 4;
        const int total = 16 * MT * pieces;
        constexpr int kBatch = 8;
        constexpr int kStride = 64 * kStreamWaves;
        for (int i0 = tid; i0 < total; i0 += kBatch * kStride) {
            uint4 v[kBatch];
#pragma unroll
            for (int b = 0; b < kBatch; ++b) {
                const int i = i0 + b * kStride;
                const int r = i / pieces;
                v[b] = make_uint4(0, 0, 0, 0);
                if (i < total && r < g.M)
                    v[b] = *reinterpret_cast<const uint4*>(g.act + int64_t(r) * kb + (i - r * pieces) * 16);
            }
#pragma unroll
            for (int b = 0; b < kBatch; ++b) {
                const int i = i0 + b * kStride;
                const int r = i / pieces;
                if (i < total) *reinterpret_cast<uint4*>(act_lds + r * pitch + (i - r * pieces) * 16) = v[b];
            }
        }
        if (tid < g.M) scale_lds[tid] = sc;
    }
    __syncthreads();

    constexpr int shift = AccShift<ABITS, WBITS>::value;
    if (!loader) {
        // the storing wave: one barrier per group, then the group's epilogue
        for (int i = 0, buf = 0; i < gcount; ++i, buf ^= 1) {
            const int gi = group_of(i);
            __syncthreads();
            const v4i* const rb = red + buf * (kLoadWaves * MT * 64);
            v4i sum[1][MT];
            int mm[MT];
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                sum[0][t] = rb[t * 64 + lane];
#pragma unroll
                for (int w = 1; w < kLoadWaves; ++w) sum[0][t] += rb[(w * MT + t) * 64 + lane];
                mm[t] = t * 16 + (lane & 15);
            }
            const int nn[1] = {gi * 16 + q * 4};
            store_tiles<1, MT>(sum, shift, mm, nn, g.M, g.N, scale_lds, g.wscale, g.bias, g.residual, g.ldr, g.y,
                               g.ldy, g.acc, g.head_dim);
        }
        return;
    }
    v4i acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = v4i{0, 0, 0, 0};
    int buf = 0;
    const uint8_t* const arow = act_lds + (lane & 15) * pitch + q * U::ALANE;
    auto step = [&](uint4 (&cur)[CH], uint4 (&nxt)[CH], int j) {
        issue(nxt, j + 1 < last ? j + 1 : last);
        const int b = j % nb;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int u = u_begin + b * CH + c;
            if (u < u_end) {  // wave-uniform
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    ActReg a;
                    lds_act<ABITS, WBITS>(a, arow + t * 16 * pitch + u * U::AROW);
                    acc[t] = unit_mfma<ABITS, WBITS>(cur[c], a, acc[t]);
                }
            }
        }
        if (b == nb - 1) {  // the group is done: partial tiles -> LDS for the storing wave
            v4i* const rb = red + buf * (kLoadWaves * MT * 64);
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                rb[(wave * MT + t) * 64 + lane] = acc[t];
                acc[t] = v4i{0, 0, 0, 0};
            }
            __syncthreads();
            buf ^= 1;
        }
    };
    for (int j = 0; j < J; j += 2) {
        step(wa, wb, j);
        if (j + 1 < J) step(wb, wa, j + 1);
    }
}

int stream_mt(int M) { return M <= 16 ? 1 : 2; }

bool stream_fits(const GemmArgs& g) {
    if (g.M < kStreamMinM || g.M > kGemvMaxM) return false;
    if (hooks().gemv_split.load(std::memory_order_relaxed)) return false;  // test hook gemv=split
    return stream_lds_bytes(stream_mt(g.M), act_pitch(g.K * g.abits / 8)) <= size_t(kMaxLds);
}

int mix_index(int abits, int wbits) { return abits == 8 ? (wbits == 8 ? 0 : 2) : (wbits == 4 ? 1 : 3); }

template <int ABITS, int WBITS, int MT>
hipError_t launch_stream_t(const GemmArgs& g, const DeviceInfo& dev, hipStream_t st) {
    const int pitch = act_pitch(g.K * ABITS / 8);
    const size_t lds = stream_lds_bytes(MT, pitch);
    // resident workgroups per CU: the register-limited count (from the device's
    // set-up) or what the CU's LDS holds, whichever is smaller.  The kernel is
    // correct for any grid; this only sizes it to one round of residents.
    int per_cu = dev.stream_regs_wg[mix_index(ABITS, WBITS)][MT - 1];
    const int by_lds = int(size_t(dev.lds_per_cu) / lds);
    per_cu = per_cu < by_lds ? per_cu : by_lds;
    per_cu = per_cu < 1 ? 1 : per_cu;
    const int groups = (g.N + 15) / 16;
    const int grid = groups < per_cu * dev.cus ? groups : per_cu * dev.cus;
    hipLaunchKernelGGL((stream_kernel<ABITS, WBITS, MT>), dim3(grid), dim3(64 * kStreamWaves), lds, st, g, pitch,
                       groups);
    return hipGetLastError();
}

template <int ABITS, int WBITS>
hipError_t launch_stream_bits(const GemmArgs& g, const DeviceInfo& dev, hipStream_t st) {
    return stream_mt(g.M) == 1 ? launch_stream_t<ABITS, WBITS, 1>(g, dev, st)
                               : launch_stream_t<ABITS, WBITS, 2>(g, dev, st);
}

hipError_t launch_stream(const GemmArgs& g, const DeviceInfo& dev, hipStream_t st) {
    if (g.abits == 8 && g.wbits == 8) return launch_stream_bits<8, 8>(g, dev, st);
    if (g.abits == 4 && g.wbits == 4) return launch_stream_bits<4, 4>(g, dev, st);
    if (g.abits == 8 && g.wbits == 4) return launch_stream_bits<8, 4>(g, dev, st);
    return launch_stream_bits<4, 8>(g, dev, st);
}

// The streaming kernels' part of a device's set-up: raise the dynamic-LDS
// limit and record the register-limited residency (dynamic LDS 0).
template <int ABITS, int WBITS, int MT>
hipError_t init_stream_kernel(DeviceInfo& d) {
    const void* kern = reinterpret_cast<const void*>(stream_kernel<ABITS, WBITS, MT>);
    hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
    if (e != hipSuccess) return e;
    int n = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, stream_kernel<ABITS, WBITS, MT>, 64 * kStreamWaves, 0);
    if (e != hipSuccess) return e;
    if (n < 1) return hipErrorInvalidValue;
    d.stream_regs_wg[mix_index(ABITS, WBITS)][MT - 1] = n;
    return hipSuccess;
}

template <int ABITS, int WBITS>
hipError_t init_stream_bits(DeviceInfo& d) {
    const hipError_t e = init_stream_kernel<ABITS, WBITS, 1>(d);
    return e != hipSuccess ? e : init_stream_kernel<ABITS, WBITS, 2>(d);
}

}  // namespace

hipError_t init_gemv_device(DeviceInfo& d) {
    hipError_t e = init_stream_bits<8, 8>(d);
    if (e == hipSuccess) e = init_stream_bits<4, 4>(d);
    if (e == hipSuccess) e = init_stream_bits<8, 4>(d);
    if (e == hipSuccess) e = init_stream_bits<4, 8>(d);
    return e;
}

hipError_t launch_gemv(const GemmArgs& g, const DeviceInfo& dev, hipStream_t stream) {
    if (g.M > kGemvMaxM) return hipErrorInvalidValue;
    if (stream_fits(g)) return launch_stream(g, dev, stream);
    if (g.abits == 8 && g.wbits == 8)
        launch_bits<8, 8>(g, stream);
    else if (g.abits == 4 && g.wbits == 4)
        launch_bits<4, 4>(g, stream);
    else if (g.abits == 8 && g.wbits == 4)
        launch_bits<8, 4>(g, stream);
    else
        launch_bits<4, 8>(g, stream);
    return hipGetLastError();
}

}  // namespace fq

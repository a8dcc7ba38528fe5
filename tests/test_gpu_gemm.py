"""GPU parity of fq_gemm (tiled MFMA kernel for M > 32, weight-streaming GEMV for
M <= 32) on identical codes: the int32 accumulators must equal the oracle's
bit for bit (the SYCL commit of the vla.cpp FoldQuant page: integer sums are
exact in any order), and each bf16 output must sit within the epilogue's
rounding bound of the oracle's float64 value."""
import numpy as np
import pytest

import oracle
from fqtest import assert_y_elementwise, dev, host, log, rand_codes

pytestmark = pytest.mark.gpu


def run_gemm(M, N, K, abits, wbits, seed, bias=False, residual=False, extreme=False, ldy=None, ldr=None):
    rng = np.random.default_rng(seed)
    ca = rand_codes(rng, M, K, abits, extreme)
    cw = rand_codes(rng, N, K, wbits, extreme)
    sa = rng.uniform(0.001, 0.05, M).astype(np.float32)
    sw = rng.uniform(0.0001, 0.002, N).astype(np.float32)
    b = (rng.standard_normal(N) * 0.1).astype(np.float32) if bias else None
    ldr = ldr or N
    res = None
    if residual:
        res = np.zeros((M, ldr), np.uint16)
        res[:, :N] = (rng.standard_normal((M, N)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    acc_ref = oracle.gemm_i32(ca, abits, cw, wbits, K)
    y_ref, yf = oracle.epilogue(acc_ref, sa, sw, b, None if res is None else res[:, :N], want_f64=True)
    ldy = ldy or N
    y = dev(np.zeros((M, ldy), np.uint16))
    acc = dev(np.zeros((M, N), np.int32))
    from w4a4_integer_gemm_amd import fq_gemm
    fq_gemm(dev(ca), dev(sa), M, abits, dev(cw), dev(sw), N, K, wbits, None if b is None else dev(b),
            None if res is None else dev(res), ldr, y, ldy, acc)
    yg = host(y, np.uint16)[:, :N]
    return host(acc), acc_ref, yg, yf, sa, sw, b, None if res is None else res[:, :N]


SHAPES = [
    # M, N, K  (M <= 32 takes the GEMV kernel)
    (1, 8, 128), (1, 520, 3584), (5, 136, 384), (16, 512, 256), (17, 264, 768), (32, 1000, 1024),
    (33, 8, 128), (33, 136, 384), (64, 128, 128), (100, 392, 768), (128, 256, 3584), (130, 520, 256),
    (300, 1000, 2048), (816, 264, 1024),
]

TILES = ["128x128", "128x144", "128x112", "128x96", "64x128", "64x224", "64x256", "64x288", "64x128x2"]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "M{}_N{}_K{}".format(*s))
@pytest.mark.parametrize("bits", [(8, 8), (4, 4), (8, 4), (4, 8)], ids=lambda b: "A{}W{}".format(*b))
def test_gemm_bit_exact_on_identical_codes(shape, bits):
    M, N, K = shape
    abits, wbits = bits
    log(f"gemm M={M} N={N} K={K} A{abits}W{wbits}")
    acc, acc_ref, yg, yf, sa, sw, b, res = run_gemm(M, N, K, abits, wbits, seed=M * 7 + N + K + abits,
                                                    bias=(M % 2 == 1), residual=(N % 16 == 8))
    assert np.array_equal(acc, acc_ref), f"{np.count_nonzero(acc != acc_ref)} accumulators differ"
    assert_y_elementwise(yg, yf, acc_ref, sa, sw, b, res, what=f"M{M} N{N} K{K}")


@pytest.mark.parametrize("M", [16, 256])
@pytest.mark.parametrize("bits", [(8, 8), (4, 4)], ids=lambda b: "A{}W{}".format(*b))
def test_gemm_extreme_codes_longest_row(M, bits):
    """Every code at +-qmax on K = 18944 (the largest accumulator of the workloads)."""
    log(f"gemm extreme codes M={M} bits={bits}")
    acc, acc_ref, yg, yf, sa, sw, b, res = run_gemm(M, 256, 18944, bits[0], bits[1], seed=5, extreme=True)
    assert np.array_equal(acc, acc_ref)
    assert_y_elementwise(yg, yf, acc_ref, sa, sw, what="extreme")


def test_gemm_strided_output_and_residual():
    log("gemm strided ldy/ldr")
    for M in (8, 200):
        acc, acc_ref, yg, yf, sa, sw, b, res = run_gemm(M, 136, 256, 8, 8, seed=9, residual=True, ldy=144, ldr=152)
        assert np.array_equal(acc, acc_ref)
        assert_y_elementwise(yg, yf, acc_ref, sa, sw, None, res, what=f"strided M={M}")


def _tile_case(tile, bits):
    # (97, 264, 1408): with a 4-bit operand, five full 256-deep stages and a
    # half-deep last one
    for M, N, K in ((300, 392, 768), (33, 1000, 1280), (97, 264, 1408)):
        acc, acc_ref, yg, yf, sa, sw, b, res = run_gemm(M, N, K, bits[0], bits[1], seed=M + N, bias=True,
                                                        residual=True)
        assert np.array_equal(acc, acc_ref), f"{tile}: {np.count_nonzero(acc != acc_ref)} accumulators differ"
        assert_y_elementwise(yg, yf, acc_ref, sa, sw, b, res, what=f"{tile} M{M} N{N} K{K}")


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("bits", [(8, 8), (4, 4), (8, 4), (4, 8)], ids=lambda b: "A{}W{}".format(*b))
def test_gemm_every_tile_shape(tile, bits, hook):
    """Each tile shape of the MFMA kernel (forced through the gemm_tile test hook)
    on ragged problems: M and N not multiples of the tile, several k stages, and
    a half-deep last stage for 4-bit operands."""
    hook(f"gemm_tile={tile}")
    log(f"gemm tile {tile} bits {bits}")
    _tile_case(tile, bits)


@pytest.mark.parametrize("tile", TILES)
def test_gemm_every_tile_shape_32x32x32_form(tile, hook):
    """8-bit x 8-bit codes take v_mfma_i32_16x16x64_i8 by default; the 32x32x32
    form (gemm_mfma=32 test hook) must give the same exact sums."""
    hook(f"gemm_tile={tile},gemm_mfma=32")
    log(f"gemm tile {tile} 32x32x32 form")
    _tile_case(tile, (8, 8))


@pytest.mark.parametrize("bits", [(8, 8), (4, 4)], ids=lambda b: "A{}W{}".format(*b))
def test_gemm_two_workgroups_per_cu_many_tiles(bits, hook):
    """The two-per-CU 64 x 128 tile on 2048 tiles (two workgroups share each
    CU, several waves of them): every int32 sum equals the 128 x 128 tile's
    (the sums do not depend on the tiling), and sampled token rows equal the
    oracle's exactly.  The samples include rows 32..63 of several tiles, whose
    partial sums pass between waves through LDS in the epilogue."""
    from w4a4_integer_gemm_amd import fq_gemm
    M, N, K = 1024, 8192, 1024
    abits, wbits = bits
    log(f"gemm two per CU M={M} N={N} K={K} A{abits}W{wbits}")
    rng = np.random.default_rng(11 + abits)
    ca, cw = rand_codes(rng, M, K, abits), rand_codes(rng, N, K, wbits)
    sa = rng.uniform(0.001, 0.05, M).astype(np.float32)
    sw = rng.uniform(0.0001, 0.002, N).astype(np.float32)
    d_ca, d_cw, d_sa, d_sw = dev(ca), dev(cw), dev(sa), dev(sw)
    out = {}
    for tile in ("64x128x2", "128x128"):
        hook(f"gemm_tile={tile}")
        y = dev(np.zeros((M, N), np.uint16))
        acc = dev(np.zeros((M, N), np.int32))
        fq_gemm(d_ca, d_sa, M, abits, d_cw, d_sw, N, K, wbits, None, None, N, y, N, acc)
        out[tile] = (host(acc), host(y, np.uint16))
    acc2, y2 = out["64x128x2"]
    assert np.array_equal(acc2, out["128x128"][0]), f"{np.count_nonzero(acc2 != out['128x128'][0])} sums differ"
    rows = sorted(set([0, M - 1] + [64 * t + r for t in (0, 7, 15) for r in (0, 32, 33, 35, 48, 51, 63)]
                      + rng.choice(M, 16, replace=False).tolist()))
    acc_ref = oracle.gemm_i32(ca[rows], abits, cw, wbits, K)
    assert np.array_equal(acc2[rows], acc_ref)
    _, yf = oracle.epilogue(acc_ref, sa[rows], sw, want_f64=True)
    assert_y_elementwise(y2[rows], yf, acc_ref, sa[rows], sw, what="two per CU")


GEMV_SHAPES = [
    # M, N, K: both GEMV kernels split K over the waves of a workgroup and walk
    # each wave's share in batches; these cover one and several batches, shares
    # that do not divide K evenly, a last wave with nothing to do, and M on both
    # sides of 16.  The streaming kernel (codes in LDS) takes 5 <= M <= 32 when
    # the codes fit; M <= 4, K = 18944 and 65536 (and K = 16384 at 8-bit codes)
    # stay on the split-K kernel either way.  N = 8200 .. 16400 gives a
    # streaming workgroup several row groups.
    (1, 24, 1408), (2, 40, 1152), (15, 8, 640), (16, 72, 2304), (17, 24, 896),
    (31, 16, 4608), (32, 8, 18944), (1, 3592, 3584), (16, 8, 65536), (3, 2056, 8192),
    (1, 16400, 256), (16, 8200, 2304), (32, 10248, 640), (5, 1032, 16384), (8, 16400, 3584),
]


@pytest.mark.parametrize("shape", GEMV_SHAPES, ids=lambda s: "M{}_N{}_K{}".format(*s))
@pytest.mark.parametrize("bits", [(8, 8), (4, 4), (8, 4), (4, 8)], ids=lambda b: "A{}W{}".format(*b))
@pytest.mark.parametrize("kernel", ["default", "split"])
def test_gemv_split_k_shapes(shape, bits, kernel, hook):
    """Decode-sized M through the default kernel choice and through the split-K
    kernel forced by the gemv=split test hook."""
    M, N, K = shape
    if kernel == "split":
        hook("gemv=split")
    log(f"gemv {kernel} M={M} N={N} K={K} A{bits[0]}W{bits[1]}")
    acc, acc_ref, yg, yf, sa, sw, b, res = run_gemm(M, N, K, bits[0], bits[1], seed=M + N + K, bias=True,
                                                    residual=(M % 2 == 0))
    assert np.array_equal(acc, acc_ref), f"{np.count_nonzero(acc != acc_ref)} accumulators differ"
    assert_y_elementwise(yg, yf, acc_ref, sa, sw, b, res, what=f"gemv M{M} N{N} K{K}")


@pytest.mark.parametrize("shape", [(1, 256, 512), (16, 384, 256), (17, 128, 1024), (33, 256, 384), (300, 1152, 768)],
                         ids=lambda s: "M{}_N{}_K{}".format(*s))
@pytest.mark.parametrize("bits", [(8, 8), (4, 4)], ids=lambda b: "A{}W{}".format(*b))
@pytest.mark.parametrize("head_dim", [8, 64, 128])
def test_gemm_heads_is_the_row_major_output_per_head(shape, bits, head_dim):
    """fq_gemm_heads writes exactly fq_gemm's outputs, each head's features as a
    dense [M][head_dim] block: y_heads[h][m][d] == y[m][h * head_dim + d]."""
    M, N, K = shape
    if N % head_dim:
        pytest.skip("N is not a whole number of heads")
    abits, wbits = bits
    log(f"gemm heads M={M} N={N} K={K} A{abits}W{wbits} head_dim={head_dim}")
    rng = np.random.default_rng(M + N + K + head_dim)
    ca, cw = rand_codes(rng, M, K, abits), rand_codes(rng, N, K, wbits)
    sa = rng.uniform(0.001, 0.05, M).astype(np.float32)
    sw = rng.uniform(0.0001, 0.002, N).astype(np.float32)
    b = (rng.standard_normal(N) * 0.1).astype(np.float32)
    res = (rng.standard_normal((M, N)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    from w4a4_integer_gemm_amd import fq_gemm, fq_gemm_heads
    args = (dev(ca), dev(sa), M, abits, dev(cw), dev(sw), N, K, wbits, dev(b), dev(res), N)
    y = dev(np.zeros((M, N), np.uint16))
    fq_gemm(*args, y, N, None)
    yh = dev(np.zeros((N // head_dim, M, head_dim), np.uint16))
    fq_gemm_heads(*args, head_dim, yh, None)
    ref = host(y, np.uint16)
    got = host(yh, np.uint16).transpose(1, 0, 2).reshape(M, N)
    assert np.array_equal(got, ref)


def test_linear_heads_on_the_qkv_shape():
    """fq_linear_heads on the fused QKV site (head_dim 128: 28 query, 4 key, 4 value heads)."""
    import synth
    from w4a4_integer_gemm_amd import DeviceSite
    wl = synth.make_workload("qkv_w8a8", M=64)
    site = DeviceSite(wl.W, wl.hblock, wl.wbits, wl.abits, gamma=wl.gamma, ascale=wl.ascale, eps=wl.eps)
    x = site.upload(wl.x)
    y = host(site.linear(x), np.uint16)
    yh = host(site.linear_heads(x, 128), np.uint16)
    assert np.array_equal(yh.transpose(1, 0, 2).reshape(wl.M, wl.N), y)

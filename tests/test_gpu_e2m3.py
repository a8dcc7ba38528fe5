"""GPU parity of the E2M3 storage of the 4-bit codes (code width 6): the prologue
writes the same codes as the 4-bit path in E2M3 form, and the FP6 GEMM
(v_mfma_scale_f32_16x16x128_f8f6f4, float32 sums of integer products) gives the
int32 accumulators of the oracle bit for bit (the SYCL commit of the vla.cpp
FoldQuant page: integer sums are exact in any order; every sum here stays below
2^24), so every output equals the 4-bit path's."""
import dataclasses

import numpy as np
import pytest

import oracle
import synth
import w4a4_integer_gemm_amd as fq
from fqtest import assert_codes, assert_y_elementwise, dev, host, log, rand_codes

pytestmark = pytest.mark.gpu
E2 = fq.E2M3


def run_gemm(M, N, K, seed, bias=False, residual=False, extreme=False):
    rng = np.random.default_rng(seed)
    if extreme:
        # +-7 with one sign per row (and 1 % of codes flipped): sums near +-49 K
        qa = np.where(rng.random((M, 1)) < 0.5, -7, 7) * np.ones((1, K), np.int64)
        qw = np.where(rng.random((N, 1)) < 0.5, -7, 7) * np.ones((1, K), np.int64)
        qa = np.where(rng.random((M, K)) < 0.01, -qa, qa)
        ca, cw = oracle.pack_e2m3(qa), oracle.pack_e2m3(qw)
    else:
        ca = rand_codes(rng, M, K, E2)
        cw = rand_codes(rng, N, K, E2)
    sa = rng.uniform(0.001, 0.05, M).astype(np.float32)
    sw = rng.uniform(0.0001, 0.002, N).astype(np.float32)
    b = (rng.standard_normal(N) * 0.1).astype(np.float32) if bias else None
    res = None
    if residual:
        res = (rng.standard_normal((M, N)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    acc_ref = oracle.gemm_i32(ca, E2, cw, E2, K)
    y_ref, yf = oracle.epilogue(acc_ref, sa, sw, b, res, want_f64=True)
    y = dev(np.zeros((M, N), np.uint16))
    acc = dev(np.zeros((M, N), np.int32))
    fq.fq_gemm(dev(ca), dev(sa), M, E2, dev(cw), dev(sw), N, K, E2, None if b is None else dev(b),
               None if res is None else dev(res), N, y, N, acc)
    return host(acc), acc_ref, host(y, np.uint16), yf, sa, sw, b, res


SHAPES = [  # M, N, K: one and several 128 x 128 tiles, ragged M and N, short and long K
    (1, 8, 128), (5, 136, 384), (32, 1000, 1024), (33, 8, 128), (64, 128, 128), (100, 392, 768),
    (128, 256, 3584), (130, 520, 256), (257, 264, 2048), (300, 1000, 2048), (816, 264, 1024),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "M{}_N{}_K{}".format(*s))
def test_e2m3_gemm_bit_exact(shape):
    M, N, K = shape
    log(f"e2m3 gemm M={M} N={N} K={K}")
    acc, acc_ref, yg, yf, sa, sw, b, res = run_gemm(M, N, K, seed=M + 3 * N + K, bias=M % 2 == 1,
                                                    residual=N % 16 == 8)
    assert np.array_equal(acc, acc_ref), f"{np.count_nonzero(acc != acc_ref)} accumulators differ"
    assert_y_elementwise(yg, yf, acc_ref, sa, sw, b, res, what=f"e2m3 M{M} N{N} K{K}")


@pytest.mark.parametrize("K", [18944, 65536])
def test_e2m3_gemm_extreme_codes(K):
    """Every code at +-7: the largest sums (49 K, below 2^24 even at K = 65536) stay exact."""
    log(f"e2m3 gemm extreme codes K={K}")
    acc, acc_ref, yg, yf, sa, sw, b, res = run_gemm(136, 264, K, seed=K, extreme=True)
    assert np.abs(acc_ref).max() > 0.9 * 49 * K
    assert np.array_equal(acc, acc_ref)
    assert_y_elementwise(yg, yf, acc_ref, sa, sw, what=f"e2m3 extreme K={K}")


PRO_CASES = [  # M, K, hblock, norm, amode, fold_after
    (3, 256, 64, True, "gain", 0), (40, 2048, 128, True, "gain", 0), (7, 3584, 128, False, "explicit", 1),
    (5, 16384, 128, False, "none", 0), (2, 18944, 256, True, "explicit", 0), (2, 65536, 128, True, "gain", 0),
]


@pytest.mark.parametrize("case", PRO_CASES, ids=lambda c: "M{}_K{}_b{}".format(*c[:3]))
def test_e2m3_prologue_matches_oracle_and_4bit_codes(case):
    M, K, b, norm, amode, fa = case
    log(f"e2m3 prologue {case}")
    wl = synth.random_workload(M, K, 8, b, 8, 4, seed=M + K, norm=norm, ascale=amode, fold_after=fa)
    gamma, a = wl.gamma, None
    if amode == "gain":
        gamma = oracle.fold_gain(wl.gamma, wl.ascale)
    elif amode == "explicit":
        a = wl.ascale
    ref6, rs6 = oracle.prologue(wl.x, gamma, wl.eps, a, fa, b, E2)
    out = {}
    for bits in (4, E2):
        codes = dev(np.zeros(fq.fq_act_bytes(M, K, bits), np.uint8))
        scale = dev(np.zeros(M, np.float32))
        fq.fq_prologue(dev(wl.x), M, K, K, None if gamma is None else dev(gamma), wl.eps,
                       None if a is None else dev(a), fa, b, bits, codes, scale)
        out[bits] = (host(codes).reshape(M, -1), host(scale))
    assert_codes(out[E2][0], out[E2][1], ref6, rs6, K, E2, what=f"e2m3 prologue {case}")
    # the same integers and scales as the 4-bit storage on this GPU
    assert np.array_equal(oracle.unpack_codes(out[E2][0], K, E2), oracle.unpack_codes(out[4][0], K, 4))
    assert np.array_equal(out[E2][1], out[4][1])


def _e2m3(wl):
    return dataclasses.replace(wl, wbits=E2, abits=E2)


def _site(wl):
    return fq.DeviceSite(wl.W, wl.hblock, wl.wbits, wl.abits, gamma=wl.gamma, ascale=wl.ascale,
                         fold_after=wl.fold_after, fold_into_gain=wl.fold_into_gain, bias=wl.bias, eps=wl.eps)


LINEAR_CASES = [  # M, K, N, hblock, norm, ascale, fold_after, bias, residual
    (16, 256, 512, 64, True, "gain", 0, False, False),
    (1, 1024, 264, 128, True, "gain", 0, True, False),
    (32, 1024, 520, 32, True, "explicit", 1, False, True),
    (33, 2048, 392, 128, False, "none", 0, True, True),
    (129, 1024, 1000, 256, False, "explicit", 1, True, True),
]


@pytest.mark.parametrize("case", LINEAR_CASES, ids=lambda c: "M{}_K{}_N{}_b{}".format(*c[:4]))
def test_e2m3_linear_equals_4bit_linear_and_oracle(case):
    M, K, N, b, norm, amode, fa, bias, resid = case
    log(f"e2m3 linear {case}")
    wl4 = synth.random_workload(M, K, N, b, 4, 4, seed=M + K + N, norm=norm, ascale=amode, fold_after=fa,
                                bias=bias, residual=resid)
    wl6 = _e2m3(wl4)
    x = dev(wl4.x)
    res = dev(wl4.residual) if wl4.residual is not None else None
    s4, s6 = _site(wl4), _site(wl6)
    y4 = host(s4.linear(x, residual=res), np.uint16)
    y6 = host(s6.linear(x, residual=res), np.uint16)
    assert np.array_equal(y4, y6), f"{np.count_nonzero(y4 != y6)} outputs differ from the 4-bit path"
    out = oracle.linear(wl6, codes_w=s6.codes_host, wscale=s6.wscale_host)
    c6, sc6 = s6.workspace_codes(M)
    assert_codes(host(c6).reshape(M, -1), host(sc6), out["codes_a"], out["act_scale"], K, E2, what=str(case))
    same = np.all(host(c6).reshape(M, -1) == out["codes_a"], axis=1)
    r = np.nonzero(same)[0]
    assert_y_elementwise(y6[r], out["y_f64"][r], out["acc"][r], out["act_scale"][r], out["wscale"], wl6.bias,
                         None if wl6.residual is None else wl6.residual[r], what=f"e2m3 linear {case}")


@pytest.mark.parametrize("name", ["gateup_w4a4", "down_w4a4"])
def test_e2m3_workload_full_size(name):
    """The Gemma W4A4 layers at full size in E2M3 form: every output equals the 4-bit
    path's, and sampled tokens match the oracle."""
    log(f"e2m3 workload {name}: building inputs")
    wl4 = synth.make_workload(name)
    wl6 = _e2m3(wl4)
    x = dev(wl4.x)
    res = dev(wl4.residual) if wl4.residual is not None else None
    s4, s6 = _site(wl4), _site(wl6)
    y4 = host(s4.linear(x, residual=res), np.uint16)
    y6 = host(s6.linear(x, residual=res), np.uint16)
    log(f"e2m3 workload {name}: M={wl4.M} K={wl4.K} N={wl4.N}")
    assert np.array_equal(y4, y6), f"{np.count_nonzero(y4 != y6)} outputs differ from the 4-bit path"
    rows = np.array([0, 1, 137, 400, wl4.M - 1])
    sub = dataclasses.replace(wl6, x=wl6.x[rows], M=len(rows),
                              residual=None if wl6.residual is None else wl6.residual[rows])
    out = oracle.linear(sub, codes_w=s6.codes_host, wscale=s6.wscale_host)
    c6, sc6 = s6.workspace_codes(wl4.M)
    gc = host(c6).reshape(wl4.M, -1)[rows]
    assert_codes(gc, host(sc6)[rows], out["codes_a"], out["act_scale"], wl4.K, E2, what=name)
    same = np.all(gc == out["codes_a"], axis=1)
    r = np.nonzero(same)[0]
    assert_y_elementwise(y6[rows][r], out["y_f64"][r], out["acc"][r], out["act_scale"][r], out["wscale"], wl6.bias,
                         None if wl6.residual is None else wl6.residual[rows][r], what=name)


def test_e2m3_heads_and_noalloc_match_row_major():
    log("e2m3 heads + noalloc")
    wl = _e2m3(synth.random_workload(70, 1024, 512, 128, 4, 4, seed=5, norm=True, ascale="gain"))
    s = _site(wl)
    x = dev(wl.x)
    y = host(s.linear(x), np.uint16)
    yh = host(s.linear_heads(x, 128), np.uint16)  # [N/128][M][128]
    assert np.array_equal(yh.transpose(1, 0, 2).reshape(wl.M, wl.N), y)
    yn = host(s.linear_noalloc(x), np.uint16)
    assert np.array_equal(yn, y)


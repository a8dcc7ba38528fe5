"""End-to-end GPU parity of fq_linear (prologue + GEMM/GEMV + epilogue) against
the oracle, on the option matrix of the vla.cpp FoldQuant page's SYCL test
(gamma, ascale before/after, bias, residual, narrowed and no rotation, the four
precisions) and on the five workloads at their full sizes (sampled tokens)."""
import numpy as np
import pytest

import oracle
import synth
import w4a4_integer_gemm_amd as fq
from fqtest import assert_codes, assert_y_elementwise, assert_y_fro, assert_y_within, dev, host, log

pytestmark = pytest.mark.gpu


def site_for(wl):
    return fq.DeviceSite(wl.W, wl.hblock, wl.wbits, wl.abits, gamma=wl.gamma, ascale=wl.ascale,
                         fold_after=wl.fold_after, fold_into_gain=wl.fold_into_gain, bias=wl.bias, eps=wl.eps)


def check_linear(wl, site, rows=None, what=""):
    """Run fq_linear on all M tokens; check the given token rows against the oracle."""
    M = wl.M
    x = dev(wl.x)
    res = dev(wl.residual) if wl.residual is not None else None
    y = site.linear(x, residual=res)
    codes_d, scales_d = site.workspace_codes(M)
    yg = host(y, np.uint16)
    gcodes = host(codes_d).reshape(M, -1)
    gscale = host(scales_d)
    rows = np.arange(M) if rows is None else np.asarray(rows)
    # oracle on the sampled tokens, with the product packer's codes (checked equal to
    # the oracle packer by the CPU tests)
    sub = synth.Workload(**{**wl.__dict__, "x": wl.x[rows], "M": len(rows),
                            "residual": None if wl.residual is None else wl.residual[rows]})
    out = oracle.linear(sub, codes_w=site.codes_host, wscale=site.wscale_host)
    frac = assert_codes(gcodes[rows], gscale[rows], out["codes_a"], out["act_scale"], wl.K, wl.abits, what=what)
    assert_y_fro(yg[rows], out["y_f64"], what=what)
    # tokens whose codes all agree must meet the element-wise epilogue bound
    same = np.all(gcodes[rows] == out["codes_a"], axis=1) & (gscale[rows] == out["act_scale"])
    if np.any(same):
        r = np.nonzero(same)[0]
        assert_y_elementwise(yg[rows][r], out["y_f64"][r], out["acc"][r], out["act_scale"][r], out["wscale"],
                             wl.bias, None if wl.residual is None else wl.residual[rows][r], what=what + " same-codes")
    return frac


OPTION_CASES = [
    # M, K, N, hblock, wbits, abits, norm, ascale, fold_after, bias, residual
    (16, 256, 512, 64, 8, 8, True, "gain", 0, False, False),
    (1, 512, 264, 128, 8, 8, True, "gain", 0, True, False),
    (32, 1024, 520, 32, 4, 4, True, "explicit", 1, False, True),
    (33, 2048, 392, 128, 4, 4, False, "none", 0, True, True),
    (300, 2048, 256, 1, 8, 8, True, "none", 0, False, False),      # no rotation
    (300, 6144, 136, 16, 4, 8, False, "explicit", 0, True, False),  # W4A8, narrowed block
    (70, 16384, 128, 128, 8, 4, True, "gain", 0, False, True),      # W8A4
    (129, 1024, 1000, 256, 8, 8, False, "explicit", 1, True, True),
]


@pytest.mark.parametrize("case", OPTION_CASES, ids=lambda c: "M{}_K{}_N{}_b{}_W{}A{}_{}".format(*c[:7]))
def test_linear_option_matrix(case):
    M, K, N, b, wb, ab, norm, amode, fa, bias, resid = case
    log(f"linear option case {case}")
    wl = synth.random_workload(M, K, N, b, wb, ab, seed=M + K + N, norm=norm, ascale=amode, fold_after=fa,
                               bias=bias, residual=resid)
    check_linear(wl, site_for(wl), what=str(case))


def test_linear_tiny_workload_full():
    wl = synth.make_workload("tiny_w8a8")
    log("linear tiny_w8a8 (16x256x512)")
    check_linear(wl, site_for(wl), what="tiny_w8a8")


@pytest.mark.parametrize("name", ["qkv_w8a8", "down_w8a8", "decode_m1_w8a8", "decode_m16_w8a8", "gateup_w4a4",
                                  "down_w4a4"])
def test_linear_workload_full_size_sampled(name):
    """Full-size workload through fq_linear in the benchmark's launch configuration;
    the oracle recomputes a sample of tokens (all output features of each)."""
    log(f"linear workload {name}: building inputs")
    wl = synth.make_workload(name)
    site = site_for(wl)
    rng = np.random.default_rng(1)
    rows = np.unique(np.concatenate([[0, wl.M - 1], rng.choice(wl.M, size=min(wl.M, 24), replace=False)]))
    log(f"linear workload {name}: M={wl.M} K={wl.K} N={wl.N} rows checked {len(rows)}")
    check_linear(wl, site, rows=rows, what=name)


@pytest.mark.parametrize("name,max_rel", [("qkv_w8a8", 0.03), ("gateup_w4a4", 0.35)])
def test_dequant_float_path_agrees_with_integer_path(name, max_rel):
    """The page's dequant mode: a float GEMM with the rows fq_dequant_rows
    rebuilds (the smoothing vector stays in the folded norm gain).

    Exact check: the GPU's own activation codes, dequantised and rotated back
    to the original frame (x_deq = R(s_a q_a); R is its own inverse), times
    the dequantised rows give the integer path's result up to float64
    rounding, because R(s_a q_a) . R(s_w q_w) = (s_a q_a) . (s_w q_w): every
    GPU output must be that value rounded to bf16 (half a bf16 ulp plus the
    epilogue's float32 rounding).  Informational: the float layer on the
    unquantised activations differs by the activations' quantisation only
    (8-bit: ~1 %, 4-bit: 15 levels), reported and bounded by max_rel."""
    wl = synth.make_workload(name, M=64, N=512)
    site = site_for(wl)
    y = host(site.linear(dev(wl.x)), np.uint16)
    codes_d, scales_d = site.workspace_codes(wl.M)
    qa = oracle.unpack_codes(host(codes_d).reshape(wl.M, -1), wl.K, wl.abits).astype(np.float64)
    sa = host(scales_d).astype(np.float64)
    W_deq = fq.fq_dequant_rows(site.codes_host, site.wscale_host, wl.K, None, 0, wl.hblock, wl.wbits)
    x_deq = np.stack([oracle.rotate_f64(sa[m] * qa[m], wl.hblock) for m in range(wl.M)])
    y_exact = x_deq @ W_deq.astype(np.float64).T
    acc = (qa @ oracle.unpack_codes(site.codes_host, wl.K, wl.wbits).astype(np.float64).T)
    # bound: the epilogue's float32 rounding of acc s_a s_w, plus the float32
    # rounding of the dequantised rows (2^-24 of sum |x_deq| |W_deq|, written
    # as a quarter of that sum on the 2^-21 scale of assert_y_within)
    w_round = (np.abs(x_deq) @ np.abs(W_deq.astype(np.float64)).T) * 0.25
    assert_y_within(y, y_exact, np.abs(acc * sa[:, None] * site.wscale_host.astype(np.float64)[None, :]) + w_round,
                    what=f"{name} dequant rows x dequantised codes")
    y_int = synth.bf16_bits_to_f32(y).astype(np.float64)
    gamma_f = oracle.fold_gain(wl.gamma, wl.ascale).astype(np.float64)
    x = synth.bf16_bits_to_f32(wl.x).astype(np.float64)
    xn = x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + wl.eps) * gamma_f
    y_float = xn @ W_deq.astype(np.float64).T
    rel = np.linalg.norm(y_int - y_float) / np.linalg.norm(y_float)
    cos = float(np.sum(y_int * y_float) / (np.linalg.norm(y_int) * np.linalg.norm(y_float)))
    log(f"dequant vs integer {name}: rel {rel:.3e} cosine {cos:.6f} (unquantised activations, informational)")
    assert rel <= max_rel and cos >= 1 - max_rel ** 2


def test_decode_with_changing_token_counts():
    """One site (one workspace) serving decode calls with different M, as a
    serving loop would: both GEMV kernels (split-K below 5 tokens, streaming
    above) against the oracle on every token."""
    wl = synth.random_workload(32, 1024, 1032, 64, 8, 8, seed=5, norm=True, ascale="gain")
    site = site_for(wl)
    site.workspace(32)
    for M in (32, 1, 16, 3, 32, 1, 17, 5):
        sub = synth.Workload(**{**wl.__dict__, "x": wl.x[:M], "M": M})
        check_linear(sub, site, what=f"M={M}")

"""GPU parity of fq_prologue against the oracle (RMSNorm with the folded gain,
smoothing divide, block Hadamard, per-token quantisation: the act node of the
vla.cpp FoldQuant page).  Codes may differ by 1 LSB on at most 0.1 % of
elements (a rounding tie under a different float reduction order, as the page's
OpenVINO commit notes); scales within 1e-5 relative."""
import numpy as np
import pytest

import oracle
import synth
import w4a4_integer_gemm_amd as fq
from fqtest import assert_codes, dev, host, log

pytestmark = pytest.mark.gpu

CASES = [
    # M, K, hblock, abits, norm, ascale mode, fold_after.  Values per lane: 8 for
    # M <= 32, K <= 2048 and hblock <= 128 (a 128-block spans 16 lanes), else 16
    # for K <= 8192 (a 256-block then spans 16 lanes: the xor-8 exchange), 32 up
    # to K = 32768, 64 beyond
    (1, 64, 1, 8, False, "none", 0),
    (4, 2016, 8, 8, True, "gain", 0),       # 8 values per lane, 252 lanes (last wave ragged)
    (32, 1024, 128, 8, True, "explicit", 1),  # the last token count with 8 values per lane
    (3, 64, 64, 4, True, "gain", 0),
    (16, 256, 64, 8, True, "gain", 0),
    (7, 256, 2, 8, True, "explicit", 0),
    (7, 256, 4, 4, False, "explicit", 1),
    (33, 512, 8, 8, True, "explicit", 1),
    (5, 512, 16, 4, True, "none", 0),
    (9, 1024, 32, 8, False, "explicit", 0),
    (2, 2048, 256, 8, True, "gain", 0),
    (17, 2048, 128, 4, True, "gain", 0),
    (64, 3584, 128, 8, True, "gain", 0),
    (8, 3584, 128, 4, False, "explicit", 1),
    (4, 8192, 128, 8, True, "none", 0),
    (3, 8160, 32, 8, True, "gain", 0),      # 16 values per lane, 510 lanes (last wave ragged)
    (5, 7936, 256, 4, True, "gain", 0),     # 16 per lane, 256-blocks over 16 lanes
    (3, 8256, 64, 8, True, "gain", 0),      # 32 values per lane, 258 lanes
    (3, 8224, 32, 4, True, "none", 0),      # 32 values per lane, 257 lanes
    (2, 32768, 256, 8, False, "explicit", 1),
    (6, 16384, 128, 4, False, "none", 0),
    (5, 18944, 128, 8, False, "none", 0),
    (2, 18944, 256, 4, True, "explicit", 0),
    (2, 65536, 128, 8, True, "gain", 0),    # the largest K the ABI takes (1024 lanes of 64)
]


def run_case(M, K, b, abits, norm, amode, fold_after, seed=0, x_scale=1.0, ldx=None):
    wl = synth.random_workload(M, K, 8, b, 8, abits, seed=seed + K + M, norm=norm,
                               ascale=("gain" if amode == "gain" else ("explicit" if amode == "explicit" else "none")),
                               fold_after=fold_after, x_scale=x_scale)
    gamma, a = wl.gamma, None
    if amode == "gain":
        gamma = oracle.fold_gain(wl.gamma, wl.ascale)
    elif amode == "explicit":
        a = wl.ascale
    ref_codes, ref_scale = oracle.prologue(wl.x, gamma, wl.eps, a, fold_after, b, abits)
    x = wl.x
    if ldx is not None:
        xp = np.zeros((M, ldx), np.uint16)
        xp[:, :K] = x
        x = xp
    xd = dev(x)
    codes = dev(np.zeros(fq.fq_act_bytes(M, K, abits), np.uint8))
    scale = dev(np.zeros(M, np.float32))
    fq.fq_prologue(xd, M, K, x.shape[1], None if gamma is None else dev(gamma), wl.eps,
                   None if a is None else dev(a), fold_after, b, abits, codes, scale)
    return host(codes).reshape(ref_codes.shape), host(scale), ref_codes, ref_scale


@pytest.mark.parametrize("case", CASES, ids=lambda c: "M{}_K{}_b{}_a{}_{}_{}_{}".format(
    c[0], c[1], c[2], c[3], "norm" if c[4] else "nonorm", c[5], "after" if c[6] else "before"))
def test_prologue_matches_oracle(case):
    log(f"prologue case {case}")
    M, K, b, abits = case[:4]
    gc, gs, rc, rs = run_case(*case)
    assert_codes(gc, gs, rc, rs, K, abits, what=str(case))


def test_prologue_strided_rows():
    log("prologue strided ldx")
    gc, gs, rc, rs = run_case(6, 512, 64, 8, True, "gain", 0, ldx=520)
    assert_codes(gc, gs, rc, rs, 512, 8, what="ldx=520")


@pytest.mark.parametrize("abits", [8, 4])
def test_prologue_degenerate_tokens(abits):
    """All-zero token (scale 0, codes 0), a constant token, a single spike, huge and tiny magnitudes."""
    log(f"prologue degenerate tokens abits={abits}")
    K, b = 512, 128
    x = np.zeros((6, K), np.float32)
    x[1] = 3.0
    x[2, 77] = -5.0
    x[3] = np.linspace(-1e30, 1e30, K)
    x[4] = np.linspace(-1e-30, 2e-30, K)
    x[5, ::3] = 1.0
    xb = synth.f32_to_bf16_bits(x)
    for gamma in (None, np.ones(K, np.float32)):
        ref_codes, ref_scale = oracle.prologue(xb, gamma, 1e-6, None, 0, b, abits)
        codes = dev(np.zeros(fq.fq_act_bytes(6, K, abits), np.uint8))
        scale = dev(np.zeros(6, np.float32))
        fq.fq_prologue(dev(xb), 6, K, K, None if gamma is None else dev(gamma), 1e-6, None, 0, b, abits, codes, scale)
        gc, gs = host(codes).reshape(ref_codes.shape), host(scale)
        assert gs[0] == 0 and np.all(gc[0] == 0)
        assert_codes(gc, gs, ref_codes, ref_scale, K, abits, what=f"degenerate gamma={gamma is not None}")


def test_prologue_on_workload_tokens():
    """The five workloads' own activation recipes (sampled tokens)."""
    for name in ("tiny_w8a8", "qkv_w8a8", "down_w8a8", "gateup_w4a4", "down_w4a4"):
        log(f"prologue workload {name}")
        wl = synth.make_workload(name, M=64, N=8)
        gamma = oracle.fold_gain(wl.gamma, wl.ascale) if wl.gamma is not None else None
        ref_codes, ref_scale = oracle.prologue(wl.x, gamma, wl.eps, None, 0, wl.hblock, wl.abits)
        codes = dev(np.zeros(fq.fq_act_bytes(wl.M, wl.K, wl.abits), np.uint8))
        scale = dev(np.zeros(wl.M, np.float32))
        fq.fq_prologue(dev(wl.x), wl.M, wl.K, wl.K, None if gamma is None else dev(gamma), wl.eps, None, 0,
                       wl.hblock, wl.abits, codes, scale)
        assert_codes(host(codes).reshape(ref_codes.shape), host(scale), ref_codes, ref_scale, wl.K, wl.abits,
                     what=name)

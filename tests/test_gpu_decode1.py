"""One-token fq_linear in one launch (fq_decode1.hip): every workgroup
quantises the token itself while its weight loads are in flight.  Its codes,
scale and outputs must be those of the two-launch path (prologue, then the
split-K GEMV) bit for bit, and meet the oracle: the SYCL commit of the vla.cpp
FoldQuant page switches to a GEMV for decode-sized M, and the codes follow its
OpenVINO commit's act steps.  Covers the four bit mixes, RMSNorm on and off,
the three smoothing modes, the three Hadamard blocks it takes, K from 128 to
4096 (one to eight units per wave, the last unit repeated), ragged N, bias,
residual and the head layout."""
import numpy as np
import pytest
import torch

import oracle
import synth
import w4a4_integer_gemm_amd as fq
from fqtest import assert_codes, assert_y_elementwise, assert_y_fro, dev, host, log

pytestmark = pytest.mark.gpu


def site_for(wl):
    return fq.DeviceSite(wl.W, wl.hblock, wl.wbits, wl.abits, gamma=wl.gamma, ascale=wl.ascale,
                         fold_after=wl.fold_after, fold_into_gain=wl.fold_into_gain, bias=wl.bias, eps=wl.eps)


CASES = [
    # K, N, hblock, wbits, abits, norm, ascale, fold_after, bias, residual
    (3584, 1032, 128, 8, 8, True, "gain", 0, False, False),
    (4096, 264, 128, 8, 8, True, "gain", 0, True, True),
    (128, 40, 32, 8, 8, True, "gain", 0, False, False),
    (512, 520, 64, 4, 4, True, "gain", 0, True, False),
    (2048, 392, 128, 4, 4, False, "none", 0, False, True),
    (1024, 136, 64, 8, 4, True, "explicit", 1, True, False),
    (3072, 256, 32, 4, 8, False, "explicit", 0, False, False),
    (2304, 1000, 128, 8, 8, True, "explicit", 1, True, True),
    (640, 24, 128, 4, 4, True, "gain", 0, False, False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "K{}_N{}_b{}_W{}A{}_{}_{}".format(*c[:5], "norm" if c[5] else
                                                                                         "nonorm", c[6]))
def test_decode1_equals_two_launches_and_oracle(case, hook):
    K, N, b, wb, ab, norm, amode, fa, bias, resid = case
    log(f"decode1 K={K} N={N} b={b} W{wb}A{ab} norm={norm} ascale={amode} fold_after={fa}")
    wl = synth.random_workload(1, K, N, b, wb, ab, seed=K + N + b + wb, norm=norm, ascale=amode, fold_after=fa,
                               bias=bias, residual=resid)
    site = site_for(wl)
    x = dev(wl.x)
    res = dev(wl.residual) if wl.residual is not None else None
    out = {}
    for mode in ("auto", "off"):
        hook(f"decode1={mode}")
        ws = site.workspace(1)
        ws.fill_(0xA5)
        y = site.linear(x, residual=res)
        c, s = site.workspace_codes(1)
        torch.cuda.synchronize()
        out[mode] = (host(y, np.uint16), host(c).copy(), host(s).copy())
    for a, b_, what in zip(out["auto"], out["off"], ("outputs", "codes", "scale")):
        assert np.array_equal(a, b_), f"one launch and two launches differ in the {what}"
    ref = oracle.linear(wl, codes_w=site.codes_host, wscale=site.wscale_host)
    y, codes, scale = out["auto"]
    assert_codes(codes.reshape(1, -1), scale, ref["codes_a"], ref["act_scale"], K, ab, what="decode1")
    assert_y_fro(y, ref["y_f64"], what="decode1")
    if np.array_equal(codes.reshape(1, -1), ref["codes_a"]):
        assert_y_elementwise(y, ref["y_f64"], ref["acc"], ref["act_scale"], ref["wscale"], wl.bias,
                             wl.residual, what="decode1 same codes")


def test_decode1_heads_layout(hook):
    """fq_linear_heads with one token takes the same kernel; y[h][0][d] against the oracle."""
    wl = synth.make_workload("qkv_w8a8", M=1)
    site = site_for(wl)
    x = site.upload(wl.x)
    yh = host(site.linear_heads(x, 128), np.uint16)
    hook("decode1=off")
    yh2 = host(site.linear_heads(x, 128), np.uint16)
    assert np.array_equal(yh, yh2)
    ref = oracle.linear(wl, codes_w=site.codes_host, wscale=site.wscale_host)
    assert_y_fro(yh.transpose(1, 0, 2).reshape(1, wl.N), ref["y_f64"], what="decode1 heads")


def test_decode1_repeated_calls_and_other_sizes():
    """A serving loop on one site: one-token calls between calls with more
    tokens (which take the two-launch path); each against the oracle."""
    wl = synth.random_workload(8, 3584, 2056, 128, 8, 8, seed=3, norm=True, ascale="gain")
    site = site_for(wl)
    for M in (1, 8, 1, 3, 1):
        sub = synth.Workload(**{**wl.__dict__, "x": wl.x[:M], "M": M})
        y = host(site.linear(dev(sub.x)), np.uint16)
        c, s = site.workspace_codes(M)
        ref = oracle.linear(sub, codes_w=site.codes_host, wscale=site.wscale_host)
        assert_codes(host(c).reshape(M, -1), host(s), ref["codes_a"], ref["act_scale"], wl.K, wl.abits,
                     what=f"M={M}")
        assert_y_fro(y, ref["y_f64"], what=f"M={M}")

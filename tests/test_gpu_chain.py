"""Chained MLP block on the GPU: gate+up site -> GeGLU -> down site with the
residual (the Gemma-style MLP of the pi0.5 backbone that the vla.cpp FoldQuant
page runs W4A4, also with INT8 o/down sites), with the node-by-node CPU
recompute diagnostic of that page's CUDA path: after each GPU node the oracle
recomputes the node from host copies of that node's own GPU inputs, and the
byte differences are reported.  Every node must meet the parity bar on its
own inputs, so a mismatch is pinned to the node that made it."""
import numpy as np
import pytest

import oracle
import synth
import w4a4_integer_gemm_amd as fq
from fqtest import assert_codes, assert_y_fro, bf16_half_ulp, bf16_to_f64, dev, host, log

pytestmark = pytest.mark.gpu


def site_for(wl):
    return fq.DeviceSite(wl.W, wl.hblock, wl.wbits, wl.abits, gamma=wl.gamma, ascale=wl.ascale,
                         fold_after=wl.fold_after, fold_into_gain=wl.fold_into_gain, bias=wl.bias, eps=wl.eps)


def diag_linear(name, wl, site, y_gpu, rows):
    """Recompute a linear node with the oracle from its own inputs; report and check."""
    codes_d, scales_d = site.workspace_codes(wl.M)
    gcodes = host(codes_d).reshape(wl.M, -1)[rows]
    gscale = host(scales_d)[rows]
    sub = synth.Workload(**{**wl.__dict__, "x": wl.x[rows], "M": len(rows),
                            "residual": None if wl.residual is None else wl.residual[rows]})
    out = oracle.linear(sub, codes_w=site.codes_host, wscale=site.wscale_host)
    yg = host(y_gpu, np.uint16)[rows]
    nbytes = int(np.count_nonzero(yg != out["y"]))
    log(f"  node {name}: {len(rows)} tokens recomputed; codes differing "
        f"{int(np.count_nonzero(gcodes != out['codes_a']))}/{gcodes.size} bytes, "
        f"outputs differing {nbytes}/{yg.size} bf16")
    assert_codes(gcodes, gscale, out["codes_a"], out["act_scale"], wl.K, wl.abits, what=name)
    assert_y_fro(yg, out["y_f64"], what=name)


def diag_geglu(gu_bits, F, h_gpu_bits):
    """Recompute GeGLU from the GPU's own gate+up output: each bf16 value within half
    a bf16 ulp of the float64 value plus the float32 evaluation error."""
    h_ora, hf = oracle.geglu(gu_bits, F, want_f64=True)
    nb = int(np.count_nonzero(h_gpu_bits != h_ora))
    log(f"  node geglu: outputs differing {nb}/{h_ora.size} bf16")
    g = bf16_to_f64(gu_bits[:, :F])
    u = bf16_to_f64(gu_bits[:, F:])
    # float32 evaluation: a few float32 roundings of |g| |u| (tanh from the device library)
    bound = bf16_half_ulp(hf) * (1 + 1e-6) + np.abs(g * u) * 2.0 ** -20 + 1e-38
    err = np.abs(bf16_to_f64(h_gpu_bits) - hf)
    assert np.all(err <= bound), f"geglu: worst excess {np.max(err - bound):.3e}"
    assert nb <= max(1, h_ora.size // 1000), f"geglu: {nb} outputs differ from the oracle's rounding"


def run_chain(M, K, F, hb, up_bits, down_bits, seed, rows=None):
    wa, aa = up_bits
    wd, ad = down_bits
    up = synth.random_workload(M, K, 2 * F, hb, wa, aa, seed=seed, norm=True, ascale="gain", outliers=8)
    site_up = site_for(up)
    x = dev(up.x)
    y1 = site_up.linear(x)
    rows = np.arange(M) if rows is None else rows
    log(f"chain M={M} K={K} F={F} b={hb} gate+up W{wa}A{aa}, down W{wd}A{ad}")
    diag_linear("gate+up", up, site_up, y1, rows)

    h = dev(np.zeros((M, F), np.uint16))
    fq.fq_geglu(y1, M, F, 2 * F, h, F)
    y1_host = host(y1, np.uint16)
    diag_geglu(y1_host, F, host(h, np.uint16))

    down = synth.random_workload(M, F, K, hb, wd, ad, seed=seed + 1, norm=False, ascale="none")
    down.x = host(h, np.uint16)          # the node's own GPU input
    down.residual = up.x                 # the block's skip connection
    site_down = site_for(down)
    y2 = site_down.linear(h, residual=x)
    diag_linear("down+residual", down, site_down, y2, rows)
    return host(y2, np.uint16)


@pytest.mark.parametrize("up_bits,down_bits", [((4, 4), (4, 4)), ((4, 4), (8, 8)), ((8, 8), (8, 8))],
                         ids=["W4A4", "W4A4_down_INT8", "W8A8"])
def test_chained_mlp_node_by_node(up_bits, down_bits):
    run_chain(48, 1024, 2048, 128, up_bits, down_bits, seed=7)


def test_chained_mlp_decode_sizes():
    """M <= 32 takes the GEMV kernel in both sites."""
    run_chain(5, 2048, 4096, 128, (4, 4), (4, 4), seed=9)


def test_chained_mlp_gemma_shapes_sampled():
    """The Gemma-2B-shaped block at the W4A4 workload size (816 tokens, K=2048,
    F=16384); the linear nodes are recomputed on 16 sampled tokens, GeGLU in full."""
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([[0, 815], rng.choice(816, 14, replace=False)]))
    run_chain(816, 2048, 16384, 128, (4, 4), (4, 4), seed=5, rows=rows)

"""Packer and prologue must agree on the fold: the smoothing vector, the fold
order and the Hadamard block.

The TensorRT-Edge-LLM pull-request page (NVFP4LinearMethod paragraph) shows a
dropped per-channel smoothing vector giving not a degraded layer but a wrong
one; the vla.cpp FoldQuant page's dequant-mode commit gives the two fold
orders, R(x/a) and R(x)/a.  Each case below packs the weights with one
setting and quantises the activations with another, and checks that the
layer's output is then far from the float layer (relative error and cosine
recorded), while the matched settings stay within the parity tolerance.  The
CPU test shows it on the oracle alone; the GPU test shows that libfq computes
exactly what the oracle computes for the same mismatched settings, so that
such a mistake is visible in the output rather than hidden by the kernels."""
import numpy as np
import pytest

import oracle
import synth
from fqtest import dev, host, log

# A matched layer differs from the float layer only by its quantisation: about
# 5e-3 on these workloads with the smoothing vector in the gain (within the
# 1e-2 parity tolerance), 2e-2 to 1e-1 with the same vector applied after the
# rotation (it was chosen to even out channels before the rotation mixes
# them).  Every mismatch is at least WRONG_REL away (0.79 and more measured).
MATCHED_REL = {"gain": 1e-2, "after": 0.15}
WRONG_REL = 0.3


def float_layer(wl):
    """RMSNorm(x) gamma W^T in float64, no quantisation: the layer the fold must preserve."""
    x = synth.bf16_bits_to_f32(wl.x).astype(np.float64)
    xn = x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + wl.eps) * wl.gamma.astype(np.float64)
    return xn @ wl.W.astype(np.float64).T


def cases(wl):
    """(name, packer settings (ascale, fold_after, hblock), prologue settings
    (gain, explicit ascale, fold_after, hblock), the matched kind or None)."""
    b, a, g = wl.hblock, wl.ascale, wl.gamma
    gf = oracle.fold_gain(g, a)
    return [
        ("matched, a in the gain", (a, 0, b), (gf, None, 0, b), "gain"),
        ("matched, explicit a after the rotation", (a, 1, b), (g, a, 1, b), "after"),
        ("a dropped from the gain", (a, 0, b), (g, None, 0, b), None),
        ("a dropped from the packer", (None, 0, b), (gf, None, 0, b), None),
        ("fold order flipped: packed after, prologue before", (a, 1, b), (g, a, 0, b), None),
        ("fold order flipped: packed before, prologue after", (a, 0, b), (g, a, 1, b), None),
        ("Hadamard block b/2 in the packer, b in the prologue", (a, 0, b // 2), (gf, None, 0, b), None),
    ]


def oracle_y(wl, pack, pro):
    cw, ws = oracle.pack_weights(wl.W, pack[0], pack[1], pack[2], wl.wbits)
    ca, sa = oracle.prologue(wl.x, pro[0], wl.eps, pro[1], pro[2], pro[3], wl.abits)
    acc = oracle.gemm_i32(ca, wl.abits, cw, wl.wbits, wl.K)
    _, yf = oracle.epilogue(acc, sa, ws, want_f64=True)
    return cw, ws, ca, sa, yf


def rel_cos(y, ref):
    rel = float(np.linalg.norm(y - ref) / np.linalg.norm(ref))
    cos = float(np.sum(y * ref) / (np.linalg.norm(y) * np.linalg.norm(ref)))
    return rel, cos


WORKLOADS = [("tiny_w8a8", None), ("qkv_w8a8", 48)]


@pytest.mark.parametrize("name,M", WORKLOADS)
def test_mismatched_fold_is_a_wrong_layer_oracle(name, M):
    wl = synth.make_workload(name, M=M)
    ref = float_layer(wl)
    for what, pack, pro, matched in cases(wl):
        rel, cos = rel_cos(oracle_y(wl, pack, pro)[4], ref)
        log(f"{name} {what}: rel {rel:.3e} cosine {cos:.4f}")
        if matched:
            assert rel <= MATCHED_REL[matched], f"{what}: {rel:.3e}"
        else:
            assert rel >= WRONG_REL, f"{what}: a mismatched fold gave rel {rel:.3e}, too close to the layer"


@pytest.mark.gpu
@pytest.mark.parametrize("name,M", WORKLOADS + [("qkv_w8a8", 1024)])
def test_mismatched_fold_gpu_matches_oracle(name, M):
    """libfq with the same mismatched settings: codes as the oracle's, output as
    the oracle's (rel Frobenius 1e-2), hence as far from the float layer."""
    import w4a4_integer_gemm_amd as fq
    wl = synth.make_workload(name, M=M)
    rows = np.unique(np.linspace(0, wl.M - 1, num=min(wl.M, 24)).astype(int))
    sub = synth.Workload(**{**wl.__dict__, "x": wl.x[rows], "M": len(rows)})
    ref = float_layer(sub)
    x = dev(wl.x)
    for what, pack, pro, matched in cases(wl):
        codes, ws = fq.fq_pack_weights(wl.W, pack[0], pack[1], pack[2], wl.wbits)
        cw, wso, ca, sa, yf = oracle_y(sub, pack, pro)
        assert np.array_equal(codes, cw) and np.array_equal(ws, wso), f"{what}: packer differs from the oracle's"
        gain, a_explicit, fold_after, hb = pro
        site = fq.DeviceSite(None, hb, wl.wbits, wl.abits, gamma=gain, ascale=a_explicit, fold_after=fold_after,
                             fold_into_gain=False, eps=wl.eps, codes=codes, wscale=ws)
        y = host(site.linear(x), np.uint16)[rows]
        gcodes, gscale = (host(t) for t in site.workspace_codes(wl.M))
        ga = oracle.unpack_codes(gcodes.reshape(wl.M, -1)[rows], wl.K, wl.abits)
        oa = oracle.unpack_codes(ca, wl.K, wl.abits)
        yg = synth.bf16_bits_to_f32(y).astype(np.float64)
        rel_o = float(np.linalg.norm(yg - yf) / np.linalg.norm(yf))
        rel, cos = rel_cos(yg, ref)
        log(f"{name} M={M} {what}: GPU vs float layer rel {rel:.3e} cosine {cos:.4f}; GPU vs oracle rel "
            f"{rel_o:.2e}, codes differing {int(np.count_nonzero(ga != oa))}/{ga.size}")
        assert np.abs(ga - oa).max() <= 1 and np.count_nonzero(ga != oa) <= 1e-3 * ga.size
        assert np.allclose(gscale[rows], sa, rtol=1e-5, atol=0)
        assert rel_o <= 1e-2
        if matched:
            assert rel <= MATCHED_REL[matched], f"{what}: {rel:.3e}"
        else:
            assert rel >= WRONG_REL, f"{what}: a mismatched fold gave rel {rel:.3e} on the GPU"

"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a library
routine (scipy's Sylvester Hadamard, numpy's matmul and half-to-even round,
torch's RMSNorm and bfloat16 cast), a closed form, an invariant of exact
arithmetic, or brute force on tiny inputs.  The definitions come from the vla.cpp
page "FoldQuant W8A8/W4A4 inference and FoldQuantVLA quantized-model converter"
(dequant-mode commit: the fold algebra and R; OpenVINO commit: the act-node
steps and the 15 INT4 levels; SYCL commit: exact integer sums).
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.linalg
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
POW2 = [1, 2, 4, 8, 16, 32, 64, 128, 256]


def _R(b, K):
    """R_b over K as an explicit float64 matrix built from scipy's Hadamard."""
    H = scipy.linalg.hadamard(b).astype(np.float64) / math.sqrt(b)
    return scipy.linalg.block_diag(*([H] * (K // b)))


# ---------------------------------------------------------------- Hadamard, R_b
@pytest.mark.parametrize("b", POW2)
def test_hadamard_entries_match_scipy_and_are_orthogonal(b):
    H = np.array([[oracle.hadamard_entry(b, i, j) for j in range(b)] for i in range(b)])
    assert np.array_equal(H, scipy.linalg.hadamard(b))
    assert np.array_equal(H @ H.T, b * np.eye(b, dtype=H.dtype))   # H H^T = b I
    assert np.array_equal(H, H.T)                                  # symmetric


@pytest.mark.parametrize("b", POW2)
def test_butterfly_columns_are_sylvester_columns(b):
    # the butterfly of unit vector e_j must be column j of H_b (natural order)
    H = scipy.linalg.hadamard(b).astype(np.float32)
    for j in range(b):
        e = np.zeros(b, np.float32)
        e[j] = 1.0
        assert np.array_equal(oracle.butterfly_f32(e, b), H[:, j])


@pytest.mark.parametrize("b", POW2)
def test_rotation_is_block_normalised_orthonormal(b):
    K = 3 * max(b, 4)
    rng = np.random.default_rng(b)
    v = rng.standard_normal(K)
    Rv = oracle.rotate_f64(v, b)
    assert np.allclose(Rv, _R(b, K) @ v, rtol=0, atol=1e-13)
    assert abs(np.linalg.norm(Rv) - np.linalg.norm(v)) <= 1e-12 * np.linalg.norm(v)
    assert np.allclose(oracle.rotate_f64(Rv, b), v, rtol=0, atol=1e-13)   # R R = I
    # contiguous blocks: a vector living in block 1 stays in block 1
    w = np.zeros(K)
    w[b:2 * b] = rng.standard_normal(b)
    Rw = oracle.rotate_f64(w, b)
    assert np.all(Rw[:b] == 0) and np.all(Rw[2 * b:] == 0)


def test_float32_butterfly_tracks_float64():
    rng = np.random.default_rng(7)
    v = rng.standard_normal(4096).astype(np.float32)
    got = oracle.butterfly_f32(v, 128).astype(np.float64)
    ref = _R(128, 4096) @ v.astype(np.float64) * math.sqrt(128)
    assert np.max(np.abs(got - ref)) <= 1e-5 * np.max(np.abs(ref))


# ---------------------------------------------------------------- weight fold and pack
@pytest.mark.parametrize("fold_after", [0, 1])
@pytest.mark.parametrize("b", [1, 32, 128])
def test_fold_weights_matches_matrix_definition(fold_after, b):
    rng = np.random.default_rng(11 + b)
    N, K = 5, 256
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    a = rng.uniform(0.2, 5.0, K).astype(np.float32)
    U = oracle.fold_weights(W, a, fold_after, b)
    R = _R(b, K)
    W64, a64 = W.astype(np.float64), a.astype(np.float64)
    ref = (R @ (a64 * W64).T).T if fold_after == 0 else a64 * (R @ W64.T).T
    assert np.allclose(U, ref, rtol=0, atol=1e-14)


@pytest.mark.parametrize("wbits", [8, 4])
@pytest.mark.parametrize("fold_after", [0, 1])
@pytest.mark.parametrize("b", [1, 64, 128])
def test_pack_within_half_step_and_unfold(wbits, fold_after, b):
    rng = np.random.default_rng(100 + b + wbits + fold_after)
    N, K = 7, 512
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[:, 3] *= 40.0
    a = rng.uniform(0.1, 6.4, K).astype(np.float32)
    qmax = oracle.qmax(wbits)
    codes, s = oracle.pack_weights(W, a, fold_after, b, wbits)
    q = oracle.unpack_codes(codes, K, wbits)
    U = oracle.fold_weights(W, a, fold_after, b)
    s64 = s.astype(np.float64)[:, None]
    # folded frame: every code within half a quantisation step of the folded weight
    assert np.all(np.abs(U - s64 * q) <= s64 / 2 * (1 + 1e-12))
    assert np.all(np.abs(q) <= qmax)
    assert np.all(np.abs(q).max(axis=1) == qmax)
    # scale is the float32 rounding of the row's amax / qmax
    assert np.array_equal(s, (np.abs(U).max(axis=1) / qmax).astype(np.float32))
    # original frame: unfold(fold(W)) within the propagated half step
    What = oracle.unfold_weights(codes, s, K, a, fold_after, b, wbits)
    a64 = a.astype(np.float64)
    if fold_after == 0:      # a (.) (W - What) = R(u - s q)
        err = np.linalg.norm(a64 * (W - What), axis=1)
        bound = math.sqrt(K) * s64[:, 0] / 2
    else:                    # W - What = R((u - s q) / a)
        err = np.linalg.norm(W - What, axis=1)
        bound = np.sqrt(np.sum((s64 / 2 / a64) ** 2, axis=1))
    assert np.all(err <= bound * (1 + 1e-9))


@pytest.mark.parametrize("fold_after", [0, 1])
def test_unfold_of_unquantised_fold_is_identity(fold_after):
    # fold then unfold without rounding: scale 1 and "codes" are the folded values
    # themselves is not expressible with integer codes, so use the algebra on R:
    rng = np.random.default_rng(3)
    N, K, b = 4, 256, 64
    W = rng.standard_normal((N, K)).astype(np.float32)
    a = rng.uniform(0.5, 2.0, K).astype(np.float32)
    U = oracle.fold_weights(W, a, fold_after, b)
    a64 = a.astype(np.float64)
    back = np.stack([oracle.rotate_f64(u, b) / a64 if fold_after == 0 else
                     oracle.rotate_f64(u / a64, b) for u in U])
    assert np.allclose(back, W.astype(np.float64), rtol=0, atol=1e-12)


@pytest.mark.parametrize("wbits", [8, 4])
def test_pack_without_rotation_is_textbook_per_row_rtn(wbits):
    rng = np.random.default_rng(5)
    N, K = 9, 128
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    qmax = oracle.qmax(wbits)
    codes, s = oracle.pack_weights(W, None, 0, 1, wbits)
    W64 = W.astype(np.float64)
    s_ref = (np.abs(W64).max(axis=1) / qmax).astype(np.float32)
    q_ref = np.clip(np.round(W64 / s_ref.astype(np.float64)[:, None]), -qmax, qmax)  # half-to-even
    assert np.array_equal(s, s_ref)
    assert np.array_equal(oracle.unpack_codes(codes, K, wbits), q_ref.astype(np.int32))


def test_nibble_order_fixture():
    fx = json.load(open(os.path.join(GOLDEN, "nibble_order.json")))
    codes = np.array(fx["codes"], np.float32)
    # a weight row whose per-row RTN reproduces these codes exactly: scale 1/8
    W = (codes / 8.0).astype(np.float32)[None, :]
    packed, s = oracle.pack_weights(W, None, 0, 1, 4)
    assert s[0] == np.float32(1.0 / 8.0)
    assert list(packed[0]) == fx["bytes"]
    assert [oracle.code_at(packed[0], k, 4) for k in range(len(codes))] == fx["codes"]


# ---------------------------------------------------------------- activation prologue
def _bf16(x):
    return synth.f32_to_bf16_bits(np.asarray(x, np.float32))


@pytest.mark.parametrize("abits", [8, 4])
def test_prologue_without_norm_or_rotation_is_per_token_rtn(abits):
    rng = np.random.default_rng(17)
    xb = _bf16(rng.standard_normal((6, 64)) * 3)
    x = synth.bf16_bits_to_f32(xb)
    qmax = oracle.qmax(abits)
    codes, s = oracle.prologue(xb, None, 1e-6, None, 0, 1, abits)
    s_ref = np.abs(x).max(axis=1) / np.float32(qmax)          # float32 numpy division
    q_ref = np.clip(np.round(x / s_ref[:, None]), -qmax, qmax)  # float32, half-to-even
    assert s.dtype == np.float32 and np.array_equal(s, s_ref.astype(np.float32))
    assert np.array_equal(oracle.unpack_codes(codes, 64, abits), q_ref.astype(np.int32))


def test_rmsnorm_matches_torch():
    rng = np.random.default_rng(19)
    xb = _bf16(rng.standard_normal((8, 256)) * 2)
    g = rng.uniform(0.5, 1.5, 256).astype(np.float32)
    h = oracle.act_frame(xb, g, 1e-6, None, 0, 1)
    xt = torch.from_numpy(synth.bf16_bits_to_f32(xb).astype(np.float64))
    ref = torch.nn.functional.rms_norm(xt, (256,), torch.from_numpy(g.astype(np.float64)), 1e-6)
    assert np.allclose(h, ref.numpy(), rtol=3e-7, atol=0)


@pytest.mark.parametrize("mode", ["gain", "explicit_before", "explicit_after", "none"])
@pytest.mark.parametrize("b", [1, 16, 128])
def test_rotation_invariance_of_float_path(mode, b):
    """Without quantisation, frame(x) . fold(W) = (RMSNorm(x) gamma) . W in exact arithmetic."""
    rng = np.random.default_rng(23 + b)
    M, K, N = 4, 256, 6
    xb = _bf16(rng.standard_normal((M, K)))
    g = rng.uniform(0.5, 1.5, K).astype(np.float32)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    a = rng.uniform(0.2, 5.0, K).astype(np.float32)
    fold_after = 1 if mode == "explicit_after" else 0
    if mode == "gain":
        h = oracle.act_frame(xb, oracle.fold_gain(g, a), 1e-6, None, 0, b)
    elif mode == "none":
        a = None
        h = oracle.act_frame(xb, g, 1e-6, None, 0, b)
    else:
        h = oracle.act_frame(xb, g, 1e-6, a, fold_after, b)
    U = oracle.fold_weights(W, a, fold_after, b)
    got = h.astype(np.float64) @ U.T
    xt = torch.from_numpy(synth.bf16_bits_to_f32(xb).astype(np.float64))
    xn = torch.nn.functional.rms_norm(xt, (K,), torch.from_numpy(g.astype(np.float64)), 1e-6).numpy()
    ref = xn @ W.astype(np.float64).T
    scale = np.abs(xn) @ np.abs(W.astype(np.float64)).T
    assert np.all(np.abs(got - ref) <= 2e-6 * scale)


def test_gain_fold_equals_explicit_smoothing_before_rotation():
    rng = np.random.default_rng(29)
    xb = _bf16(rng.standard_normal((5, 512)))
    g = rng.uniform(0.5, 1.5, 512).astype(np.float32)
    a = rng.uniform(0.2, 5.0, 512).astype(np.float32)
    h1 = oracle.act_frame(xb, oracle.fold_gain(g, a), 1e-6, None, 0, 128)
    h2 = oracle.act_frame(xb, g, 1e-6, a, 0, 128)
    assert np.allclose(h1, h2, rtol=0, atol=2e-6 * np.abs(h2).max())


@pytest.mark.parametrize("abits", [8, 4])
@pytest.mark.parametrize("norm", [False, True])
def test_prologue_invariances(abits, norm):
    rng = np.random.default_rng(31)
    K = 1024
    x = (rng.standard_normal((8, K)) * 2).astype(np.float32)
    x[:, 5] *= 30
    g = rng.uniform(0.5, 1.5, K).astype(np.float32) if norm else None
    eps = 0.0   # with eps = 0 a power-of-two rescale is exact at norm sites too
    c0, s0 = oracle.prologue(_bf16(x), g, eps, None, 0, 128, abits)
    c4, s4 = oracle.prologue(_bf16(x * 4), g, eps, None, 0, 128, abits)
    cn, sn = oracle.prologue(_bf16(-x), g, eps, None, 0, 128, abits)
    assert np.array_equal(c0, c4)
    assert np.array_equal(s4, s0 if norm else s0 * 4)
    q0 = oracle.unpack_codes(c0, K, abits)
    assert np.array_equal(oracle.unpack_codes(cn, K, abits), -q0)
    assert np.array_equal(sn, s0)
    qmax = oracle.qmax(abits)
    assert np.all(np.abs(q0) <= qmax) and np.all(np.abs(q0).max(axis=1) == qmax)


def test_prologue_zero_token_gives_zero_codes_and_scale():
    x = np.zeros((3, 256), np.float32)
    x[1] = 1.0
    for abits in (8, 4):
        c, s = oracle.prologue(_bf16(x), None, 1e-6, None, 0, 64, abits)
        assert s[0] == 0 and s[2] == 0 and s[1] > 0
        q = oracle.unpack_codes(c, 256, abits)
        assert np.all(q[0] == 0) and np.all(q[2] == 0)
    # a norm site with a zero token: rms = sqrt(eps), still all-zero codes
    c, s = oracle.prologue(_bf16(x), np.ones(256, np.float32), 1e-6, None, 0, 64, 8)
    assert s[0] == 0 and np.all(c[0] == 0)


def test_spike_token_fixture():
    fx = json.load(open(os.path.join(GOLDEN, "spike_token.json")))
    K, b = fx["K"], fx["hblock"]
    x = np.zeros((1, K), np.float32)
    x[0, fx["x_index"]] = fx["x_value"]
    for abits, key in ((8, "codes_a8"), (4, "codes_a4")):
        c, s = oracle.prologue(_bf16(x), None, 1e-6, None, 0, b, abits)
        assert oracle.unpack_codes(c, K, abits)[0].tolist() == fx[key]
        assert abs(s[0] - fx[f"scale_a{abits}_approx"]) <= 1e-6 * s[0]


# ---------------------------------------------------------------- integer GEMM
@pytest.mark.parametrize("abits,wbits", [(8, 8), (4, 4), (4, 8), (8, 4)])
def test_gemm_equals_integer_matmul(abits, wbits):
    rng = np.random.default_rng(37 + abits + 2 * wbits)
    M, N, K = 13, 21, 320

    def rand_codes(rows, bits):
        q = rng.integers(-oracle.qmax(bits), oracle.qmax(bits) + 1, size=(rows, K))
        if bits == 8:
            return q.astype(np.int8).view(np.uint8), q
        lo, hi = q[:, 0::2] & 0xF, q[:, 1::2] & 0xF
        return (lo | (hi << 4)).astype(np.uint8), q

    ca, qa = rand_codes(M, abits)
    cw, qw = rand_codes(N, wbits)
    assert np.array_equal(oracle.unpack_codes(ca, K, abits), qa)
    acc = oracle.gemm_i32(ca, abits, cw, wbits, K)
    assert np.array_equal(acc, (qa.astype(np.int64) @ qw.astype(np.int64).T).astype(np.int32))


def test_gemm_brute_force_tiny_and_extremes():
    rng = np.random.default_rng(41)
    for K in (2, 4, 8, 16):
        qa = rng.choice([-127, 127], size=(3, K))
        qw = rng.integers(-127, 128, size=(4, K))
        acc = oracle.gemm_i32(qa.astype(np.int8).view(np.uint8), 8, qw.astype(np.int8).view(np.uint8), 8, K)
        for m in range(3):
            for n in range(4):
                assert acc[m, n] == sum(int(qa[m, k]) * int(qw[n, k]) for k in range(K))
    # all codes at +-qmax on the longest row of the workloads (K = 18944)
    K = 18944
    qa = np.full((2, K), 127, np.int8)
    qa[1] = -127
    qw = np.full((3, K), 127, np.int8)
    acc = oracle.gemm_i32(qa.view(np.uint8), 8, qw.view(np.uint8), 8, K)
    assert acc[0, 0] == 127 * 127 * K and acc[1, 2] == -127 * 127 * K


def test_gemm_reports_int32_overflow():
    K = 140000  # 127 * 127 * K > 2^31 - 1
    qa = np.full((1, K), 127, np.int8).view(np.uint8)
    with pytest.raises(OverflowError):
        oracle.gemm_i32(qa, 8, qa, 8, K)


# ---------------------------------------------------------------- bf16 rounding, epilogue
def test_bf16_rounding_matches_torch_on_float32_values():
    rng = np.random.default_rng(43)
    v = np.concatenate([
        rng.standard_normal(4000).astype(np.float32) * 100,
        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.4e38, -3.4e38, 1e-40, -1e-41,
                  np.inf, -np.inf, 2 ** -133, 2 ** -134, 3 * 2 ** -135], np.float32),
        (rng.integers(0, 2 ** 32, 4000, dtype=np.uint64).astype(np.uint32).view(np.float32)),
    ])
    v = v[np.isfinite(v) | np.isinf(v)]
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.bf16_from_f64(float(t)) for t in v], np.uint16)
    assert np.array_equal(got, ref)


def test_bf16_rounding_is_single_rounding_from_float64():
    # just above the tie between 1 and 1 + 2^-7: one rounding goes up; rounding
    # through float32 first would land on the tie and go to even (1.0)
    assert oracle.bf16_from_f64(1 + 2 ** -8 + 2 ** -40) == 0x3F81
    assert oracle.bf16_from_f64(1 + 2 ** -8) == 0x3F80          # exact tie -> even
    assert oracle.bf16_from_f64(1 + 3 * 2 ** -8) == 0x3F82      # tie -> even (up)
    assert oracle.bf16_from_f64(-(1 + 2 ** -8 + 2 ** -40)) == 0xBF81


def test_epilogue_closed_forms():
    acc = np.array([[1, -3, 0, 1 << 20]], np.int32)
    sa = np.array([0.5], np.float32)
    sw = np.array([2.0, 0.25, 1.0, 2 ** -20], np.float32)
    bias = np.array([0.0, 1.0, -2.0, 0.0], np.float32)
    res = _bf16([[0.0, 0.0, 0.5, 1.0]])
    y, yf = oracle.epilogue(acc, sa, sw, bias, res, want_f64=True)
    assert yf.tolist() == [[1.0, 1.0 - 0.375, -1.5, 1.5]]
    assert y.tolist() == [[0x3F80, 0x3F20, 0xBFC0, 0x3FC0]]


# ---------------------------------------------------------------- whole site, tiny shapes
@pytest.mark.parametrize("wbits,abits", [(8, 8), (4, 4)])
def test_tiny_site_within_closed_form_bound(wbits, abits):
    wl = synth.random_workload(8, 256, 32, 64, wbits, abits, seed=47, norm=True, ascale="gain",
                               residual=True, bias=True)
    out = oracle.linear(wl)
    K = wl.K
    qa = oracle.unpack_codes(out["codes_a"], K, abits).astype(np.float64)
    qw = oracle.unpack_codes(out["codes_w"], K, wbits).astype(np.float64)
    sa = out["act_scale"].astype(np.float64)[:, None]
    sw = out["wscale"].astype(np.float64)[:, None]
    res = synth.bf16_bits_to_f32(wl.residual).astype(np.float64)
    extra = wl.bias.astype(np.float64)[None, :] + res
    # 1. the epilogue value is the dequantised product
    deq = (qa * sa) @ (qw * sw).T + extra
    assert np.allclose(out["y_f64"], deq, rtol=1e-12, atol=1e-12)
    # 2. bf16 output is the single rounding of that value
    assert np.array_equal(out["y"], np.vectorize(oracle.bf16_from_f64, otypes=[np.uint16])(out["y_f64"]))
    # 3. against the unquantised float layer, within the per-element quantisation bound
    h = oracle.act_frame(wl.x, out["gamma_folded"], wl.eps, None, 0, wl.hblock).astype(np.float64)
    U = oracle.fold_weights(wl.W, wl.ascale, 0, wl.hblock)
    exact = h @ U.T + extra
    bound = (np.abs(h) @ (np.ones_like(U) * sw).T / 2 + sa / 2 * np.abs(U).sum(axis=1)[None, :]
             + sa * sw.T * K / 4)
    assert np.all(np.abs(out["y_f64"] - exact) <= bound * (1 + 1e-9) + 1e-6 * np.abs(exact))


def test_rotation_reduces_error_on_outlier_site():
    """The point of the block rotation (runtime summary: codes in a block-Hadamard
    frame): on an activation with outlier channels and no smoothing, b = 128 loses
    less than b = 1."""
    errs = {}
    for b in (1, 128):
        wl = synth.random_workload(16, 1024, 64, b, 8, 8, seed=53, norm=True, ascale="none",
                                   outliers=8, outlier_factor=40.0)
        out = oracle.linear(wl)
        h = oracle.act_frame(wl.x, wl.gamma, wl.eps, None, 0, 1).astype(np.float64)
        exact = h @ wl.W.astype(np.float64).T
        errs[b] = np.linalg.norm(out["y_f64"] - exact) / np.linalg.norm(exact)
    assert errs[128] < errs[1]


def test_geglu_matches_torch_tanh_gelu_and_rounds_once():
    """GeGLU of the chained MLP block: the float64 value is torch's tanh-approximate
    GELU (a library routine) times up, and the bf16 output is its single
    nearest-even rounding."""
    import torch
    rng = np.random.default_rng(5)
    F = 96
    gu = synth.f32_to_bf16_bits((rng.standard_normal((6, 2 * F)) * 2.5).astype(np.float32))
    h, hf = oracle.geglu(gu, F, want_f64=True)
    g = torch.from_numpy(synth.bf16_bits_to_f32(gu[:, :F]).astype(np.float64))
    u = torch.from_numpy(synth.bf16_bits_to_f32(gu[:, F:]).astype(np.float64))
    ref = (torch.nn.functional.gelu(g, approximate="tanh") * u).numpy()
    assert np.allclose(hf, ref, rtol=1e-13, atol=1e-300)
    want = np.array([[oracle.bf16_from_f64(v) for v in row] for row in ref], np.uint16)
    assert np.array_equal(h, want)


def test_geglu_special_values():
    """gelu(0) = 0; gelu(g) -> g for large g and -> 0 for very negative g."""
    one = synth.f32_to_bf16_bits(np.float32(1.0))
    rows = []
    for gate in (0.0, 20.0, -20.0, 3.0):
        rows.append([synth.f32_to_bf16_bits(np.float32(gate)), one])
    gu = np.array(rows, np.uint16).reshape(4, 2)
    h, hf = oracle.geglu(gu, 1, want_f64=True)
    assert hf[0, 0] == 0.0
    assert abs(hf[1, 0] - 20.0) < 1e-12
    assert abs(hf[2, 0]) < 1e-12
    # gelu_tanh(3) from its definition with tanh evaluated by numpy
    c = np.sqrt(2 / np.pi)
    assert abs(hf[3, 0] - 1.5 * (1 + np.tanh(c * (3 + 0.044715 * 27)))) < 1e-14


# ---------------------------------------------------------------- E2M3 storage of the 4-bit codes
def test_e2m3_values_follow_the_format_definition():
    # closed forms of FP6 E2M3 (bias 1, subnormals at exponent 0, no inf/NaN)
    assert oracle.e2m3_value(0b011111) == 7.5     # largest normal: 2^2 x 1.875
    assert oracle.e2m3_value(0b001000) == 1.0     # smallest normal
    assert oracle.e2m3_value(0b000001) == 0.125   # smallest subnormal: 1/8
    assert oracle.e2m3_value(0b000111) == 0.875   # largest subnormal
    assert oracle.e2m3_value(0b010100) == 3.0
    assert oracle.e2m3_value(0b011010) == 5.0
    z = oracle.e2m3_value(0b100000)
    assert z == 0.0 and math.copysign(1.0, z) < 0
    pos = [oracle.e2m3_value(c) for c in range(32)]
    assert all(a < b for a, b in zip(pos, pos[1:]))  # magnitudes grow with the pattern
    assert all(oracle.e2m3_value(c | 32) == -pos[c] for c in range(32))


def test_e2m3_holds_every_4bit_code_exactly():
    codes = [oracle.e2m3_code(v) for v in range(-7, 8)]
    assert len(set(codes)) == 15
    assert [oracle.e2m3_value(c) for c in codes] == [float(v) for v in range(-7, 8)]
    integral = [c for c in range(64) if oracle.e2m3_value(c) == int(oracle.e2m3_value(c))]
    assert len(integral) == 16  # the 15 codes and -0
    with pytest.raises(ValueError):
        oracle.e2m3_code(8)


def test_e2m3_row_fixture():
    fx = json.load(open(os.path.join(GOLDEN, "e2m3_row.json")))
    q = np.array([fx["codes"]])
    assert [oracle.e2m3_code(v) for v in fx["codes"]] == fx["fields"]
    packed = oracle.pack_e2m3(q)
    assert list(packed[0]) == fx["bytes"]
    assert np.array_equal(oracle.unpack_codes(packed, q.shape[1], oracle.E2M3), q)
    assert [oracle.code_at(packed[0], k, oracle.E2M3) for k in range(q.shape[1])] == fx["codes"]


def test_e2m3_bit_positions_one_value_at_a_time():
    # value k alone in a row sets exactly bits 6k .. 6k+5 of the little-endian bit string
    K = 16
    for k in range(K):
        for v in (1, -3, 7):
            q = np.zeros((1, K), np.int64)
            q[0, k] = v
            row = oracle.pack_e2m3(q)[0]
            word = int.from_bytes(bytes(row), "little")
            assert word == oracle.e2m3_code(v) << (6 * k)


def test_e2m3_storage_is_the_4bit_quantiser():
    # packer, prologue and contraction give the same integers as with 4-bit storage
    rng = np.random.default_rng(51)
    N, M, K = 9, 5, 256
    W = rng.normal(0, 0.02, (N, K)).astype(np.float32)
    a = rng.uniform(0.5, 2.0, K).astype(np.float32)
    c4, s4 = oracle.pack_weights(W, a, 0, 64, 4)
    c6, s6 = oracle.pack_weights(W, a, 0, 64, oracle.E2M3)
    assert c6.shape == (N, 3 * K // 4)
    assert np.array_equal(s4, s6)
    assert np.array_equal(oracle.unpack_codes(c4, K, 4), oracle.unpack_codes(c6, K, oracle.E2M3))
    x = _bf16(rng.normal(0, 1, (M, K)))
    g = rng.uniform(0.5, 1.5, K).astype(np.float32)
    a4, sa4 = oracle.prologue(x, g, 1e-6, None, 0, 64, 4)
    a6, sa6 = oracle.prologue(x, g, 1e-6, None, 0, 64, oracle.E2M3)
    assert np.array_equal(sa4, sa6)
    qa = oracle.unpack_codes(a4, K, 4)
    assert np.array_equal(qa, oracle.unpack_codes(a6, K, oracle.E2M3))
    acc6 = oracle.gemm_i32(a6, oracle.E2M3, c6, oracle.E2M3, K)
    qw = oracle.unpack_codes(c4, K, 4)
    assert np.array_equal(acc6, (qa.astype(np.int64) @ qw.astype(np.int64).T).astype(np.int32))
    u4 = oracle.unfold_weights(c4, s4, K, a, 0, 64, 4)
    u6 = oracle.unfold_weights(c6, s6, K, a, 0, 64, oracle.E2M3)
    assert np.array_equal(u4, u6)


def test_e2m3_unpack_rejects_non_code_patterns():
    row = np.zeros((1, 3), np.uint8)
    row[0, 0] = 0b011111  # 7.5 in field 0: no integer code
    with pytest.raises(ValueError):
        oracle.unpack_codes(row, 4, oracle.E2M3)

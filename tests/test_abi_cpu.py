"""CPU-only checks of libfq: it loads, exports every symbol include/fq.h declares,
its host packer and gain fold match the oracle bit for bit, and every device
entry point rejects bad arguments before touching the GPU (the page's
convention: refuse an impossible request up front, naming the argument and
the arithmetic)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import synth
import w4a4_integer_gemm_amd as fq
from w4a4_integer_gemm_amd import _binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fq.h")

# a fake but aligned "device pointer": validation never dereferences it
DEV = 0x10000
BAD = 0x10001


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fq_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = fq.lib()
    names = header_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(_binding.SIGNATURES), "binding and header disagree"
    assert fq.abi_version() == 2


def test_sizes():
    assert fq.fq_weight_bytes(4608, 3584, 8) == 4608 * 3584
    assert fq.fq_weight_bytes(32768, 2048, 4) == 32768 * 1024
    assert fq.fq_act_bytes(816, 16384, 4) == 816 * 8192
    assert fq.fq_weight_bytes(0, 64, 8) == 0 and fq.fq_weight_bytes(4, 64, 3) == 0
    assert fq.fq_weight_bytes(32768, 2048, fq.E2M3) == 32768 * 1536
    assert fq.fq_act_bytes(816, 16384, fq.E2M3) == 816 * 12288
    ws = fq.fq_linear_workspace_bytes(1024, 3584, 8)
    assert ws >= 1024 * 3584 + 4 * 1024 and ws % 256 == 0


@pytest.mark.parametrize("wbits", [8, 4, 6])
@pytest.mark.parametrize("fold_after", [0, 1])
@pytest.mark.parametrize("hblock", [1, 2, 8, 32, 64, 128, 256])
@pytest.mark.parametrize("with_a", [False, True])
def test_host_packer_matches_oracle(wbits, fold_after, hblock, with_a):
    rng = np.random.default_rng(hblock * 7 + wbits + fold_after)
    N, K = 24, 512
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[:, 7] *= 50
    W[3] = 0.0  # an all-zero row: scale 0, codes 0
    a = rng.uniform(0.15, 6.4, K).astype(np.float32) if with_a else None
    c1, s1 = fq.fq_pack_weights(W, a, fold_after, hblock, wbits)
    c2, s2 = oracle.pack_weights(W, a, fold_after, hblock, wbits)
    assert np.array_equal(s1, s2)
    assert np.array_equal(c1, c2)
    assert s1[3] == 0 and np.all(c1[3] == 0)


def test_host_packer_matches_oracle_on_workload_shapes():
    wl = synth.make_workload("qkv_w8a8", N=256)
    c1, s1 = fq.fq_pack_weights(wl.W, wl.ascale, 0, wl.hblock, 8)
    c2, s2 = oracle.pack_weights(wl.W, wl.ascale, 0, wl.hblock, 8)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
    wl = synth.make_workload("gateup_w4a4", N=256)
    for bits in (4, fq.E2M3):
        c1, s1 = fq.fq_pack_weights(wl.W, wl.ascale, 0, wl.hblock, bits)
        c2, s2 = oracle.pack_weights(wl.W, wl.ascale, 0, wl.hblock, bits)
        assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


def test_e2m3_storage_holds_the_4bit_codes():
    """The E2M3 rows carry the 4-bit packer's integers, scale for scale, and
    dequantise to the same floats."""
    rng = np.random.default_rng(61)
    N, K = 40, 1024
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    a = rng.uniform(0.3, 3.0, K).astype(np.float32)
    c4, s4 = fq.fq_pack_weights(W, a, 1, 64, 4)
    c6, s6 = fq.fq_pack_weights(W, a, 1, 64, fq.E2M3)
    assert c6.shape == (N, 3 * K // 4) and np.array_equal(s4, s6)
    assert np.array_equal(oracle.unpack_codes(c4, K, 4), oracle.unpack_codes(c6, K, oracle.E2M3))
    d4 = fq.fq_dequant_rows(c4, s4, K, a, 1, 64, 4)
    d6 = fq.fq_dequant_rows(c6, s6, K, a, 1, 64, fq.E2M3)
    assert np.array_equal(d4, d6)


def _ulp_diff(a32, b32):
    """Distance in float32 units in the last place (same sign assumed near equality)."""
    ai = a32.view(np.int32).astype(np.int64)
    bi = b32.view(np.int32).astype(np.int64)
    ai = np.where(ai < 0, -(ai & 0x7FFFFFFF), ai)
    bi = np.where(bi < 0, -(bi & 0x7FFFFFFF), bi)
    return np.abs(ai - bi)


@pytest.mark.parametrize("wbits", [8, 4])
@pytest.mark.parametrize("fold_after", [0, 1])
@pytest.mark.parametrize("hblock", [1, 16, 128])
@pytest.mark.parametrize("with_a", [False, True])
def test_dequant_rows_match_oracle_unfold(wbits, fold_after, hblock, with_a):
    """fq_dequant_rows against the oracle's float64 unfold, rounded once to
    float32: equal to within one float32 unit in the last place (the two sum
    the butterfly in different orders)."""
    rng = np.random.default_rng(hblock + 3 * wbits + fold_after)
    N, K = 20, 384
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    a = rng.uniform(0.2, 5.0, K).astype(np.float32) if with_a else None
    codes, ws = oracle.pack_weights(W, a, fold_after, hblock, wbits)
    got = fq.fq_dequant_rows(codes, ws, K, a, fold_after, hblock, wbits)
    ref = oracle.unfold_weights(codes, ws, K, a, fold_after, hblock, wbits).astype(np.float32)
    d = _ulp_diff(got, ref)
    small = np.abs(ref) < 1e-30
    assert np.all(d[~small] <= 1), f"max ulp diff {d[~small].max()}"
    assert np.all(np.abs(got[small]) < 1e-29)


@pytest.mark.parametrize("wbits", [8, 4])
@pytest.mark.parametrize("fold_after", [0, 1])
def test_dequant_rows_undo_the_fold_up_to_rounding(wbits, fold_after):
    """The rebuild returns the original rows up to the codes' rounding: per row,
    in the smoothing-weighted norm the fold preserves, the error is at most
    half a quantisation step per element (sqrt(K) s_n / 2)."""
    rng = np.random.default_rng(11 + wbits + fold_after)
    N, K, b = 16, 512, 64
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    a = rng.uniform(0.3, 3.0, K).astype(np.float32)
    codes, ws = fq.fq_pack_weights(W, a, fold_after, b, wbits)
    back = fq.fq_dequant_rows(codes, ws, K, a, fold_after, b, wbits).astype(np.float64)
    err = back - W.astype(np.float64)
    for n in range(N):
        bound = np.sqrt(K) * ws[n] / 2 * (1 + 1e-6)
        weighted = err[n] * a if fold_after == 0 else err[n]
        scale = 1.0 if fold_after == 0 else 1.0 / a.min()
        assert np.linalg.norm(weighted) <= bound * scale + 1e-12


def test_dequant_rows_rejects():
    codes = np.zeros((4, 256), np.uint8)
    ws = np.ones(4, np.float32)
    with pytest.raises(fq.FqError, match="fq_dequant_rows: K=100"):
        fq.fq_dequant_rows(codes, ws, 100, None, 0, 1, 8)
    with pytest.raises(fq.FqError, match="fq_dequant_rows: K=256 not divisible by hblock=512|hblock=512"):
        fq.fq_dequant_rows(codes, ws, 256, None, 0, 512, 8)
    bad = ws.copy()
    bad[2] = np.nan
    with pytest.raises(fq.FqError, match=r"wscale\[2\]"):
        fq.fq_dequant_rows(codes, bad, 256, None, 0, 1, 8)


def test_fold_gain_matches_oracle():
    rng = np.random.default_rng(1)
    g = rng.uniform(0.5, 1.5, 3584).astype(np.float32)
    a = rng.uniform(0.1, 160.0, 3584).astype(np.float32)
    assert np.array_equal(fq.fq_fold_gain(g, a), oracle.fold_gain(g, a))
    assert np.array_equal(fq.fq_fold_gain(g, None), g)
    with pytest.raises(fq.FqError, match="ascale\\[2\\]"):
        a2 = a.copy()
        a2[2] = 0
        fq.fq_fold_gain(g, a2)


@pytest.mark.parametrize("kw,match", [
    (dict(wbits=3), "wbits=3"),
    (dict(K=100), "K=100"),
    (dict(K=192), r"K=192 must be a multiple of 128"),
    (dict(K=384, hblock=256), r"K=384 not divisible by hblock=256 \(384/256 = 1.50\)"),
    (dict(hblock=3), "hblock=3"),
    (dict(hblock=512), "hblock=512"),
    (dict(fold_after=2), "fold_after=2"),
])
def test_host_packer_rejects(kw, match):
    args = dict(N=4, K=256, hblock=64, wbits=8, fold_after=0)
    args.update(kw)
    W = np.zeros((args["N"], args["K"]), np.float32)
    with pytest.raises(fq.FqError, match=match):
        fq.fq_pack_weights(W, None, args["fold_after"], args["hblock"], args["wbits"])


def _prologue(**kw):
    a = dict(x=DEV, M=4, K=256, ldx=256, gamma=DEV, eps=1e-6, ascale=None, fold_after=0, hblock=64, abits=8,
             codes=DEV, scale=DEV)
    a.update(kw)
    L = fq.lib()
    return L.fq_prologue(a["x"], a["M"], a["K"], a["ldx"], a["gamma"], a["eps"], a["ascale"], a["fold_after"],
                         a["hblock"], a["abits"], a["codes"], a["scale"], None)


@pytest.mark.parametrize("kw,status,match", [
    (dict(x=None), 1, "x_bf16 is NULL"),
    (dict(codes=None), 1, "act_codes is NULL"),
    (dict(scale=None), 1, "act_scale is NULL"),
    (dict(M=0), 2, "M=0"),
    (dict(K=100, ldx=104), 2, r"K=100 is not a multiple of 32 \(100/32 = 3.12\)"),
    (dict(K=131072, ldx=131072), 2, "K=131072 outside"),
    (dict(K=40992, ldx=40992, hblock=32), 2, r"K=40992 above 32768 must be a multiple of 64"),
    (dict(hblock=48), 2, "hblock=48"),
    (dict(K=320, ldx=320, hblock=128), 2, r"K=320 not divisible by hblock=128 \(320/128 = 2.50\)"),
    (dict(abits=2), 3, "abits=2"),
    (dict(ldx=255), 2, "ldx=255 < K=256"),
    (dict(ldx=260), 4, "ldx=260 is not a multiple of 8"),
    (dict(x=BAD), 4, "x_bf16 is not 16-byte aligned"),
    (dict(codes=BAD), 4, "act_codes is not 16-byte aligned"),
    (dict(fold_after=5), 1, "fold_after=5"),
    (dict(eps=float("nan")), 1, "eps=nan"),
])
def test_prologue_rejects_before_device_work(kw, status, match):
    rc = _prologue(**kw)
    assert rc == status
    msg = fq.last_error()
    assert msg.startswith("fq_prologue:")
    assert re.search(match, msg), msg


def _gemm(**kw):
    a = dict(act=DEV, sa=DEV, M=64, abits=8, w=DEV, sw=DEV, N=128, K=256, wbits=8, bias=None, res=None, ldr=0,
             y=DEV, ldy=128, acc=None)
    a.update(kw)
    return fq.lib().fq_gemm(a["act"], a["sa"], a["M"], a["abits"], a["w"], a["sw"], a["N"], a["K"], a["wbits"],
                            a["bias"], a["res"], a["ldr"], a["y"], a["ldy"], a["acc"], None)


@pytest.mark.parametrize("kw,status,match", [
    (dict(w=None), 1, "w_codes is NULL"),
    (dict(y=None), 1, "y_bf16 is NULL"),
    (dict(N=0), 2, "N=0"),
    (dict(N=100, ldy=100), 2, r"N=100 is not a multiple of 8 \(100/8 = 12.500\)"),
    (dict(ldy=64), 2, "ldy=64 < N=128"),
    (dict(res=DEV, ldr=64), 2, "ldr=64 < N=128"),
    (dict(res=DEV, ldr=132), 4, "ldr=132 is not a multiple of 8"),
    (dict(wbits=5), 3, "wbits=5"),
    (dict(wbits=6), 3, "abits=8 with wbits=6: E2M3 codes"),
    (dict(abits=6, wbits=4), 3, "abits=6 with wbits=4"),
    (dict(w=BAD), 4, "w_codes is not 16-byte aligned"),
    (dict(acc=BAD), 4, "acc_i32 is not 16-byte aligned"),
    (dict(K=0), 2, "K=0"),
    (dict(K=192), 2, r"K=192 is not a multiple of 128 \(192/128 = 1.50\)"),
])
def test_gemm_rejects_before_device_work(kw, status, match):
    rc = _gemm(**kw)
    assert rc == status
    msg = fq.last_error()
    assert msg.startswith("fq_gemm:") and re.search(match, msg), msg


@pytest.mark.parametrize("kw,status,match", [
    (dict(hd=12), 2, "head_dim=12 is not a multiple of 8"),
    (dict(hd=48), 2, r"N=128 is not a whole number of heads of head_dim=48 \(128/48 = 2.667\)"),
    (dict(hd=-8), 2, "head_dim=-8 must be > 0"),
    (dict(hd=64, y=None), 1, "y_bf16 is NULL"),
])
def test_gemm_heads_rejects_before_device_work(kw, status, match):
    a = dict(hd=64, y=DEV)
    a.update(kw)
    rc = fq.lib().fq_gemm_heads(DEV, DEV, 64, 8, DEV, DEV, 128, 256, 8, None, None, 0, a["hd"], a["y"], None, None)
    assert rc == status
    msg = fq.last_error()
    assert msg.startswith("fq_gemm_heads:") and re.search(match, msg), msg


def test_linear_heads_rejects_before_device_work():
    rc = fq.lib().fq_linear_heads(DEV, 16, 256, 256, DEV, 1e-6, None, 0, 64, 8, DEV, DEV, 128, 8, None, None, 0,
                                  24, DEV, 0x100000, 1 << 20, None)
    assert rc == 2
    assert fq.last_error().startswith("fq_linear_heads: head_dim=24") or "head_dim=24" in fq.last_error()


def _linear(**kw):
    a = dict(x=DEV, M=16, K=256, ldx=256, gamma=DEV, eps=1e-6, ascale=None, fold_after=0, hblock=64, abits=8,
             w=DEV, sw=DEV, N=128, wbits=8, bias=None, res=None, ldr=0, y=DEV, ldy=128, ws=0x100000,
             wsb=1 << 20)
    a.update(kw)
    return fq.lib().fq_linear(a["x"], a["M"], a["K"], a["ldx"], a["gamma"], a["eps"], a["ascale"], a["fold_after"],
                              a["hblock"], a["abits"], a["w"], a["sw"], a["N"], a["wbits"], a["bias"], a["res"],
                              a["ldr"], a["y"], a["ldy"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status,match", [
    (dict(ws=None), 1, "workspace is NULL"),
    (dict(ws=0x100010), 4, "workspace is not 256-byte aligned"),
    (dict(wsb=100), 1, r"workspace_bytes=100 < \d+ needed for M=16 K=256 abits=8"),
    (dict(hblock=7), 2, "hblock=7"),
    (dict(N=12, ldy=16), 2, "N=12 is not a multiple of 8"),
    (dict(abits=5), 3, "abits=5"),
])
def test_linear_rejects_before_device_work(kw, status, match):
    rc = _linear(**kw)
    assert rc == status
    msg = fq.last_error()
    assert msg.startswith("fq_linear:") and re.search(match, msg), msg


def test_error_message_is_cleared_by_a_good_host_call():
    _gemm(N=0)
    assert fq.last_error()
    fq.fq_pack_weights(np.ones((2, 128), np.float32), None, 0, 64, 8)
    assert fq.last_error() == ""


def test_binding_refuses_host_tensors_for_device_calls():
    import torch
    with pytest.raises(ValueError, match="GPU tensors"):
        fq.fq_prologue(torch.zeros(4, 64, dtype=torch.int16), 4, 64, 64, None, 1e-6, None, 0, 64, 8,
                       torch.zeros(256, dtype=torch.uint8), torch.zeros(4), None)


def test_test_hook_parses_and_rejects():
    """fq_test_hook takes "key=value" items and rejects unknown keys or values
    with a message (host only: it touches no device)."""
    L = _binding.lib()
    for good in ("", "default", "gemm_tile=64x128x2", "gemm_tile=auto,gemm_mfma=32", "gemv=split",
                 "gemm_tile=128x144,gemm_mfma=16,gemv=auto"):
        assert L.fq_test_hook(good.encode()) == 0, good
    assert L.fq_test_hook(None) == 0
    for bad, what in (("gemm_tile=100x100", "unknown gemm_tile"), ("gemm_mfma=8", "gemm_mfma must be"),
                      ("gemv=fast", "gemv must be"), ("tile=64x128", "unknown hook")):
        assert L.fq_test_hook(bad.encode()) == 1, bad
        assert what in _binding.last_error(), _binding.last_error()
    assert L.fq_test_hook(b"") == 0


def test_linear_noalloc_rejects_before_device_work():
    """fq_linear_noalloc refuses a workspace larger than its scratch array (and
    the usual bad arguments) before it touches the device."""
    L = _binding.lib()
    cap = L.fq_linear_noalloc_max_bytes()
    assert cap == 24 << 20
    # 2048 tokens x 16384 8-bit codes = 32 MiB of codes > 24 MiB
    rc = L.fq_linear_noalloc(DEV, 2048, 16384, 16384, None, 1e-6, None, 0, 128, 8, DEV, DEV, 512, 8, None, None, 0,
                             DEV, 512, None)
    assert rc == 3 and "scratch array" in _binding.last_error() and "fq_linear" in _binding.last_error()
    assert L.fq_linear_workspace_bytes(2048, 16384, 8) > cap
    rc = L.fq_linear_noalloc(DEV, 16, 3584, 3584, None, 1e-6, None, 0, 100, 8, DEV, DEV, 512, 8, None, None, 0,
                             DEV, 512, None)
    assert rc == 2 and "hblock" in _binding.last_error()
    rc = L.fq_linear_noalloc(DEV, 16, 3584, 3584, None, 1e-6, None, 0, 128, 8, DEV, DEV, 500, 8, None, None, 0,
                             DEV, 512, None)
    assert rc == 2 and "N=500" in _binding.last_error()
    rc = L.fq_linear_noalloc(BAD, 16, 3584, 3584, None, 1e-6, None, 0, 128, 8, DEV, DEV, 512, 8, None, None, 0,
                             DEV, 512, None)
    assert rc == 4 and "x_bf16" in _binding.last_error()

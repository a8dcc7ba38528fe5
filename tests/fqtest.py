"""Shared helpers of the GPU parity tests (comparison rules, device upload)."""
from __future__ import annotations

import sys

import numpy as np

import oracle
import synth

# Tolerances (the build's parity bar):
#  - int32 accumulators: bit-exact for identical codes
#  - activation codes: at most 1 LSB apart on at most 0.1 % of elements
#  - bf16 output: relative Frobenius error <= 1e-2 against the oracle's float64 value;
#    with identical codes, every element within half a bf16 ulp plus the float32
#    rounding of the epilogue's three operations (2^-21 of the summed magnitudes)
CODE_MISMATCH_FRAC = 1e-3
Y_REL_FRO = 1e-2


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def host(t, dtype=None):
    a = t.detach().cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


def rand_codes(rng, rows, K, bits, extreme=False):
    """Random codes in [-qmax, qmax] (or all +-qmax), stored as the kernels read them."""
    qmax = oracle.qmax(bits)
    if extreme:
        q = rng.choice([-qmax, qmax], size=(rows, K))
    else:
        q = rng.integers(-qmax, qmax + 1, size=(rows, K))
    if bits == 8:
        return q.astype(np.int8).view(np.uint8)
    if bits == oracle.E2M3:
        return oracle.pack_e2m3(q)
    return ((q[:, 0::2] & 0xF) | ((q[:, 1::2] & 0xF) << 4)).astype(np.uint8)


def bf16_to_f64(bits):
    return synth.bf16_bits_to_f32(np.ascontiguousarray(bits).view(np.uint16)).astype(np.float64)


def compare_codes(gpu_codes, ora_codes, K, bits):
    """Return (fraction of mismatched codes, max |difference|)."""
    g = oracle.unpack_codes(np.asarray(gpu_codes).reshape(ora_codes.shape), K, bits)
    o = oracle.unpack_codes(ora_codes, K, bits)
    d = np.abs(g - o)
    return float(np.count_nonzero(d)) / d.size, int(d.max()) if d.size else 0


def assert_codes(gpu_codes, gpu_scale, ora_codes, ora_scale, K, bits, what=""):
    frac, dmax = compare_codes(gpu_codes, ora_codes, K, bits)
    log(f"  {what} codes: mismatch fraction {frac:.2e}, max diff {dmax}")
    assert dmax <= 1, f"{what}: a code differs by {dmax} LSB"
    assert frac <= CODE_MISMATCH_FRAC, f"{what}: {frac:.3e} of codes differ"
    gs = np.asarray(gpu_scale, np.float32)
    rel = np.abs(gs.astype(np.float64) - ora_scale.astype(np.float64)) / np.maximum(np.abs(ora_scale), 1e-30)
    assert np.all(rel <= 1e-5), f"{what}: act_scale rel diff {rel.max():.3e}"
    return frac


def bf16_half_ulp(v):
    a = np.abs(v)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 8)


def epilogue_magnitude(acc, sa, sw, bias=None, residual_bits=None):
    """|acc * s_m * s_n| + |bias_n| + |residual_mn| per output: the scale of the
    epilogue's float32 rounding."""
    mag = np.abs(acc.astype(np.float64) * sa.astype(np.float64)[:, None] * sw.astype(np.float64)[None, :])
    if bias is not None:
        mag = mag + np.abs(bias.astype(np.float64))[None, :]
    if residual_bits is not None:
        mag = mag + np.abs(bf16_to_f64(residual_bits))
    return mag


def assert_y_within(y_gpu_bits, y_f64, mag, what=""):
    """Each bf16 output within half a bf16 ulp of the oracle's float64 value plus
    the float32 rounding of the epilogue's three operations (2^-21 of `mag`)."""
    yg = bf16_to_f64(y_gpu_bits)
    bound = bf16_half_ulp(y_f64) * (1 + 1e-6) + mag * 2.0 ** -21
    err = np.abs(yg - y_f64)
    bad = err > bound
    log(f"  {what} y: max err/bound {np.max(err / np.maximum(bound, 1e-300)):.3f}")
    assert not np.any(bad), f"{what}: {np.count_nonzero(bad)} outputs outside the bound, e.g. " \
                            f"{yg[bad][:4]} vs {y_f64[bad][:4]}"


def assert_y_elementwise(y_gpu_bits, y_f64, acc, sa, sw, bias=None, residual_bits=None, what=""):
    """Identical codes: each bf16 output within half a bf16 ulp of the oracle's
    float64 value plus the float32 rounding of the epilogue."""
    assert_y_within(y_gpu_bits, y_f64, epilogue_magnitude(acc, sa, sw, bias, residual_bits), what)


def rel_fro(y_gpu_bits, y_f64):
    yg = bf16_to_f64(y_gpu_bits)
    return float(np.linalg.norm(yg - y_f64) / max(np.linalg.norm(y_f64), 1e-300))


def assert_y_fro(y_gpu_bits, y_f64, what=""):
    r = rel_fro(y_gpu_bits, y_f64)
    log(f"  {what} y: rel Frobenius {r:.3e}")
    assert r <= Y_REL_FRO, f"{what}: rel Frobenius {r:.3e} > {Y_REL_FRO}"
    return r

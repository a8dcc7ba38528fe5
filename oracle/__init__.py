"""FoldQuant CPU oracle -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct CPU implementation of the FoldQuant integer
linear layer (C in ``fqo.c``, loaded here with ctypes).  Only ``tests/``, the
package smoke check and the benchmark's CPU-baseline leg may use it; the HIP
library never does, and the two share no code.

Every function below cites the passage of the vla.cpp pull request page
"FoldQuant W8A8/W4A4 inference and FoldQuantVLA quantized-model converter" that
it follows (section named in the docstring), and documents the reading taken
where that page leaves a step open.

Code width 6 (``E2M3``) is a storage form of the 4-bit codes, not a third
quantiser: the same integers in [-7, 7] (qmax 7), each kept as a 6-bit OCP FP6
E2M3 number (sign bit 5, two exponent bits with bias 1, three mantissa bits;
exponent 0 is subnormal), which represents every one of them exactly.  Value k
of a row sits in bits 6k .. 6k+5 of the row's bytes read as one little-endian
bit string (3K/4 bytes per row).  Here it is a conversion wrapped around the
4-bit functions: quantise with 4 bits, then re-store (``pack_e2m3``), and read
back (``unpack_codes``) before the integer contraction.

Pins: every function here is checked by ``tests/test_oracle_pins.py`` against
closed forms, library routines (scipy's Sylvester Hadamard, numpy matmul and
round-half-even, torch's bfloat16 cast), invariants and brute force.  The
bit-level float details beyond those (reduction order of the float sums, the
exact float32 constant 1/sqrt(b)) are *parity unpinned*: they are readings.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

from .build import LIB, build

__all__ = [
    "lib", "hadamard_entry", "rotate_f64", "butterfly_f32", "fold_gain", "fold_weights",
    "pack_weights", "unfold_weights", "act_frame", "prologue", "gemm_i32", "epilogue",
    "bf16_from_f64", "code_at", "num_threads", "unpack_codes", "linear", "row_bytes", "qmax", "geglu",
    "E2M3", "e2m3_value", "e2m3_code", "pack_e2m3", "storage_bits",
]

E2M3 = 6  # code width argument: 4-bit codes stored as FP6 E2M3

_lib = None

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_F = ctypes.c_float


def lib():
    """Load (building first if absent) the oracle shared library."""
    global _lib
    if _lib is None:
        path = os.environ.get("FQO_LIB") or LIB  # FQO_LIB: the host-sanitizer build of the oracle
        if path == LIB and not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(path)
        L.fqo_hadamard_entry.argtypes = [_I32, _I32, _I32]
        L.fqo_rotate_f64.argtypes = [_P, _I64, _I32]
        L.fqo_butterfly_f32.argtypes = [_P, _I64, _I32]
        L.fqo_fold_gain.argtypes = [_P, _P, _I32, _P]
        L.fqo_fold_weights.argtypes = [_P, _I32, _I32, _P, _I32, _I32, _P]
        L.fqo_pack_weights.argtypes = [_P, _I32, _I32, _P, _I32, _I32, _I32, _P, _P]
        L.fqo_unfold_weights.argtypes = [_P, _P, _I32, _I32, _P, _I32, _I32, _I32, _P]
        L.fqo_act_frame.argtypes = [_P, _I32, _I32, _I64, _P, _F, _P, _I32, _I32, _P]
        L.fqo_prologue.argtypes = [_P, _I32, _I32, _I64, _P, _F, _P, _I32, _I32, _I32, _P, _P]
        L.fqo_gemm_i32.argtypes = [_P, _I32, _I32, _P, _I32, _I32, _I32, _P]
        L.fqo_geglu.argtypes = [_P, _I32, _I32, _I64, _P, _I64, _P]
        L.fqo_epilogue.argtypes = [_P, _I32, _I32, _P, _P, _P, _P, _I64, _P, _P]
        L.fqo_bf16_from_f64.argtypes = [ctypes.c_double]
        L.fqo_bf16_from_f64.restype = ctypes.c_uint16
        L.fqo_code_at.argtypes = [_P, _I32, _I32]
        L.fqo_num_threads.argtypes = []
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _check(rc: int, what: str):
    if rc < 0:
        raise ValueError(f"oracle {what}: bad argument (rc={rc})")


def qmax(bits: int) -> int:
    """Symmetric code range: +-127 for 8 bits, +-7 for 4 bits ("15 activation levels",
    OpenVINO commit); the E2M3 storage holds the 4-bit codes."""
    return {8: 127, 4: 7, E2M3: 7}[bits]


def storage_bits(bits: int) -> int:
    """The quantiser width behind a code width argument (E2M3 stores 4-bit codes)."""
    return 4 if bits == E2M3 else bits


def row_bytes(K: int, bits: int) -> int:
    return {8: K, 4: K // 2, E2M3: 3 * K // 4}[bits]


def e2m3_value(code: int) -> float:
    """The number a 6-bit FP6 E2M3 code stands for (OCP Microscaling formats
    specification, FP6 E2M3: exponent bias 1, no infinities or NaN): sign bit 5,
    exponent e = bits 4..3, mantissa m = bits 2..0; e = 0 gives m/8, otherwise
    2^(e-1) (1 + m/8)."""
    if not 0 <= code < 64:
        raise ValueError(f"e2m3_value: {code} is not a 6-bit code")
    sign = -1.0 if code & 32 else 1.0
    e, m = (code >> 3) & 3, code & 7
    mag = m / 8.0 if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 8.0)
    return sign * mag


def e2m3_code(v: int) -> int:
    """The E2M3 code of an integer code v in [-7, 7]: the 6-bit pattern whose value
    is v (+0 for zero), found by search over the 64 patterns."""
    if not -7 <= v <= 7:
        raise ValueError(f"e2m3_code: {v} is outside [-7, 7]")
    if v == 0:
        return 0
    for c in range(64):
        if e2m3_value(c) == float(v):
            return c
    raise AssertionError("unreachable: every integer in [-7, 7] is an E2M3 number")


_E2M3_OF = None  # code of v + 7, v in [-7, 7]
_VAL_OF = None   # integer value of each 6-bit pattern (or 99 where it is no integer code)


def _tables():
    global _E2M3_OF, _VAL_OF
    if _E2M3_OF is None:
        _E2M3_OF = np.array([e2m3_code(v) for v in range(-7, 8)], np.uint32)
        vals = [e2m3_value(c) for c in range(64)]
        _VAL_OF = np.array([int(x) if x == int(x) and abs(x) <= 7 else 99 for x in vals], np.int32)
    return _E2M3_OF, _VAL_OF


def pack_e2m3(ints: np.ndarray) -> np.ndarray:
    """Rows of integer codes in [-7, 7] -> E2M3 rows: value k in bits 6k .. 6k+5 of the
    row's little-endian bit string (four values = three bytes)."""
    q = np.asarray(ints)
    if q.ndim != 2 or q.shape[1] % 4:
        raise ValueError("pack_e2m3: rows of a multiple of 4 codes")
    if q.size and (q.min() < -7 or q.max() > 7):
        raise ValueError("pack_e2m3: codes outside [-7, 7]")
    enc, _ = _tables()
    c = enc[q.astype(np.int64) + 7].reshape(q.shape[0], q.shape[1] // 4, 4)
    word = c[..., 0] | (c[..., 1] << 6) | (c[..., 2] << 12) | (c[..., 3] << 18)
    out = np.empty((q.shape[0], q.shape[1] // 4, 3), np.uint8)
    out[..., 0] = word & 0xFF
    out[..., 1] = (word >> 8) & 0xFF
    out[..., 2] = (word >> 16) & 0xFF
    return out.reshape(q.shape[0], 3 * q.shape[1] // 4)


def _to_nibbles(codes, K: int) -> np.ndarray:
    """E2M3 rows -> the packed 4-bit rows of the same integers."""
    q = unpack_codes(codes, K, E2M3)
    lo = (q[:, 0::2] & 0xF).astype(np.uint8)
    hi = (q[:, 1::2] & 0xF).astype(np.uint8)
    return lo | (hi << 4)


def hadamard_entry(b: int, i: int, j: int) -> int:
    """H_b[i][j] of the Sylvester construction (dequant-mode commit)."""
    return lib().fqo_hadamard_entry(b, i, j)


def rotate_f64(v: np.ndarray, b: int) -> np.ndarray:
    """R_b v in float64: block butterfly then 1/sqrt(b) (dequant-mode commit)."""
    out = np.array(v, dtype=np.float64, copy=True, order="C")
    _check(lib().fqo_rotate_f64(_p(out), out.size, b), "rotate_f64")
    return out


def butterfly_f32(v: np.ndarray, b: int) -> np.ndarray:
    """Unnormalised H_b per block in float32, stage spans 1, 2, ..., b/2."""
    out = np.array(v, dtype=np.float32, copy=True, order="C")
    _check(lib().fqo_butterfly_f32(_p(out), out.size, b), "butterfly_f32")
    return out


def fold_gain(gamma: np.ndarray, ascale: Optional[np.ndarray]) -> np.ndarray:
    """gamma / a in float32: the smoothing vector folded into the RMSNorm gain
    (dequant-mode commit: the LLM sites' SmoothQuant vector is in the norm gains)."""
    g = _c(gamma, np.float32)
    a = _c(ascale, np.float32)
    out = np.empty_like(g)
    _check(lib().fqo_fold_gain(_p(g), _p(a), g.size, _p(out)), "fold_gain")
    return out


def fold_weights(W, ascale, fold_after: int, hblock: int) -> np.ndarray:
    """Folded float64 weight rows u_n = R(a.w_n) or a.R(w_n), unquantised."""
    W = _c(W, np.float32)
    a = _c(ascale, np.float32)
    N, K = W.shape
    U = np.empty((N, K), np.float64)
    _check(lib().fqo_fold_weights(_p(W), N, K, _p(a), fold_after, hblock, _p(U)), "fold_weights")
    return U


def pack_weights(W, ascale, fold_after: int, hblock: int, wbits: int):
    """Per-row symmetric RTN (ties to even) of the folded rows; returns (codes, wscale).
    Runtime summary ("INT8 or INT4 codes with per-row scales") and the converter's
    bring-up export ("rotation and per-row RTN")."""
    W = _c(W, np.float32)
    a = _c(ascale, np.float32)
    N, K = W.shape
    qb = storage_bits(wbits)
    codes = np.zeros((N, row_bytes(K, qb)), np.uint8)
    ws = np.empty(N, np.float32)
    _check(lib().fqo_pack_weights(_p(W), N, K, _p(a), fold_after, hblock, qb, _p(codes), _p(ws)),
           "pack_weights")
    if wbits == E2M3:
        codes = pack_e2m3(unpack_codes(codes, K, 4))
    return codes, ws


def unfold_weights(codes, wscale, K: int, ascale, fold_after: int, hblock: int, wbits: int):
    """Dequantised rows in the original frame: R(s q)/a or R(s q / a) (dequant-mode commit)."""
    if wbits == E2M3:
        codes, wbits = _to_nibbles(codes, K), 4
    codes = _c(codes, np.uint8)
    ws = _c(wscale, np.float32)
    a = _c(ascale, np.float32)
    N = codes.shape[0]
    out = np.empty((N, K), np.float64)
    _check(lib().fqo_unfold_weights(_p(codes), _p(ws), N, K, _p(a), fold_after, hblock, wbits,
                                    _p(out)), "unfold_weights")
    return out


def act_frame(x_bits, gamma, eps: float, ascale, fold_after: int, hblock: int) -> np.ndarray:
    """Float32 activation frame before quantisation (OpenVINO commit's act-node steps)."""
    x = _c(x_bits, np.uint16)
    M, K = x.shape
    h = np.empty((M, K), np.float32)
    _check(lib().fqo_act_frame(_p(x), M, K, K, _p(_c(gamma, np.float32)), eps,
                               _p(_c(ascale, np.float32)), fold_after, hblock, _p(h)), "act_frame")
    return h


def prologue(x_bits, gamma, eps: float, ascale, fold_after: int, hblock: int, abits: int):
    """Codes and per-token scales: amax scale, round-half-even, clamp (OpenVINO commit)."""
    x = _c(x_bits, np.uint16)
    M, K = x.shape
    qb = storage_bits(abits)
    codes = np.zeros((M, row_bytes(K, qb)), np.uint8)
    sc = np.empty(M, np.float32)
    _check(lib().fqo_prologue(_p(x), M, K, K, _p(_c(gamma, np.float32)), eps,
                              _p(_c(ascale, np.float32)), fold_after, hblock, qb, _p(codes),
                              _p(sc)), "prologue")
    if abits == E2M3:
        codes = pack_e2m3(unpack_codes(codes, K, 4))
    return codes, sc


def gemm_i32(act_codes, abits: int, w_codes, wbits: int, K: int) -> np.ndarray:
    """Exact integer contraction of the codes (runtime summary: integer GEMMs;
    SYCL commit: integer sums are exact in any order).  E2M3 rows are read back to
    their integers first."""
    if abits == E2M3:
        act_codes, abits = _to_nibbles(act_codes, K), 4
    if wbits == E2M3:
        w_codes, wbits = _to_nibbles(w_codes, K), 4
    A = _c(act_codes, np.uint8)
    B = _c(w_codes, np.uint8)
    M, N = A.shape[0], B.shape[0]
    acc = np.empty((M, N), np.int32)
    rc = lib().fqo_gemm_i32(_p(A), M, abits, _p(B), N, K, wbits, _p(acc))
    _check(rc, "gemm_i32")
    if rc == 1:
        raise OverflowError("oracle gemm_i32: a sum does not fit in int32")
    return acc


def epilogue(acc, act_scale, wscale, bias=None, residual_bits=None, want_f64: bool = False):
    """y = bf16(acc * s_a * s_w + bias + residual) from float64 (runtime summary:
    residual add in the epilogue; OpenVINO commit: dequantised by wscale)."""
    acc = _c(acc, np.int32)
    M, N = acc.shape
    y = np.empty((M, N), np.uint16)
    yf = np.empty((M, N), np.float64) if want_f64 else None
    res = _c(residual_bits, np.uint16)
    _check(lib().fqo_epilogue(_p(acc), M, N, _p(_c(act_scale, np.float32)),
                              _p(_c(wscale, np.float32)), _p(_c(bias, np.float32)), _p(res),
                              N if res is None else res.shape[1], _p(y), _p(yf)), "epilogue")
    return (y, yf) if want_f64 else y


def geglu(gu_bits, F: int, want_f64: bool = False):
    """h = bf16(gelu_tanh(gate) * up) for rows [gate F | up F] (the chained MLP
    block between the gate+up and down sites); float64 inside, one rounding."""
    gu = _c(gu_bits, np.uint16)
    M = gu.shape[0]
    h = np.empty((M, F), np.uint16)
    hf = np.empty((M, F), np.float64) if want_f64 else None
    _check(lib().fqo_geglu(_p(gu), M, F, gu.shape[1], _p(h), F, _p(hf)), "geglu")
    return (h, hf) if want_f64 else h


def bf16_from_f64(v: float) -> int:
    """Nearest-even bfloat16 bits of a float64 (one rounding)."""
    return int(lib().fqo_bf16_from_f64(float(v)))


def num_threads() -> int:
    """Threads the oracle's OpenMP loops use."""
    return int(lib().fqo_num_threads())


def code_at(row: np.ndarray, k: int, bits: int) -> int:
    if bits == E2M3:
        return int(unpack_codes(np.asarray(row, np.uint8).reshape(1, -1), 4 * len(row) // 3, E2M3)[0, k])
    r = _c(row, np.uint8)
    return int(lib().fqo_code_at(_p(r), k, bits))


def unpack_codes(codes: np.ndarray, K: int, bits: int) -> np.ndarray:
    """Integer codes [rows][K] from int8, packed 4-bit (even k in the low nibble) or
    E2M3 storage (value k in bits 6k .. 6k+5; a pattern that is no integer code
    in [-7, 7] raises)."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    if bits == E2M3:
        _, val = _tables()
        b = c.reshape(c.shape[0], K // 4, 3).astype(np.uint32)
        word = b[..., 0] | (b[..., 1] << 8) | (b[..., 2] << 16)
        f = np.stack([(word >> (6 * j)) & 63 for j in range(4)], axis=-1).reshape(c.shape[0], K)
        out = val[f]
        if (out == 99).any():
            raise ValueError("unpack_codes: an E2M3 pattern that is not an integer code in [-7, 7]")
        return out
    if bits == 8:
        return c.view(np.int8).astype(np.int32).reshape(c.shape[0], K)
    lo = (c & 0xF).astype(np.int32)
    hi = (c >> 4).astype(np.int32)
    out = np.empty((c.shape[0], K), np.int32)
    out[:, 0::2] = np.where(lo >= 8, lo - 16, lo)
    out[:, 1::2] = np.where(hi >= 8, hi - 16, hi)
    return out


def linear(wl, codes_w=None, wscale=None):
    """Whole site for a ``synth.Workload``: fold gain (norm sites), pack, prologue,
    GEMM, epilogue.  Returns a dict with every intermediate."""
    gamma = wl.gamma
    pro_a = None
    if gamma is not None and wl.fold_into_gain:
        gamma = fold_gain(wl.gamma, wl.ascale)
    elif wl.ascale is not None:
        pro_a = wl.ascale
    if codes_w is None:
        codes_w, wscale = pack_weights(wl.W, wl.ascale, wl.fold_after, wl.hblock, wl.wbits)
    codes_a, sa = prologue(wl.x, gamma, wl.eps, pro_a, wl.fold_after, wl.hblock, wl.abits)
    acc = gemm_i32(codes_a, wl.abits, codes_w, wl.wbits, wl.K)
    y, yf = epilogue(acc, sa, wscale, wl.bias, wl.residual, want_f64=True)
    return dict(gamma_folded=gamma, prologue_ascale=pro_a, codes_w=codes_w, wscale=wscale,
                codes_a=codes_a, act_scale=sa, acc=acc, y=y, y_f64=yf)

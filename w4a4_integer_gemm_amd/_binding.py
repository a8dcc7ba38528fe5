"""ctypes binding of libfq (include/fq.h).  Argument marshalling only.

Device entry points take torch tensors that already live on the GPU and pass
their data pointers plus the current HIP stream; every step of the layer runs
in libfq's kernels.  Host entry points take numpy arrays.  There is no
fallback: if libfq.so is missing or a call fails, an exception says why.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# FQ_LIB selects another build of the same library (the host-sanitizer build)
LIB_PATH = os.environ.get("FQ_LIB") or os.path.join(HERE, "libfq.so")

E2M3 = 6  # FQ_CODES_E2M3: the 4-bit codes stored as FP6 E2M3 (include/fq.h)

FQ_OK = 0
_STATUS = {0: "FQ_OK", 1: "FQ_ERR_ARG", 2: "FQ_ERR_SHAPE", 3: "FQ_ERR_UNSUPPORTED", 4: "FQ_ERR_ALIGN",
           5: "FQ_ERR_DEVICE"}

# exported symbols and their signatures (must match include/fq.h)
_P, _I32, _I64, _F, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "fq_last_error": ([], ctypes.c_char_p),
    "fq_abi_version": ([], ctypes.c_int),
    "fq_device_init": ([], ctypes.c_int),
    "fq_test_hook": ([ctypes.c_char_p], ctypes.c_int),
    "fq_weight_bytes": ([_I32, _I32, _I32], _SZ),
    "fq_act_bytes": ([_I32, _I32, _I32], _SZ),
    "fq_fold_gain": ([_P, _P, _I32, _P], ctypes.c_int),
    "fq_pack_weights": ([_P, _I32, _I32, _P, _I32, _I32, _I32, _P, _P], ctypes.c_int),
    "fq_dequant_rows": ([_P, _P, _I32, _I32, _P, _I32, _I32, _I32, _P], ctypes.c_int),
    "fq_prologue": ([_P, _I32, _I32, _I64, _P, _F, _P, _I32, _I32, _I32, _P, _P, _P], ctypes.c_int),
    "fq_gemm": ([_P, _P, _I32, _I32, _P, _P, _I32, _I32, _I32, _P, _P, _I64, _P, _I64, _P, _P], ctypes.c_int),
    "fq_geglu": ([_P, _I32, _I32, _I64, _P, _I64, _P], ctypes.c_int),
    "fq_gemm_heads": ([_P, _P, _I32, _I32, _P, _P, _I32, _I32, _I32, _P, _P, _I64, _I32, _P, _P, _P], ctypes.c_int),
    "fq_linear_workspace_bytes": ([_I32, _I32, _I32], _SZ),
    "fq_linear": ([_P, _I32, _I32, _I64, _P, _F, _P, _I32, _I32, _I32, _P, _P, _I32, _I32, _P, _P, _I64, _P,
                   _I64, _P, _SZ, _P], ctypes.c_int),
    "fq_linear_noalloc": ([_P, _I32, _I32, _I64, _P, _F, _P, _I32, _I32, _I32, _P, _P, _I32, _I32, _P, _P, _I64, _P,
                           _I64, _P], ctypes.c_int),
    "fq_linear_noalloc_max_bytes": ([], _SZ),
    "fq_linear_heads": ([_P, _I32, _I32, _I64, _P, _F, _P, _I32, _I32, _I32, _P, _P, _I32, _I32, _P, _P, _I64,
                         _I32, _P, _P, _SZ, _P], ctypes.c_int),
}


class FqError(RuntimeError):
    """A libfq call returned a status other than FQ_OK."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status
        self.message = message


_lib = None


def lib() -> ctypes.CDLL:
    """Load libfq.so from the package directory (built by build.py)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libfq.so not found at {LIB_PATH}; build it with "
                               "`python w4a4_integer_gemm_amd/build.py` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _check(rc: int):
    if rc != FQ_OK:
        raise FqError(rc, lib().fq_last_error().decode())


def last_error() -> str:
    return lib().fq_last_error().decode()


def abi_version() -> int:
    return lib().fq_abi_version()


def fq_device_init():
    """Per-device set-up of the current device (optional; see include/fq.h)."""
    _check(lib().fq_device_init())


def fq_test_hook(spec: Optional[str]):
    """Force kernel choices for the tests ("gemm_tile=64x128,gemm_mfma=32,gemv=split"; "" resets)."""
    _check(lib().fq_test_hook(None if spec is None else spec.encode()))


# ------------------------------------------------------------------ host entry points
def _np_ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def fq_weight_bytes(N: int, K: int, wbits: int) -> int:
    return lib().fq_weight_bytes(N, K, wbits)


def fq_act_bytes(M: int, K: int, abits: int) -> int:
    return lib().fq_act_bytes(M, K, abits)


def fq_linear_workspace_bytes(M: int, K: int, abits: int) -> int:
    return lib().fq_linear_workspace_bytes(M, K, abits)


def fq_fold_gain(gamma: np.ndarray, ascale: Optional[np.ndarray]) -> np.ndarray:
    g = np.ascontiguousarray(gamma, dtype=np.float32)
    a = None if ascale is None else np.ascontiguousarray(ascale, dtype=np.float32)
    out = np.empty_like(g)
    _check(lib().fq_fold_gain(_np_ptr(g), _np_ptr(a), g.size, _np_ptr(out)))
    return out


def fq_pack_weights(W: np.ndarray, ascale: Optional[np.ndarray], fold_after: int, hblock: int, wbits: int):
    """Host packer; returns (codes uint8 [N][K, K/2 or 3K/4 (E2M3)], wscale float32 [N])."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    a = None if ascale is None else np.ascontiguousarray(ascale, dtype=np.float32)
    nbytes = fq_weight_bytes(N, K, wbits)
    codes = np.zeros((N, nbytes // N if nbytes else 0), np.uint8)
    ws = np.empty(N, np.float32)
    _check(lib().fq_pack_weights(_np_ptr(W), N, K, _np_ptr(a), fold_after, hblock, wbits, _np_ptr(codes),
                                 _np_ptr(ws)))
    return codes, ws


def fq_dequant_rows(codes: np.ndarray, wscale: np.ndarray, K: int, ascale: Optional[np.ndarray], fold_after: int,
                    hblock: int, wbits: int) -> np.ndarray:
    """Host dequantisation to float rows in the original frame; returns float32 [N][K]."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    ws = np.ascontiguousarray(wscale, dtype=np.float32)
    N = ws.shape[0]
    a = None if ascale is None else np.ascontiguousarray(ascale, dtype=np.float32)
    out = np.empty((N, K), np.float32)
    _check(lib().fq_dequant_rows(_np_ptr(codes), _np_ptr(ws), N, K, _np_ptr(a), fold_after, hblock, wbits,
                                 _np_ptr(out)))
    return out


# ------------------------------------------------------------------ device entry points
def _dptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("device entry points need GPU tensors")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    """The hipStream_t of `stream`, or of the current device's current stream.
    (torch.cuda.current_stream() builds a Stream object: about 2.7 us per call,
    a fifth of a small layer's host time; the raw accessor returns the handle.)"""
    import torch
    if stream is not None:
        return stream.cuda_stream
    C = torch._C
    if hasattr(C, "_cuda_getCurrentRawStream"):
        return C._cuda_getCurrentRawStream(C._cuda_getDevice())
    return torch.cuda.current_stream().cuda_stream


def fq_prologue(x, M: int, K: int, ldx: int, gamma_folded, eps: float, ascale, fold_after: int, hblock: int,
                abits: int, act_codes, act_scale, stream=None):
    _check(lib().fq_prologue(_dptr(x), M, K, ldx, _dptr(gamma_folded), eps, _dptr(ascale), fold_after, hblock,
                             abits, _dptr(act_codes), _dptr(act_scale), _stream(stream)))


def fq_gemm(act_codes, act_scale, M: int, abits: int, w_codes, wscale, N: int, K: int, wbits: int, bias,
            residual, ldr: int, y, ldy: int, acc=None, stream=None):
    _check(lib().fq_gemm(_dptr(act_codes), _dptr(act_scale), M, abits, _dptr(w_codes), _dptr(wscale), N, K, wbits,
                         _dptr(bias), _dptr(residual), ldr, _dptr(y), ldy, _dptr(acc), _stream(stream)))


def fq_linear(x, M: int, K: int, ldx: int, gamma_folded, eps: float, ascale, fold_after: int, hblock: int,
              abits: int, w_codes, wscale, N: int, wbits: int, bias, residual, ldr: int, y, ldy: int, workspace,
              workspace_bytes: int, stream=None):
    _check(lib().fq_linear(_dptr(x), M, K, ldx, _dptr(gamma_folded), eps, _dptr(ascale), fold_after, hblock, abits,
                           _dptr(w_codes), _dptr(wscale), N, wbits, _dptr(bias), _dptr(residual), ldr, _dptr(y),
                           ldy, _dptr(workspace), workspace_bytes, _stream(stream)))


def fq_linear_noalloc(x, M: int, K: int, ldx: int, gamma_folded, eps: float, ascale, fold_after: int, hblock: int,
                      abits: int, w_codes, wscale, N: int, wbits: int, bias, residual, ldr: int, y, ldy: int,
                      stream=None):
    _check(lib().fq_linear_noalloc(_dptr(x), M, K, ldx, _dptr(gamma_folded), eps, _dptr(ascale), fold_after, hblock,
                                   abits, _dptr(w_codes), _dptr(wscale), N, wbits, _dptr(bias), _dptr(residual), ldr,
                                   _dptr(y), ldy, _stream(stream)))


def fq_linear_noalloc_max_bytes() -> int:
    return lib().fq_linear_noalloc_max_bytes()


def fq_gemm_heads(act_codes, act_scale, M: int, abits: int, w_codes, wscale, N: int, K: int, wbits: int, bias,
                  residual, ldr: int, head_dim: int, y, acc=None, stream=None):
    _check(lib().fq_gemm_heads(_dptr(act_codes), _dptr(act_scale), M, abits, _dptr(w_codes), _dptr(wscale), N, K,
                               wbits, _dptr(bias), _dptr(residual), ldr, head_dim, _dptr(y), _dptr(acc),
                               _stream(stream)))


def fq_linear_heads(x, M: int, K: int, ldx: int, gamma_folded, eps: float, ascale, fold_after: int, hblock: int,
                    abits: int, w_codes, wscale, N: int, wbits: int, bias, residual, ldr: int, head_dim: int, y,
                    workspace, workspace_bytes: int, stream=None):
    _check(lib().fq_linear_heads(_dptr(x), M, K, ldx, _dptr(gamma_folded), eps, _dptr(ascale), fold_after, hblock,
                                 abits, _dptr(w_codes), _dptr(wscale), N, wbits, _dptr(bias), _dptr(residual), ldr,
                                 head_dim, _dptr(y), _dptr(workspace), workspace_bytes, _stream(stream)))


def fq_geglu(gateup, M: int, F: int, ld_in: int, h, ld_out: int, stream=None):
    _check(lib().fq_geglu(_dptr(gateup), M, F, ld_in, _dptr(h), ld_out, _stream(stream)))

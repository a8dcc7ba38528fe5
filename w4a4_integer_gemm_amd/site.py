"""A FoldQuant linear site resident on the GPU (device buffers + calls into libfq).

Holds the packed weight codes, scales, folded gain, smoothing vector and the
workspace as torch tensors, and calls the C ABI on them.  Packing runs in
libfq's host packer; everything else runs in libfq's kernels.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from . import _binding as B


def _to_dev(a: Optional[np.ndarray], device):
    import torch
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


class DeviceSite:
    """One linear site: x [M][K] bf16 -> y [M][N] bf16.

    gamma: RMSNorm gain (None for a quant-only site); ascale: smoothing vector;
    fold_into_gain: carry ascale inside the gain (gamma / a, fold before) rather
    than as an explicit divide in the prologue."""

    def __init__(self, W: np.ndarray, hblock: int, wbits: int, abits: int, gamma=None, ascale=None,
                 fold_after: int = 0, fold_into_gain: bool = True, bias=None, eps: float = 1e-6,
                 device="cuda", codes=None, wscale=None):
        import torch
        # (code bytes per row: K * bits / 8, with 6 bits for the E2M3 storage)
        self.N, self.K = W.shape if W is not None else (codes.shape[0], codes.shape[1] * 8 // wbits)
        self.hblock, self.wbits, self.abits = hblock, wbits, abits
        self.eps, self.fold_after = float(eps), int(fold_after)
        self.device = torch.device(device)
        if codes is None:
            codes, wscale = B.fq_pack_weights(W, ascale, fold_after, hblock, wbits)
        self.codes_host, self.wscale_host = codes, wscale
        self.codes = _to_dev(codes, self.device)
        self.wscale = _to_dev(wscale, self.device)
        if gamma is not None and fold_into_gain:
            if fold_after:
                raise ValueError("a gain fold is a fold before the rotation; pass fold_after=0")
            self.gamma_host = B.fq_fold_gain(gamma, ascale)
            self.ascale_host = None
        else:
            self.gamma_host = None if gamma is None else np.ascontiguousarray(gamma, np.float32)
            self.ascale_host = None if ascale is None else np.ascontiguousarray(ascale, np.float32)
        self.gamma = _to_dev(self.gamma_host, self.device)
        self.ascale = _to_dev(self.ascale_host, self.device)
        self.bias = _to_dev(None if bias is None else np.ascontiguousarray(bias, np.float32), self.device)
        self._ws = None
        self._ws_bytes = {}  # M -> fq_linear_workspace_bytes

    # -- buffers
    def workspace(self, M: int):
        import torch
        nbytes = self._ws_bytes.get(M)
        if nbytes is None:
            nbytes = self._ws_bytes[M] = B.fq_linear_workspace_bytes(M, self.K, self.abits)
        if self._ws is None or self._ws.numel() < nbytes:
            self._ws = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        return self._ws

    def empty_out(self, M: int):
        import torch
        return torch.empty((M, self.N), dtype=torch.int16, device=self.device)

    def empty_codes(self, M: int):
        import torch
        return (torch.empty(B.fq_act_bytes(M, self.K, self.abits), dtype=torch.uint8, device=self.device),
                torch.empty(M, dtype=torch.float32, device=self.device))

    # -- calls
    def prologue(self, x, codes=None, scales=None, stream=None):
        M = x.shape[0]
        if codes is None:
            codes, scales = self.empty_codes(M)
        B.fq_prologue(x, M, self.K, x.stride(0), self.gamma, self.eps, self.ascale, self.fold_after,
                      self.hblock, self.abits, codes, scales, stream)
        return codes, scales

    def gemm(self, codes, scales, M: int, residual=None, y=None, acc=None, stream=None):
        if y is None:
            y = self.empty_out(M)
        B.fq_gemm(codes, scales, M, self.abits, self.codes, self.wscale, self.N, self.K, self.wbits, self.bias,
                  residual, 0 if residual is None else residual.stride(0), y, y.stride(0), acc, stream)
        return y

    def linear(self, x, residual=None, y=None, stream=None):
        M = x.shape[0]
        if y is None:
            y = self.empty_out(M)
        ws = self.workspace(M)
        B.fq_linear(x, M, self.K, x.stride(0), self.gamma, self.eps, self.ascale, self.fold_after, self.hblock,
                    self.abits, self.codes, self.wscale, self.N, self.wbits, self.bias, residual,
                    0 if residual is None else residual.stride(0), y, y.stride(0), ws, ws.numel(), stream)
        return y

    def linear_noalloc(self, x, residual=None, y=None, stream=None):
        """fq_linear_noalloc: as linear(), with the library's per-GPU scratch array as the workspace."""
        M = x.shape[0]
        if y is None:
            y = self.empty_out(M)
        B.fq_linear_noalloc(x, M, self.K, x.stride(0), self.gamma, self.eps, self.ascale, self.fold_after,
                            self.hblock, self.abits, self.codes, self.wscale, self.N, self.wbits, self.bias, residual,
                            0 if residual is None else residual.stride(0), y, y.stride(0), stream)
        return y

    def linear_heads(self, x, head_dim: int, residual=None, y=None, stream=None):
        """fq_linear_heads: y is [N / head_dim][M][head_dim] (int16 tensor of bf16 bits)."""
        import torch
        M = x.shape[0]
        if y is None:
            y = torch.empty((self.N // head_dim, M, head_dim), dtype=torch.int16, device=self.device)
        ws = self.workspace(M)
        B.fq_linear_heads(x, M, self.K, x.stride(0), self.gamma, self.eps, self.ascale, self.fold_after, self.hblock,
                          self.abits, self.codes, self.wscale, self.N, self.wbits, self.bias, residual,
                          0 if residual is None else residual.stride(0), head_dim, y, ws, ws.numel(), stream)
        return y

    def workspace_codes(self, M: int):
        """(codes, scales) views of the workspace after fq_linear."""
        import torch
        ws = self.workspace(M)
        nb = B.fq_act_bytes(M, self.K, self.abits)
        off = (nb + 255) // 256 * 256
        return ws[:nb], ws[off:off + 4 * M].view(torch.float32)

    @staticmethod
    def upload(a, device="cuda"):
        return _to_dev(a, device)

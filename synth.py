"""Seeded synthetic inputs for the FoldQuant integer linear layer.

This module is shared by the tests, the benchmark and the CPU oracle's callers.
It only draws random numbers and arranges them into the shapes, value
distributions and structure of the workloads described on the pages (a VLA
language backbone's projections: Qwen2.5-7B-shaped QKV, MLP down projection and
fused gate+up decode, and a Gemma-2B-shaped W4A4 MLP).  It holds none of the
FoldQuant arithmetic (no Hadamard rotation, no quantisation, no GEMM).

Conventions
- bf16 tensors are carried as ``numpy.uint16`` bit patterns; ``f32_to_bf16_bits``
  rounds float32 draws to nearest-even, ``bf16_bits_to_f32`` widens exactly.
- Every tensor of a workload gets its own child seed from
  ``numpy.random.SeedSequence(seed).spawn``, so changing how one tensor is drawn
  never shifts another (the Alpamayo reflection page, section on the diffusion
  noise seed, shows what a shared stream does to reproducibility).
- The smoothing vector ``ascale`` follows SmoothQuant's migration rule
  a_j = max_m|X_mj|^alpha / max_n|W_nj|^(1-alpha) with alpha = 0.5, taken over a
  *separate* calibration batch drawn with the same recipe.  X is the raw
  activation channel maximum times the RMSNorm gain; the per-token RMS factor of
  the norm is left out of the statistic (it is a per-token scalar close to 1
  for these distributions).  This is an input recipe, not part of the method:
  the pages take the vector from a calibrated checkpoint.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

__all__ = [
    "f32_to_bf16_bits", "bf16_bits_to_f32", "Workload", "CONFIGS", "make_workload",
    "random_workload",
]


def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    f = np.ascontiguousarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    nan = np.isnan(f)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclass
class Workload:
    """One FoldQuant linear site with its inputs (all host numpy arrays)."""
    name: str
    M: int
    K: int
    N: int
    hblock: int
    wbits: int
    abits: int
    x: np.ndarray                      # uint16 bf16 bits [M][K]
    W: np.ndarray                      # float32 [N][K] (nn.Linear layout)
    gamma: Optional[np.ndarray] = None  # float32 [K] RMSNorm gain (None: quant-only site)
    ascale: Optional[np.ndarray] = None  # float32 [K] smoothing vector (None: a = 1)
    fold_after: int = 0                # 0: x' = R(x/a); 1: x' = R(x)/a
    fold_into_gain: bool = True        # norm sites carry a inside the gain (gamma/a)
    residual: Optional[np.ndarray] = None  # uint16 bf16 bits [M][N]
    bias: Optional[np.ndarray] = None  # float32 [N]
    eps: float = 1e-6
    seed: int = 0
    recipe: str = ""
    extra: Dict[str, object] = field(default_factory=dict)


def _children(seed: int, n: int = 12):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(n)]


def _smoothing(act_absmax: np.ndarray, W: np.ndarray, alpha: float = 0.5) -> np.ndarray:
    """SmoothQuant migration vector from channel maxima (input recipe, see module doc)."""
    wmax = np.abs(W).max(axis=0).astype(np.float64)
    amax = act_absmax.astype(np.float64)
    a = np.power(np.maximum(amax, 1e-12), alpha) / np.power(np.maximum(wmax, 1e-12), 1.0 - alpha)
    return np.maximum(a, 1e-5).astype(np.float32)


def _normal_bf16(rng, M, K):
    return rng.standard_normal((M, K), dtype=np.float32)


def _outlier_channels(rng, K, count):
    return np.sort(rng.choice(K, size=count, replace=False))


def _act_scaled_outliers(rng_x, ch, M, K, factor):
    x = _normal_bf16(rng_x, M, K)
    x[:, ch] *= np.float32(factor)
    return x


def _act_heavy_tail(rng_x, rng_t, ch, M, K, factor, df):
    x = _normal_bf16(rng_x, M, K)
    x[:, ch] = (np.float32(factor) * rng_t.standard_t(df, size=(M, len(ch)))).astype(np.float32)
    return x


def _weights(rng, N, K, std=0.02):
    W = rng.standard_normal((N, K), dtype=np.float32)
    W *= np.float32(std)
    return W


def _silu(a):
    return a / (1.0 + np.exp(-a))


def _gelu_tanh(a):
    return 0.5 * a * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (a + 0.044715 * a ** 3)))


# name -> (M, K, N, hblock, wbits, abits, seed)
CONFIGS = {
    # tiny W8A8 site: 16 tokens, K=256, N=512, block 64, 4 outlier channels x30
    "tiny_w8a8": (16, 256, 512, 64, 8, 8, 0),
    # Qwen2.5-7B fused QKV projection (3584 + 512 + 512 outputs), 1024-token prefill
    "qkv_w8a8": (1024, 3584, 4608, 128, 8, 8, 2),
    # Qwen2.5-7B MLP down projection with the residual add in the epilogue
    "down_w8a8": (1024, 18944, 3584, 128, 8, 8, 3),
    # decode GEMV against the fused gate+up weight (2 x 18944 rows)
    "decode_m1_w8a8": (1, 3584, 37888, 128, 8, 8, 4),
    "decode_m16_w8a8": (16, 3584, 37888, 128, 8, 8, 4),
    # Gemma-2B-shaped W4A4 MLP: gate+up (2 x 16384) then down with residual
    "gateup_w4a4": (816, 2048, 32768, 128, 4, 4, 5),
    "down_w4a4": (816, 16384, 2048, 128, 4, 4, 5),
}


def make_workload(name: str, M: Optional[int] = None, N: Optional[int] = None,
                  with_weights: bool = True) -> Workload:
    """Build one of the named workloads.  ``M``/``N`` may shrink a workload for
    quick tests (same recipe, fewer tokens/rows)."""
    M0, K, N0, hb, wb, ab, seed = CONFIGS[name]
    M = M0 if M is None else M
    N = N0 if N is None else N
    g = _children(seed)
    # children: 0 x, 1 channels, 2 t-draws, 3 gamma, 4 W, 5 calib x, 6 residual, 7 second x
    gamma = None
    ascale = None
    residual = None
    recipe = ""
    W = _weights(g[4], N, K) if with_weights else np.zeros((0, K), np.float32)
    if name == "tiny_w8a8":
        ch = _outlier_channels(g[1], K, 4)
        x = _act_scaled_outliers(g[0], ch, M, K, 30.0)
        xc = _act_scaled_outliers(g[5], ch, 128, K, 30.0)
        recipe = "x ~ N(0,1) bf16 with 4 channels x30; gamma ~ U(0.5,1.5); SmoothQuant alpha=0.5 folded into gamma; W ~ N(0,0.02^2)"
    elif name in ("qkv_w8a8", "decode_m1_w8a8", "decode_m16_w8a8"):
        ch = _outlier_channels(g[1], K, int(round(0.01 * K)))
        x = _act_heavy_tail(g[0], g[2], ch, M, K, 20.0, 2.0)
        xc = _act_heavy_tail(g[5], g[7], ch, 128, K, 20.0, 2.0)
        recipe = "x ~ N(0,1) bf16 with round(1% of K) channels replaced by 20*t(df=2); gamma ~ U(0.5,1.5); SmoothQuant alpha=0.5 folded into gamma; W ~ N(0,0.02^2)"
    elif name == "gateup_w4a4":
        ch = _outlier_channels(g[1], K, 8)
        x = _act_scaled_outliers(g[0], ch, M, K, 25.0)
        xc = _act_scaled_outliers(g[5], ch, 128, K, 25.0)
        recipe = "x ~ N(0,1) bf16 with 8 channels x25; gamma ~ U(0.5,1.5); SmoothQuant alpha=0.5 folded into gamma; W ~ N(0,0.02^2) to INT4"
    elif name == "down_w8a8":
        A = g[0].standard_normal((M, K), dtype=np.float32)
        B = g[2].standard_normal((M, K), dtype=np.float32)
        x = (_silu(A) * B).astype(np.float32)
        residual = f32_to_bf16_bits(g[6].standard_normal((M, N), dtype=np.float32))
        recipe = "x = bf16(SiLU(A)*B), A,B ~ N(0,1); quant-only prologue (no RMSNorm, a = 1); residual ~ N(0,1) bf16; W ~ N(0,0.02^2)"
    elif name == "down_w4a4":
        A = g[0].standard_normal((M, K), dtype=np.float32)
        B = g[2].standard_normal((M, K), dtype=np.float32)
        x = (_gelu_tanh(A) * B).astype(np.float32)
        # residual is the gate+up site's input x (the block's skip connection)
        gu = make_workload("gateup_w4a4", M=M, N=1, with_weights=False)
        residual = gu.x.copy() if gu.K == N else f32_to_bf16_bits(g[6].standard_normal((M, N), dtype=np.float32))
        recipe = "x = bf16(gelu_tanh(A)*B), A,B ~ N(0,1); quant-only prologue; residual = the gate+up site's bf16 input; W ~ N(0,0.02^2) to INT4"
    else:  # pragma: no cover
        raise KeyError(name)

    xb = f32_to_bf16_bits(x)
    if name in ("tiny_w8a8", "qkv_w8a8", "decode_m1_w8a8", "decode_m16_w8a8", "gateup_w4a4"):
        gamma = g[3].uniform(0.5, 1.5, size=K).astype(np.float32)
        if with_weights:
            act_absmax = np.abs(bf16_bits_to_f32(f32_to_bf16_bits(xc))).max(axis=0) * gamma
            ascale = _smoothing(act_absmax, W)
        else:
            ascale = np.ones(K, np.float32)
    return Workload(name=name, M=M, K=K, N=N, hblock=hb, wbits=wb, abits=ab, x=xb, W=W,
                    gamma=gamma, ascale=ascale, fold_after=0, fold_into_gain=gamma is not None,
                    residual=residual, bias=None, eps=1e-6, seed=seed, recipe=recipe)


def random_workload(M: int, K: int, N: int, hblock: int, wbits: int, abits: int, seed: int,
                    norm: bool = True, ascale: str = "none", fold_after: int = 0,
                    bias: bool = False, residual: bool = False, outliers: int = 4,
                    outlier_factor: float = 30.0, x_scale: float = 1.0) -> Workload:
    """A small workload for the option matrix of the tests.

    ``ascale``: "none" (a = 1), "gain" (folded into the RMSNorm gain; needs
    ``norm``) or "explicit" (passed to the prologue as its own vector, applied
    before or after the rotation according to ``fold_after``)."""
    g = _children(seed)
    x = g[0].standard_normal((M, K), dtype=np.float32) * np.float32(x_scale)
    if outliers:
        ch = _outlier_channels(g[1], K, min(outliers, K))
        x[:, ch] *= np.float32(outlier_factor)
    W = _weights(g[4], N, K)
    gamma = g[3].uniform(0.5, 1.5, size=K).astype(np.float32) if norm else None
    a = None
    if ascale != "none":
        amax = np.abs(x).max(axis=0) * (gamma if gamma is not None else 1.0)
        a = _smoothing(np.maximum(amax, 1e-3), W)
    res = f32_to_bf16_bits(g[6].standard_normal((M, N), dtype=np.float32)) if residual else None
    b = (g[8].standard_normal(N, dtype=np.float32) * np.float32(0.1)) if bias else None
    return Workload(name=f"rand_m{M}_k{K}_n{N}_b{hblock}_w{wbits}a{abits}", M=M, K=K, N=N,
                    hblock=hblock, wbits=wbits, abits=abits, x=f32_to_bf16_bits(x), W=W,
                    gamma=gamma, ascale=a, fold_after=fold_after,
                    fold_into_gain=(ascale == "gain"), residual=res, bias=b, eps=1e-6, seed=seed,
                    recipe="random option-matrix case")

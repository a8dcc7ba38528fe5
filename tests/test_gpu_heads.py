"""Head-layout epilogue (fq_gemm_heads / fq_linear_heads) against the oracle.

The vla.cpp FoldQuant page's CUDA path puts the residual add and the head
layout in the GEMM epilogue (Runtime summary); the SYCL path keeps plain
[N][T] outputs.  Here the oracle's float64 outputs, permuted to
y[h][m][d] for feature n = h * head_dim + d, are the reference: every
accumulator must equal the oracle's, and every bf16 output must sit within
the epilogue's rounding bound of the oracle's value, with bias and a
row-major residual.  Covers the split-K GEMV (M <= 4, and any M forced with
gemv=split), the streaming GEMV (5 <= M <= 32, one and two token tiles) and
the tiled MFMA GEMM (M > 32)."""
import numpy as np
import pytest

import oracle
import synth
from fqtest import assert_codes, assert_y_fro, assert_y_within, dev, epilogue_magnitude, host, log, rand_codes

pytestmark = pytest.mark.gpu


def to_heads(a, head_dim):
    """[M][N] -> [N / head_dim][M][head_dim]."""
    M, N = a.shape
    return np.ascontiguousarray(a.reshape(M, N // head_dim, head_dim).transpose(1, 0, 2))


HEAD_CASES = [
    # M, N, K, head_dim, gemv hook
    (1, 256, 512, 64, "auto"), (3, 384, 1024, 128, "auto"), (5, 136, 384, 8, "auto"), (16, 512, 768, 128, "auto"),
    (16, 512, 768, 128, "split"), (17, 640, 384, 64, "auto"), (32, 1024, 2048, 128, "auto"),
    (33, 264, 256, 8, "auto"), (130, 1152, 768, 128, "auto"), (300, 4608, 1024, 128, "auto"),
]


@pytest.mark.parametrize("case", HEAD_CASES, ids=lambda c: "M{}_N{}_K{}_hd{}_{}".format(*c))
@pytest.mark.parametrize("bits", [(8, 8), (4, 4)], ids=lambda b: "A{}W{}".format(*b))
def test_gemm_heads_against_oracle(case, bits, hook):
    from w4a4_integer_gemm_amd import fq_gemm_heads
    M, N, K, head_dim, gemv = case
    abits, wbits = bits
    hook(f"gemv={gemv}")
    log(f"gemm heads vs oracle M={M} N={N} K={K} head_dim={head_dim} A{abits}W{wbits} gemv={gemv}")
    rng = np.random.default_rng(M * 31 + N + K + head_dim + abits)
    ca, cw = rand_codes(rng, M, K, abits), rand_codes(rng, N, K, wbits)
    sa = rng.uniform(0.001, 0.05, M).astype(np.float32)
    sw = rng.uniform(0.0001, 0.002, N).astype(np.float32)
    b = (rng.standard_normal(N) * 0.1).astype(np.float32)
    res = synth.f32_to_bf16_bits(rng.standard_normal((M, N)).astype(np.float32))
    acc_ref = oracle.gemm_i32(ca, abits, cw, wbits, K)
    _, yf = oracle.epilogue(acc_ref, sa, sw, b, res, want_f64=True)
    yh = dev(np.zeros((N // head_dim, M, head_dim), np.uint16))
    acc = dev(np.zeros((M, N), np.int32))
    fq_gemm_heads(dev(ca), dev(sa), M, abits, dev(cw), dev(sw), N, K, wbits, dev(b), dev(res), N, head_dim, yh,
                  acc)
    assert np.array_equal(host(acc), acc_ref), f"{np.count_nonzero(host(acc) != acc_ref)} accumulators differ"
    got = host(yh, np.uint16)
    # element (h, m, d) against the oracle's (m, h * head_dim + d), with that element's bound
    assert_y_within(got, to_heads(yf, head_dim), to_heads(epilogue_magnitude(acc_ref, sa, sw, b, res), head_dim),
                    what=f"heads M{M} N{N}")


@pytest.mark.parametrize("M", [1024, 16, 3])
def test_linear_heads_qkv_against_oracle(M):
    """fq_linear_heads on the fused QKV site (K = 3584, N = 4608, head_dim 128:
    28 query, 4 key and 4 value heads) against oracle.linear on sampled tokens,
    through the MFMA GEMM (M = 1024), the streaming GEMV (16) and the split-K
    GEMV (3)."""
    import w4a4_integer_gemm_amd as fq
    wl = synth.make_workload("qkv_w8a8", M=M)
    log(f"linear heads qkv M={M}")
    site = fq.DeviceSite(wl.W, wl.hblock, wl.wbits, wl.abits, gamma=wl.gamma, ascale=wl.ascale, eps=wl.eps)
    yh = host(site.linear_heads(site.upload(wl.x), 128), np.uint16)
    codes_d, scales_d = site.workspace_codes(M)
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, size=min(M, 16), replace=False)]))
    sub = synth.Workload(**{**wl.__dict__, "x": wl.x[rows], "M": len(rows)})
    out = oracle.linear(sub, codes_w=site.codes_host, wscale=site.wscale_host)
    gcodes = host(codes_d).reshape(M, -1)[rows]
    assert_codes(gcodes, host(scales_d)[rows], out["codes_a"], out["act_scale"], wl.K, wl.abits, what="qkv heads")
    got = yh[:, rows, :]  # [h][sampled m][d]
    ref = to_heads(out["y_f64"], 128)
    assert_y_fro(got.transpose(1, 0, 2).reshape(len(rows), wl.N), out["y_f64"], what="qkv heads")
    same = np.all(gcodes == out["codes_a"], axis=1)
    if np.any(same):
        r = np.nonzero(same)[0]
        mag = epilogue_magnitude(out["acc"][r], out["act_scale"][r], out["wscale"])
        assert_y_within(got[:, r, :], ref[:, r, :], to_heads(mag, 128), what="qkv heads same-codes")

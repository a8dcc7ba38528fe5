"""fq_linear_noalloc, the variant of fq_linear for callers that cannot
allocate: its workspace is the library's per-GPU scratch array.  Checked
through the C ABI against fq_linear with a caller workspace on the same
inputs (the same kernels, so the outputs must be equal bit for bit), on two
calls in a row per case with the second one smaller, on the tiled GEMM and
both GEMV kernels; and replayed from a HIP graph."""
import numpy as np
import pytest
import torch

import synth
import w4a4_integer_gemm_amd as fq
from fqtest import log

pytestmark = pytest.mark.gpu


def site_for(wl):
    return fq.DeviceSite(wl.W, wl.hblock, wl.wbits, wl.abits, gamma=wl.gamma, ascale=wl.ascale,
                         fold_after=wl.fold_after, fold_into_gain=wl.fold_into_gain, bias=wl.bias, eps=wl.eps)


CASES = [
    # workload, first M, second (smaller) M
    ("qkv_w8a8", 1024, 16),
    ("down_w8a8", 1024, 3),
    ("gateup_w4a4", 816, 64),
    ("decode_m16_w8a8", 16, 1),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}_M{c[1]}_then_M{c[2]}")
def test_noalloc_equals_fq_linear(case):
    name, m1, m2 = case
    wl = synth.make_workload(name, M=m1)
    log(f"noalloc {name}: M={m1} then M={m2} (K={wl.K} N={wl.N})")
    site = site_for(wl)
    x = site.upload(wl.x)
    res = site.upload(wl.residual) if wl.residual is not None else None
    for M in (m1, m2):
        xm = x[:M]
        rm = None if res is None else res[:M]
        want = site.linear(xm, residual=rm)
        got = site.empty_out(M)
        got.fill_(0x7FC0)  # NaN pattern: every output must be written
        site.linear_noalloc(xm, residual=rm, y=got)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"{name} M={M}: {int((got != want).sum())} outputs differ from fq_linear"


def test_noalloc_rejects_oversize_and_keeps_working():
    """A request beyond the scratch array is refused before any work; the next
    call in range still matches fq_linear."""
    wl = synth.make_workload("qkv_w8a8", M=32)
    site = site_for(wl)
    cap = fq.fq_linear_noalloc_max_bytes()
    M_big = cap // wl.K + 1
    xb = torch.zeros((M_big, wl.K), dtype=torch.int16, device="cuda")
    yb = torch.zeros((M_big, wl.N), dtype=torch.int16, device="cuda")
    with pytest.raises(fq.FqError) as e:
        site.linear_noalloc(xb, y=yb)
    assert e.value.status == 3 and "scratch array" in e.value.message
    assert int(yb.abs().sum()) == 0
    x = site.upload(wl.x)
    assert torch.equal(site.linear_noalloc(x), site.linear(x))


def test_noalloc_graph_replays():
    """Captured in a HIP graph and replayed with new inputs between replays:
    every replay equals an eager fq_linear call."""
    wl = synth.make_workload("gateup_w4a4", M=96, N=2048)
    site = site_for(wl)
    x = site.upload(wl.x)
    y = site.empty_out(wl.M)
    site.linear_noalloc(x, y=y)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        site.linear_noalloc(x, y=y)
    rng = np.random.default_rng(5)
    for rep in range(3):
        x.copy_(site.upload(wl.x[rng.permutation(wl.M)]))
        want = site.linear(x)
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, want), f"replay {rep} differs"
    del g

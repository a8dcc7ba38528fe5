"""fq_linear captured in a HIP graph (as the benchmark replays it) gives the
eager result on every replay: several replays, with eager work (new inputs
written into the captured buffers, an eager fq_linear, host
synchronizations) between them, each compared bit for bit with an eager
call on the same inputs.  Covers the MFMA GEMM with a residual, the W4A4
GEMM, the streaming decode GEMV (M = 16, weights rotated over two sites as
in the benchmark) and the split-K GEMV (M = 1)."""
import numpy as np
import pytest
import torch

import synth
import w4a4_integer_gemm_amd as fq
from fqtest import dev, log

pytestmark = pytest.mark.gpu

CASES = [
    # workload, M, N (shrunk where the full size adds nothing), copies
    ("qkv_w8a8", 96, 1152, 1),
    ("down_w8a8", 64, 512, 1),
    ("gateup_w4a4", 80, 1024, 1),
    ("decode_m16_w8a8", 16, 4096, 2),
    ("decode_m1_w8a8", 1, 4096, 2),
]


def site_for(wl, codes=None, wscale=None):
    return fq.DeviceSite(None if codes is not None else wl.W, wl.hblock, wl.wbits, wl.abits, gamma=wl.gamma,
                         ascale=wl.ascale, fold_after=wl.fold_after, fold_into_gain=wl.fold_into_gain,
                         bias=wl.bias, eps=wl.eps, codes=codes, wscale=wscale)


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}_M{c[1]}_N{c[2]}")
def test_graph_replays_match_eager(case):
    name, M, N, copies = case
    log(f"graph case {case}")
    wl = synth.make_workload(name, M=M, N=N)
    base = site_for(wl)
    sites = [base] + [site_for(wl, base.codes_host, base.wscale_host) for _ in range(copies - 1)]
    x = dev(wl.x)
    res = dev(wl.residual) if wl.residual is not None else None
    ys = [s.empty_out(M) for s in sites]
    for s in sites:
        s.workspace(M)

    def step_all():
        for s, y in zip(sites, ys):
            s.linear(x, residual=res, y=y)

    step_all()  # first calls outside the capture (one-time device queries)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step_all()
    rng = np.random.default_rng(7)
    for rep in range(4):
        # eager work between replays: fresh inputs into the captured buffers, and
        # an eager call on them whose results the replay must reproduce
        xn = wl.x if rep == 0 else wl.x[rng.permutation(M)]
        if rep % 2:
            xn = xn[:, ::-1]  # the same values in another order along K
        x.copy_(dev(xn))
        step_all()
        torch.cuda.synchronize()
        want = [y.clone() for y in ys]
        want_codes = [torch.cat([c.view(torch.uint8).flatten() for c in s.workspace_codes(M)]).clone()
                      for s in sites]
        for y in ys:
            y.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (s, y) in enumerate(zip(sites, ys)):
            got_codes = torch.cat([c.view(torch.uint8).flatten() for c in s.workspace_codes(M)])
            assert torch.equal(got_codes, want_codes[i]), f"{name} replay {rep} site {i}: codes differ from eager"
            assert torch.equal(y, want[i]), f"{name} replay {rep} site {i}: y differs from eager"
    del g


FIRST_CALL_SCRIPT = r"""
import sys
sys.path.insert(0, {root!r})
import numpy as np, torch
import synth
import w4a4_integer_gemm_amd as fq
init = {init!r}
print("first-call capture: W4A4 decode MLP block, M =", {M}, "device_init first:", init, flush=True)
M, K, F, hb = {M}, 2048, 16384, 128
up = synth.random_workload(M, K, 2 * F, hb, 4, 4, seed=21, norm=True, ascale="gain", outliers=8)
down = synth.random_workload(M, F, K, hb, 4, 4, seed=22, norm=False, ascale="none")
mk = lambda wl: fq.DeviceSite(wl.W, wl.hblock, wl.wbits, wl.abits, gamma=wl.gamma, ascale=wl.ascale,
                              fold_after=wl.fold_after, fold_into_gain=wl.fold_into_gain, eps=wl.eps)
s_up, s_down = mk(up), mk(down)
x = s_up.upload(up.x)
y1 = s_up.empty_out(M)
h = torch.empty((M, F), dtype=torch.int16, device="cuda")
y2 = s_down.empty_out(M)
s_up.workspace(M)
s_down.workspace(M)
torch.cuda.synchronize()
if init:
    fq.fq_device_init()

def block():
    s_up.linear(x, y=y1)
    fq.fq_geglu(y1, M, F, 2 * F, h, F)
    s_down.linear(h, residual=x, y=y2)

g = torch.cuda.CUDAGraph()
with torch.cuda.graph(g):   # the process's first libfq device calls happen inside this capture
    block()
outs = []
for rep in range(3):
    x.copy_(s_up.upload(up.x if rep == 0 else up.x[::-1].copy()))
    y1.zero_(); h.zero_(); y2.zero_()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    got = [t.clone() for t in (y1, h, y2)]
    block()
    torch.cuda.synchronize()
    for a, b, name in zip(got, (y1, h, y2), ("gate+up", "geglu", "down")):
        assert torch.equal(a, b), f"replay {{rep}}: {{name}} differs from the eager call"
print("first-call capture ok", flush=True)
"""


@pytest.mark.parametrize("M,init", [(8, False), (16, True), (3, False)])
def test_graph_capture_of_the_first_calls(M, init):
    """A fresh process whose first libfq device calls are inside a graph capture
    (the per-device set-up then runs during the capture, or beforehand through
    fq_device_init): a chained W4A4 decode MLP block, gate+up (K = 2048) ->
    GeGLU -> down (K = 16384) with the residual, whose two sites give the
    streaming GEMV two different LDS sizes.  Every replay must equal eager calls."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = FIRST_CALL_SCRIPT.format(root=root, M=M, init=init)
    log(f"first-call capture subprocess M={M} init={init}")
    p = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    log(p.stdout[-2000:] + p.stderr[-4000:])
    assert p.returncode == 0, f"subprocess failed ({p.returncode})"
    assert "first-call capture ok" in p.stdout

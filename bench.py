#!/usr/bin/env python3
"""Benchmark of the FoldQuant integer linear layer on one MI355X.

One step = one fq_linear call (prologue + integer GEMM + fused epilogue) over
the Qwen2.5-7B-shaped fused QKV projection: 1024 tokens, K = 3584,
N = 4608 (3584 + 512 + 512), W8A8, Hadamard block 128.  Inputs are seeded
synthetic bf16 activations with heavy-tailed channels and N(0, 0.02) weights,
already resident in HBM when the timed region starts.

Prints ONE JSON line: throughput in TOPS (2*M*N*K integer ops per step), the
roofline of the dominant kernel (the MFMA GEMM, timed with HIP events on the
stream it runs on), the CPU oracle timed on the host, secondary lines for the
other prefill shape (MLP down projection with residual), the W4A4 sites and
the decode GEMV (GB/s, weights rotated over copies larger than the 256 MB
Infinity Cache), the measured MFMA-i8 and HBM-read ceilings of this GPU next
to the datasheet peaks, and amd-smi clocks and power (idle before, under
load, after).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fq_linear TOPS @ M=1024 Qwen2.5-7B shapes (% INT8 peak); decode GB/s (% HBM)"
PEAK_INT8_TOPS = 5000.0      # MI355X dense INT8 MFMA, 5.0 POP/s
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, 8 TB/s


def site_for(wl):
    import w4a4_integer_gemm_amd as fq
    return fq.DeviceSite(wl.W, wl.hblock, wl.wbits, wl.abits, gamma=wl.gamma, ascale=wl.ascale,
                         fold_after=wl.fold_after, fold_into_gain=wl.fold_into_gain, bias=wl.bias, eps=wl.eps)


WARM_MS = 25.0  # untimed work before a timed region: the clock needs 5-10 ms of load to settle


def warm_up(step, warmup, min_ms=WARM_MS):
    """At least `warmup` calls, and then more in groups of 20 until min_ms of
    wall time has passed (host-synchronized), so that a timed region starts at
    the clock the part holds under steady load.  Returns the calls run."""
    import torch
    n = 0
    t0 = time.perf_counter()
    for _ in range(warmup):
        step()
        n += 1
    torch.cuda.synchronize()
    while (time.perf_counter() - t0) * 1e3 < min_ms:
        for _ in range(20):
            step()
        n += 20
        torch.cuda.synchronize()
    return n


def timed_steps(step, steps, batch=20):
    """Time `steps` back-to-back calls launched from Python between two
    synchronizations (the value reported; the graph-replayed figure goes next
    to it);
    HIP events recorded every `batch` calls inside the same region give the
    spread: median, p10 and p90 of the batch means (ms per call)."""
    import torch
    s = torch.cuda.current_stream()
    marks = []
    t0 = time.perf_counter()
    for i in range(steps):
        if i % batch == 0:
            e = torch.cuda.Event(enable_timing=True)
            e.record(s)
            marks.append((i, e))
        step()
    end = torch.cuda.Event(enable_timing=True)
    end.record(s)
    marks.append((steps, end))
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    means = [a[1].elapsed_time(b[1]) / (b[0] - a[0]) for a, b in zip(marks, marks[1:]) if b[0] - a[0] == batch]
    stats = None
    if means:
        stats = {"batch": batch, "batches": len(means), "median_ms": float(np.median(means)),
                 "p10_ms": float(np.percentile(means, 10)), "p90_ms": float(np.percentile(means, 90))}
    return ms, stats


def graph_steps(step, steps, batch=20):
    """Time `steps` calls of step() replayed from HIP graphs: one graph holds
    `batch` calls (replayed steps // batch times), another the remainder.
    The timed region runs between two synchronizations; HIP events recorded
    between replays give the spread: median, p10 and p90 of the batch means.
    Returns (ms per call over the whole region, spread)."""
    import torch
    full, rem = divmod(steps, batch)

    def capture(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n):
                step()
        return g

    gb = capture(batch) if full else None
    gr = capture(rem) if rem else None
    for g in (gb, gr):  # untimed first replays
        if g is not None:
            g.replay()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    marks = []
    t0 = time.perf_counter()
    for _ in range(full):
        e = torch.cuda.Event(enable_timing=True)
        e.record(s)
        marks.append(e)
        gb.replay()
    e = torch.cuda.Event(enable_timing=True)
    e.record(s)
    marks.append(e)
    if gr is not None:
        gr.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    means = [a.elapsed_time(b) / batch for a, b in zip(marks, marks[1:])]
    stats = None
    if means:
        stats = {"batch": batch, "batches": len(means), "median_ms": float(np.median(means)),
                 "p10_ms": float(np.percentile(means, 10)), "p90_ms": float(np.percentile(means, 90))}
    del gb, gr
    return ms, stats


E2M3_SUFFIX = "_e2m3"  # a W4A4 workload with its 4-bit codes stored as FP6 E2M3 (code width 6)


def load_workload(name):
    import dataclasses
    import synth
    if name.endswith(E2M3_SUFFIX):
        return dataclasses.replace(synth.make_workload(name[:-len(E2M3_SUFFIX)]), wbits=6, abits=6)
    return synth.make_workload(name)


def bench_prefill(name, steps, warmup):
    import torch
    wl = load_workload(name)
    site = site_for(wl)
    x = site.upload(wl.x)
    res = site.upload(wl.residual) if wl.residual is not None else None
    y = site.empty_out(wl.M)
    site.workspace(wl.M)
    step = lambda: site.linear(x, residual=res, y=y)
    nwarm = warm_up(step, warmup)
    ms, batches = timed_steps(step, steps)
    ms_graph, _ = graph_steps(step, steps)
    ops = 2.0 * wl.M * wl.N * wl.K
    codes, scales = site.workspace_codes(wl.M)
    # per-kernel averages (HIP events around graph replays of back-to-back launches of one kernel)
    ms_pro, _ = graph_steps(lambda: site.prologue(x, codes, scales), steps)
    ms_gemm, _ = graph_steps(lambda: site.gemm(codes, scales, wl.M, residual=res, y=y), steps)
    site.linear(x, residual=res, y=y)
    torch.cuda.synchronize()
    ok, detail = parity(wl, site, y, codes, scales)
    return dict(wl=wl, site=site, step=step, ms=ms, tops=ops / (ms * 1e-3) / 1e12, ms_prologue=ms_pro,
                ms_gemm=ms_gemm, ms_graph=ms_graph,
                warmup_run=nwarm,
                tops_graph=ops / (ms_graph * 1e-3) / 1e12,
                gemm_tops=ops / (ms_gemm * 1e-3) / 1e12, parity=detail, parity_ok=ok, ops=ops, batches=batches)


def parity(wl, site, y, codes, scales, nrows=8):
    import oracle
    import synth
    rows = np.linspace(0, wl.M - 1, num=min(nrows, wl.M)).astype(int)
    sub = synth.Workload(**{**wl.__dict__, "x": wl.x[rows], "M": len(rows),
                            "residual": None if wl.residual is None else wl.residual[rows]})
    out = oracle.linear(sub, codes_w=site.codes_host, wscale=site.wscale_host)
    gc = codes.cpu().numpy().reshape(wl.M, -1)[rows]
    ga = oracle.unpack_codes(gc, wl.K, wl.abits)
    oa = oracle.unpack_codes(out["codes_a"], wl.K, wl.abits)
    mism = float(np.count_nonzero(ga != oa)) / ga.size
    maxd = int(np.abs(ga - oa).max())
    yg = synth.bf16_bits_to_f32(y.cpu().numpy().view(np.uint16)[rows]).astype(np.float64)
    fro = float(np.linalg.norm(yg - out["y_f64"]) / np.linalg.norm(out["y_f64"]))
    ok = maxd <= 1 and mism <= 1e-3 and fro <= 1e-2
    return ok, dict(rows_checked=len(rows), code_mismatch_frac=mism, code_max_diff=maxd, y_rel_fro=fro)


def bench_mlp_block(steps, warmup):
    """The Gemma-shaped W4A4 MLP block chained on the GPU: gate+up site (816 x
    2048 -> 32768) -> GeGLU -> down site (16384 -> 2048) with the residual, the
    down site reading the GeGLU output of the gate+up site.  TOPS over the two
    GEMMs' 2*M*N*K; the parity control recomputes sampled tokens of each node
    with the oracle from that node's own GPU inputs."""
    import torch
    import synth
    import w4a4_integer_gemm_amd as fq
    up = synth.make_workload("gateup_w4a4")
    F = up.N // 2
    dn = synth.make_workload("down_w4a4")
    s_up, s_dn = site_for(up), site_for(dn)
    x = s_up.upload(up.x)
    y1 = s_up.empty_out(up.M)
    h = torch.empty((up.M, F), dtype=torch.int16, device="cuda")
    y2 = s_dn.empty_out(up.M)
    s_up.workspace(up.M)
    s_dn.workspace(up.M)

    def step():
        s_up.linear(x, y=y1)
        fq.fq_geglu(y1, up.M, F, 2 * F, h, F)
        s_dn.linear(h, residual=x, y=y2)
    nwarm = warm_up(step, warmup)
    ms, batches = timed_steps(step, steps)
    ms_graph, _ = graph_steps(step, steps)
    step()
    torch.cuda.synchronize()
    # parity of the down node from its own GPU input h
    dn.x = h.cpu().numpy().view(np.uint16)
    dn.residual = up.x
    ok, detail = parity(dn, s_dn, y2, *s_dn.workspace_codes(up.M))
    ops = 2.0 * up.M * (up.N * up.K + dn.N * dn.K)
    return dict(ms=ms, tops=ops / (ms * 1e-3) / 1e12, ms_graph=ms_graph, tops_graph=ops / (ms_graph * 1e-3) / 1e12,
                batches=batches, parity=detail, parity_ok=ok, warmup_run=nwarm)


def bench_decode(name, steps, warmup, copies=5):
    """Decode GEMV GB/s with the weights rotated over `copies` device copies
    (5 x 136 MB > 2 x the 256 MB Infinity Cache) so each call streams from HBM."""
    import torch
    import synth
    import w4a4_integer_gemm_amd as fq
    wl = synth.make_workload(name)
    base = site_for(wl)
    sites = [base] + [fq.DeviceSite(None, wl.hblock, wl.wbits, wl.abits, gamma=wl.gamma, ascale=wl.ascale,
                                    fold_after=wl.fold_after, fold_into_gain=wl.fold_into_gain, bias=wl.bias,
                                    eps=wl.eps, codes=base.codes_host, wscale=base.wscale_host)
                      for _ in range(copies - 1)]
    wl.W = None
    x = base.upload(wl.x)
    ys = [s.empty_out(wl.M) for s in sites]
    for s in sites:
        s.workspace(wl.M)
    i = [0]

    def step():
        k = i[0] % copies
        sites[k].linear(x, y=ys[k])
        i[0] += 1

    nwarm = warm_up(step, warmup)
    ms, batches = timed_steps(step, steps)
    ms_graph, _ = graph_steps(step, steps)
    wbytes = wl.N * wl.K * wl.wbits / 8
    # algorithmic bytes: weight codes + weight scales + x + y + activation codes written and read back
    nbytes = wbytes + 4 * wl.N + 2 * wl.M * wl.K + 2 * wl.M * wl.N + 2 * wl.M * wl.K * wl.abits / 8 + 8 * wl.M
    # GEMV kernel alone (same rotation)
    codes_scales = [s.workspace_codes(wl.M) for s in sites]
    j = [0]

    def gemv():
        k = j[0] % copies
        c, sc = codes_scales[k]
        sites[k].gemm(c, sc, wl.M, y=ys[k])
        j[0] += 1

    ms_gemv, _ = graph_steps(gemv, steps)
    gemv_bytes = wbytes + 4 * wl.N + wl.M * wl.K * wl.abits / 8 + 4 * wl.M + 2 * wl.M * wl.N
    return dict(name=name, M=wl.M, ms=ms, gbs=nbytes / (ms * 1e-3) / 1e9, ms_gemv=ms_gemv, ms_graph=ms_graph,
                warmup_run=nwarm,
                gbs_graph=nbytes / (ms_graph * 1e-3) / 1e9,
                gemv_gbs=gemv_bytes / (ms_gemv * 1e-3) / 1e9, bytes=nbytes, gemv_bytes=gemv_bytes, batches=batches)


def cpu_baseline(name, min_seconds=10.0, max_reps=400):
    """The oracle (plain C + OpenMP) on the same workload, repeated until about
    min_seconds of CPU work: whole fq_linear (prologue, integer GEMM, epilogue)."""
    import oracle
    import synth
    wl = synth.make_workload(name)
    codes_w, wscale = oracle.pack_weights(wl.W, wl.ascale, wl.fold_after, wl.hblock, wl.wbits)
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        oracle.linear(wl, codes_w=codes_w, wscale=wscale)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start >= min_seconds or len(times) >= max_reps:
            break
    t = float(np.median(times))
    ops = 2.0 * wl.M * wl.N * wl.K
    out = dict(value=ops / t / 1e12, unit="TOP/s", cores=oracle.num_threads(), cpu_model=cpu_model(), kind="oracle",
               sample=f"whole {name} fq_linear (M={wl.M} K={wl.K} N={wl.N}) on the oracle, "
                      f"{len(times)} repetitions ({sum(times):.1f} s), median {t * 1e3:.1f} ms; weights packed once")
    out["one_core"] = cpu_one_core(name)
    return out


ONE_CORE_SCRIPT = """
import json, sys, time
sys.path.insert(0, {root!r})
import numpy as np, oracle, synth
wl = synth.make_workload({name!r}, M={m})
codes_w, wscale = oracle.pack_weights(wl.W, wl.ascale, wl.fold_after, wl.hblock, wl.wbits)
ts = []
t_start = time.perf_counter()
while time.perf_counter() - t_start < {seconds} or len(ts) < 2:
    t0 = time.perf_counter()
    oracle.linear(wl, codes_w=codes_w, wscale=wscale)
    ts.append(time.perf_counter() - t0)
t = float(np.median(ts))
print(json.dumps(dict(value=2.0 * wl.M * wl.N * wl.K / t / 1e12, unit="TOP/s", cores=oracle.num_threads(),
                      sample=f"{{wl.M}} tokens of {name} (K={{wl.K}} N={{wl.N}}), {{len(ts)}} repetitions, "
                             f"median {{t * 1e3:.1f}} ms")))
"""


def cpu_one_core(name, tokens=64, seconds=4.0):
    """The same oracle on one host core (OMP_NUM_THREADS=1, a child process that
    never touches the GPU) over the first `tokens` tokens: the per-core rate."""
    import subprocess
    code = ONE_CORE_SCRIPT.format(root=ROOT, name=name, m=tokens, seconds=seconds)
    env = {**os.environ, "OMP_NUM_THREADS": "1"}
    try:
        p = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
        return json.loads(p.stdout.strip().splitlines()[-1]) if p.returncode == 0 else None
    except (subprocess.SubprocessError, ValueError, IndexError):
        return None


def gemm_bytes(wl):
    """Bytes the GEMM must move at least once: both code matrices, both scale
    vectors, the bf16 output (and the bf16 residual when there is one)."""
    n = wl.M * wl.K * wl.abits // 8 + wl.N * wl.K * wl.wbits // 8 + 4 * (wl.M + wl.N) + 2 * wl.M * wl.N
    return n + (2 * wl.M * wl.N if wl.residual is not None else 0)


def copy_probe(nbytes=256 << 20):
    """One plain device copy kernel of known size (reads and writes nbytes): the
    scale for the FETCH_SIZE / WRITE_SIZE counters of a profiled run."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.mul(src, 1.0, out=dst)  # one elementwise kernel: nbytes in, nbytes out
    torch.cuda.synchronize()
    del src, dst
    return nbytes


def load_traffic(kernel_key, sources):
    """Scaled FETCH_SIZE + WRITE_SIZE bytes per launch of a kernel from the committed
    rocprofv3 counter summary; None if absent or taken on other kernel sources."""
    import hashlib
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    e = json.load(open(p)).get(kernel_key)
    if e is None:
        return None
    h = hashlib.sha256()
    for src in sources:
        with open(os.path.join(ROOT, "w4a4_integer_gemm_amd", "csrc", src), "rb") as f:
            h.update(f.read())
    return e["bytes"] if h.hexdigest() == e.get("source_sha256") else None


CEILING_LIB = os.path.join(ROOT, "w4a4_integer_gemm_amd", "libfq_ceiling.so")


def _ceiling_lib():
    import ctypes
    if not os.path.exists(CEILING_LIB):
        raise RuntimeError(f"{CEILING_LIB} not found; build it with `python w4a4_integer_gemm_amd/build.py`")
    L = ctypes.CDLL(CEILING_LIB)
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    L.fqc_mfma_i8.argtypes = [P, I64, I32, I32, P, P]
    L.fqc_mfma_i8.restype = ctypes.c_int
    L.fqc_mfma_i8_ops.argtypes = [I32, I32]
    L.fqc_mfma_i8_ops.restype = I64
    L.fqc_stream_read.argtypes = [P, I64, I32, I32, P, P]
    L.fqc_stream_read.restype = ctypes.c_int
    return L


def _event_ms(run, reps):
    """Mean ms of `reps` back-to-back run() calls, HIP events on the current stream."""
    import torch
    s = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(s)
    for _ in range(reps):
        run()
    b.record(s)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def measure_ceilings(stream_bytes=135_790_592, copies=5):
    """Measured ceilings of this part, next to the datasheet peaks:
    - the v_mfma_i32_16x16x64_i8 rate on random operand bytes (the codes' power
      draw) and on zero bytes, one and two waves per SIMD;
    - the HBM read rate of a plain grid-stride read of `copies` rotated buffers
      of the decode layer's weight size (37888 x 3584 bytes), best over the
      launch shapes swept."""
    import torch
    L = _ceiling_lib()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream().cuda_stream
    out = torch.zeros(4, dtype=torch.int32, device="cuda")
    res = {"mfma_i8": {}, "stream_read": {}}
    iters = 4000
    best_rand = 0.0
    for kind in ("random", "zero"):
        for per_cu in (1, 2):
            blocks = cus * per_cu
            n16 = blocks * 256 * 16
            src = (torch.randint(-128, 128, (n16 * 16,), dtype=torch.int8, device="cuda") if kind == "random"
                   else torch.zeros(n16 * 16, dtype=torch.int8, device="cuda"))
            run = lambda: L.fqc_mfma_i8(src.data_ptr(), n16, blocks, iters, out.data_ptr(), stream)
            rc = run()
            if rc != 0:
                raise RuntimeError(f"fqc_mfma_i8 failed: hip error {rc}")
            t0 = time.perf_counter()
            while time.perf_counter() - t0 < WARM_MS * 1e-3 * 4:  # settle the clock under this load
                run()
                torch.cuda.synchronize()
            ms = _event_ms(run, 5)
            tops = L.fqc_mfma_i8_ops(blocks, iters) / (ms * 1e-3) / 1e12
            res["mfma_i8"][f"{kind}_{per_cu}wave_per_simd"] = tops
            if kind == "random":
                best_rand = max(best_rand, tops)
            del src
    res["mfma_i8_random_tops"] = best_rand
    n16 = stream_bytes // 16
    bufs = [torch.randint(-128, 128, (stream_bytes,), dtype=torch.int8, device="cuda") for _ in range(copies)]
    best = (0.0, None)
    i = [0]

    def reader(per_cu, u):
        def run():
            L.fqc_stream_read(bufs[i[0] % copies].data_ptr(), n16, cus * per_cu, u, out.data_ptr(), stream)
            i[0] += 1
        return run
    warm_up(reader(8, 4), 20)  # the memory system under load before the sweep
    # two passes over the launch shapes, 100 launches (about 2 ms) each; the best pass counts
    for _ in range(2):
        for per_cu in (4, 8, 16):
            for u in (4, 8, 16):
                run = reader(per_cu, u)
                for _ in range(10):
                    run()
                ms = _event_ms(run, 100)
                gbs = n16 * 16 / (ms * 1e-3) / 1e9
                key = f"{per_cu}wg_per_cu_u{u}"
                res["stream_read"][key] = max(gbs, res["stream_read"].get(key, 0.0))
                if gbs > best[0]:
                    best = (gbs, f"{cus * per_cu} workgroups of 256, {u} x 16-byte loads in flight per lane")
    res["stream_read_gbs"] = best[0]
    res["stream_read_config"] = best[1]
    res["stream_read_buffers"] = f"{copies} rotated buffers of {stream_bytes} bytes"
    del bufs
    torch.cuda.empty_cache()
    return res


def _smi_value(v):
    if isinstance(v, dict):
        v = v.get("value", None)
    try:
        return float(v)
    except (TypeError, ValueError):
        return None


def amd_smi_sample():
    """Current gfx and memory clocks (MHz) and socket power (W) of GPU 0 from
    amd-smi, or None when amd-smi is unavailable."""
    import subprocess
    try:
        p = subprocess.run(["amd-smi", "metric", "-g", "0", "-p", "-c", "--json"], capture_output=True, text=True,
                           timeout=30)
        data = json.loads(p.stdout)
    except (OSError, subprocess.SubprocessError, ValueError):
        return None
    if isinstance(data, list):
        data = data[0] if data else {}
    if isinstance(data, dict) and "gpu_data" in data:
        data = data["gpu_data"][0] if data["gpu_data"] else {}
    clk = data.get("clock", {}) if isinstance(data, dict) else {}
    pw = data.get("power", {}) if isinstance(data, dict) else {}
    gfx = [_smi_value(c.get("clk")) for k, c in sorted(clk.items()) if k.startswith("gfx_") and isinstance(c, dict)]
    gfx = [g for g in gfx if g is not None]
    mem = _smi_value(clk.get("mem_0", {}).get("clk")) if isinstance(clk.get("mem_0"), dict) else None
    return {"sclk_mhz": (sum(gfx) / len(gfx)) if gfx else None, "sclk_per_xcd_mhz": gfx or None, "mclk_mhz": mem,
            "socket_power_w": _smi_value(pw.get("socket_power"))}


def sample_under_load(step, seconds=1.5):
    """amd-smi sampled from a helper thread while step() runs back to back."""
    import threading
    import torch
    box = {}
    th = threading.Thread(target=lambda: box.update(s=amd_smi_sample()))
    t0 = time.perf_counter()
    th.start()
    while th.is_alive() or time.perf_counter() - t0 < seconds:
        for _ in range(50):
            step()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 > 60:
            break
    th.join()
    return box.get("s")


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or None


WORKLOAD_DESC = {
    "qkv_w8a8": "Qwen2.5-7B-shaped fused QKV projection",
    "down_w8a8": "Qwen2.5-7B-shaped MLP down projection with the residual",
    "gateup_w4a4": "Gemma-2B-shaped MLP gate+up projection",
    "down_w4a4": "Gemma-2B-shaped MLP down projection with the residual",
    "tiny_w8a8": "tiny 16-token site",
    "decode_m1_w8a8": "decode GEMV (fused gate+up), 1 token",
    "decode_m16_w8a8": "decode GEMV (fused gate+up), 16 tokens",
    "gateup_w4a4_e2m3": "Gemma-2B-shaped MLP gate+up projection, 4-bit codes stored as FP6 E2M3 (FP6 MFMA)",
    "down_w4a4_e2m3": "Gemma-2B-shaped MLP down projection with the residual, 4-bit codes stored as FP6 E2M3",
}


def describe(name, wl):
    return (f"{name}: {WORKLOAD_DESC.get(name, name)}, M={wl.M} K={wl.K} N={wl.N} W{wl.wbits}A{wl.abits} "
            f"hblock={wl.hblock}, weights warm in HBM")


def vendor_gemms(steps=200):
    """Context only: the vendor GEMMs (hipBLASLt through torch: int8 torch._int_mm with an int32 result, fp8
    e4m3 torch._scaled_mm with a bf16 result, bf16 matmul) on the four prefill layers' M x N x K, next to this
    library's fq_gemm on the same shapes.  Operands are random codes; the library GEMMs do no quantisation
    and no epilogue beyond their own output type, so they do less work than fq_gemm."""
    import torch
    import synth
    out = {}
    for name in ("qkv_w8a8", "down_w8a8", "gateup_w4a4", "down_w4a4"):
        wl = synth.make_workload(name)
        M, N, K = wl.M, wl.N, wl.K
        ops = 2.0 * M * N * K
        site = site_for(wl)
        x = site.upload(wl.x)
        res = site.upload(wl.residual) if wl.residual is not None else None
        y = site.empty_out(M)
        site.workspace(M)
        site.linear(x, residual=res, y=y)
        codes, scales = site.workspace_codes(M)

        def timed(step):
            warm_up(step, 20)
            return min(graph_steps(step, steps)[0] for _ in range(3))
        r = {"shape": f"M={M} N={N} K={K}"}
        ms = timed(lambda: site.gemm(codes, scales, M, residual=res, y=y))
        r[f"fq_gemm W{wl.wbits}A{wl.abits} (bf16 out, fused epilogue)"] = {"us": ms * 1e3, "tops": ops / ms / 1e9}
        a = torch.randint(-127, 128, (M, K), dtype=torch.int8, device="cuda")
        w = torch.randint(-127, 128, (N, K), dtype=torch.int8, device="cuda")
        ms = timed(lambda: torch._int_mm(a, w.t()))
        r["torch._int_mm int8 (int32 out)"] = {"us": ms * 1e3, "tops": ops / ms / 1e9}
        try:
            af = torch.randn(M, K, device="cuda").to(torch.float8_e4m3fn)
            wf = torch.randn(N, K, device="cuda").to(torch.float8_e4m3fn)
            one = torch.ones((), device="cuda")
            ms = timed(lambda: torch._scaled_mm(af, wf.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16))
            r["torch._scaled_mm fp8 e4m3 (bf16 out)"] = {"us": ms * 1e3, "tops": ops / ms / 1e9}
        except RuntimeError as e:
            r["torch._scaled_mm fp8 e4m3 (bf16 out)"] = f"unavailable: {str(e)[:120]}"
        ab = torch.randn(M, K, device="cuda", dtype=torch.bfloat16)
        wb = torch.randn(N, K, device="cuda", dtype=torch.bfloat16)
        ms = timed(lambda: torch.matmul(ab, wb.t()))
        r["torch.matmul bf16"] = {"us": ms * 1e3, "tflops": ops / ms / 1e9}
        out[name] = r
        del a, w, ab, wb
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="qkv_w8a8")
    ap.add_argument("--no-secondary", action="store_true", help="skip the down-projection and decode lines")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one 256 MiB elementwise copy kernel (scale for HBM byte counters)")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the measured MFMA and HBM-read ceilings")
    ap.add_argument("--no-clocks", action="store_true", help="skip the amd-smi clock and power samples")
    ap.add_argument("--ceilings-only", action="store_true", help="print the measured ceilings only")
    ap.add_argument("--vendor-only", action="store_true",
                    help="print the vendor GEMMs (hipBLASLt via torch) next to fq_gemm on the prefill shapes")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} requested, but this build measures one GPU only: the FoldQuant "
              "layer is benchmarked on a single MI355X (one GPU's share at its real shape). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    import w4a4_integer_gemm_amd as fq
    fq.lib()  # fail loudly if the HIP library is missing
    if args.ceilings_only:
        print(json.dumps({"ceilings": measure_ceilings()}), flush=True)
        return
    if args.vendor_only:
        print(json.dumps({"vendor_gemms": vendor_gemms()}), flush=True)
        return

    clocks = {}
    if not args.no_clocks:
        clocks["idle_before"] = amd_smi_sample()
    r = bench_prefill(args.workload, args.steps, args.warmup)
    wl = r["wl"]
    achieved = r["ops"] / (r["ms_gemm"] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": f"gemm_kernel<{wl.abits},{wl.wbits}> (fq_gemm, MFMA i8)",
                "achieved": achieved, "peak": PEAK_INT8_TOPS, "unit": "TOP/s",
                "unit_note": "tera integer operations per second (2*M*N*K per GEMM)",
                "frac": achieved / PEAK_INT8_TOPS,
                "traffic": load_traffic(f"gemm:{args.workload}", ("fq_gemm.hip", "fq_ring.h", "fq_device.h")),
                "traffic_unit": "bytes per launch (scaled FETCH_SIZE + WRITE_SIZE)",
                "algorithmic_bytes": gemm_bytes(wl)}
    secondary = []
    if not args.no_secondary:
        # the other 1024-token prefill shape (part of the headline metric), then the
        # W4A4 Gemma-shaped MLP sites (parity configs, reported for completeness)
        for name in ("down_w8a8", "gateup_w4a4", "down_w4a4", "gateup_w4a4" + E2M3_SUFFIX,
                     "down_w4a4" + E2M3_SUFFIX):
            s = bench_prefill(name, max(20, args.steps // 4), args.warmup)
            secondary.append({"workload": name, "metric": "fq_linear TOPS", "value": s["tops"],
                              "frac_int8_peak": s["tops"] / PEAK_INT8_TOPS, "ms_per_call": s["ms"],
                              "graph": {"value": s["tops_graph"], "ms_per_call": s["ms_graph"]},
                              "batch_spread": s["batches"], "gemm_tops": s["gemm_tops"],
                              "ms_prologue": s["ms_prologue"], "ms_gemm": s["ms_gemm"], "parity": s["parity"]})
            del s
            torch.cuda.empty_cache()
        m = bench_mlp_block(max(20, args.steps // 4), args.warmup)
        secondary.append({"workload": "gemma_mlp_block_w4a4", "metric": "MLP block TOPS (two GEMMs)",
                          "value": m["tops"], "frac_int8_peak": m["tops"] / PEAK_INT8_TOPS, "ms_per_call": m["ms"],
                          "graph": {"value": m["tops_graph"], "ms_per_call": m["ms_graph"]},
                          "batch_spread": m["batches"], "parity_down_node": m["parity"],
                          "chain": "gate+up fq_linear (816x2048->32768) -> fq_geglu -> down fq_linear "
                                   "(16384->2048, residual = the block input)"})
        del m
        torch.cuda.empty_cache()
        # the tiny 16-token site: latency only
        s = bench_prefill("tiny_w8a8", max(50, args.steps), args.warmup)
        secondary.append({"workload": "tiny_w8a8", "metric": "fq_linear latency", "value": s["ms"] * 1e3,
                          "unit": "us", "batch_spread": s["batches"], "graph": {"value": s["ms_graph"] * 1e3},
                          "parity": s["parity"]})
        del s
        for name in ("decode_m1_w8a8", "decode_m16_w8a8"):
            d = bench_decode(name, max(50, args.steps), args.warmup)
            secondary.append({"workload": name, "metric": "decode GB/s", "value": d["gbs"],
                              "frac_hbm": d["gbs"] / PEAK_HBM_GBS, "ms_per_call": d["ms"],
                              "graph": {"value": d["gbs_graph"], "ms_per_call": d["ms_graph"]},
                              "batch_spread": d["batches"],
                              "gemv_gbs": d["gemv_gbs"], "gemv_frac_hbm": d["gemv_gbs"] / PEAK_HBM_GBS,
                              "ms_gemv": d["ms_gemv"], "algorithmic_bytes": d["bytes"],
                              "weights": "rotated over 5 device copies (679 MB) to defeat the Infinity Cache"})
        torch.cuda.empty_cache()
    ceilings = None if args.no_ceilings else measure_ceilings()
    if ceilings:
        mf, sr = ceilings["mfma_i8_random_tops"], ceilings["stream_read_gbs"]
        roofline["measured_peak"] = mf
        roofline["frac_of_measured"] = achieved / mf
        roofline["measured_peak_note"] = "v_mfma_i32_16x16x64_i8 back to back on random operand bytes, this GPU"
        for e in secondary:
            if e.get("metric") == "decode GB/s":
                e["frac_measured_read"] = e["value"] / sr
                e["gemv_frac_measured_read"] = e["gemv_gbs"] / sr
            elif e.get("metric") == "fq_linear TOPS":
                e["frac_measured_mfma"] = e["value"] / mf
    if not args.no_clocks:
        clocks["under_load"] = sample_under_load(r["step"])
        clocks["under_load_note"] = f"sampled while {args.workload} fq_linear ran back to back"
        clocks["after"] = amd_smi_sample()
    probe = copy_probe() if args.copy_probe else None
    cpu = None if args.no_cpu_baseline else cpu_baseline(args.workload)
    out = {
        "metric": METRIC,
        "value": r["tops"],
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": describe(args.workload, wl), "global_batch": wl.M, "parallelism": "single GPU"},
        "frac_int8_peak": r["tops"] / PEAK_INT8_TOPS,
        "frac_measured_mfma": (r["tops"] / ceilings["mfma_i8_random_tops"]) if ceilings else None,
        "timing": "value: the calls launched back to back from Python; 'graph': the same calls replayed from HIP "
                  "graphs of 20 (no launch gaps; the large kernels then run slower); ms_prologue, ms_gemm "
                  "and the roofline: one kernel replayed from graphs",
        "graph": {"value": r["tops_graph"], "ms_per_step": r["ms_graph"]},
        "warmup_steps_run": r["warmup_run"],
        "warmup_rule": f"at least --warmup steps and at least {WARM_MS:g} ms of them before each timed region",
        "batch_spread": r["batches"],
        "ms_prologue": r["ms_prologue"],
        "ms_gemm": r["ms_gemm"],
        "parity": r["parity"],
        "roofline": roofline,
        "cpu_baseline": cpu,
        "ceilings": ceilings,
        "clocks": clocks or None,
        "secondary": secondary,
    }
    if probe:
        out["copy_probe_bytes"] = probe
    print(json.dumps(out), flush=True)
    if not r["parity_ok"]:
        print("bench.py: parity control FAILED on the timed buffers", file=sys.stderr)
        sys.exit(3)


if __name__ == "__main__":
    main()

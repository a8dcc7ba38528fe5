"""Build libfq.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

Every object is compiled for gfx950 only, with IEEE float32 divide and sqrt,
no floating-point contraction (the exactness rules of the vla.cpp FoldQuant
page), packed-FP32 instructions disabled and MFMA accumulators in VGPRs."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libfq.so")
CEILING_LIB = os.path.join(HERE, "libfq_ceiling.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["fq_api.cpp", "fq_pack.cpp", "fq_prologue.hip", "fq_gemm.hip", "fq_gemm_fp6.hip", "fq_gemv.hip", "fq_geglu.hip",
           "fq_noalloc.hip", "fq_decode1.hip"]
# the benchmark's ceiling probes: a library of their own, outside the layer's ABI
CEILING_SOURCES = ["fq_ceiling.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA accumulators in ordinary VGPRs: the mixed AGPR/VGPR assignment
    # the default heuristic picks shuffles accumulators between the two files
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    f"-I{os.path.join(ROOT, 'include')}",
]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *CFLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out: str, verbose: bool):
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + CEILING_SOURCES
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, verbose), srcs)))
    _link([objs[s] for s in SOURCES], LIB, verbose)
    _link([objs[s] for s in CEILING_SOURCES], CEILING_LIB, verbose)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

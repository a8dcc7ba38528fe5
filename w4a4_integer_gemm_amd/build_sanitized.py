"""Host-side sanitizer build of libfq and of the CPU oracle, and the CPU test
run under it (AddressSanitizer + UndefinedBehaviorSanitizer).

The host code -- argument validation, error messages, the weight packer and
dequantiser (fq_api.cpp, fq_pack.cpp) -- and the oracle (fqo.c) are compiled
with g++/gcc and -fsanitize=address,undefined; the HIP kernel objects are
taken unchanged from the ordinary build (run build.py first), since device
code is not sanitized.  The result, libfq_san.so and oracle/liboracle_san.so,
is loaded instead of the ordinary libraries through FQ_LIB / FQO_LIB, with
the gcc ASan runtime preloaded into the Python process:

    python w4a4_integer_gemm_amd/build_sanitized.py --test

builds both and runs the CPU tests of the ABI, the packer, the oracle pins and
the fold-consistency checks under the sanitizers (no GPU needed).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libfq_san.so")
ORACLE_LIB = os.path.join(ROOT, "oracle", "liboracle_san.so")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]
HOST_SOURCES = ["fq_api.cpp", "fq_pack.cpp"]
# the library's kernels, as the ordinary build compiled them (its list of sources)
sys.path.insert(0, ROOT)
from w4a4_integer_gemm_amd.build import SOURCES as _LIB_SOURCES  # noqa: E402

DEVICE_OBJECTS = [os.path.splitext(s)[0] + ".o" for s in _LIB_SOURCES if s.endswith(".hip")]
TESTS = ["tests/test_abi_cpu.py", "tests/test_oracle_pins.py", "tests/test_fold_consistency.py"]


def run(cmd):
    print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build():
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + "_san.o")
        run(["g++", "-std=c++17", "-O1", "-fPIC", "-Wall", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
             f"-I{os.path.join(ROOT, 'include')}", "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    dev = [os.path.join(BUILD_DIR, o) for o in DEVICE_OBJECTS]
    missing = [o for o in dev if not os.path.exists(o)]
    if missing:
        raise SystemExit(f"missing {missing}: run `python w4a4_integer_gemm_amd/build.py` first")
    run(["g++", "-shared", "-fPIC", *SAN, "-o", LIB, *objs, *dev, "-L/opt/rocm/lib", "-lamdhip64",
         "-Wl,-rpath,/opt/rocm/lib"])
    run(["gcc", "-std=c11", "-O1", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-Wall",
         "-Wextra", *SAN, "-o", ORACLE_LIB, os.path.join(ROOT, "oracle", "fqo.c"), "-lm"])


def test():
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()
    ubsan = subprocess.run(["gcc", "-print-file-name=libubsan.so"], capture_output=True, text=True,
                           check=True).stdout.strip()
    env = {**os.environ, "FQ_LIB": LIB, "FQO_LIB": ORACLE_LIB, "LD_PRELOAD": f"{asan}:{ubsan}",
           # Python itself is not built with ASan: its allocations at exit are not leaks of ours
           "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:strict_string_checks=1",
           "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider", *TESTS]
    print(" ".join(cmd), flush=True)
    return subprocess.run(cmd, cwd=ROOT, env=env).returncode


if __name__ == "__main__":
    build()
    sys.exit(test() if "--test" in sys.argv else 0)

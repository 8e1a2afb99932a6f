"""Build libbitlinear.so in-tree with hipcc for gfx950.

    python -m ternary_weight_linear_absmean_amd.build [-v] [-j N]

Each source is compiled to an object (in parallel), then linked into
``ternary_weight_linear_absmean_amd/libbitlinear.so``.  Device code is built
with FMA contraction off (every fp32 step of the quantisers and the rescale
is one IEEE rounding), without packed-fp32 instructions, and with the leading
kernel arguments preloaded into SGPRs.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libbitlinear.so")

SOURCES = ["api.cpp", "quant.hip", "gemv.hip", "gemm.hip", "gemm_skinny.hip", "ffn.hip",
           "stack.hip", "stack_persistent.hip", "backward.hip", "t5.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
         "-ffp-contract=off", "-fno-fast-math", "-fvisibility=hidden",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # kernarg preload: the leading kernel arguments (up to 16 dwords) are
         # placed in SGPRs at wave launch, so a kernel reads them without a
         # scalar load round trip (the fused decode kernel passes its job
         # boundaries there; the few-token product gains ~0.15 us per launch)
         "-mllvm", "-amdgpu-kernarg-preload-count=16",
         "-Wall", "-Wno-unused-function",
         "-I", INCLUDE, "-I", CSRC]


def _compile(src, verbose):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err and verbose:
        print(err, flush=True)
    return obj


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(SOURCES)))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    jobs = 8
    if "-j" in sys.argv:
        jobs = int(sys.argv[sys.argv.index("-j") + 1])
    print(build(verbose="-v" in sys.argv, jobs=jobs))

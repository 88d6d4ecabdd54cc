"""Build libnvfp4.so (the HIP kernels and the C ABI of include/nvfp4.h) for
gfx950 with hipcc, in-tree, next to this file.

Compiler flags that matter for exactness: fp32 division and square root
stay correctly rounded, no fast-math, no denormal flushing; packed fp32
instructions are disabled (``-packed-fp32-ops``)."""
import concurrent.futures
import os
import shlex
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libnvfp4.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["quantize.hip", "gemm_tiled.hip", "gemm_decode.hip", "gemm_simple.hip", "int4_gemm.hip", "int4_asym.hip", "lora.hip", "api.cpp"]

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(shlex.quote(c) for c in cmd), flush=True)
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the device-only feature flag; drop that note
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    if out.strip() and verbose:
        print(out)
    return out


def build(verbose=False, jobs=None):
    """Compile every source and link libnvfp4.so; returns the library path."""
    os.makedirs(OBJDIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(OBJDIR, src + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmds.append([HIPCC, *FLAGS, *lang, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj])
    jobs = jobs or min(len(cmds), os.cpu_count() or 4, 8)
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


def build_peak(verbose=False):
    """Compile peak/peak.hip (bench.py's roofline microbenchmarks, not part
    of the library) into peak/libpeak.so; returns its path."""
    src = os.path.join(ROOT, "peak", "peak.hip")
    out = os.path.join(ROOT, "peak", "libpeak.so")
    tmp = out + ".tmp"
    _run([HIPCC, *FLAGS, "-shared", src, "-o", tmp], verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

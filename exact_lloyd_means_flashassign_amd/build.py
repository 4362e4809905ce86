"""Build libfk.so (the HIP library) in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libfk.so")
OBJDIR = os.path.join(HERE, "_build")

SOURCES = ["fk_api.hip", "fk_assign.hip", "fk_sort.hip", "fk_update.hip"]
# on-box microbenchmarks (HBM stream, row gather, matrix-product loops): a
# library of their own, loaded only by the benchmark
MICRO_SOURCE = "fk_micro.hip"
MICRO_LIB = os.path.join(HERE, "libfk_micro.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed-fp32 VALU forms are turned off for every HIP file; the compiler's host
# pass warns that it does not know the feature, which is harmless.
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def build(verbose: bool = False) -> str:
    """Compile every source and link libfk.so; always recompiles."""
    os.makedirs(OBJDIR, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(OBJDIR, src.replace(".hip", ".o"))
        cmd = [HIPCC, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
        if verbose and r.stderr.strip():
            sys.stderr.write(r.stderr)
        return obj

    with ThreadPoolExecutor(len(SOURCES) + 1) as ex:
        objs = list(ex.map(compile_one, SOURCES + [MICRO_SOURCE]))
    micro_obj = objs.pop()
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    tmp = MICRO_LIB + ".tmp%d" % os.getpid()
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, micro_obj],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of the microbenchmarks failed:\n{r.stderr}")
    os.replace(tmp, MICRO_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

"""Build libtide.so (HIP kernels + host planner + C ABI) for gfx950 in-tree."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libtide.so")
SOURCES = [os.path.join(CSRC, "kernels.hip"), os.path.join(CSRC, "plan.cpp"),
           os.path.join(CSRC, "sdma.cpp"), os.path.join(CSRC, "noalloc.hip")]
HEADERS = [os.path.join(CSRC, "tide_internal.hpp"), os.path.join(CSRC, "sdma.hpp"),
           os.path.join(ROOT, "include", "tide.h")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Werror", "-Wno-unused-command-line-argument",
    # fp32 arithmetic exactly as written: no flush-to-zero, no contraction,
    # and no packed fp32 instructions.
    "-fno-gpu-flush-denormals-to-zero", "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.sep not in c or os.path.exists(c)):
            return c
    return "hipcc"


def build(out: str = LIB, extra=(), verbose: bool = False) -> str:
    objs = []
    bdir = os.path.join(ROOT, "_build")
    os.makedirs(bdir, exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(bdir, os.path.basename(src) + ".o")
        cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed for %s:\n%s%s" % (src, r.stdout, r.stderr))
        objs.append(obj)
    tmp = out + ".tmp%d" % os.getpid()
    # The DMA-engine path calls the HSA runtime directly.
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs,
           "-L/opt/rocm/lib", "-lhsa-runtime64"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s%s" % (r.stdout, r.stderr))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))

"""Build tests/c_abi_e2e, the plain-C end-to-end test of the C ABI.

Test infrastructure: the program links libtide.so (the library under test),
the HIP runtime and the CPU oracle (oracle/libtide_oracle.so), which it uses
to check the library's results. gcc compiles it as C11 against include/tide.h.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "c_abi_e2e.c")
EXE = os.path.join(HERE, "c_abi_e2e")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(out: str = EXE) -> str:
    cc = os.environ.get("CC", "gcc")
    libdir = os.path.join(ROOT, "mixed_precision_rs_amd")
    odir = os.path.join(ROOT, "oracle")
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [cc, "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           SRC, "-o", tmp,
           "-L", libdir, "-ltide", "-L", odir, "-ltide_oracle",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../mixed_precision_rs_amd:$ORIGIN/../oracle:" + os.path.join(ROCM, "lib")]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())

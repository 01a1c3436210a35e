"""Compile the CPU oracle into oracle/libtide_oracle.so with gcc.

Test infrastructure: the oracle is a plain C11 file built without fast-math,
contraction or vectorising flags that could change its binary32 arithmetic.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "tide_oracle.c")
LIB = os.path.join(HERE, "libtide_oracle.so")
CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-fPIC", "-shared",
          "-Wall", "-Wextra", "-Werror"]


def build(src: str = SRC, out: str = LIB, extra=()) -> str:
    cc = os.environ.get("CC", "gcc")
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run([cc, *CFLAGS, *extra, "-o", tmp, src], check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())

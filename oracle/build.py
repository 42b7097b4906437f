"""Builds the CPU oracle library (test infrastructure only).

The oracle is plain C compiled with gcc; it needs no GPU toolchain and shares
no source with the HIP library.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gg_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
          "-std=c11", "-shared", "-fPIC", "-Wall"]


def build(force=True):
    """Compile gg_oracle.c into liboracle.so (always, unless force is False
    and the library is newer than its source)."""
    if (not force and os.path.exists(LIB)
            and os.path.getmtime(LIB) >= os.path.getmtime(SRC)):
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())

"""Build the CPU oracle shared library with gcc.

Test infrastructure only: the oracle is what the tests, the smoke check and the
benchmark's CPU-baseline leg compare against.  Nothing on the product path
imports or loads it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(OUT_DIR, "libmoe_oracle.so")


def build(src=SRC, out=LIB, extra_flags=()):
    """Compile ``src`` into the shared library ``out`` (plain -O2, IEEE math)."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
           *extra_flags, "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    print(build())
    sys.exit(0)

"""Build the CPU oracle shared library (test infrastructure only).

The oracle is plain C compiled with gcc at -O2 with floating-point
contraction off, so every fp32 operation is one IEEE operation.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libhkv_oracle.so")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "hkv_oracle.c")
    cmd = ["gcc", "-O2", "-std=gnu11", "-ffp-contract=off", "-fno-fast-math",
           "-Wall", "-Wextra", "-fPIC", "-shared", "-o", LIB + ".tmp", src,
           "-lm", "-lpthread"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

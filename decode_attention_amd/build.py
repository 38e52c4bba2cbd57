"""Build libhkv.so (the HIP kernels and the C ABI) for gfx950, in-tree.

Flags: -ffp-contract=off so no multiply-add is fused behind the code's back
(the packed cache bytes depend on every fp32 rounding), HIP's default
correctly rounded fp32 division and square root, and packed-fp32 VALU
instructions disabled.
"""
import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libhkv.so")
# Measurement aid for the benchmark (a streaming-read probe) and a check of
# the library's reciprocal, not the library.
PROBE_LIB = os.path.join(HERE, "libhkv_probe.so")
ARCH = os.environ.get("HKV_OFFLOAD_ARCH", "gfx950")


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def build(verbose: bool = False) -> str:
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    cmd = [hipcc, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-ffp-contract=off", "-Wall",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
           "-o", LIB + ".tmp"] + sources()
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    probe = [hipcc, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
             "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
             "-o", PROBE_LIB + ".tmp", os.path.join(HERE, "probe", "hkv_probe.hip")]
    if verbose:
        print(" ".join(probe))
    subprocess.run(probe, check=True)
    os.replace(PROBE_LIB + ".tmp", PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

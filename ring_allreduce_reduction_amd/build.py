"""Build libar.so (the C-ABI library with the gfx950 kernels) in-tree with hipcc."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libar.so")
SOURCES = ["ar_kernels.hip", "ar_comm.cpp", "ar_tune.cpp", "ar_group.cpp"]
ARCH = os.environ.get("AR_OFFLOAD_ARCH", "gfx950")


def build(verbose: bool = False) -> str:
    cmd = ["hipcc", "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-Wno-unused-function",
           # every add is one IEEE add; binary32 subnormals are kept
           "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
           # no packed-FP32 instructions: each float add is one lane's own add
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    cmd += [os.path.join(CSRC, s) for s in SOURCES]
    cmd += ["-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    build_probe(verbose)
    return LIB


PROBE_LIB = os.path.join(HERE, "libstream_ceiling.so")


def build_probe(verbose: bool = False) -> str:
    """The streaming-ceiling probe bench.py reports beside the HBM peak."""
    cmd = ["hipcc", "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           os.path.join(CSRC, "probes", "stream_ceiling.hip"), "-o", PROBE_LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(PROBE_LIB + ".tmp", PROBE_LIB)
    return PROBE_LIB


if __name__ == "__main__":
    print(build(verbose=True))

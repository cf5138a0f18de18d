"""Build libar.so (the C-ABI library with the gfx950 kernels) in-tree with hipcc.

Every source is compiled to an object of its own, several at a time (the
kernel families live in separate translation units), and the objects are
linked into one shared library."""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libar.so")
OBJ = os.path.join(HERE, "_build")
SOURCES = ["ar_kernels_ring_simple.hip", "ar_kernels_ring_ll.hip", "ar_kernels_ring_ll128.hip", "ar_kernels_ring_batch.hip",
           "ar_kernels_ring_rs.hip", "ar_kernels_ring_ag.hip", "ar_kernels_tree.hip", "ar_kernels_tree_batch.hip",
           "ar_kernels.hip", "ar_noalloc.hip",
           "ar_comm.cpp", "ar_tune.cpp", "ar_group.cpp"]
ARCH = os.environ.get("AR_OFFLOAD_ARCH", "gfx950")
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
         # every add is one IEEE add; binary32 subnormals are kept
         "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
         # no packed-FP32 instructions: each float add is one lane's own add
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _jobs():
    return max(1, min(len(SOURCES), os.cpu_count() or 1, 16))


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]

    def compile_one(src):
        obj = os.path.join(OBJ, src + ".o")
        cmd = ["hipcc"] + FLAGS + inc + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        return obj

    with ThreadPoolExecutor(max_workers=_jobs()) as pool:
        objs = list(pool.map(compile_one, SOURCES))
    cmd = ["hipcc", "--offload-arch=" + ARCH, "-shared", "-fPIC"] + objs + ["-o", LIB + ".tmp"]
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

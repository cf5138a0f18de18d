"""Register and scratch use of the built gfx950 kernels, read from the code
object's own metadata (the device half of libar.so): the kernels on the hot
path must not spill to scratch.  CPU only (objcopy, clang-offload-bundler and
llvm-readelf from the ROCm toolchain)."""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

LLVM = "/opt/rocm/llvm/bin"


@pytest.fixture(scope="module")
def kernels():
    from ring_allreduce_reduction_amd import binding
    lib = binding.LIB_PATH
    if not os.path.exists(lib):
        from ring_allreduce_reduction_amd.build import build
        build()
    tools = [shutil.which("objcopy"), os.path.join(LLVM, "clang-offload-bundler"), os.path.join(LLVM, "llvm-readelf")]
    if not all(t and os.path.exists(t) for t in tools):
        pytest.skip("ROCm toolchain not found")
    with tempfile.TemporaryDirectory() as d:
        fat, copy = os.path.join(d, "fatbin"), os.path.join(d, "lib.copy")
        # an explicit output file: without one objcopy rewrites its input in place
        subprocess.run([tools[0], "--dump-section", ".hip_fatbin=" + fat, lib, copy], check=True)
        # one offload bundle per translation unit with kernels, back to back
        data = open(fat, "rb").read()
        magic = b"__CLANG_OFFLOAD_BUNDLE__"
        starts = []
        i = data.find(magic)
        while i >= 0:
            starts.append(i)
            i = data.find(magic, i + len(magic))
        assert starts, "no offload bundle in libar.so"
        notes = ""
        for n, (a, b) in enumerate(zip(starts, starts[1:] + [len(data)])):
            part, co = os.path.join(d, "bundle%d" % n), os.path.join(d, "gfx950_%d.co" % n)
            with open(part, "wb") as f:
                f.write(data[a:b])
            subprocess.run([tools[1], "--type=o", "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", "--input=" + part,
                            "--output=" + co, "--unbundle"], check=True)
            notes += subprocess.run([tools[2], "--notes", co], check=True, capture_output=True, text=True).stdout
    out, cur = {}, None
    for line in notes.splitlines():
        m = re.match(r"\s+\.name:\s+(\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.match(r"\s+\.(private_segment_fixed_size|vgpr_count|vgpr_spill_count):\s+(\d+)", line)
        if m and cur is not None:
            cur[m.group(1)] = int(m.group(2))
    return out


def _kernel(kernels, tmpl):
    hits = [k for k in kernels if tmpl in k]
    assert hits, "no kernel matching %s" % tmpl
    return hits


def test_headline_kernel_fits_without_spills(kernels):
    # ring, Simple, fp32, Sum, 4 and 8 KiB slots, AllReduce, single call: FIFOs in
    # device memory and in LDS
    names = _kernel(kernels, "ringAllReduceKernelILi2ELi1ELi0ELi8ELi0ELb0E")
    names += _kernel(kernels, "ringAllReduceKernelILi2ELi1ELi0ELi4ELi0ELb0ELb1ELb1ELb1E")
    assert len(names) == 2
    for name in names:
        k = kernels[name]
        assert k["private_segment_fixed_size"] == 0 and k["vgpr_spill_count"] == 0, name
        assert k["vgpr_count"] <= 128, name   # 16 wavefronts of a workgroup fit a CU's register file


def test_no_spills_on_the_fp32_int32_allreduce_paths(kernels):
    bad = []
    for name, k in kernels.items():
        m = re.search(r"(ring|tree)AllReduceKernelILi(\d)ELi(\d)E", name)   # <proto, dtype, ...>
        if not m or m.group(3) not in ("0", "1"):   # data type int32 / fp32
            continue
        if "ring" in name and "ELi0ELb" not in name:   # ring: AllReduce only
            continue
        if k.get("private_segment_fixed_size", 0) or k.get("vgpr_spill_count", 0):
            bad.append((name, k))
    assert not bad, bad


def test_tree_and_batched_kernels_do_not_spill(kernels):
    bad = [(n, k) for n, k in kernels.items()
           if ("treeAllReduceKernel" in n or "ELb1E" in n) and (k.get("vgpr_spill_count", 0) or
                                                                  k.get("private_segment_fixed_size", 0))]
    assert not bad, bad

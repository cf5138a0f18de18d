"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer: the
CPU oracle (oracle/ring_oracle.c), the tuner (ar_tune.cpp: cost model,
measured time table, AR_TUNE_FILE parsing) and the group aggregation rule
(ar_group.cpp), built with gcc / g++ (no GPU code) into one driver
(tests/sanitize/driver.cpp) that exercises them over many argument
combinations, bad ones included.  Run with the compiled table, a valid
AR_TUNE_FILE and a malformed one.  CPU only."""
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "ring_allreduce_reduction_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


@pytest.fixture(scope="module")
def driver():
    if shutil.which("g++") is None or shutil.which("gcc") is None:
        pytest.skip("gcc / g++ not found")
    sys.path.insert(0, ROOT)
    from ring_allreduce_reduction_amd import build
    d = tempfile.mkdtemp(prefix="ar_san_")
    build.write_tune_table_inc(os.path.join(d, "ar_tune_table.inc"))
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", d]
    objs = []
    for src, cc, std in [(os.path.join(ROOT, "oracle", "ring_oracle.c"), "gcc", "-std=c11"),
                         (os.path.join(CSRC, "ar_tune.cpp"), "g++", "-std=c++17"),
                         (os.path.join(CSRC, "ar_group.cpp"), "g++", "-std=c++17"),
                         (os.path.join(ROOT, "tests", "sanitize", "driver.cpp"), "g++", "-std=c++17")]:
        obj = os.path.join(d, os.path.basename(src) + ".o")
        subprocess.run([cc, std, "-Wall"] + SAN + inc + ["-c", src, "-o", obj], check=True)
        objs.append(obj)
    exe = os.path.join(d, "driver")
    subprocess.run(["g++"] + SAN + objs + ["-o", exe, "-lm"], check=True)
    yield exe, d
    shutil.rmtree(d, ignore_errors=True)


def _run(exe, tune_file=None):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("AR_TUNE_FILE", None)
    if tune_file:
        env["AR_TUNE_FILE"] = tune_file
    p = subprocess.run([exe], env=env, capture_output=True, text=True, timeout=600)
    bad = [ln for ln in p.stderr.splitlines() if "AddressSanitizer" in ln or "runtime error" in ln
           or "LeakSanitizer" in ln or "check failed" in ln]
    assert p.returncode == 0 and not bad, (p.returncode, bad[:10], p.stderr[-2000:])
    assert "0 check failures" in p.stdout


def test_host_code_clean_with_compiled_table(driver):
    _run(driver[0])


def test_host_code_clean_with_tune_file(driver):
    exe, d = driver
    path = os.path.join(d, "table.txt")
    shutil.copy(os.path.join(CSRC, "ar_tune_table.txt"), path)
    _run(exe, path)


def test_host_code_clean_with_malformed_tune_file(driver):
    exe, d = driver
    path = os.path.join(d, "bad.txt")
    with open(path, "w") as f:
        f.write("# malformed\n8 4096 1 2 3\nmodel ring simple 1 2\n9999999999999 x y z\n" + "7 " * 5000 + "\n")
    _run(exe, path)
    _run(exe, os.path.join(d, "does_not_exist.txt"))

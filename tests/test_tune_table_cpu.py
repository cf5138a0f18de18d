"""The tuner's measured time table (arTuneTableTime), no GPU needed: every
line of the calibration record the library compiles in is reproduced,
times between lines follow a restatement of the interpolation rule, rank
counts outside the table are not covered, and AR_TUNE_FILE replaces the
table (read once per process, so checked in subprocesses).  The pages let a
tuner plugin override the cost of each candidate before the argmin
["NCCL 原始碼解讀：一個 AllReduce 的 GPU 旅程", ch.5 §一, step 3]."""
import math
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TABLE = os.path.join(ROOT, "ring_allreduce_reduction_amd", "csrc", "ar_tune_table.txt")
COLS = [(0, 0), (0, 1), (0, 2), (1, 0), (1, 1), (1, 2)]   # (algo, proto) of each column


@pytest.fixture(scope="module")
def B():
    from ring_allreduce_reduction_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from ring_allreduce_reduction_amd.build import build
        build()
    binding.lib()
    return binding


def read_table(path):
    tab = {}
    for line in open(path):
        f = line.split("#")[0].split()
        if not f or f[0] == "model":
            continue
        tab.setdefault(int(f[0]), []).append((int(f[1]), [None if x == "-" else float(x) for x in f[2:8]]))
    for n in tab:
        tab[n].sort()
    return tab


def rank_time(lines, S, k):
    """Interpolation along one rank count: log-log between the lines around S;
    the smallest line's time below it; in proportion to bytes past the
    largest; None where a line it needs marks the candidate unable to run."""
    above = [i for i, (b, _) in enumerate(lines) if b >= S]
    if above and above[0] == 0:
        return lines[0][1][k]
    if not above:
        b, ts = lines[-1]
        return None if ts[k] is None else ts[k] * S / b
    (s0, a), (s1, c) = lines[above[0] - 1], lines[above[0]]
    if s1 == S:
        return c[k]
    if a[k] is None or c[k] is None:
        return None
    w = (math.log(S) - math.log(s0)) / (math.log(s1) - math.log(s0))
    return math.exp((1 - w) * math.log(a[k]) + w * math.log(c[k]))


def restated(tab, n, S, k):
    ranks = sorted(tab)
    if n < ranks[0] or n > ranks[-1]:
        return None
    if n in tab:
        return rank_time(tab[n], S, k)
    n0 = max(r for r in ranks if r < n)
    n1 = min(r for r in ranks if r > n)
    t0, t1 = rank_time(tab[n0], S, k), rank_time(tab[n1], S, k)
    if t0 is None or t1 is None:
        return None
    w = (math.log(n) - math.log(n0)) / (math.log(n1) - math.log(n0))
    return math.exp((1 - w) * math.log(t0) + w * math.log(t1))


def test_every_line_is_reproduced(B):
    tab = read_table(TABLE)
    assert len(tab) >= 16 and min(tab) == 2 and max(tab) >= 72
    for n, lines in tab.items():
        for S, ts in lines:
            for k, (a, p) in enumerate(COLS):
                got = B.arTuneTableTime(n, S, a, p)
                if ts[k] is None:
                    assert got is None, (n, S, a, p)
                else:
                    assert got == pytest.approx(ts[k], rel=2e-6), (n, S, a, p)


def test_between_lines_and_rank_counts(B):
    tab = read_table(TABLE)
    rng = np.random.default_rng(7)
    for _ in range(400):
        n = int(rng.integers(2, 129))
        S = int(2 ** rng.uniform(3, 30))
        k = int(rng.integers(0, 6))
        want = restated(tab, n, S, k)
        got = B.arTuneTableTime(n, S, *COLS[k])
        assert (got is None) == (want is None), (n, S, COLS[k])
        if want is not None:
            assert got == pytest.approx(want, rel=1e-4), (n, S, COLS[k])


def test_outside_the_table(B):
    assert B.arTuneTableTime(1, 4096, 0, 2) is None          # one rank: below the table
    assert B.arTuneTableTime(129, 4096, 0, 2) is None        # past the largest rank count
    with pytest.raises(B.ArError):
        B.arTuneTableTime(8, 0, 0, 2)
    with pytest.raises(B.ArError):
        B.arTuneTableTime(8, 4096, 2, 2)


def test_picks_follow_the_table_where_it_differs_from_the_model(B):
    # 4 ranks x 1 MiB: the tree runs faster than the ring on this GPU (the
    # fitted model would take the ring)
    assert B.arTuneTableTime(4, 1 << 20, 1, 2) < B.arTuneTableTime(4, 1 << 20, 0, 2)
    # 2 ranks x 64 B: the tree (the model would take the ring)
    assert B.arTuneTableTime(2, 64, 1, 2) < B.arTuneTableTime(2, 64, 0, 2)
    # 16 ranks x 4 MiB: the ring
    assert B.arTuneTableTime(16, 4 << 20, 0, 2) < B.arTuneTableTime(16, 4 << 20, 1, 2)


def _run_with_table(text, code):
    path = os.path.join(os.environ.get("TMPDIR", "/tmp"), "ar_tune_test_%d.txt" % os.getpid())
    with open(path, "w") as f:
        f.write(text)
    env = dict(os.environ, AR_TUNE_FILE=path)
    try:
        return subprocess.run([sys.executable, "-c", "import sys; sys.path.insert(0, %r)\n" % ROOT + code],
                              env=env, capture_output=True, text=True, timeout=120)
    finally:
        os.remove(path)


def test_tune_file_replaces_the_table():
    text = ("# two rank counts\n4 1024 10 11 12 13 14 15\n4 4096 20 21 22 23 24 -\n8 1024 30 31 32 33 34 35\n"
            "model ring simple 1 2 3 4\n")
    code = ("from ring_allreduce_reduction_amd import binding as B\n"
            "print(B.arTuneTableTime(4, 1024, 0, 2), B.arTuneTableTime(4, 2048, 1, 0), "
            "B.arTuneTableTime(6, 1024, 0, 0), B.arTuneTableTime(4, 3000, 1, 2), B.arTuneTableTime(9, 1024, 0, 0))\n")
    r = _run_with_table(text, code)
    assert r.returncode == 0, r.stderr
    a, b, c, d, e = r.stdout.split()
    assert float(a) == 12.0
    assert float(b) == pytest.approx(math.exp(0.5 * math.log(13) + 0.5 * math.log(23)), rel=1e-5)
    w = math.log(6 / 4) / math.log(8 / 4)
    assert float(c) == pytest.approx(math.exp((1 - w) * math.log(10) + w * math.log(30)), rel=1e-5)
    assert d == "None" and e == "None"   # a candidate marked "-", a rank count past the file's


def test_malformed_tune_file_keeps_the_compiled_table(B):
    code = ("from ring_allreduce_reduction_amd import binding as B\n"
            "print(B.arTuneTableTime(8, 4096, 0, 2))\n")
    r = _run_with_table("8 4096 1 2 3\n", code)
    assert r.returncode == 0, r.stderr
    assert "AR_TUNE_FILE" in r.stderr
    assert float(r.stdout) == pytest.approx(B.arTuneTableTime(8, 4096, 0, 2), rel=1e-6)

"""Two plan decisions of the library, checked on the host (CPU only):

  - the BCSR schedule: 512-wide N tiles from n = 8192 on, 256-wide below;
    four row groups and 256-wide tiles when A (8 KB per stored block) is
    larger than 2 MB and at most 16 MB, n >= 8192 and there are at least
    256 block rows; half-block stages (kh = 32) at 256 columns when block
    rows hold at most 16 blocks on average;
  - the dispatch order of tile-vector-wise row tiles: a permutation, in
    groups of four (the last may be shorter) filled heaviest first in snake
    order, each group of four ordered heaviest, second, lightest, third.

tests/schedule_driver.cpp calls the library's functions; the expected
values are worked out here from those rules."""
import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "sparse_dense_matrix_amd")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    if not os.path.exists(os.path.join(LIBDIR, "libspmm.so")):
        pytest.skip("library not built")
    exe = str(tmp_path_factory.mktemp("schedule") / "schedule_driver")
    subprocess.run([hipcc, "-O1", "-std=c++17", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "schedule_driver.cpp"), "-o", exe,
                    "-L", LIBDIR, "-lspmm", f"-Wl,-rpath,{LIBDIR}"],
                   check=True, capture_output=True)
    return exe


def ask(driver, lines):
    r = subprocess.run([driver], input="\n".join(lines) + "\n", capture_output=True, text=True,
                       check=True)
    return r.stdout.strip().split("\n")


KB8 = 8192  # bytes of one stored 64 x 64 bf16 block


@pytest.mark.parametrize("mb,n,nnzb,expect", [
    (64, 4096, 410, (256, 1, 32)),              # the 4096 case: narrow tiles, few blocks per row
    (10, 1000, 200, (256, 1, 64)),              # 20 blocks per row: whole-block stages
    (296, 65536, 1658, (256, 4, 32)),           # the 90% prefill layer: A 13.6 MB, row groups
    (296, 65536, 4973, (512, 1, 64)),           # the 70% layer: A 40.7 MB, too large for groups
    (296, 65536, 8288, (512, 1, 64)),           # the 50% layer
    (296, 8191, 1658, (256, 1, 32)),            # just below n = 8192
    (296, 8192, 256, (512, 1, 64)),             # A of 2 MB exactly: no groups
    (296, 8192, 257, (256, 4, 32)),             # just above 2 MB
    (296, 8192, 2048, (256, 4, 32)),            # 16 MB exactly: still groups
    (296, 8192, 2049, (512, 1, 64)),            # just above 16 MB
    (255, 65536, 1658, (512, 1, 64)),           # fewer than 256 block rows: no groups
    (320, 8200, 4096 + 1, (512, 1, 64)),        # A > 16 MB
    (320, 8200, 5121, (512, 1, 64)),
    (320, 8200, 420, (256, 4, 32)),             # the integer row-group test
])
def test_bcsr_schedule(driver, mb, n, nnzb, expect):
    tn, rg, kh = map(int, ask(driver, [f"schedule {mb} {n} {nnzb}"])[0].split())
    assert (tn, rg, kh) == expect
    # the rules, restated
    a_bytes = nnzb * KB8
    groups = n >= 8192 and 2 << 20 < a_bytes <= 16 << 20 and mb >= 256
    assert tn == (256 if groups or n < 8192 else 512)
    assert rg == (4 if groups else 1)
    assert kh == (32 if tn == 256 and nnzb <= 16 * mb else 64)


def snake_order(counts):
    """The rule, restated: heaviest first (lowest index on ties) into groups
    of four in snake order, each group of four ordered 0, 1, 3, 2."""
    mt = len(counts)
    by_work = sorted(range(mt), key=lambda t: (-counts[t], t))
    G = (mt + 3) // 4
    cap = [min(4, mt - 4 * g) for g in range(G)]
    members = [[] for _ in range(G)]
    g, d = 0, 1
    def step():
        nonlocal g, d
        if g + d < 0 or g + d >= G:
            d = -d
        else:
            g += d
    for t in by_work:
        while len(members[g]) >= cap[g]:
            step()
        members[g].append(t)
        step()
    out = []
    for m in members:
        if len(m) == 4:
            m = [m[0], m[1], m[3], m[2]]
        out += m
    return out


def test_tvw_row_order_hand_worked(driver):
    # 8 row tiles, counts 8..1 (tile 0 heaviest): snake over 2 groups puts
    # tiles 0, 3, 4, 7 in group 0 and 1, 2, 5, 6 in group 1; ordered
    # heaviest, second, lightest, third
    got = list(map(int, ask(driver, ["tvw 8 8 7 6 5 4 3 2 1"])[0].split()))
    assert got == [0, 3, 7, 4, 1, 2, 6, 5]


@pytest.mark.parametrize("mt", [1, 3, 4, 5, 10, 32, 33])
def test_tvw_row_order_follows_the_rule(driver, mt):
    r = np.random.default_rng(mt)
    counts = r.integers(0, 9, size=mt).tolist()
    got = list(map(int, ask(driver, [f"tvw {mt} " + " ".join(map(str, counts))])[0].split()))
    assert sorted(got) == list(range(mt))
    assert got == snake_order(counts)
    # the groups' totals differ by at most the heaviest row tile
    totals = [sum(counts[t] for t in got[i:i + 4]) for i in range(0, 4 * (mt // 4), 4)]
    if totals:
        assert max(totals) - min(totals) <= max(counts)

"""The BCSR plan's pairing of block rows (host logic, CPU only).

A paired tile computes two block rows over the union of their block
columns, so a B slab both rows use is loaded once.  The plan pairs rows
greedily: rows in order of decreasing block count (lowest index first on
ties); each unpaired row takes the unpaired row that shares most block
columns with it (lowest index on ties), or, when none shares any, the
largest row left.  tests/pairing_driver.cpp calls the library's pairing
on a pattern and prints the pairs and their units; these tests check the
units against the pattern and the pairs against that rule, restated here
independently."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "sparse_dense_matrix_amd")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    if not os.path.exists(os.path.join(LIBDIR, "libspmm.so")):
        pytest.skip("library not built")
    exe = str(tmp_path_factory.mktemp("pairing") / "pairing_driver")
    subprocess.run([hipcc, "-O1", "-std=c++17", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "pairing_driver.cpp"), "-o", exe,
                    "-L", LIBDIR, "-lspmm", f"-Wl,-rpath,{LIBDIR}"],
                   check=True, capture_output=True)
    return exe


def run_pairing(driver, rows, kb):
    """rows: list of sorted block-column lists.  Returns (saving, pairs, units)
    with pairs [(r0, r1, u0, u1)] and units [(col, b0, b1)]."""
    rp = np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(int)
    ci = [c for r in rows for c in r]
    text = f"{len(rows)} {kb} {len(ci)}\n" + " ".join(map(str, rp)) + "\n" + " ".join(map(str, ci)) + "\n"
    r = subprocess.run([driver], input=text, capture_output=True, text=True, check=True)
    lines = r.stdout.split("\n")
    saving = float(lines[0])
    npairs = int(lines[1])
    pairs = [tuple(map(int, lines[2 + p].split())) for p in range(npairs)]
    nunits = int(lines[2 + npairs])
    units = [tuple(map(int, lines[3 + npairs + u].split())) for u in range(nunits)]
    return saving, pairs, units, rp


def greedy_pairs(rows):
    """The pairing rule, restated: [(first row, second row or -1)]."""
    order = sorted(range(len(rows)), key=lambda i: (-len(rows[i]), i))
    sets = [set(r) for r in rows]
    used = [False] * len(rows)
    out = []
    for r in order:
        if used[r]:
            continue
        used[r] = True
        best, best_shared = -1, 0
        for s in range(len(rows)):
            if not used[s]:
                shared = len(sets[r] & sets[s])
                if shared > best_shared:
                    best, best_shared = s, shared
        if best < 0:
            left = [s for s in order if not used[s]]
            best = left[0] if left else -1
        if best >= 0:
            used[best] = True
        out.append((r, best))
    return out


def check_units(rows, rp, pairs, units):
    """Every stored block appears in exactly one unit, in its own row's slot,
    and a pair's units are the ascending union of its rows' block columns."""
    seen = np.zeros(rp[-1], int)
    for r0, r1, u0, u1 in pairs:
        cols = [units[u][0] for u in range(u0, u1)]
        union = sorted(set(rows[r0]) | (set(rows[r1]) if r1 >= 0 else set()))
        assert cols == union
        for u in range(u0, u1):
            col, b0, b1 = units[u]
            for row, b in ((r0, b0), (r1, b1)):
                if b < 0:
                    assert row < 0 or col not in rows[row]
                else:
                    assert rp[row] <= b < rp[row + 1] and rows[row][b - rp[row]] == col
                    seen[b] += 1
    assert (seen == 1).all()
    assert [p[2] for p in pairs] == [0] + [p[3] for p in pairs[:-1]] and pairs[-1][3] == len(units)


def test_hand_worked_pairing(driver):
    # r0 {0,1,2} takes r1 {0,1} (two shared columns, against one with r2);
    # r2 {2,3} then shares nothing with r3 {5}, and takes it as the largest
    # row left.  8 blocks in 6 units: a quarter of the B slab loads saved.
    rows = [[0, 1, 2], [0, 1], [2, 3], [5]]
    saving, pairs, units, rp = run_pairing(driver, rows, 6)
    assert [(p[0], p[1]) for p in pairs] == [(0, 1), (2, 3)]
    assert units == [(0, 0, 3), (1, 1, 4), (2, 2, -1), (2, 5, -1), (3, 6, -1), (5, -1, 7)]
    assert saving == pytest.approx(0.25, abs=1e-15)
    check_units(rows, rp, pairs, units)


def test_ties_take_the_lowest_index_and_odd_counts_leave_a_single(driver):
    # r0 {0,1} shares one column with r1 and one with r2: r1 (lower index);
    # r2 is then alone; an empty row pairs like any other
    rows = [[0, 1], [0], [1], []]
    _, pairs, units, rp = run_pairing(driver, rows, 2)
    assert [(p[0], p[1]) for p in pairs] == [(0, 1), (2, 3)]
    check_units(rows, rp, pairs, units)
    rows = [[0, 1], [0], [1]]
    _, pairs, units, rp = run_pairing(driver, rows, 2)
    assert [(p[0], p[1]) for p in pairs] == [(0, 1), (2, -1)]
    check_units(rows, rp, pairs, units)


def test_more_than_64_units_refuses(driver):
    # a pair that would walk 70 block columns: the pairing reports no saving
    # (the plan then keeps single-row tiles)
    rows = [list(range(70)), [0, 1], [3], [4]]
    saving, _, _, _ = run_pairing(driver, rows, 70)
    assert saving == 0.0


def test_search_beyond_its_bound_refuses(driver):
    # 8,000 block rows at 30% of 56 block columns: the search would visit
    # 56 * 2,400^2 = 3.2e8 rows, past the bound (2^28); no pairing.  At 7,000
    # rows (2.5e8 visits) the rows are still paired.
    r = np.random.default_rng(6)
    for mb, paired in ((8000, False), (7000, True)):
        mask = r.random((mb, 56)) < 0.3
        rows = [np.nonzero(m)[0].tolist() for m in mask]
        saving, pairs, units, rp = run_pairing(driver, rows, 56)
        assert (saving > 0.1) == paired
        if paired:
            check_units(rows, rp, pairs, units)


@pytest.mark.parametrize("name", ["bcsr_prefill_18944x3584", "bcsr_prefill_18944x3584_z70",
                                  "bcsr_4096_b64_90"])
def test_benchmark_patterns_follow_the_rule(driver, name):
    w = synth.WORKLOADS[name]
    mb, kb = w.m // 64, w.k // 64
    ids = np.sort(synth.rng(w.seed, synth.S_PATTERN).choice(mb * kb, size=w.nblocks, replace=False))
    rows = [[] for _ in range(mb)]
    for b in ids:
        rows[int(b) // kb].append(int(b) % kb)
    saving, pairs, units, rp = run_pairing(driver, rows, kb)
    assert [(p[0], p[1]) for p in pairs] == greedy_pairs(rows)
    check_units(rows, rp, pairs, units)
    assert saving == pytest.approx(1 - len(units) / len(ids), abs=1e-12)
    if name == "bcsr_prefill_18944x3584":
        assert len(units) == 1285          # 22.5% fewer B half-slab loads than 1,658 blocks


def test_random_patterns_follow_the_rule(driver):
    r = np.random.default_rng(5)
    for trial in range(20):
        mb, kb = int(r.integers(1, 40)), int(r.integers(1, 30))
        dens = float(r.uniform(0.0, 0.6))
        rows = [sorted(np.nonzero(r.random(kb) < dens)[0].tolist()) for _ in range(mb)]
        if sum(map(len, rows)) == 0:
            continue
        saving, pairs, units, rp = run_pairing(driver, rows, kb)
        assert [(p[0], p[1]) for p in pairs] == greedy_pairs(rows), trial
        check_units(rows, rp, pairs, units)

"""Row/column reordering before BCSR (spmm_pack_bcsr_csr): host logic, no GPU.

The permutation is a heuristic, so what is pinned is what must hold for any
valid one: both are permutations, the packed blocks are exactly the permuted
matrix cut into blocks (checked against the oracle's own packer), the block
count never grows, and a matrix whose block structure was hidden by shuffling
rows and columns gets all of it back.  The permutation that minimises nonzero
blocks is named on the "Daily Papers" search page (block-sparse SpMM on
tensor cores for unstructured matrices)."""
import numpy as np
import pytest

import synth


@pytest.fixture(scope="module")
def S():
    import sparse_dense_matrix_amd as S
    return S


def _arrays(S, M):
    return {w: S.spmm_matrix_array(M, w) for w in
            (S.ARRAY_ROW_PTR, S.ARRAY_COL_IDX, S.ARRAY_VALS, S.ARRAY_ROW_PERM, S.ARRAY_COL_PERM)}


def _plus_zero(a_bits):
    """-0 written as +0: the CSR keeps no zeros, so blocks built from it hold +0."""
    a = a_bits.copy()
    a[(a & 0x7FFF) == 0] = 0
    return a


def _csr_of(a_bits):
    nz = (a_bits & 0x7FFF) != 0
    rp = np.zeros(a_bits.shape[0] + 1, np.int64)
    np.cumsum(nz.sum(axis=1), out=rp[1:])
    r, c = np.nonzero(nz)
    return rp, c.astype(np.int32), a_bits[r, c].astype(np.uint16)


def test_no_reorder_matches_dense_packer(S, orc):
    a, _ = synth.block_sparse_dense_bf16(512, 768, 64, 64, 30, 0.02, 41)
    a = _plus_zero(a)
    rp, ci, v = _csr_of(a)
    M = S.spmm_pack_bcsr_csr(512, 768, rp, ci, v, reorder=False)
    got = _arrays(S, M)
    orp, oci, ov = orc.pack_bcsr(a, 64, 64)
    np.testing.assert_array_equal(got[S.ARRAY_ROW_PTR], orp)
    np.testing.assert_array_equal(got[S.ARRAY_COL_IDX], oci)
    np.testing.assert_array_equal(got[S.ARRAY_VALS], ov.reshape(-1))
    assert len(got[S.ARRAY_ROW_PERM]) == 0 and len(got[S.ARRAY_COL_PERM]) == 0


@pytest.mark.parametrize("seed", range(6))
def test_reordered_blocks_are_the_permuted_matrix(S, orc, seed):
    r = np.random.default_rng(900 + seed)
    m, k = 64 * int(r.integers(2, 9)), 64 * int(r.integers(2, 9))
    a, _ = synth.block_sparse_dense_bf16(m, k, 64, 64, int(r.integers(1, (m // 64) * (k // 64))),
                                         0.02, 50 + seed)
    # sprinkle single entries too, so not every block is clean
    extra = r.integers(0, [m, k], size=(int(r.integers(0, 40)), 2))
    a[extra[:, 0], extra[:, 1]] = 0x3F80
    rp, ci, v, _, _ = synth.scrambled_csr_bf16(a, 60 + seed)
    dense = np.zeros((m, k), np.uint16)
    dense[np.repeat(np.arange(m), np.diff(rp)), ci] = v
    M = S.spmm_pack_bcsr_csr(m, k, rp, ci, v, reorder=True)
    got = _arrays(S, M)
    rperm, cperm = got[S.ARRAY_ROW_PERM], got[S.ARRAY_COL_PERM]
    plain = orc.pack_bcsr(dense, 64, 64)
    if len(rperm) == 0:                      # no gain: the original order is kept
        np.testing.assert_array_equal(got[S.ARRAY_COL_IDX], plain[1])
        return
    np.testing.assert_array_equal(np.sort(rperm), np.arange(m))
    np.testing.assert_array_equal(np.sort(cperm), np.arange(k))
    orp, oci, ov = orc.pack_bcsr(dense[rperm][:, cperm], 64, 64)
    np.testing.assert_array_equal(got[S.ARRAY_ROW_PTR], orp)
    np.testing.assert_array_equal(got[S.ARRAY_COL_IDX], oci)
    np.testing.assert_array_equal(got[S.ARRAY_VALS], ov.reshape(-1))
    assert len(oci) < len(plain[1])          # kept only when it has fewer blocks


def test_hidden_block_structure_is_recovered(S, orc):
    # 90% of the 64 x 64 blocks zero, then rows and columns shuffled: every
    # block of the shuffled matrix holds entries, and the reordering finds
    # the original blocks again
    w = synth.WORKLOADS["bcsr_4096_b64_90"]
    a, ids = synth.block_sparse_dense_bf16(1024, 1024, 64, 64, 26, 0.02, 77)
    rp, ci, v, _, _ = synth.scrambled_csr_bf16(a, 78)
    plain = S.spmm_matrix_info(S.spmm_pack_bcsr_csr(1024, 1024, rp, ci, v, reorder=False))
    M = S.spmm_pack_bcsr_csr(1024, 1024, rp, ci, v, reorder=True)
    info = S.spmm_matrix_info(M)
    assert plain["nnzb"] >= 200
    assert info["nnzb"] == 26
    assert w.block == 64


def test_reorder_arguments(S):
    rp = np.array([0, 1, 1], np.int64)
    ci = np.array([3], np.int32)
    v = np.array([0x3F80], np.uint16)
    with pytest.raises(S.SpmmError) as e:
        S.spmm_pack_bcsr_csr(2, 64, rp, ci, v, reorder=False)      # m % 64 != 0
    assert e.value.name == "SPMM_ERR_INVALID_ARG"
    import ctypes
    rp = np.zeros(65, np.int64)
    rp[1:] = 1
    h = ctypes.c_void_p()
    st = S.lib().spmm_pack_bcsr_csr(64, 64, S.BF16, rp.ctypes.data, ci.ctypes.data, v.ctypes.data,
                                    64, 64, 2, ctypes.byref(h))       # reorder must be 0 or 1
    assert st == 1 and not h.value
    bad = np.array([0, 2] + [2] * 63, np.int64)
    with pytest.raises(S.SpmmError) as e:                          # columns not ascending
        S.spmm_pack_bcsr_csr(64, 64, bad, np.array([5, 5], np.int32),
                             np.array([1, 1], np.uint16), reorder=True)
    assert e.value.name == "SPMM_ERR_INVALID_ARG"


# ---------------------------------------------------------------------------
# the permutation itself, against the oracle's plain implementation of the
# reading (oracle.h, orc_reorder_perms)
# ---------------------------------------------------------------------------

def _oracle_case(orc, g, name):
    m, k, bm, bk = g[f"{name}_shape"][0]
    rp = np.array(g[f"{name}_row_ptr"][0], np.int64)
    ci = np.array(g[f"{name}_col_idx"][0], np.int32)
    return m, k, bm, bk, rp, ci, orc.reorder_perms(m, k, rp, ci, bm, bk)


def test_oracle_reorder_hand_examples(orc):
    from conftest import read_golden
    g = read_golden("reorder_hand.txt")
    m, k, bm, bk, rp, ci, (kept, rperm, cperm, before, after) = _oracle_case(orc, g, "case1")
    assert kept == bool(g["case1_kept"][0][0])
    np.testing.assert_array_equal(rperm, g["case1_row_perm"][0])
    np.testing.assert_array_equal(cperm, g["case1_col_perm"][0])
    assert [before, after] == g["case1_blocks"][0]
    m, k, bm, bk, rp, ci, (kept, rperm, cperm, before, after) = _oracle_case(orc, g, "case2")
    assert kept == bool(g["case2_kept"][0][0])
    np.testing.assert_array_equal(rperm, np.arange(m))
    np.testing.assert_array_equal(cperm, np.arange(k))
    assert [before, after] == g["case2_blocks"][0]


def _dense_list_less(xa, xb):
    """Lexicographic order of two ascending index lists given as 0/1 vectors,
    a prefix first: at the first position where they differ, the list that
    holds it is smaller unless the other one has nothing after it."""
    d = np.nonzero(xa != xb)[0]
    if len(d) == 0:
        return False
    r = d[0]
    if xa[r]:
        return bool(xb[r + 1:].any())
    return not bool(xa[r + 1:].any())


def _random_pattern(r, m, k, density, empty_rows=(), empty_cols=(), dup_cols=()):
    nz = r.random((m, k)) < density
    for c, src in dup_cols:
        nz[:, c] = nz[:, src]
    nz[list(empty_rows), :] = False
    nz[:, list(empty_cols)] = False
    rp = np.zeros(m + 1, np.int64)
    np.cumsum(nz.sum(axis=1), out=rp[1:])
    return nz, rp, np.nonzero(nz)[1].astype(np.int32)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_oracle_reorder_invariants(orc, seed):
    # the oracle's orders checked with a comparator written differently (on
    # 0/1 vectors), and its block counts against a direct count
    r = np.random.default_rng(seed)
    m, k, bm, bk = 48, 40, 8, 8
    nz, rp, ci = _random_pattern(r, m, k, 0.06, empty_rows=(3, 17), empty_cols=(5,),
                                 dup_cols=((9, 2), (30, 2)))
    kept, rperm, cperm, before, after = orc.reorder_perms(m, k, rp, ci, bm, bk)

    def blocks(a):
        return int(a.reshape(m // bm, bm, k // bk, bk).any(axis=(1, 3)).sum())

    assert before == blocks(nz)
    if not kept:
        return
    assert sorted(rperm) == list(range(m)) and sorted(cperm) == list(range(k))
    for a, b in zip(cperm[:-1], cperm[1:]):
        assert not _dense_list_less(nz[:, b], nz[:, a]), (a, b)
        if (nz[:, a] == nz[:, b]).all():
            assert a < b
    pc = nz[:, cperm]
    bcols = pc.reshape(m, k // bk, bk).any(axis=2)
    for a, b in zip(rperm[:-1], rperm[1:]):
        assert not _dense_list_less(bcols[b], bcols[a]), (a, b)
        if (bcols[a] == bcols[b]).all():
            assert a < b
    assert after == blocks(nz[rperm][:, cperm]) and after < before


def test_oracle_reorder_recovers_hidden_blocks(orc):
    # full blocks hidden by shuffling rows and columns: every column of a
    # block has the same row list, so the order must bring back exactly the
    # original blocks (partly filled blocks need not come back whole)
    r = np.random.default_rng(7)
    m = k = 64
    nz = np.zeros((m, k), bool)
    for b in range(8):
        nz[8 * b:8 * b + 8, 8 * ((3 * b) % 8):8 * ((3 * b) % 8) + 8] = True
    shuf = nz[r.permutation(m)][:, r.permutation(k)]
    rp = np.zeros(m + 1, np.int64)
    np.cumsum(shuf.sum(axis=1), out=rp[1:])
    kept, rperm, cperm, before, after = orc.reorder_perms(m, k, rp, np.nonzero(shuf)[1], 8, 8)
    assert kept and after == 8 and before > 8


@pytest.mark.parametrize("case", ["random_sparse", "ties_and_empties", "hidden_blocks", "no_gain"])
def test_library_permutation_equals_oracle(S, orc, case):
    r = np.random.default_rng({"random_sparse": 11, "ties_and_empties": 12, "hidden_blocks": 13,
                               "no_gain": 14}[case])
    m, k = 256, 320
    if case == "random_sparse":
        nz, rp, ci = _random_pattern(r, m, k, 0.01)
    elif case == "ties_and_empties":
        nz, rp, ci = _random_pattern(r, m, k, 0.02, empty_rows=range(0, 256, 9),
                                     empty_cols=range(1, 320, 7), dup_cols=((10, 3), (200, 3), (64, 65)))
    elif case == "hidden_blocks":
        base = np.zeros((m, k), bool)
        for b in r.choice(4 * 5, 6, replace=False):
            i, j = divmod(int(b), 5)
            base[64 * i:64 * i + 64, 64 * j:64 * j + 64] = r.random((64, 64)) < 0.5
        nz = base[r.permutation(m)][:, r.permutation(k)]
        rp = np.zeros(m + 1, np.int64)
        np.cumsum(nz.sum(axis=1), out=rp[1:])
        ci = np.nonzero(nz)[1].astype(np.int32)
    else:
        nz = np.zeros((m, k), bool)
        nz[:64, :64] = True                      # one full block: nothing to gain
        rp = np.zeros(m + 1, np.int64)
        np.cumsum(nz.sum(axis=1), out=rp[1:])
        ci = np.nonzero(nz)[1].astype(np.int32)
    vals = np.full(len(ci), 0x3F80, np.uint16)
    M = S.spmm_pack_bcsr_csr(m, k, rp, ci, vals, reorder=True)
    kept, rperm, cperm, before, after = orc.reorder_perms(m, k, rp, ci, 64, 64)
    got_r = S.spmm_matrix_array(M, S.ARRAY_ROW_PERM)
    got_c = S.spmm_matrix_array(M, S.ARRAY_COL_PERM)
    if kept:
        np.testing.assert_array_equal(got_r, rperm)
        np.testing.assert_array_equal(got_c, cperm)
    else:
        assert len(got_r) == 0 and len(got_c) == 0
    assert S.spmm_matrix_info(M)["nnzb"] == after
    assert kept == (case != "no_gain")


def test_library_permutation_equals_oracle_scrambled_4096(S, orc):
    # the scrambled 4096 workload: its 410 hidden blocks, permutations bit for bit
    w = synth.WORKLOADS["scrambled_4096_bcsr_reordered"]
    a = synth.make_a(w)
    M = S.spmm_pack_bcsr_csr(w.m, w.k, a["row_ptr"], a["col_idx"], a["vals_bf16"], reorder=True)
    kept, rperm, cperm, before, after = orc.reorder_perms(w.m, w.k, a["row_ptr"], a["col_idx"], 64, 64)
    assert kept and after == 410
    np.testing.assert_array_equal(S.spmm_matrix_array(M, S.ARRAY_ROW_PERM), rperm)
    np.testing.assert_array_equal(S.spmm_matrix_array(M, S.ARRAY_COL_PERM), cperm)

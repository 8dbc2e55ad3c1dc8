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

"""Sliding-window decomposition of (2N-2):2N weights (spmm_pack_slide): host
logic, no GPU.

The (2N-2):2N family and its decomposition into N-1 overlapping 2:4 windows
are on the "Daily Papers" search page.  What must hold for any valid
decomposition: each window is a valid 2:4 group, and folding the lifted
matrix back onto the original columns (lifted column 4w + j of group g is
original column 2N g + 2w + j) gives exactly the oracle's (2N-2):2N pruning.
Every pattern of kept positions is tried for N = 2..5."""
import itertools

import numpy as np
import pytest

import synth


@pytest.fixture(scope="module")
def S():
    import sparse_dense_matrix_amd as S
    return S


def source_column(j, group):
    per = 2 * (group - 2)
    g, o = divmod(j, per)
    return g * group + 2 * (o // 4) + o % 4


def fold(orc, S, M, m, k, group):
    v = S.spmm_matrix_array(M, S.ARRAY_VALS)
    mt = S.spmm_matrix_array(M, S.ARRAY_META)
    k_lift = len(v) // m * 2
    lifted = orc.densify24(v.reshape(m, k_lift // 2), mt.reshape(m, k_lift // 8))
    out = np.zeros((m, k), np.int64)
    for j in range(k_lift):
        out[:, source_column(j, group)] += lifted[:, j]
    return out, k_lift


@pytest.mark.parametrize("group", [4, 6, 8, 10])
def test_every_kept_pattern_folds_back(S, orc, group):
    keep = group - 2
    pats = list(itertools.combinations(range(group), keep))
    a = np.zeros((len(pats), group * 2), np.int8)
    for i, kept in enumerate(pats):
        for rank, p in enumerate(kept):
            a[i, p] = 100 - rank                        # the kept ones are the largest
            a[i, group + p] = -(60 + rank)
        for p in set(range(group)) - set(kept):
            a[i, p] = 1                                 # dropped: smaller magnitude
    if (2 * (group // 2 - 1) * 2 * 2) % 8:               # lifted row must hold whole bytes
        a = np.concatenate([a, a], axis=1)
    M = S.spmm_pack_slide(a, group)
    got, _ = fold(orc, S, M, a.shape[0], a.shape[1], group)
    np.testing.assert_array_equal(got, orc.prune_nm(a, keep, group))


@pytest.mark.parametrize("seed,group", [(0, 8), (1, 8), (2, 6), (3, 16), (4, 4)])
def test_random_matrices_fold_back(S, orc, seed, group):
    r = np.random.default_rng(1200 + seed)
    m, k = int(r.integers(1, 40)), group * 4 * int(r.integers(1, 6))
    a = synth.int8_uniform(r, (m, k))
    a[r.random(a.shape) < 0.2] = 0                      # zeros inside groups
    a[0, :group] = -128
    M = S.spmm_pack_slide(a, group)
    got, k_lift = fold(orc, S, M, m, k, group)
    np.testing.assert_array_equal(got, orc.prune_nm(a, group - 2, group))
    assert k_lift == k // group * 4 * (group // 2 - 1)
    assert S.spmm_matrix_info(M)["block_k"] == group


def test_2_of_4_is_the_plain_24_pack(S, orc):
    a = synth.int8_uniform(np.random.default_rng(9), (17, 64))
    M = S.spmm_pack_slide(a, 4)
    v, mt = orc.pack24(a)
    np.testing.assert_array_equal(S.spmm_matrix_array(M, S.ARRAY_VALS), v.reshape(-1))
    np.testing.assert_array_equal(S.spmm_matrix_array(M, S.ARRAY_META), mt.reshape(-1))


def test_slide_arguments(S):
    for shape, group in (((4, 12), 8), ((4, 16), 7), ((4, 16), 2), ((4, 8), 6), ((4, 6), 6 * 11)):
        with pytest.raises(S.SpmmError) as e:
            S.spmm_pack_slide(np.zeros(shape, np.int8), group)
        assert e.value.name == "SPMM_ERR_INVALID_ARG"

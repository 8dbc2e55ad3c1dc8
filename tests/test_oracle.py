"""Pins for the CPU oracle: hand-worked fixtures, brute force, closed forms and
invariants.  None of these re-types the oracle's own loops: each compares it
with something the definitions fix independently (a hand computation, numpy's
dense matmul on the densified matrix, an identity or permutation product, a
numpy re-derivation of the 2:4 selection rule).

Sources: AsyncSparse abstract and Figure 2 caption (BCSR, WCSR, row-window
splitting); Magicube abstract (int8 SpMM); tiled-GEMM abstract (2:4 pattern);
search-results page entries on N:M sparsity and on SpMM.
"""
import numpy as np
import pytest

import synth
from conftest import read_golden

# ---------------------------------------------------------------------------
# hand-worked fixtures
# ---------------------------------------------------------------------------


def test_golden_pack24(orc):
    g = read_golden("pack24_hand.txt")
    a = np.array(g["a"], dtype=np.int8)
    vals, meta = orc.pack24(a)
    np.testing.assert_array_equal(vals, np.array(g["vals"], dtype=np.int8))
    np.testing.assert_array_equal(meta, np.array(g["meta"], dtype=np.uint8))
    k = a.shape[1]
    B = np.zeros((k, 2), dtype=np.int8)
    B[:, 0] = np.arange(1, k + 1)
    B[:, 1] = np.where(np.arange(k) % 2 == 0, 2, -2)
    c = orc.sp24_spmm(vals, meta, B)
    np.testing.assert_array_equal(c, np.array(g["c"], dtype=np.int32))


def test_golden_csr(orc):
    g = read_golden("csr_hand.txt")
    rp = np.array(g["row_ptr"][0], dtype=np.int64)
    ci = np.array(g["col_idx"][0], dtype=np.int32)
    v = np.array(g["vals"][0], dtype=np.float32)
    B = np.array(g["b"], dtype=np.float32)
    m = g["m"][0][0]
    assert orc.csr_check(m, g["k"][0][0], rp, ci) == 0
    c = orc.csr_spmm(rp, ci, v, B)
    np.testing.assert_array_equal(c, np.array(g["c"], dtype=np.float64))
    for W, T in ((2, 1), (2, 2), (1, 8)):
        cw, cb = orc.wcsr_chunks(m, rp, W, T)
        np.testing.assert_array_equal(cw, g[f"chunks W={W} T={T} window"][0])
        np.testing.assert_array_equal(cb, g[f"chunks W={W} T={T} begin"][0])


def test_golden_bcsr(orc):
    g = read_golden("bcsr_hand.txt")
    a = np.array(g["a"], dtype=np.uint16)
    bm, bk = g["block"][0]
    rp, ci, v = orc.pack_bcsr(a, bm, bk)
    np.testing.assert_array_equal(rp, g["row_ptr"][0])
    np.testing.assert_array_equal(ci, g["col_idx"][0])
    np.testing.assert_array_equal(v.reshape(len(ci), -1), np.array(g["vals"], dtype=np.uint16))
    B = synth.f32_to_bf16_bits(np.array(g["b"], dtype=np.float32))
    c = orc.bcsr_spmm(bm, bk, rp, ci, v, B)
    np.testing.assert_array_equal(c, np.array(g["c"], dtype=np.float64))


def test_bf16_widening(orc):
    # bit patterns whose values are fixed by the IEEE binary32 layout
    assert orc.bf16_to_double(0x3F80) == 1.0
    assert orc.bf16_to_double(0xC000) == -2.0
    assert orc.bf16_to_double(0x3F00) == 0.5
    assert orc.bf16_to_double(0x0001) == 2.0 ** -133   # smallest subnormal
    assert orc.bf16_to_double(0x7F7F) == (2 - 2 ** -7) * 2.0 ** 127


# ---------------------------------------------------------------------------
# brute force on tiny random inputs: oracle vs numpy dense matmul of the
# densified matrix (a library routine that shares nothing with the oracle)
# ---------------------------------------------------------------------------


def _np_dense_from_csr(m, k, rp, ci, v):
    d = np.zeros((m, k), dtype=np.float64)
    rows = np.repeat(np.arange(m), np.diff(rp))
    d[rows, ci] = v
    return d


@pytest.mark.parametrize("seed", range(40))
def test_csr_bruteforce(orc, seed):
    r = np.random.default_rng(seed)
    m, k, n = (int(x) for x in r.integers(1, 97, size=3))
    rp, ci, v = synth.csr_uniform(m, k, float(r.uniform(0.0, 0.4)), 1000 + seed)
    B = r.standard_normal((k, n)).astype(np.float32)
    got = orc.csr_spmm(rp, ci, v, B)
    dense = _np_dense_from_csr(m, k, rp, ci, v)
    np.testing.assert_array_equal(orc.csr_densify(m, k, rp, ci, v), dense)
    ref = dense @ B.astype(np.float64)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    # the oracle's own naive dense GEMM agrees exactly: same k order, and the
    # zero products it adds do not change a double sum
    np.testing.assert_array_equal(got + 0.0, orc.gemm_f64(dense, B.astype(np.float64)) + 0.0)
    # a row subset and a column slab are slices of the full product
    rows = np.sort(r.choice(m, size=max(1, m // 3), replace=False)).astype(np.int64)
    j0, j1 = sorted(int(x) for x in r.integers(0, n + 1, size=2))
    np.testing.assert_array_equal(orc.csr_spmm(rp, ci, v, B, rows=rows, j0=j0, j1=j1),
                                  got[rows][:, j0:j1])


@pytest.mark.parametrize("seed", range(30))
def test_bcsr_bruteforce(orc, seed):
    r = np.random.default_rng(100 + seed)
    bm, bk = (int(x) for x in r.choice([1, 2, 4, 8, 16], size=2))
    mb, kb = (int(x) for x in r.integers(1, 7, size=2))
    m, k, n = mb * bm, kb * bk, int(r.integers(1, 70))
    nblocks = int(r.integers(0, mb * kb + 1))
    a, ids = synth.block_sparse_dense_bf16(m, k, bm, bk, nblocks, 0.5, 2000 + seed)
    rp, ci, v = orc.pack_bcsr(a, bm, bk)
    # block mask = the drawn blocks (N(0,0.5) never rounds a whole block to 0)
    assert len(ci) == nblocks
    assert sorted(int(x) for x in (np.repeat(np.arange(mb), np.diff(rp)) * kb + ci)) == \
        sorted(int(x) for x in ids)
    dense = synth.bf16_bits_to_f32(a).astype(np.float64)
    np.testing.assert_array_equal(orc.bcsr_densify(m, k, bm, bk, rp, ci, v), dense)
    Bb = synth.f32_to_bf16_bits(r.standard_normal((k, n)).astype(np.float32))
    got = orc.bcsr_spmm(bm, bk, rp, ci, v, Bb)
    ref = dense @ synth.bf16_bits_to_f32(Bb).astype(np.float64)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def _np_prune24(a):
    """2:4 selection re-derived with numpy: stable argsort of -|a| per group."""
    m, k = a.shape
    g = a.reshape(m, k // 4, 4).astype(np.int64)
    order = np.argsort(-np.abs(g), axis=2, kind="stable")[:, :, :2]
    keep = np.zeros_like(g, dtype=bool)
    np.put_along_axis(keep, order, True, axis=2)
    return np.where(keep, g, 0).reshape(m, k).astype(np.int8)


@pytest.mark.parametrize("seed", range(30))
def test_sp24_bruteforce(orc, seed):
    r = np.random.default_rng(300 + seed)
    m, n = int(r.integers(1, 97)), int(r.integers(1, 97))
    k = 8 * int(r.integers(1, 13))
    # small alphabets force ties; full range covers -128
    lo, hi = [(-2, 3), (-128, 128), (-127, 128)][seed % 3]
    a = r.integers(lo, hi, size=(m, k)).astype(np.int8)
    vals, meta = orc.pack24(a)
    pruned = orc.densify24(vals, meta)
    np.testing.assert_array_equal(pruned, _np_prune24(a))
    # the pruned matrix is 2:4 and idempotent under packing
    assert ((pruned.reshape(m, k // 4, 4) != 0).sum(axis=2) <= 2).all()
    v2, m2 = orc.pack24(pruned)
    np.testing.assert_array_equal(v2, vals)
    np.testing.assert_array_equal(m2, meta)
    # every stored pair is in ascending position order
    nib = np.stack([meta & 0xF, meta >> 4], axis=2).reshape(m, k // 4)
    assert ((nib & 3) < (nib >> 2)).all()
    B = r.integers(-128, 128, size=(k, n)).astype(np.int8)
    got = orc.sp24_spmm(vals, meta, B)
    ref = pruned.astype(np.int64) @ B.astype(np.int64)
    np.testing.assert_array_equal(got, ref)
    np.testing.assert_array_equal(orc.gemm_i8(pruned, B), ref)


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------


def test_identity_and_permutation_csr(orc):
    n, m = 37, 50
    r = np.random.default_rng(7)
    B = r.standard_normal((m, n)).astype(np.float32)
    rp = np.arange(m + 1, dtype=np.int64)
    ci = np.arange(m, dtype=np.int32)
    np.testing.assert_array_equal(orc.csr_spmm(rp, ci, np.ones(m, np.float32), B), B)
    perm = r.permutation(m).astype(np.int32)
    # row i of P holds a one at column perm[i] -> (P B)[i] = B[perm[i]]
    np.testing.assert_array_equal(orc.csr_spmm(rp, perm, np.ones(m, np.float32), B), B[perm])
    for e in (-3, 0, 5):
        got = orc.csr_spmm(rp, ci, np.full(m, 2.0 ** e, np.float32), B)
        np.testing.assert_array_equal(got, B.astype(np.float64) * 2.0 ** e)


def test_identity_and_permutation_bcsr(orc):
    bm = 4
    m = 6 * bm
    r = np.random.default_rng(8)
    B = synth.f32_to_bf16_bits(r.standard_normal((m, 29)).astype(np.float32))
    Bf = synth.bf16_bits_to_f32(B).astype(np.float64)
    eye = synth.f32_to_bf16_bits(np.eye(m, dtype=np.float32))
    rp, ci, v = orc.pack_bcsr(eye, bm, bm)
    assert len(ci) == m // bm                      # only diagonal blocks stored
    np.testing.assert_array_equal(orc.bcsr_spmm(bm, bm, rp, ci, v, B), Bf)
    perm = r.permutation(m)
    P = np.zeros((m, m), dtype=np.float32)
    P[np.arange(m), perm] = 1.0
    rp, ci, v = orc.pack_bcsr(synth.f32_to_bf16_bits(P), bm, bm)
    np.testing.assert_array_equal(orc.bcsr_spmm(bm, bm, rp, ci, v, B), Bf[perm])
    # single nonzero a at (i, k): row i = a * B[k], all other rows zero
    S = np.zeros((m, m), dtype=np.float32)
    S[5, 17] = -0.375
    rp, ci, v = orc.pack_bcsr(synth.f32_to_bf16_bits(S), bm, bm)
    got = orc.bcsr_spmm(bm, bm, rp, ci, v, B)
    exp = np.zeros_like(got)
    exp[5] = -0.375 * Bf[17]
    np.testing.assert_array_equal(got, exp)


def test_identity_and_linearity_sp24(orc):
    m = 64
    eye = np.eye(m, dtype=np.int8)
    vals, meta = orc.pack24(eye)
    np.testing.assert_array_equal(orc.densify24(vals, meta), eye)   # I is 2:4 already
    r = np.random.default_rng(9)
    B1 = r.integers(-64, 64, size=(m, 33)).astype(np.int8)
    B2 = r.integers(-63, 64, size=(m, 33)).astype(np.int8)
    np.testing.assert_array_equal(orc.sp24_spmm(vals, meta, B1), B1.astype(np.int32))
    a = r.integers(-127, 128, size=(40, m)).astype(np.int8)
    v, mt = orc.pack24(a)
    lhs = orc.sp24_spmm(v, mt, (B1.astype(np.int16) + B2).astype(np.int8))
    rhs = orc.sp24_spmm(v, mt, B1).astype(np.int64) + orc.sp24_spmm(v, mt, B2)
    np.testing.assert_array_equal(lhs, rhs)


def test_sp24_extreme_sum_is_exact(orc):
    # |C| = (k/2) * 128 * 128 with every kept value -128 and B = -128:
    # k = 8192 gives 4096 * 16384 = 2^26, well inside int32
    k = 8192
    a = np.full((2, k), -128, dtype=np.int8)
    v, mt = orc.pack24(a)
    B = np.full((k, 3), -128, dtype=np.int8)
    np.testing.assert_array_equal(orc.sp24_spmm(v, mt, B), np.full((2, 3), (k // 2) * 16384))


# ---------------------------------------------------------------------------
# invariants of the packers
# ---------------------------------------------------------------------------


def test_bcsr_zero_matrix(orc):
    a = np.zeros((128, 192), dtype=np.uint16)
    a[5, 7] = 0x8000    # -0.0 is zero
    rp, ci, v = orc.pack_bcsr(a, 64, 64)
    assert len(ci) == 0 and (rp == 0).all()
    B = synth.f32_to_bf16_bits(np.ones((192, 10), np.float32))
    assert (orc.bcsr_spmm(64, 64, rp, ci, v, B) == 0).all()


def test_bcsr_nan_block_kept(orc):
    a = np.zeros((64, 128), dtype=np.uint16)
    a[3, 70] = 0x7FC0   # NaN counts as nonzero
    rp, ci, v = orc.pack_bcsr(a, 64, 64)
    assert list(ci) == [1] and list(rp) == [0, 1]


def test_bcsr_rejects_ragged(orc):
    with pytest.raises(ValueError):
        orc.pack_bcsr(np.zeros((65, 64), dtype=np.uint16), 64, 64)


@pytest.mark.parametrize("seed", range(20))
def test_wcsr_chunk_invariants(orc, seed):
    r = np.random.default_rng(500 + seed)
    m = int(r.integers(1, 400))
    lens = r.integers(0, 3, size=m) * r.integers(0, 60, size=m)
    rp = np.zeros(m + 1, dtype=np.int64)
    np.cumsum(lens, out=rp[1:])
    W, T = int(r.integers(1, 40)), int(r.integers(1, 200))
    cw, cb = orc.wcsr_chunks(m, rp, W, T)
    nnz = int(rp[-1])
    assert cb[0] == 0 and cb[-1] == nnz and (np.diff(cb) >= 0).all()
    assert (np.diff(cw) >= 0).all() and cw[-1] == (m - 1) // W
    expected = 0
    for w in range((m + W - 1) // W):
        s, e = int(rp[w * W]), int(rp[min(m, (w + 1) * W)])
        mine = np.nonzero(cw == w)[0]
        assert len(mine) >= 1
        expected += max(1, -(-(e - s) // T))
        assert cb[mine[0]] == s and cb[mine[-1] + 1] == e           # covers the window
        assert (np.diff(cb[mine[0]:mine[-1] + 2]) <= T).all()        # at most T each
        if e - s <= T:
            assert len(mine) == 1
    assert len(cw) == expected


def test_csr_check_codes(orc):
    rp = np.array([0, 2, 2, 4], dtype=np.int64)
    ci = np.array([1, 3, 0, 2], dtype=np.int32)
    assert orc.csr_check(3, 4, rp, ci) == 0
    assert orc.csr_check(3, 4, np.array([1, 2, 2, 4]), ci) == 1
    assert orc.csr_check(3, 4, np.array([0, 3, 2, 4]), ci) == 2
    assert orc.csr_check(3, 4, np.array([0, 2, 2, 3]), ci) == 3
    assert orc.csr_check(3, 4, rp, np.array([1, 4, 0, 2])) == 4
    assert orc.csr_check(3, 4, rp, np.array([3, 1, 0, 2])) == 5
    assert orc.csr_check(3, 4, rp, np.array([1, 1, 0, 2])) == 5


def test_rel_frobenius(orc):
    assert orc.rel_frobenius([3.0, 4.0], [3.0, 4.0]) == 0.0
    assert orc.rel_frobenius([3.0, 4.0 + 5e-3], [3.0, 4.0]) == pytest.approx(1e-3)
    assert orc.rel_frobenius([0.0], [0.0]) == 0.0
    assert orc.rel_frobenius([1.0], [0.0]) == float("inf")


# ---------------------------------------------------------------------------
# sampled dense-dense product (SDDMM): brute force and closed forms
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("seed", range(20))
def test_sddmm_bruteforce(orc, seed):
    # oracle vs numpy's dense X @ Y^T read at the pattern's positions
    r = np.random.default_rng(700 + seed)
    m, k, kd = (int(x) for x in r.integers(1, 80, size=3))
    rp, ci, _ = synth.csr_uniform(m, k, float(r.uniform(0.0, 0.5)), 3000 + seed)
    X = r.standard_normal((m, kd)).astype(np.float32)
    Y = r.standard_normal((k, kd)).astype(np.float32)
    got = orc.sddmm(rp, ci, X, Y)
    rows = np.repeat(np.arange(m), np.diff(rp))
    ref = (X.astype(np.float64) @ Y.astype(np.float64).T)[rows, ci]
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    # a row subset gives those rows' entries, in stored order
    sub = np.sort(r.choice(m, size=max(1, m // 2), replace=False)).astype(np.int64)
    want = np.concatenate([got[rp[i]:rp[i + 1]] for i in sub])
    np.testing.assert_array_equal(orc.sddmm(rp, ci, X, Y, rows=sub), want)


def test_sddmm_closed_forms(orc):
    r = np.random.default_rng(11)
    m, kd = 40, 24
    X = r.standard_normal((m, kd)).astype(np.float32)
    # diagonal pattern with Y = X: squared row norms
    rp = np.arange(m + 1, dtype=np.int64)
    ci = np.arange(m, dtype=np.int32)
    np.testing.assert_allclose(orc.sddmm(rp, ci, X, X),
                               (X.astype(np.float64) ** 2).sum(axis=1), rtol=1e-13)
    # one-hot rows of X pick single columns of Y: exact
    Y = r.standard_normal((30, kd)).astype(np.float32)
    hot = r.integers(0, kd, size=m)
    Xh = np.zeros((m, kd), np.float32)
    Xh[np.arange(m), hot] = 1.0
    cols = r.integers(0, 30, size=m).astype(np.int32)
    np.testing.assert_array_equal(orc.sddmm(rp, cols, Xh, Y), Y[cols, hot].astype(np.float64))
    # an empty pattern gives nothing; empty rows are skipped
    assert len(orc.sddmm(np.zeros(m + 1, np.int64), np.zeros(0, np.int32), X, X)) == 0


def _block_pattern(r, mb, kb, bm, bk, density):
    """A BCSR pattern from the oracle's own pack of a bf16 matrix whose
    blocks are nonzero with the given probability."""
    keep = r.random((mb, kb)) < density
    a = np.zeros((mb * bm, kb * bk), np.uint16)
    for I, J in zip(*np.nonzero(keep)):
        a[I * bm + r.integers(bm), J * bk + r.integers(bk)] = 0x3F80   # 1.0
    return a


@pytest.mark.parametrize("seed", range(12))
def test_sddmm_bcsr_bruteforce(orc, seed):
    # oracle vs numpy's dense X @ Y^T cut into the stored blocks
    r = np.random.default_rng(800 + seed)
    bm, bk = (int(x) for x in r.choice([1, 2, 4, 8], size=2))
    mb, kb, kd = int(r.integers(1, 7)), int(r.integers(1, 7)), int(r.integers(1, 70))
    rp, ci, _ = orc.pack_bcsr(_block_pattern(r, mb, kb, bm, bk, 0.5), bm, bk)
    brow = np.repeat(np.arange(mb), np.diff(rp))
    # bf16 operands: exact widening, fp64 sums
    Xb = synth.f32_to_bf16_bits(r.standard_normal((mb * bm, kd)).astype(np.float32))
    Yb = synth.f32_to_bf16_bits(r.standard_normal((kb * bk, kd)).astype(np.float32))
    full = synth.bf16_bits_to_f32(Xb).astype(np.float64) @ synth.bf16_bits_to_f32(Yb).astype(np.float64).T
    ref = np.stack([full[I * bm:(I + 1) * bm, J * bk:(J + 1) * bk] for I, J in zip(brow, ci)]) \
        if len(ci) else np.zeros((0, bm, bk))
    got = orc.sddmm_bcsr(bm, bk, rp, ci, Xb, Yb)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    # int8 operands: exact
    Xi = r.integers(-128, 128, size=(mb * bm, kd)).astype(np.int8)
    Yi = r.integers(-128, 128, size=(kb * bk, kd)).astype(np.int8)
    fi = Xi.astype(np.int64) @ Yi.astype(np.int64).T
    refi = np.stack([fi[I * bm:(I + 1) * bm, J * bk:(J + 1) * bk] for I, J in zip(brow, ci)]) \
        if len(ci) else np.zeros((0, bm, bk))
    np.testing.assert_array_equal(orc.sddmm_bcsr(bm, bk, rp, ci, Xi, Yi), refi)
    # a block subset gives those blocks, in the order asked
    if len(ci):
        sub = r.permutation(len(ci))[: max(1, len(ci) // 2)].astype(np.int64)
        np.testing.assert_array_equal(orc.sddmm_bcsr(bm, bk, rp, ci, Xb, Yb, blocks=sub), got[sub])


def test_sddmm_bcsr_closed_forms(orc):
    r = np.random.default_rng(12)
    bm = bk = 64
    rp, ci, _ = orc.pack_bcsr(_block_pattern(r, 3, 4, bm, bk, 0.6), bm, bk)
    brow = np.repeat(np.arange(3), np.diff(rp))
    kd = 96
    # one-hot rows of X pick single elements of Y: exact
    hot = r.integers(0, kd, size=3 * bm)
    Xh = np.zeros((3 * bm, kd), np.uint16)
    Xh[np.arange(3 * bm), hot] = 0x3F80
    Yb = synth.dense_bf16_normal(4 * bk, kd, 90)
    Yf = synth.bf16_bits_to_f32(Yb).astype(np.float64)
    got = orc.sddmm_bcsr(bm, bk, rp, ci, Xh, Yb)
    for q, (I, J) in enumerate(zip(brow, ci)):
        rows = np.arange(I * bm, (I + 1) * bm)
        np.testing.assert_array_equal(got[q], Yf[J * bk:(J + 1) * bk][:, hot[rows]].T)
    # int8 extremes: all -128 gives kd * 16384 everywhere, exact
    Xi = np.full((3 * bm, kd), -128, np.int8)
    Yi = np.full((4 * bk, kd), -128, np.int8)
    assert (orc.sddmm_bcsr(bm, bk, rp, ci, Xi, Yi) == kd * 16384).all()
    # ... and an inner dimension past 2^31 / 16384 overflows int32: reported
    big = 131073
    rp1, ci1 = np.array([0, 1], np.int32), np.array([0], np.int32)
    with pytest.raises(OverflowError):
        orc.sddmm_bcsr(1, 1, rp1, ci1, np.full((1, big), -128, np.int8), np.full((1, big), -128, np.int8))
    # an empty pattern gives no blocks
    z = orc.sddmm_bcsr(bm, bk, np.zeros(4, np.int32), np.zeros(0, np.int32), Xh, Yb)
    assert z.shape == (0, bm, bk)


# ---- N:M pruning (the (2N-2):2N family) -------------------------------------

def test_prune_nm_is_the_24_rule_at_2_of_4(orc):
    for seed in range(10):
        a = synth.int8_uniform(np.random.default_rng(1100 + seed), (int(5 + seed), 64))
        a[0, :8] = [-128, 127, 127, -128, 0, 0, 0, 5]        # ties and -128
        v, m = orc.pack24(a)
        np.testing.assert_array_equal(orc.prune_nm(a, 2, 4), orc.densify24(v, m))


@pytest.mark.parametrize("keep,group", [(6, 8), (4, 6), (14, 16), (1, 2), (3, 3), (0, 4)])
def test_prune_nm_invariants(orc, keep, group):
    r = np.random.default_rng(keep * 100 + group)
    a = r.integers(-128, 128, size=(40, group * 12)).astype(np.int8)
    a[::3] = r.integers(-3, 4, size=a[::3].shape)            # many ties
    out = orc.prune_nm(a, keep, group)
    ga = a.reshape(40, -1, group).astype(np.int64)
    go = out.reshape(40, -1, group).astype(np.int64)
    kept = (go == ga) & ((go != 0) | (ga == 0))
    for i in range(40):
        for g in range(ga.shape[1]):
            vals = np.abs(ga[i, g])
            # the kept set: `keep` positions, by (larger |a|, lower position)
            order = sorted(range(group), key=lambda t: (-vals[t], t))[:keep]
            mask = np.zeros(group, bool)
            mask[order] = True
            np.testing.assert_array_equal(go[i, g][mask], ga[i, g][mask])
            assert (go[i, g][~mask] == 0).all()
            if keep and (~mask).any():
                assert vals[mask].min() >= vals[~mask].max()
    assert kept.shape == ga.shape


def test_prune_nm_hand_cases(orc):
    a = np.array([[3, -3, 3, -3, 1, 0, -128, 127]], np.int8)
    np.testing.assert_array_equal(orc.prune_nm(a, 6, 8), [[3, -3, 3, -3, 0, 0, -128, 127]])
    a = np.array([[0, 0, 0, 0, 0, 0, 0, 1]], np.int8)
    np.testing.assert_array_equal(orc.prune_nm(a, 6, 8), a)    # zeros kept as zeros
    a = np.array([[5, 5, 5, 5, 5, 5, 5, 5]], np.int8)           # all tie: lowest six survive
    np.testing.assert_array_equal(orc.prune_nm(a, 6, 8), [[5, 5, 5, 5, 5, 5, 0, 0]])
    with pytest.raises(ValueError):
        orc.prune_nm(np.zeros((1, 12), np.int8), 6, 8)


# ---- N:M pruning of bf16 (the 2:4 pattern of tile-vector-wise bf16) ------------

def _bf(x):
    return synth.f32_to_bf16_bits(np.asarray(x, np.float32))


def test_prune_nm_bf16_reduces_to_the_int8_rule(orc):
    # int8 values are exact in bf16 and keep their magnitude order
    for seed in range(6):
        a = synth.int8_uniform(np.random.default_rng(1200 + seed), (7, 64))
        a[0, :8] = [-128, 127, 127, -128, 0, 0, 0, 5]
        a[1, :8] = [1, -1, 1, -1, 0, 0, 0, 0]
        for keep, group in ((2, 4), (6, 8), (3, 16), (0, 4)):
            got = orc.prune_nm(_bf(a.astype(np.float32)), keep, group)
            exp = _bf(orc.prune_nm(a, keep, group).astype(np.float32))
            np.testing.assert_array_equal(got, exp)


def test_prune_nm_bf16_hand_cases(orc):
    inf, nan = np.inf, np.nan
    rows = [
        ([1.5, -2.0, 0.25, -0.0], [1.5, -2.0, 0.0, 0.0]),
        ([-1.0, 1.0078125, 0.5, 1.0], [-1.0, 1.0078125, 0.0, 0.0]),    # 1 and -1 tie
        ([3.0, -3.0, 3.0, -3.0], [3.0, -3.0, 0.0, 0.0]),
        ([inf, nan, 1.0, -inf], [inf, nan, 0.0, 0.0]),                 # NaN first, then inf
        ([0.5, -inf, 65504.0, 1e30], [0.0, -inf, 0.0, 1e30]),
    ]
    a = _bf([r[0] for r in rows])
    exp = _bf([r[1] for r in rows])
    got = orc.prune_nm(a, 2, 4)
    np.testing.assert_array_equal(got, exp)
    # signed zeros tie (kept as they are), subnormals beat zero, NaNs tie
    bits = np.array([[0x8000, 0x0000, 0x0000, 0x8000],
                     [0x0001, 0x8002, 0x0000, 0x0001],
                     [0x7FC0, 0x7FFF, 0xFFC1, 0x3F80],
                     [0x0000, 0x0000, 0x0000, 0x0001]], np.uint16)
    exp = np.array([[0x8000, 0x0000, 0, 0],
                    [0x0001, 0x8002, 0, 0],
                    [0x7FC0, 0x7FFF, 0, 0],
                    [0x0000, 0, 0, 0x0001]], np.uint16)
    np.testing.assert_array_equal(orc.prune_nm(bits, 2, 4), exp)
    with pytest.raises(ValueError):
        orc.prune_nm(np.zeros((1, 6), np.uint16), 2, 4)


@pytest.mark.parametrize("keep,group", [(2, 4), (6, 8), (1, 3)])
def test_prune_nm_bf16_brute_force(orc, keep, group):
    # against a sort of each group by (NaN first, larger |a|, lower position)
    r = np.random.default_rng(1300 + keep + group)
    pool = np.array([0.0, -0.0, 1.0, -1.0, 2.5, -2.5, np.inf, -np.inf, np.nan, 1e-39, 7.0],
                    np.float32)
    a = _bf(r.choice(pool, size=(30, group * 6)))
    a[:, ::5] = r.integers(0, 1 << 16, size=a[:, ::5].shape, dtype=np.uint16)  # any pattern
    got = orc.prune_nm(a, keep, group)
    with np.errstate(invalid="ignore"):
        x = synth.bf16_bits_to_f32(a).astype(np.float64)
    for i in range(a.shape[0]):
        for g in range(a.shape[1] // group):
            seg = x[i, g * group:(g + 1) * group]
            order = sorted(range(group), key=lambda t: (0 if np.isnan(seg[t]) else 1,
                                                        -abs(seg[t]) if not np.isnan(seg[t]) else 0.0,
                                                        t))
            mask = np.zeros(group, bool)
            mask[order[:keep]] = True
            o = got[i, g * group:(g + 1) * group]
            src = a[i, g * group:(g + 1) * group]
            np.testing.assert_array_equal(o[mask], src[mask])
            assert (o[~mask] == 0).all()

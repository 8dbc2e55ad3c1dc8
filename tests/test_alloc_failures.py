"""Out-of-memory handling of the C ABI, on the host (no GPU needed).

With SPMM_TEST_FAIL_ALLOC = n the n-th allocation an ABI call makes fails as
it would when memory runs out.  Walking n = 1, 2, ... through every
allocation of each packer, every failing call must return
SPMM_ERR_OUT_OF_MEMORY with *out set to NULL and a message, and the first n
that reaches the end must produce exactly the arrays of an unhooked call.
Leaks on these paths are checked by the sanitizer run (tests/test_sanitizers.py).

Packers: BCSR and WCSR (AsyncSparse page, abstract and Figure 2 caption),
2:4 (tiled-GEMM page, abstract), tile-vector-wise (same), (2N-2):2N (search
page), reordered BCSR (search page)."""
import ctypes
import os

import numpy as np
import pytest

import synth

OOM = 3


@pytest.fixture(scope="module")
def S():
    import sparse_dense_matrix_amd as S
    return S


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def walk(S, call, limit=400):
    """Run call(out_ref) with the n-th allocation failing for n = 1, 2, ...
    until it succeeds; returns (failures seen, handle of the successful
    call)."""
    n = 0
    try:
        while True:
            n += 1
            assert n < limit, "no successful call"
            os.environ["SPMM_TEST_FAIL_ALLOC"] = str(n)
            out = ctypes.c_void_p(0xDEAD)
            st = call(ctypes.byref(out))
            if st == 0:
                assert out.value
                return n - 1, out
            assert st == OOM, (n, S.spmm_status_str(st), S.spmm_last_error())
            assert out.value is None, f"allocation {n}: *out not NULL on failure"
            assert S.spmm_last_error(), "no message"
    finally:
        os.environ.pop("SPMM_TEST_FAIL_ALLOC", None)


def same_arrays(S, h, ref, which):
    m = S.Matrix(h)
    for w in which:
        np.testing.assert_array_equal(S.spmm_matrix_array(m, w), S.spmm_matrix_array(ref, w))
    return m


def test_hook_off_by_default(S):
    a = synth.SMALL["bcsr_small"]
    M = S.spmm_pack_bcsr(synth.make_a(a)["dense"])
    assert M.info()["nnzb"] > 0


def test_pack_bcsr_oom_paths(S):
    a = np.ascontiguousarray(synth.make_a(synth.SMALL["bcsr_small"])["dense"])
    ref = S.spmm_pack_bcsr(a)
    fails, h = walk(S, lambda o: S._lib.spmm_pack_bcsr(a.shape[0], a.shape[1], 64, 64, S.BF16, _p(a),
                                                         a.shape[1], o))
    assert fails >= 3
    same_arrays(S, h, ref, (S.ARRAY_ROW_PTR, S.ARRAY_COL_IDX, S.ARRAY_VALS))


def test_pack_wcsr_oom_paths(S):
    w = synth.SMALL["csr_powerlaw_small"]
    a = synth.make_a(w)
    rp, ci, v = (np.ascontiguousarray(a["row_ptr"], np.int64), np.ascontiguousarray(a["col_idx"], np.int32),
                 np.ascontiguousarray(a["vals"], np.float32))
    ref = S.spmm_pack_wcsr(w.m, w.k, rp, ci, v, 16, 64)
    fails, h = walk(S, lambda o: S._lib.spmm_pack_wcsr(w.m, w.k, S.F32, _p(rp), _p(ci), _p(v), 16, 64, o))
    assert fails >= 4
    same_arrays(S, h, ref, (S.ARRAY_ROW_PTR, S.ARRAY_COL_IDX, S.ARRAY_VALS, S.ARRAY_CHUNK_WINDOW,
                            S.ARRAY_CHUNK_BEGIN))


@pytest.mark.parametrize("elem", ["i8", "bf16"])
def test_pack_24_and_tvw_oom_paths(S, elem):
    r = np.random.default_rng(71)
    if elem == "i8":
        a, dt = synth.int8_uniform(r, (256, 512)), S.I8
    else:
        a, dt = synth.f32_to_bf16_bits(synth.normal_f32(r, (256, 512), 0.02)), S.BF16
    a[:, 128:256] = 0      # one zero tile for the tile-vector-wise pattern
    a = np.ascontiguousarray(a)
    ref = S.spmm_pack_24(a)
    fails, h = walk(S, lambda o: S._lib.spmm_pack_24(256, 512, dt, _p(a), 512, o))
    assert fails >= 2
    same_arrays(S, h, ref, (S.ARRAY_VALS, S.ARRAY_META))
    ref = S.spmm_pack_tvw(a, 256, 128)
    fails, h = walk(S, lambda o: S._lib.spmm_pack_tvw(256, 512, dt, _p(a), 512, 256, 128, o))
    assert fails >= 3
    same_arrays(S, h, ref, (S.ARRAY_ROW_PTR, S.ARRAY_COL_IDX, S.ARRAY_VALS, S.ARRAY_META))


def test_pack_slide_oom_paths(S):
    a = np.ascontiguousarray(synth.int8_uniform(np.random.default_rng(72), (64, 256)))
    ref = S.spmm_pack_slide(a, 8)
    fails, h = walk(S, lambda o: S._lib.spmm_pack_slide(64, 256, _p(a), 256, 8, o))
    assert fails >= 3
    same_arrays(S, h, ref, (S.ARRAY_VALS, S.ARRAY_META))


@pytest.mark.parametrize("reorder", [0, 1])
def test_pack_bcsr_csr_oom_paths(S, reorder):
    m, k = 256, 512
    r = np.random.default_rng(73)
    dense = np.zeros((m, k), np.float32)
    for b in r.choice((m // 64) * (k // 64), 6, replace=False):
        i, j = divmod(int(b), k // 64)
        dense[i * 64:(i + 1) * 64, j * 64:(j + 1) * 64] = r.uniform(-1, 1, (64, 64))
    dense = dense[r.permutation(m)][:, r.permutation(k)]
    rows, cols = np.nonzero(dense)
    rp = np.zeros(m + 1, np.int64)
    np.add.at(rp, rows + 1, 1)
    rp = np.cumsum(rp)
    ci = np.ascontiguousarray(cols, np.int32)
    v = np.ascontiguousarray(synth.f32_to_bf16_bits(dense[rows, cols]))
    ref = S.spmm_pack_bcsr_csr(m, k, rp, ci, v, reorder=bool(reorder))
    fails, h = walk(S, lambda o: S._lib.spmm_pack_bcsr_csr(m, k, S.BF16, _p(rp), _p(ci), _p(v), 64, 64,
                                                             reorder, o))
    assert fails >= (8 if reorder else 3)
    same_arrays(S, h, ref, (S.ARRAY_ROW_PTR, S.ARRAY_COL_IDX, S.ARRAY_VALS, S.ARRAY_ROW_PERM,
                            S.ARRAY_COL_PERM))


def test_hook_does_not_outlive_its_call(S):
    # the count is read at the start of each allocating call: a matrix
    # packed after the variable is removed is unaffected
    a = np.ascontiguousarray(synth.int8_uniform(np.random.default_rng(74), (16, 64)))
    os.environ["SPMM_TEST_FAIL_ALLOC"] = "1"
    try:
        with pytest.raises(S.SpmmError) as ei:
            S.spmm_pack_24(a)
        assert ei.value.name == "SPMM_ERR_OUT_OF_MEMORY"
    finally:
        os.environ.pop("SPMM_TEST_FAIL_ALLOC", None)
    assert S.spmm_pack_24(a).info()["nnz"] == 16 * 32

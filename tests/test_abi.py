"""Host-side checks of the C-ABI library (no GPU needed): every symbol the
header declares is exported, the library's packers reproduce the oracle's
canonical arrays bit for bit, and bad input is rejected with the documented
status and a message.

Packing rules: AsyncSparse abstract and Figure 2 caption (BCSR, WCSR row
windows split into chunks); tiled-GEMM abstract and the N:M search-results
entry (2:4)."""
import ctypes
import os
import re

import numpy as np
import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def S():
    import sparse_dense_matrix_amd as S
    return S


def header_functions():
    text = open(os.path.join(ROOT, "include", "spmm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spmm_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(S):
    declared = header_functions()
    assert len(declared) >= 12
    assert sorted(S.EXPORTS) == declared
    lib = ctypes.CDLL(S.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings(S):
    assert S.spmm_status_str(0) == "SPMM_OK"
    assert S.spmm_status_str(1) == "SPMM_ERR_INVALID_ARG"
    assert S.spmm_status_str(4) == "SPMM_ERR_HIP"


# ---------------------------------------------------------------------------
# packers vs oracle (bit-exact)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["bcsr_small"])
def test_pack_bcsr_matches_oracle(S, orc, name):
    w = synth.SMALL[name]
    a = synth.make_a(w)["dense"]
    M = S.spmm_pack_bcsr(a, 64, 64)
    rp, ci, v = orc.pack_bcsr(a, 64, 64)
    np.testing.assert_array_equal(S.spmm_matrix_array(M, S.ARRAY_ROW_PTR), rp)
    np.testing.assert_array_equal(S.spmm_matrix_array(M, S.ARRAY_COL_IDX), ci)
    np.testing.assert_array_equal(S.spmm_matrix_array(M, S.ARRAY_VALS), v.ravel())
    info = S.spmm_matrix_info(M)
    assert info["nnzb"] == len(ci) == w.nblocks and info["nnz"] == len(ci) * 4096


@pytest.mark.parametrize("seed", range(12))
def test_pack_bcsr_random_blocks(S, orc, seed):
    r = np.random.default_rng(seed)
    bm, bk = (int(x) for x in r.choice([2, 4, 8, 16, 64], size=2))
    m, k = bm * int(r.integers(1, 6)), bk * int(r.integers(1, 6))
    a = np.zeros((m, k), dtype=np.uint16)
    mask = r.random((m, k)) < 0.05
    a[mask] = r.integers(1, 0xFFFF, size=int(mask.sum()), dtype=np.uint16)
    a[r.random((m, k)) < 0.02] = 0x8000          # -0.0 stays zero
    M = S.spmm_pack_bcsr(a, bm, bk)
    rp, ci, v = orc.pack_bcsr(a, bm, bk)
    np.testing.assert_array_equal(S.spmm_matrix_array(M, S.ARRAY_ROW_PTR), rp)
    np.testing.assert_array_equal(S.spmm_matrix_array(M, S.ARRAY_COL_IDX), ci)
    np.testing.assert_array_equal(S.spmm_matrix_array(M, S.ARRAY_VALS), v.ravel())


@pytest.mark.parametrize("W,T", [(1, 1), (16, 512), (16, 4096), (3, 7), (64, 100)])
@pytest.mark.parametrize("name", ["csr_uniform_small", "csr_powerlaw_small"])
def test_pack_wcsr_matches_oracle(S, orc, name, W, T):
    w = synth.SMALL[name]
    a = synth.make_a(w)
    M = S.spmm_pack_wcsr(w.m, w.k, a["row_ptr"], a["col_idx"], a["vals"], W, T)
    cw, cb = orc.wcsr_chunks(w.m, a["row_ptr"], W, T)
    np.testing.assert_array_equal(S.spmm_matrix_array(M, S.ARRAY_CHUNK_WINDOW), cw)
    np.testing.assert_array_equal(S.spmm_matrix_array(M, S.ARRAY_CHUNK_BEGIN), cb)
    np.testing.assert_array_equal(S.spmm_matrix_array(M, S.ARRAY_ROW_PTR), a["row_ptr"])
    np.testing.assert_array_equal(S.spmm_matrix_array(M, S.ARRAY_COL_IDX), a["col_idx"])
    np.testing.assert_array_equal(S.spmm_matrix_array(M, S.ARRAY_VALS), a["vals"])
    info = S.spmm_matrix_info(M)
    assert info["num_chunks"] == len(cw) and info["num_windows"] == -(-w.m // W)


@pytest.mark.parametrize("m,W_expected", [(256, 1), (20000, 1), (65536, 4), (1_000_000, 16)])
def test_pack_wcsr_default_window(S, orc, m, W_expected):
    # window_rows = 0 / max_chunk_nnz = 0 pick min(16, max(1, m / 16384)) and
    # 512; the chunk tables are then the oracle's for those values
    rp = (np.arange(m + 1, dtype=np.int64) * 3)
    ci = np.tile(np.array([0, 5, 9], dtype=np.int32), m)
    v = np.ones(3 * m, dtype=np.float32)
    M = S.spmm_pack_wcsr(m, 10, rp, ci, v, 0, 0)
    info = S.spmm_matrix_info(M)
    assert info["window_rows"] == W_expected and info["max_chunk_nnz"] == 512
    cw, cb = orc.wcsr_chunks(m, rp, W_expected, 512)
    np.testing.assert_array_equal(S.spmm_matrix_array(M, S.ARRAY_CHUNK_WINDOW), cw)
    np.testing.assert_array_equal(S.spmm_matrix_array(M, S.ARRAY_CHUNK_BEGIN), cb)


@pytest.mark.parametrize("seed", range(12))
def test_pack_24_matches_oracle(S, orc, seed):
    r = np.random.default_rng(40 + seed)
    m, k = int(r.integers(1, 70)), 8 * int(r.integers(1, 20))
    lo, hi = [(-2, 3), (-128, 128), (-127, 128), (0, 1)][seed % 4]
    a = r.integers(lo, hi, size=(m, k)).astype(np.int8)
    M = S.spmm_pack_24(a)
    v, mt = orc.pack24(a)
    np.testing.assert_array_equal(S.spmm_matrix_array(M, S.ARRAY_VALS), v.ravel())
    np.testing.assert_array_equal(S.spmm_matrix_array(M, S.ARRAY_META), mt.ravel())


@pytest.mark.parametrize("seed", range(4))
def test_pack_24_bf16_is_the_oracle_prune(S, orc, seed):
    # densify the library's arrays and compare with the oracle's bf16 pruning
    r = np.random.default_rng(60 + seed)
    m, k = int(r.integers(1, 40)), 8 * int(r.integers(1, 12))
    a = synth.f32_to_bf16_bits(r.normal(size=(m, k)).astype(np.float32))
    a[r.random((m, k)) < 0.2] = 0
    specials = np.array([0x7FC0, 0x7F80, 0xFF80, 0x8000, 0x0001, 0x3F80, 0xBF80], np.uint16)
    idx = r.integers(0, [m, k], size=(min(m * k, 12), 2))
    a[idx[:, 0], idx[:, 1]] = r.choice(specials, size=len(idx))
    M = S.spmm_pack_24(a)
    v = S.spmm_matrix_array(M, S.ARRAY_VALS).reshape(m, k // 2)
    mt = S.spmm_matrix_array(M, S.ARRAY_META).reshape(m, k // 8)
    assert v.dtype == np.uint16 and S.spmm_matrix_info(M)["dtype"] == S.BF16
    dense = np.zeros((m, k), np.uint16)
    rows = np.arange(m)
    for g in range(k // 4):
        nib = (mt[:, g // 2] >> (4 * (g % 2))) & 0xF
        i0, i1 = nib & 3, nib >> 2
        assert (i0 < i1).all()
        dense[rows, 4 * g + i0] = v[:, 2 * g]
        dense[rows, 4 * g + i1] = v[:, 2 * g + 1]
    np.testing.assert_array_equal(dense, orc.prune_nm(a, 2, 4))


def test_pack_24_full_config(S, orc):
    w = synth.WORKLOADS["sp24_i8_8192"]
    a = synth.make_a(w)["dense"]
    M = S.spmm_pack_24(a)
    v, mt = orc.pack24(a)
    np.testing.assert_array_equal(S.spmm_matrix_array(M, S.ARRAY_VALS), v.ravel())
    np.testing.assert_array_equal(S.spmm_matrix_array(M, S.ARRAY_META), mt.ravel())


def test_pack_bcsr_full_configs(S, orc):
    # the 4096 case and the 18944 x 3584 prefill layer, bit for bit
    for name in ("bcsr_4096_b64_90", "bcsr_prefill_18944x3584"):
        w = synth.WORKLOADS[name]
        a = synth.make_a(w)["dense"]
        M = S.spmm_pack_bcsr(a, 64, 64)
        rp, ci, v = orc.pack_bcsr(a, 64, 64)
        assert len(ci) == w.nblocks
        np.testing.assert_array_equal(S.spmm_matrix_array(M, S.ARRAY_ROW_PTR), rp)
        np.testing.assert_array_equal(S.spmm_matrix_array(M, S.ARRAY_COL_IDX), ci)
        np.testing.assert_array_equal(S.spmm_matrix_array(M, S.ARRAY_VALS), v.ravel())


def test_pack_wcsr_full_config(S, orc):
    # the 10^6-row power-law CSR at the bench's window shape (W = 16 rows, at
    # most T = 512 entries per chunk): the CSR copy and both chunk tables, bit
    # for bit
    w = synth.WORKLOADS["csr_powerlaw_1m"]
    a = synth.make_a(w)
    M = S.spmm_pack_wcsr(w.m, w.k, a["row_ptr"], a["col_idx"], a["vals"], 16, 512)
    info = S.spmm_matrix_info(M)
    assert (info["window_rows"], info["max_chunk_nnz"]) == (16, 512)
    cw, cb = orc.wcsr_chunks(w.m, a["row_ptr"], 16, 512)
    assert info["num_chunks"] == len(cw) and len(cw) > w.m // 16
    np.testing.assert_array_equal(S.spmm_matrix_array(M, S.ARRAY_CHUNK_WINDOW), cw)
    np.testing.assert_array_equal(S.spmm_matrix_array(M, S.ARRAY_CHUNK_BEGIN), cb)
    np.testing.assert_array_equal(S.spmm_matrix_array(M, S.ARRAY_ROW_PTR), a["row_ptr"])
    np.testing.assert_array_equal(S.spmm_matrix_array(M, S.ARRAY_COL_IDX), a["col_idx"])
    np.testing.assert_array_equal(S.spmm_matrix_array(M, S.ARRAY_VALS).view(np.uint32),
                                  np.asarray(a["vals"], np.float32).view(np.uint32))
    # the packer's default shape is the same for this matrix
    D = S.spmm_pack_wcsr(w.m, w.k, a["row_ptr"], a["col_idx"], a["vals"])
    assert S.spmm_matrix_info(D)["num_chunks"] == len(cw)


# ---------------------------------------------------------------------------
# error paths
# ---------------------------------------------------------------------------

def _status(S, fn, *args):
    with pytest.raises(S.SpmmError) as ei:
        fn(*args)
    assert ei.value.message, "failing call left no message"
    return ei.value.name


def test_wcsr_rejects_non_canonical(S):
    rp = np.array([0, 2, 2, 4], dtype=np.int64)
    ci = np.array([1, 3, 0, 2], dtype=np.int32)
    v = np.ones(4, np.float32)
    assert S.spmm_pack_wcsr(3, 4, rp, ci, v, 2, 2) is not None
    bad = [
        (np.array([1, 2, 2, 4]), ci),     # row_ptr[0] != 0
        (np.array([0, 3, 2, 4]), ci),     # decreasing
        (rp, np.array([1, 4, 0, 2])),     # column out of range
        (rp, np.array([1, -1, 0, 2])),    # negative column
        (rp, np.array([3, 1, 0, 2])),     # unsorted
        (rp, np.array([1, 1, 0, 2])),     # duplicate
    ]
    for r_, c_ in bad:
        assert _status(S, S.spmm_pack_wcsr, 3, 4, r_, c_, v, 2, 2) == "SPMM_ERR_INVALID_ARG"
    assert _status(S, S.spmm_pack_wcsr, 3, 4, rp, ci, v, -1, 2) == "SPMM_ERR_INVALID_ARG"
    assert _status(S, S.spmm_pack_wcsr, 3, 4, rp, ci, v, 2, -1) == "SPMM_ERR_INVALID_ARG"
    assert _status(S, S.spmm_pack_wcsr, 3, 4, rp, ci, v, 2, 2, S.BF16) == "SPMM_ERR_UNSUPPORTED"


def test_bcsr_and_24_shape_errors(S):
    assert _status(S, S.spmm_pack_bcsr, np.zeros((65, 64), np.uint16)) == "SPMM_ERR_INVALID_ARG"
    assert _status(S, S.spmm_pack_bcsr, np.zeros((64, 64), np.uint16), 64, 64,
                   S.F32) == "SPMM_ERR_UNSUPPORTED"
    assert _status(S, S.spmm_pack_24, np.zeros((4, 12), np.int8)) == "SPMM_ERR_INVALID_ARG"
    import ctypes
    h, buf = ctypes.c_void_p(), np.zeros(32, np.float32)
    assert S.lib().spmm_pack_24(4, 8, S.F32, buf.ctypes.data, 8, ctypes.byref(h)) == 2  # UNSUPPORTED
    assert not h.value


def test_null_out_and_handles(S):
    lib = S.lib()
    assert lib.spmm_pack_24(4, 8, S.I8, None, 8, None) == 1
    assert lib.spmm_matrix_info(None, None) == 1
    assert lib.spmm_execute(None, None, 0, None, 0, None) == 1
    lib.spmm_matrix_destroy(None)
    lib.spmm_plan_destroy(None)


def test_empty_matrices_pack(S, orc):
    M = S.spmm_pack_wcsr(5, 7, np.zeros(6, np.int64), np.zeros(0, np.int32),
                         np.zeros(0, np.float32), 2, 4)
    info = S.spmm_matrix_info(M)
    assert info["nnz"] == 0 and info["num_chunks"] == 3
    np.testing.assert_array_equal(S.spmm_matrix_array(M, S.ARRAY_CHUNK_BEGIN), [0, 0, 0, 0])
    M = S.spmm_pack_bcsr(np.zeros((128, 64), np.uint16))
    assert S.spmm_matrix_info(M)["nnzb"] == 0
    np.testing.assert_array_equal(S.spmm_matrix_array(M, S.ARRAY_ROW_PTR), [0, 0, 0])

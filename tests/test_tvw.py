"""Tile-vector-wise packing (spmm_pack_tvw): host logic, no GPU.

The pattern is the tile-wise sparsity of "Accelerating Sparse DNNs Based on
Tiled GEMM" (abstract) combined with 2:4: tiles holding a nonzero are stored,
pruned 2:4 along k.  Pinned against the oracle's own 2:4 packer: every stored
tile must be bit-for-bit the oracle's 2:4 arrays of that region, and the
stored tiles must be exactly the nonzero ones."""
import numpy as np
import pytest

import synth


@pytest.fixture(scope="module")
def S():
    import sparse_dense_matrix_amd as S
    return S


def _check_tvw(S, orc, a, tm, tk):
    M = S.spmm_pack_tvw(a, tm, tk)
    rp = S.spmm_matrix_array(M, S.ARRAY_ROW_PTR)
    ci = S.spmm_matrix_array(M, S.ARRAY_COL_IDX)
    tv = S.spmm_matrix_array(M, S.ARRAY_VALS).reshape(-1, tm, tk // 2)
    tmeta = S.spmm_matrix_array(M, S.ARRAY_META).reshape(-1, tm, tk // 8)
    m, k = a.shape
    v24, m24 = orc.pack24(a)
    nonzero = (a.reshape(m // tm, tm, k // tk, tk) != 0).any(axis=(1, 3))
    q = 0
    for T in range(m // tm):
        kept = np.nonzero(nonzero[T])[0]
        np.testing.assert_array_equal(ci[rp[T]:rp[T + 1]], kept)
        for s in kept:
            np.testing.assert_array_equal(tv[q], v24[T * tm:(T + 1) * tm, s * tk // 2:(s + 1) * tk // 2])
            np.testing.assert_array_equal(tmeta[q], m24[T * tm:(T + 1) * tm, s * tk // 8:(s + 1) * tk // 8])
            q += 1
    assert q == len(ci) == S.spmm_matrix_info(M)["nnzb"]
    return M


@pytest.mark.parametrize("seed", range(5))
def test_tvw_tiles_are_the_24_pack_of_nonzero_tiles(S, orc, seed):
    r = np.random.default_rng(1000 + seed)
    tm, tk = [(256, 128), (64, 64), (32, 16), (16, 8), (256, 128)][seed]
    m, k = tm * int(r.integers(1, 4)), tk * int(r.integers(1, 5))
    a = synth.tile_sparse_i8(m, k, tm, tk, int(r.integers(0, (m // tm) * (k // tk) + 1)), 70 + seed)
    # a few stray entries, some equal to -128, and a tile holding only one
    extra = r.integers(0, [m, k], size=(int(r.integers(0, 6)), 2))
    a[extra[:, 0], extra[:, 1]] = r.choice([-128, 1, -1, 127], size=len(extra))
    _check_tvw(S, orc, a, tm, tk)


def test_tvw_all_tiles_and_no_tiles(S, orc):
    a = synth.int8_uniform(synth.rng(5, 1), (256, 256))
    M = _check_tvw(S, orc, a, 256, 128)          # every tile stored: the plain 2:4 pack
    assert S.spmm_matrix_info(M)["nnzb"] == 2
    Z = S.spmm_pack_tvw(np.zeros((256, 256), np.int8), 256, 128)
    assert S.spmm_matrix_info(Z)["nnzb"] == 0
    assert len(S.spmm_matrix_array(Z, S.ARRAY_VALS)) == 0


def test_tvw_arguments(S):
    for shape, tm, tk in (((256, 100), 256, 128), ((200, 128), 256, 128), ((256, 132), 256, 12)):
        with pytest.raises(S.SpmmError) as e:
            S.spmm_pack_tvw(np.zeros(shape, np.int8), tm, tk)
        assert e.value.name == "SPMM_ERR_INVALID_ARG"


# ---- bf16 -------------------------------------------------------------------------

def _densify_tiles(tv, tmeta, tk):
    """Expand stored tiles ([nt, tm, tk/2] kept values, [nt, tm, tk/8] nibble
    bytes) to dense [nt, tm, tk], checking that positions ascend."""
    nt, tm = tv.shape[:2]
    out = np.zeros((nt, tm, tk), tv.dtype)
    t_i, r_i = np.indices((nt, tm))
    for g in range(tk // 4):
        nib = (tmeta[:, :, g // 2] >> (4 * (g % 2))) & 0xF
        i0, i1 = nib & 3, nib >> 2
        assert (i0 < i1).all()
        out[t_i, r_i, 4 * g + i0] = tv[:, :, 2 * g]
        out[t_i, r_i, 4 * g + i1] = tv[:, :, 2 * g + 1]
    return out


def _check_tvw_bf16(S, orc, a, tm, tk):
    M = S.spmm_pack_tvw(a, tm, tk)
    info = S.spmm_matrix_info(M)
    assert info["dtype"] == S.BF16
    rp = S.spmm_matrix_array(M, S.ARRAY_ROW_PTR)
    ci = S.spmm_matrix_array(M, S.ARRAY_COL_IDX)
    tv = S.spmm_matrix_array(M, S.ARRAY_VALS)
    assert tv.dtype == np.uint16
    tv = tv.reshape(-1, tm, tk // 2)
    tmeta = S.spmm_matrix_array(M, S.ARRAY_META).reshape(-1, tm, tk // 8)
    m, k = a.shape
    dense = _densify_tiles(tv, tmeta, tk)
    pruned = orc.prune_nm(a, 2, 4)
    nonzero = ((a & 0x7FFF) != 0).reshape(m // tm, tm, k // tk, tk).any(axis=(1, 3))
    q = 0
    for T in range(m // tm):
        kept = np.nonzero(nonzero[T])[0]
        np.testing.assert_array_equal(ci[rp[T]:rp[T + 1]], kept)
        for s in kept:
            np.testing.assert_array_equal(dense[q], pruned[T * tm:(T + 1) * tm, s * tk:(s + 1) * tk])
            q += 1
    assert q == len(ci) == info["nnzb"]
    return M


@pytest.mark.parametrize("seed", range(4))
def test_tvw_bf16_tiles_are_the_pruned_nonzero_tiles(S, orc, seed):
    r = np.random.default_rng(1400 + seed)
    tm, tk = [(256, 128), (256, 64), (32, 16), (16, 8)][seed]
    m, k = tm * int(r.integers(1, 4)), tk * int(r.integers(1, 5))
    nt = int(r.integers(0, (m // tm) * (k // tk) + 1))
    a, _ = synth.block_sparse_dense_bf16(m, k, tm, tk, nt, 1.0, 80 + seed)
    # specials: NaN, infinities, signed zeros, subnormals, equal magnitudes;
    # a tile holding only -0 stays unstored
    extra = r.integers(0, [m, k], size=(int(r.integers(0, 12)), 2))
    a[extra[:, 0], extra[:, 1]] = r.choice(
        np.array([0x7FC0, 0x7F80, 0xFF80, 0x8000, 0x0001, 0x8001, 0x3F80, 0xBF80], np.uint16),
        size=len(extra))
    _check_tvw_bf16(S, orc, a, tm, tk)


def test_tvw_bf16_negative_zero_tile_is_not_stored(S, orc):
    a = np.zeros((256, 256), np.uint16)
    a[:, :128] = 0x8000                               # -0 everywhere: numerically zero
    a[5, 200] = 0x3F80
    M = _check_tvw_bf16(S, orc, a, 256, 128)
    np.testing.assert_array_equal(S.spmm_matrix_array(M, S.ARRAY_COL_IDX), [1])


def test_tvw_dtype_argument(S):
    with pytest.raises(TypeError):
        S.spmm_pack_tvw(np.zeros((256, 128), np.float32), 256, 128)

"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle
on the same seeded inputs.

Bars: int8 2:4 bit-exact; fp32 WCSR relative Frobenius error <= 1e-5; bf16
BCSR (fp32 accumulate, bf16 round-to-nearest-even output) <= 2e-3.  Every
element of C must be written (C is pre-filled with a sentinel).

Formats: BCSR / WCSR from the AsyncSparse page (abstract, Figure 2 caption,
row-window splitting in the summary); 2:4 from the tiled-GEMM page
(abstract) and the N:M search-results entry; int8 SpMM from the Magicube
page (abstract).
"""
import numpy as np
import pytest

import synth
from gpu_helpers import (TOL_BF16, TOL_F32, assert_all_written, bf16_to_f64, empty_out, from_dev,
                         run, to_dev)

pytestmark = pytest.mark.gpu

I32_SENTINEL = 0x7ABCDEF1   # an int32 no tested sum takes


@pytest.fixture(scope="module")
def S():
    import sparse_dense_matrix_amd as S
    import torch
    assert torch.cuda.is_available()
    return S


def _say(msg):
    print(msg, flush=True)


# ---------------------------------------------------------------------------
# BCSR bf16
# ---------------------------------------------------------------------------

def bcsr_case(S, orc, a_bits, B_bits, rows=None, pad=0):
    m, n = a_bits.shape[0], B_bits.shape[1]
    M = S.spmm_pack_bcsr(a_bits, 64, 64)
    P = S.spmm_plan(M, n, S.BF16, S.BF16)
    got = run(S, P, B_bits, m, n, "bf16", pad)
    assert_all_written(got, "bf16")
    rp, ci, v = orc.pack_bcsr(a_bits, 64, 64)
    ref = orc.bcsr_spmm(64, 64, rp, ci, v, B_bits, rows=rows)
    g = bf16_to_f64(got if rows is None else got[rows])
    assert np.isfinite(g).all(), "non-finite outputs"
    return g, ref, got


def test_bcsr_small_ragged_n(S, orc):
    w = synth.SMALL["bcsr_small"]            # 640 x 512, n = 1000 (ragged tile)
    a = synth.make_a(w)["dense"]
    B = synth.make_b(w)
    for pad in (0, 24):
        g, ref, _ = bcsr_case(S, orc, a, B, pad=pad)
        err = orc.rel_frobenius(g, ref)
        _say(f"bcsr_small pad={pad} rel_frob={err:.3e}")
        assert err <= TOL_BF16


def test_bcsr_identity_exact(S, orc):
    m = 256
    eye = synth.f32_to_bf16_bits(np.eye(m, dtype=np.float32))
    B = synth.dense_bf16_normal(m, 264, 77)
    M = S.spmm_pack_bcsr(eye)
    P = S.spmm_plan(M, 264, S.BF16, S.BF16)
    got = run(S, P, B, m, 264, "bf16")
    np.testing.assert_array_equal(got, B)


def test_bcsr_single_nonzero_is_rne(S, orc):
    # one product of two bf16 values is exact in fp32, so the output must be
    # exactly its round-to-nearest-even bf16
    m, k, n = 128, 192, 512
    a = np.zeros((m, k), np.float32)
    a[70, 100] = -1.3671875           # bf16-exact, many mantissa bits
    a_bits = synth.f32_to_bf16_bits(a)
    B = synth.dense_bf16_normal(k, n, 78)
    M = S.spmm_pack_bcsr(a_bits)
    P = S.spmm_plan(M, n, S.BF16, S.BF16)
    got = run(S, P, B, m, n, "bf16")
    exp = np.zeros((m, n), np.uint16)
    prod = (np.float32(-1.3671875) * synth.bf16_bits_to_f32(B[100])).astype(np.float32)
    exp[70] = synth.f32_to_bf16_bits(prod)
    np.testing.assert_array_equal(got & 0x7FFF, exp & 0x7FFF)        # zeros may be -0
    np.testing.assert_array_equal(got[70], exp[70])


def test_bcsr_empty_and_dense_block_rows(S, orc):
    m, k, n = 256, 512, 256
    a = np.zeros((m, k), np.uint16)
    a[64:128, :] = synth.dense_bf16_normal(64, k, 79, sigma=0.02)  # one full block row
    B = synth.dense_bf16_normal(k, n, 80)
    g, ref, got = bcsr_case(S, orc, a, B)
    assert (got[:64] & 0x7FFF == 0).all() and (got[128:] & 0x7FFF == 0).all()
    assert orc.rel_frobenius(g, ref) <= TOL_BF16
    zero = np.zeros((m, k), np.uint16)
    _, _, got0 = bcsr_case(S, orc, zero, B)
    assert (got0 & 0x7FFF == 0).all()


def test_bcsr_4096_config(S, orc):
    # every row and column of C against the oracle
    w = synth.WORKLOADS["bcsr_4096_b64_90"]
    a = synth.make_a(w)["dense"]
    B = synth.make_b(w)
    g, ref, _ = bcsr_case(S, orc, a, B)
    err = orc.rel_frobenius(g, ref)
    _say(f"bcsr_4096 all {w.m} rows rel_frob={err:.3e}")
    assert err <= TOL_BF16


# column ranges of the prefill layer checked over every row: the first and
# the last 1024 columns and two interior ranges that straddle N-tile
# boundaries of every tile width the plan may take (256 and 512); C's columns
# are independent, so these check the same sums as whole rows
PREFILL_COLS = ((0, 1024), (16128, 17152), (40704, 41728), (65536 - 1024, 65536))


@pytest.mark.parametrize("name", ["bcsr_prefill_18944x3584", "bcsr_prefill_18944x3584_z70",
                                  "bcsr_prefill_18944x3584_z50"])
def test_bcsr_prefill_config(S, orc, name):
    w = synth.WORKLOADS[name]
    a = synth.make_a(w)["dense"]
    B = synth.make_b(w)
    M = S.spmm_pack_bcsr(a, 64, 64)
    P = S.spmm_plan(M, w.n, S.BF16, S.BF16)
    _say(f"{name}: plan tile_n={P.info()['tile_n']} grid={P.info()['grid']}")
    got = run(S, P, B, w.m, w.n, "bf16")
    assert_all_written(got, "bf16")
    rp, ci, v = orc.pack_bcsr(a, 64, 64)
    for j0, j1 in PREFILL_COLS:
        ref = orc.bcsr_spmm(64, 64, rp, ci, v, B, j0=j0, j1=j1)
        err = orc.rel_frobenius(bf16_to_f64(got[:, j0:j1]), ref)
        _say(f"{name} all {w.m} rows cols=[{j0},{j1}) rel_frob={err:.3e}")
        assert err <= TOL_BF16


def _int_bcsr(m, k, nblocks, seed, empty_rows=()):
    """bf16 bits of an m x k matrix with `nblocks` uniformly placed 64 x 64
    blocks of small integers (-3..3, zeros included) and the given block rows
    emptied."""
    r = np.random.default_rng(seed)
    mb, kb = m // 64, k // 64
    a = np.zeros((m, k), np.float32)
    for b in r.choice(mb * kb, nblocks, replace=False):
        i, j = divmod(int(b), kb)
        a[i * 64:(i + 1) * 64, j * 64:(j + 1) * 64] = r.integers(-3, 4, size=(64, 64))
    for i in empty_rows:
        a[i * 64:(i + 1) * 64] = 0
    return synth.f32_to_bf16_bits(a)


def _assert_int_exact(got, ref):
    """Integer-valued inputs: every fp32 partial sum is exact, so C must be
    exactly the round-to-nearest-even bf16 of the exact sum (zeros may carry
    either sign)."""
    assert np.abs(ref).max() < 2 ** 24
    exp = synth.f32_to_bf16_bits(ref.astype(np.float32))
    np.testing.assert_array_equal(got & 0x7FFF, exp & 0x7FFF)
    nz = ref != 0
    np.testing.assert_array_equal(got[nz], exp[nz])


def test_bcsr_integer_values_many_blocks_per_row_exact(S, orc):
    # about 20 stored blocks per block row (whole-block stages), an empty
    # block row, a ragged n; bit-exact against the oracle's exact sums
    m, k, n = 640, 2048, 1032
    a = _int_bcsr(m, k, 200, 91, empty_rows=(3,))
    B = synth.f32_to_bf16_bits(np.random.default_rng(92).integers(-4, 5, size=(k, n)).astype(np.float32))
    M = S.spmm_pack_bcsr(a, 64, 64)
    P = S.spmm_plan(M, n, S.BF16, S.BF16)
    got = run(S, P, B, m, n, "bf16")
    assert_all_written(got, "bf16")
    rp, ci, v = orc.pack_bcsr(a, 64, 64)
    assert np.diff(rp).max() > 16 and np.diff(rp).mean() > 16
    _say(f"bcsr integer many blocks: blocks={len(ci)} tile_n={P.info()['tile_n']}")
    _assert_int_exact(got, orc.bcsr_spmm(64, 64, rp, ci, v, B))


def test_bcsr_integer_values_row_groups_exact(S, orc):
    # A of ~3.4 MB at n >= 8192 takes the row-group schedule (each XCD serves
    # a quarter of the block rows over half the N tiles); ragged last N tile,
    # empty block rows;
    # every row bit-exact over the first, an interior and the last columns
    m, k, n = 20480, 1024, 8200
    a = _int_bcsr(m, k, 420, 93, empty_rows=(0, 1, 2, 150))
    B = synth.f32_to_bf16_bits(np.random.default_rng(94).integers(-4, 5, size=(k, n)).astype(np.float32))
    M = S.spmm_pack_bcsr(a, 64, 64)
    P = S.spmm_plan(M, n, S.BF16, S.BF16)
    got = run(S, P, B, m, n, "bf16")
    assert_all_written(got, "bf16")
    rp, ci, v = orc.pack_bcsr(a, 64, 64)
    _say(f"bcsr integer row groups: blocks={len(ci)} tile_n={P.info()['tile_n']} grid={P.info()['grid']}")
    for j0, j1 in ((0, 512), (3968, 4480), (n - 520, n)):
        _assert_int_exact(got[:, j0:j1], orc.bcsr_spmm(64, 64, rp, ci, v, B, j0=j0, j1=j1))


def test_bcsr_paired_block_rows_exact(S, orc):
    # enough 64-row block rows at n < 8192 for the plan to pair them (tile_m
    # 128: two block rows walk the union of their block columns): rows that
    # share every column, rows that share none, empty rows next to full
    # ones, an odd block-row count and a ragged last N tile; integer values,
    # bit-exact over every row
    m, k, n = 64 * 131, 1024, 8120
    mb, kb = m // 64, k // 64
    r = np.random.default_rng(95)
    mask = np.zeros((mb, kb), bool)
    mask[0:10, [0, 3, 5]] = True                  # identical columns
    for i in range(10, 26):
        mask[i, i - 10] = True                    # one column each, all different
    # rows 26..31 stay empty
    mask[32, :] = True                            # a full block row
    for i in range(33, mb):
        mask[i, r.choice(kb, 3, replace=False)] = True
    a = np.zeros((m, k), np.float32)
    for i, j in zip(*np.nonzero(mask)):
        a[i * 64:(i + 1) * 64, j * 64:(j + 1) * 64] = r.integers(-3, 4, size=(64, 64))
    a = synth.f32_to_bf16_bits(a)
    B = synth.f32_to_bf16_bits(r.integers(-4, 5, size=(k, n)).astype(np.float32))
    M = S.spmm_pack_bcsr(a, 64, 64)
    P = S.spmm_plan(M, n, S.BF16, S.BF16)
    info = P.info()
    _say(f"bcsr paired rows: tile_m={info['tile_m']} tile_n={info['tile_n']} grid={info['grid']}")
    assert info["tile_m"] == 128 and info["tile_n"] == 256
    rp, ci, v = orc.pack_bcsr(a, 64, 64)
    refs = [(j0, j1, orc.bcsr_spmm(64, 64, rp, ci, v, B, j0=j0, j1=j1))
            for j0, j1 in ((0, 520), (3840, 4352), (n - 440, n))]
    for pad in (0, 24):                 # B and C with ld = n and ld = n + 24
        got = run(S, P, B, m, n, "bf16", pad)
        assert_all_written(got, "bf16")
        assert (got[26 * 64:32 * 64] & 0x7FFF == 0).all()
        for j0, j1, ref in refs:
            _assert_int_exact(got[:, j0:j1], ref)


def test_bcsr_pair_over_64_units_keeps_single_rows(S, orc):
    # a block row with 80 stored blocks: its pair would walk more than 64
    # block columns, more than a wave holds descriptors for, so the plan keeps
    # single-row tiles (tile_m 64); the result is still exact
    m, k, n = 64 * 131, 64 * 80, 8120
    mb, kb = m // 64, k // 64
    r = np.random.default_rng(96)
    mask = np.zeros((mb, kb), bool)
    mask[5, :] = True
    for i in range(mb):
        if i != 5:
            mask[i, r.choice(kb, 3, replace=False)] = True
    a = np.zeros((m, k), np.float32)
    for i, j in zip(*np.nonzero(mask)):
        a[i * 64:(i + 1) * 64, j * 64:(j + 1) * 64] = r.integers(-3, 4, size=(64, 64))
    a = synth.f32_to_bf16_bits(a)
    B = synth.f32_to_bf16_bits(r.integers(-4, 5, size=(k, n)).astype(np.float32))
    M = S.spmm_pack_bcsr(a, 64, 64)
    P = S.spmm_plan(M, n, S.BF16, S.BF16)
    info = P.info()
    _say(f"bcsr long row: tile_m={info['tile_m']} tile_n={info['tile_n']} grid={info['grid']}")
    assert info["tile_m"] == 64
    got = run(S, P, B, m, n, "bf16")
    assert_all_written(got, "bf16")
    rp, ci, v = orc.pack_bcsr(a, 64, 64)
    for j0, j1 in ((0, 264), (n - 264, n)):
        _assert_int_exact(got[:, j0:j1], orc.bcsr_spmm(64, 64, rp, ci, v, B, j0=j0, j1=j1))


def test_bcsr_many_blocks_per_row(S, orc):
    # more than 16 stored blocks per block row on average: whole-block LDS
    # stages at 256 columns (few blocks per row take half-block stages, as
    # in every other small case); an empty block row and a ragged n
    m, k, n = 320, 2048, 520
    a, _ = synth.block_sparse_dense_bf16(m, k, 64, 64, 144, 0.02, 87)
    a[128:192] = 0
    B = synth.dense_bf16_normal(k, n, 88)
    g, ref, got = bcsr_case(S, orc, a, B)
    assert (got[128:192] & 0x7FFF == 0).all()
    err = orc.rel_frobenius(g, ref)
    _say(f"bcsr many blocks per row: blocks={int(np.count_nonzero(a.reshape(5, 64, 32, 64).any(axis=(1, 3))))} "
         f"rel_frob={err:.3e}")
    assert err <= TOL_BF16


def test_bcsr_row_groups_skewed_rows(S, orc):
    # A of ~7 MB at n >= 8192 takes the row-group schedule (each XCD serves a
    # quarter of the block rows over half the N tiles, 256-wide N tiles): empty
    # block rows, one full
    # block row, a ragged block-row count and a ragged last N tile
    m, k, n = 16576, 2048, 8200
    a, _ = synth.block_sparse_dense_bf16(m, k, 64, 64, 830, 0.02, 83)
    a[: 10 * 64] = 0
    a[100 * 64: 101 * 64] = synth.dense_bf16_normal(64, k, 84, sigma=0.02)
    B = synth.dense_bf16_normal(k, n, 85)
    M = S.spmm_pack_bcsr(a, 64, 64)
    P = S.spmm_plan(M, n, S.BF16, S.BF16)
    assert P.info()["tile_n"] == 256
    got = run(S, P, B, m, n, "bf16")
    assert (got != 0xFFFF).all(), "some C element was not written"
    assert (got[: 10 * 64] & 0x7FFF == 0).all()
    r = np.random.default_rng(86)
    rows = np.unique(np.concatenate([np.arange(64), np.arange(6400, 6464), np.arange(m - 64, m),
                                     r.choice(m, 128, replace=False)])).astype(np.int64)
    rp, ci, v = orc.pack_bcsr(a, 64, 64)
    ref = orc.bcsr_spmm(64, 64, rp, ci, v, B, rows=rows)
    err = orc.rel_frobenius(bf16_to_f64(got[rows]), ref)
    _say(f"bcsr row groups m={m} n={n} blocks={S.spmm_matrix_info(M)['nnzb']} "
         f"grid={P.info()['grid']} rel_frob={err:.3e}")
    assert err <= TOL_BF16


def test_bcsr_deterministic(S, orc):
    w = synth.SMALL["bcsr_small"]
    a = synth.make_a(w)["dense"]
    B = synth.make_b(w)
    M = S.spmm_pack_bcsr(a)
    P = S.spmm_plan(M, w.n, S.BF16, S.BF16)
    x = run(S, P, B, w.m, w.n, "bf16")
    y = run(S, P, B, w.m, w.n, "bf16")
    np.testing.assert_array_equal(x, y)


def test_bcsr_schedules_agree_bitwise(S, orc):
    # The prefill layer's block pattern at three widths of B: n = 1024 takes
    # single-row tiles (too few pair tiles), n = 4288 paired block rows, n =
    # 8192 paired rows in four row groups.  Every C element sees the same
    # MFMAs in the same order under each schedule (stored blocks ascending,
    # k-steps ascending), so the columns they share are equal bit for bit.
    w = synth.SMALL["bcsr_prefill_slice"]
    a = synth.make_a(w)["dense"]
    B = synth.dense_bf16_normal(w.k, 8192, 86)
    M = S.spmm_pack_bcsr(a)
    outs, seen = {}, set()
    for n in (1024, 4288, 8192):
        P = S.spmm_plan(M, n, S.BF16, S.BF16)
        info = P.info()
        seen.add((info["tile_m"], info["tile_n"], info["grid"]))
        _say(f"bcsr schedules: n={n} tile_m={info['tile_m']} tile_n={info['tile_n']} grid={info['grid']}")
        outs[n] = run(S, P, np.ascontiguousarray(B[:, :n]), w.m, n, "bf16")
        assert_all_written(outs[n], "bf16")
    assert len(seen) == 3 and {t[0] for t in seen} == {64, 128}
    np.testing.assert_array_equal(outs[1024], outs[4288][:, :1024])
    np.testing.assert_array_equal(outs[1024], outs[8192][:, :1024])
    np.testing.assert_array_equal(outs[4288], outs[8192][:, :4288])
    # and against the oracle on a few rows, so that agreement is not shared error
    rows = np.array([0, 1, 4095, 9000, w.m - 1], np.int64)
    rp, ci, v = orc.pack_bcsr(a, 64, 64)
    ref = orc.bcsr_spmm(64, 64, rp, ci, v, np.ascontiguousarray(B[:, :1024]), rows=rows)
    assert orc.rel_frobenius(bf16_to_f64(outs[1024][rows]), ref) <= TOL_BF16


# ---------------------------------------------------------------------------
# WCSR fp32
# ---------------------------------------------------------------------------

def wcsr_case(S, orc, m, k, rp, ci, v, B, W, T, rows=None, pad=0):
    n = B.shape[1]
    M = S.spmm_pack_wcsr(m, k, rp, ci, v, W, T)
    P = S.spmm_plan(M, n, S.F32, S.F32)
    got = run(S, P, B, m, n, "f32", pad)
    assert_all_written(got, "f32")
    ref = orc.csr_spmm(rp, ci, v, B, rows=rows)
    g = got if rows is None else got[rows]
    return orc.rel_frobenius(g, ref), got, P


def test_wcsr_tiny_config(S, orc):
    w = synth.WORKLOADS["csr_tiny_256"]
    a = synth.make_a(w)
    B = synth.make_b(w)
    err, _, _ = wcsr_case(S, orc, w.m, w.k, a["row_ptr"], a["col_idx"], a["vals"], B, 16, 512)
    _say(f"csr_tiny rel_frob={err:.3e}")
    assert err <= TOL_F32


@pytest.mark.parametrize("W,T", [(16, 512), (1, 1), (3, 7), (64, 100), (16, 4096)])
@pytest.mark.parametrize("name", ["csr_uniform_small", "csr_powerlaw_small"])
def test_wcsr_small(S, orc, name, W, T):
    w = synth.SMALL[name]
    a = synth.make_a(w)
    B = synth.make_b(w)
    err, _, P = wcsr_case(S, orc, w.m, w.k, a["row_ptr"], a["col_idx"], a["vals"], B, W, T)
    _say(f"{name} W={W} T={T} split_rows={P.info()['num_split_rows']} rel_frob={err:.3e}")
    assert err <= TOL_F32


@pytest.mark.parametrize("n", [1, 3, 64, 65, 129, 300])
def test_wcsr_ragged_n(S, orc, n):
    w = synth.SMALL["csr_uniform_small"]
    a = synth.make_a(w)
    B = synth.dense_f32_normal(w.k, n, 81)
    # leading dimensions padded to whole 16-byte rows, as the ABI requires
    err, _, _ = wcsr_case(S, orc, w.m, w.k, a["row_ptr"], a["col_idx"], a["vals"], B, 8, 37,
                          pad=(-n) % 4 + 4)
    assert err <= TOL_F32


def test_wcsr_empty_and_giant_rows(S, orc):
    k, n = 30000, 128
    r = np.random.default_rng(9)
    lens = np.zeros(50, np.int64)
    lens[[3, 17, 18, 40]] = [20000, 5, 1, 7000]    # empty rows everywhere else
    rp = np.zeros(51, np.int64)
    np.cumsum(lens, out=rp[1:])
    ci = np.concatenate([np.sort(r.choice(k, L, replace=False)) for L in lens if L]).astype(np.int32)
    v = r.uniform(-1, 1, int(rp[-1])).astype(np.float32)
    B = synth.dense_f32_normal(k, n, 82)
    for W, T in ((16, 512), (4, 300), (50, 100000), (1, 64)):
        err, got, P = wcsr_case(S, orc, 50, k, rp, ci, v, B, W, T)
        _say(f"giant W={W} T={T} split_rows={P.info()['num_split_rows']} rel_frob={err:.3e}")
        assert err <= TOL_F32
        assert (got[lens == 0] == 0).all()
    # all-empty matrix
    rp0 = np.zeros(51, np.int64)
    err, got, _ = wcsr_case(S, orc, 50, k, rp0, np.zeros(0, np.int32), np.zeros(0, np.float32),
                            B, 16, 512)
    assert (got == 0).all()


def test_wcsr_powerlaw_1m_config(S, orc):
    # every row of C against the oracle (all 10^6 rows, 128 columns)
    w = synth.WORKLOADS["csr_powerlaw_1m"]
    a = synth.make_a(w)
    B = synth.make_b(w)
    err, got, P = wcsr_case(S, orc, w.m, w.k, a["row_ptr"], a["col_idx"], a["vals"], B, 16, 512)
    _say(f"csr_powerlaw_1m all {w.m} rows split_rows={P.info()['num_split_rows']} "
         f"rel_frob={err:.3e}")
    assert err <= TOL_F32
    lens = np.diff(a["row_ptr"])
    assert (got[lens == 0] == 0).all()


def test_wcsr_deterministic(S, orc):
    w = synth.SMALL["csr_powerlaw_small"]
    a = synth.make_a(w)
    B = synth.make_b(w)
    M = S.spmm_pack_wcsr(w.m, w.k, a["row_ptr"], a["col_idx"], a["vals"], 16, 64)
    P = S.spmm_plan(M, w.n, S.F32, S.F32)
    x = run(S, P, B, w.m, w.n, "f32")
    y = run(S, P, B, w.m, w.n, "f32")
    np.testing.assert_array_equal(x.view(np.uint32), y.view(np.uint32))


# ---------------------------------------------------------------------------
# 2:4 int8
# ---------------------------------------------------------------------------

def sp24_case(S, orc, a, B, rows=None, pad=0):
    m, n = a.shape[0], B.shape[1]
    M = S.spmm_pack_24(a)
    P = S.spmm_plan(M, n, S.I8, S.I32)
    got = run(S, P, B, m, n, "i32", pad)
    assert_all_written(got, "i32")
    v, mt = orc.pack24(a)
    ref = orc.sp24_spmm(v, mt, B, rows=rows)
    return got if rows is None else got[rows], ref


def test_sp24_small_ragged(S, orc):
    w = synth.SMALL["sp24_small"]       # 320 x 512, n = 400: ragged m and n tiles
    a = synth.make_a(w)["dense"]
    B = synth.make_b(w)
    for pad in (0, 32):
        got, ref = sp24_case(S, orc, a, B, pad=pad)
        np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("m,k,n", [(1, 8, 16), (17, 136, 48), (130, 264, 144), (64, 1024, 16)])
def test_sp24_shapes(S, orc, m, k, n):
    r = np.random.default_rng(m * 1000 + k)
    a = synth.int8_uniform(r, (m, k))
    B = synth.int8_uniform(r, (k, n))
    got, ref = sp24_case(S, orc, a, B)
    np.testing.assert_array_equal(got, ref)


def test_sp24_identity_and_extremes(S, orc):
    m = 256
    B = synth.int8_uniform(np.random.default_rng(3), (m, 128))
    got, _ = sp24_case(S, orc, np.eye(m, dtype=np.int8), B)
    np.testing.assert_array_equal(got, B.astype(np.int32))
    k = 8192
    a = np.full((128, k), -128, np.int8)
    Bm = np.full((k, 32), -128, np.int8)
    got, ref = sp24_case(S, orc, a, Bm)
    np.testing.assert_array_equal(got, np.full((128, 32), (k // 2) * 16384, np.int32))


def test_sp24_8192_config(S, orc):
    # every element of C bit for bit
    w = synth.WORKLOADS["sp24_i8_8192"]
    a = synth.make_a(w)["dense"]
    B = synth.make_b(w)
    got, ref = sp24_case(S, orc, a, B)
    np.testing.assert_array_equal(got, ref)
    _say(f"sp24_i8_8192 all {w.m} rows exact")


def test_sp24_empty_k_writes_zeros(S, orc):
    # k = 0 (a valid pack): the plan has no k-steps, execute takes a NULL B
    # and must write zeros without reading B; int8, bf16 and (2N-2):2N
    torch = __import__("torch")
    m, n = 300, 32
    cases = [(S.spmm_pack_24(np.zeros((m, 0), np.int8)), (S.I8, S.I32), torch.int32, "i32"),
             (S.spmm_pack_24(np.zeros((m, 0), np.uint16)), (S.BF16, S.BF16), torch.int16, "bf16"),
             (S.spmm_pack_slide(np.zeros((m, 0), np.int8), 8), (S.I8, S.I32), torch.int32, "i32")]
    for M, types, cdt, kind in cases:
        P = S.spmm_plan(M, n, *types)
        Ct = empty_out(m, n, kind)
        S.spmm_execute(P, 0, Ct.data_ptr(), ldb=n, ldc=n)
        got = from_dev(Ct, kind)
        assert (np.asarray(got).view(np.uint16 if kind == "bf16" else np.int32) & (0x7FFF if kind == "bf16" else -1) == 0).all()


# ---------------------------------------------------------------------------
# 2:4 bf16
# ---------------------------------------------------------------------------

def sp24_bf16_case(S, orc, a_bits, B_bits, rows=None, pad=0):
    """GPU result (uint16 bits) and the oracle's fp64 product of the 2:4-pruned
    A (its pruning, then its dense fp64 product: any m and k)."""
    m, n = a_bits.shape[0], B_bits.shape[1]
    M = S.spmm_pack_24(a_bits)
    P = S.spmm_plan(M, n, S.BF16, S.BF16)
    got = run(S, P, B_bits, m, n, "bf16", pad)
    assert_all_written(got, "bf16")
    pruned = orc.prune_nm(a_bits, 2, 4)
    ref = orc.gemm_f64(bf16_to_f64(pruned if rows is None else pruned[rows]), bf16_to_f64(B_bits))
    g = bf16_to_f64(got if rows is None else got[rows])
    assert np.isfinite(g).all(), "unwritten or non-finite outputs"
    return g, ref, got


def test_sp24_bf16_small_ragged(S, orc):
    w = synth.SMALL["sp24_bf16_small"]   # 320 x 512, n = 400: ragged m and n tiles
    a = synth.make_a(w)["dense"]
    B = synth.make_b(w)
    for pad in (0, 16):
        g, ref, _ = sp24_bf16_case(S, orc, a, B, pad=pad)
        err = orc.rel_frobenius(g, ref)
        assert err <= TOL_BF16, err
    _say(f"sp24_bf16_small rel={err:.2e}")


@pytest.mark.parametrize("m,k,n", [(1, 8, 16), (17, 136, 48), (130, 264, 144), (64, 1024, 16)])
def test_sp24_bf16_shapes(S, orc, m, k, n):
    r = np.random.default_rng(m * 1000 + k + 7)
    a = synth.f32_to_bf16_bits(synth.normal_f32(r, (m, k), 0.02))
    B = synth.f32_to_bf16_bits(synth.normal_f32(r, (k, n), 1.0))
    g, ref, _ = sp24_bf16_case(S, orc, a, B)
    err = orc.rel_frobenius(g, ref)
    assert err <= TOL_BF16, err


def test_sp24_bf16_integer_values_are_exact(S, orc):
    # small integers: every fp32 partial sum is exact, so C must be exactly the
    # round-to-nearest-even bf16 of the exact sum; pins the kept positions, the
    # k order of B and the epilogue bit for bit, over ragged m, k and n
    r = np.random.default_rng(46)
    m, k, n = 330, 520, 272
    a = r.integers(-3, 4, size=(m, k)).astype(np.float32)
    a[100:164] = 0                               # an all-zero row band
    a_bits = synth.f32_to_bf16_bits(a)
    B = synth.f32_to_bf16_bits(r.integers(-4, 5, size=(k, n)).astype(np.float32))
    _, ref, got = sp24_bf16_case(S, orc, a_bits, B)
    assert np.abs(ref).max() < 2 ** 24
    np.testing.assert_array_equal(got & 0x7FFF, synth.f32_to_bf16_bits(ref.astype(np.float32)) & 0x7FFF)
    nz = ref != 0
    np.testing.assert_array_equal(got[nz], synth.f32_to_bf16_bits(ref[nz].astype(np.float32)))


def test_sp24_bf16_ragged_k_padding_meets_zeros(S, orc):
    # k = 72 is not a whole number of 64-deep steps: the last step's slab
    # k-rows past k must be zeros, not copies of a B row, or a padded zero of
    # A times an infinite B element would turn whole columns into NaN.  B row
    # 0 holds +Inf in every third column and every row keeps A[i, 0] = 1 (the
    # largest of its group), so those columns must come out exactly +Inf
    r = np.random.default_rng(49)
    m, k, n = 130, 72, 96
    a = synth.normal_f32(r, (m, k), 0.02)
    a[:, 0] = 1.0
    a_bits = synth.f32_to_bf16_bits(a)
    B = synth.f32_to_bf16_bits(synth.normal_f32(r, (k, n), 1.0))
    B[0, ::3] = 0x7F80
    M = S.spmm_pack_24(a_bits)
    P = S.spmm_plan(M, n, S.BF16, S.BF16)
    got = run(S, P, B, m, n, "bf16")
    assert (got[:, ::3] == 0x7F80).all(), "infinite columns"
    fin = np.ones(n, bool)
    fin[::3] = False
    pruned = orc.prune_nm(a_bits, 2, 4)
    ref = orc.gemm_f64(bf16_to_f64(pruned), bf16_to_f64(B[:, fin]))
    g = bf16_to_f64(got[:, fin])
    assert np.isfinite(g).all()
    assert orc.rel_frobenius(g, ref) <= TOL_BF16


def test_sp24_bf16_identity_and_zero(S, orc):
    m = 256
    eye = synth.f32_to_bf16_bits(np.eye(m, dtype=np.float32))   # one nonzero per group: kept
    B = synth.dense_bf16_normal(m, 272, 47)
    _, _, got = sp24_bf16_case(S, orc, eye, B)
    np.testing.assert_array_equal(got, B)
    Z = np.zeros((128, 192), np.uint16)
    M = S.spmm_pack_24(Z)
    P = S.spmm_plan(M, 32, S.BF16, S.BF16)
    got = run(S, P, synth.dense_bf16_normal(192, 32, 48), 128, 32, "bf16")
    assert (got & 0x7FFF == 0).all()
    for types in ((S.I8, S.I32), (S.BF16, S.F32)):
        with pytest.raises(S.SpmmError) as ei:
            S.spmm_plan(M, 32, *types)
        assert ei.value.name == "SPMM_ERR_UNSUPPORTED"


def test_sp24_bf16_8192_sampled(S, orc):
    w = synth.WORKLOADS["sp24_bf16_8192"]
    a = synth.make_a(w)["dense"]
    B = synth.make_b(w)
    r = np.random.default_rng(25)
    rows = np.unique(np.concatenate([np.arange(16), np.arange(w.m - 16, w.m),
                                     r.choice(w.m, 48, replace=False)])).astype(np.int64)
    g, ref, _ = sp24_bf16_case(S, orc, a, B, rows=rows)
    err = orc.rel_frobenius(g, ref)
    assert err <= TOL_BF16, err
    _say(f"sp24_bf16_8192 rows={len(rows)} rel={err:.2e}")


# ---------------------------------------------------------------------------
# boundary behaviour on the device
# ---------------------------------------------------------------------------

def test_plan_rejects_unsupported(S):
    a = np.zeros((64, 64), np.uint16)
    M = S.spmm_pack_bcsr(a)
    with pytest.raises(S.SpmmError) as ei:
        S.spmm_plan(M, 12, S.BF16, S.BF16)          # n % 8 != 0
    assert ei.value.name == "SPMM_ERR_UNSUPPORTED"
    with pytest.raises(S.SpmmError) as ei:
        S.spmm_plan(M, 16, S.F32, S.F32)
    assert ei.value.name == "SPMM_ERR_UNSUPPORTED"
    M24 = S.spmm_pack_24(np.zeros((16, 16), np.int8))
    with pytest.raises(S.SpmmError) as ei:
        S.spmm_plan(M24, 24, S.I8, S.I32)
    assert ei.value.name == "SPMM_ERR_UNSUPPORTED"


def test_execute_rejects_bad_layouts(S):
    torch = pytest.importorskip("torch")
    M = S.spmm_pack_bcsr(np.zeros((64, 64), np.uint16))
    P = S.spmm_plan(M, 64, S.BF16, S.BF16)
    B = torch.zeros((64, 72), dtype=torch.int16, device="cuda")
    Cw = torch.zeros((64, 64), dtype=torch.int16, device="cuda")
    with pytest.raises(S.SpmmError) as ei:          # misaligned B
        S.spmm_execute(P, B.data_ptr() + 2, Cw.data_ptr(), ldb=72, ldc=64)
    assert ei.value.name == "SPMM_ERR_INVALID_ARG"
    with pytest.raises(S.SpmmError) as ei:          # ldb < n
        S.spmm_execute(P, B.data_ptr(), Cw.data_ptr(), ldb=32, ldc=64)
    assert ei.value.name == "SPMM_ERR_INVALID_ARG"
    # leading dimensions past the kernels' 32-bit B offsets are refused before
    # any launch (nothing reads B here)
    with pytest.raises(S.SpmmError) as ei:
        S.spmm_execute(P, B.data_ptr(), Cw.data_ptr(), ldb=(1 << 24) + 8, ldc=64)
    assert ei.value.name == "SPMM_ERR_UNSUPPORTED"
    M24 = S.spmm_pack_24(np.ones((16, 8192), np.int8))
    P24 = S.spmm_plan(M24, 16, S.I8, S.I32)
    C24 = torch.zeros((16, 16), dtype=torch.int32, device="cuda")
    with pytest.raises(S.SpmmError) as ei:
        S.spmm_execute(P24, B.data_ptr(), C24.data_ptr(), ldb=1 << 20, ldc=16)
    assert ei.value.name == "SPMM_ERR_UNSUPPORTED"


def test_binding_checks_tensors_against_the_plan(S):
    # torch tensors handed to execute must have the plan's shapes, element
    # sizes and device; a mismatch is refused before anything is launched
    torch = pytest.importorskip("torch")
    M = S.spmm_pack_bcsr(np.zeros((128, 64), np.uint16))
    P = S.spmm_plan(M, 64, S.BF16, S.BF16)
    B = torch.zeros((64, 64), dtype=torch.int16, device="cuda")
    Cm = torch.zeros((128, 64), dtype=torch.int16, device="cuda")
    S.spmm_execute(P, B, Cm)
    for b, c, what in ((B[:32], Cm, "shape"), (B, Cm[:, :32], "shape"),
                       (B.float(), Cm, "element"), (B, Cm.cpu(), "cuda"),
                       (torch.zeros((64, 128), dtype=torch.int16, device="cuda"), Cm, "shape")):
        with pytest.raises(ValueError, match=what):
            S.spmm_execute(P, b, c)
    Mw = S.spmm_pack_wcsr(4, 8, np.array([0, 1, 1, 2, 3], np.int64), np.array([0, 7, 3], np.int32),
                          np.ones(3, np.float32))
    Q = S.spmm_plan_sddmm(Mw, 16)
    X = torch.zeros((4, 16), device="cuda")
    Y = torch.zeros((8, 16), device="cuda")
    out = torch.zeros(3, device="cuda")
    S.spmm_execute_sddmm(Q, X, Y, out)
    torch.cuda.synchronize()
    for x, y, o, what in ((X[:, :8], Y, out, "shape"), (X, Y[:4], out, "shape"),
                          (X, Y, out[:2], "at least 3"), (X, Y, out.double(), "element")):
        with pytest.raises(ValueError, match=what):
            S.spmm_execute_sddmm(Q, x, y, o)


def test_two_plans_two_streams(S, orc):
    torch = pytest.importorskip("torch")
    w1, w2 = synth.SMALL["csr_powerlaw_small"], synth.SMALL["bcsr_small"]
    a1, a2 = synth.make_a(w1), synth.make_a(w2)["dense"]
    B1, B2 = synth.make_b(w1), synth.make_b(w2)
    P1 = S.spmm_plan(S.spmm_pack_wcsr(w1.m, w1.k, a1["row_ptr"], a1["col_idx"], a1["vals"], 16, 64),
                     w1.n, S.F32, S.F32)
    P2 = S.spmm_plan(S.spmm_pack_bcsr(a2), w2.n, S.BF16, S.BF16)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    Bt1, Bt2 = to_dev(B1), to_dev(B2)
    C1, C2 = empty_out(w1.m, w1.n, "f32"), empty_out(w2.m, w2.n, "bf16")
    torch.cuda.synchronize()
    for _ in range(3):
        S.spmm_execute(P1, Bt1, C1, stream=s1)
        S.spmm_execute(P2, Bt2, C2, stream=s2)
    torch.cuda.synchronize()
    ref1 = orc.csr_spmm(a1["row_ptr"], a1["col_idx"], a1["vals"], B1)
    assert orc.rel_frobenius(from_dev(C1, "f32"), ref1) <= TOL_F32
    rp, ci, v = orc.pack_bcsr(a2, 64, 64)
    ref2 = orc.bcsr_spmm(64, 64, rp, ci, v, B2)
    assert orc.rel_frobenius(bf16_to_f64(from_dev(C2, "bf16")), ref2) <= TOL_BF16


# ---------------------------------------------------------------------------
# SDDMM fp32: out[p] = X[i] . Y[j] over the stored entries of a WCSR pattern
# ---------------------------------------------------------------------------

def sddmm_case(S, orc, m, k, rp, ci, X, Y, W=0, T=0, rows=None, extra=0):
    """X and Y go to the device as column slices of allocations whose rows are
    whole 16-byte multiples (kd rounded up to 4 floats, plus `extra`)."""
    torch = pytest.importorskip("torch")
    M = S.spmm_pack_wcsr(m, k, rp, ci, np.ones(len(ci), np.float32), W, T)
    kd = X.shape[1]
    P = S.spmm_plan_sddmm(M, kd)
    nnz = len(ci)
    out = torch.full((max(nnz, 1),), float("nan"), dtype=torch.float32, device="cuda")
    pad = (-kd) % 4 + extra
    S.spmm_execute_sddmm(P, to_dev(X, pad), to_dev(Y, pad), out)
    got = from_dev(out, "f32")[:nnz]
    if rows is None:
        ref = orc.sddmm(rp, ci, X, Y)
        sel = got
    else:
        ref = orc.sddmm(rp, ci, X, Y, rows=rows)
        sel = np.concatenate([got[rp[i]:rp[i + 1]] for i in rows]) if len(rows) else got[:0]
    assert np.isfinite(got).all(), "unwritten or non-finite outputs"
    return orc.rel_frobenius(sel, ref), got, P


@pytest.mark.parametrize("kd", [1, 4, 32, 63, 64, 96, 128, 200, 300, 301, 1000])
def test_sddmm_small(S, orc, kd):
    w = synth.SMALL["sddmm_small"]          # 20000 x 20000 power-law pattern
    a = synth.make_a(w)
    X, Y = synth.make_xy(w, kd)
    for W, T, extra in ((0, 0, 0), (16, 64, 4), (1, 5, 0)):
        err, _, P = sddmm_case(S, orc, w.m, w.k, a["row_ptr"], a["col_idx"], X, Y, W, T,
                               extra=extra)
        _say(f"sddmm_small kd={kd} W={W} T={T} ld+{extra} grid={P.info()['grid']} "
             f"rel_frob={err:.3e}")
        assert err <= TOL_F32


def test_sddmm_empty_giant_rows_and_kd0(S, orc):
    k, kd = 30000, 128
    r = np.random.default_rng(19)
    lens = np.zeros(50, np.int64)
    lens[[3, 17, 18, 40]] = [20000, 5, 1, 7000]
    rp = np.zeros(51, np.int64)
    np.cumsum(lens, out=rp[1:])
    ci = np.concatenate([np.sort(r.choice(k, L, replace=False)) for L in lens if L]).astype(np.int32)
    X = synth.dense_f32_normal(50, kd, 83)
    Y = synth.dense_f32_normal(k, kd, 84)
    for W, T in ((16, 512), (4, 300), (1, 64)):
        err, _, _ = sddmm_case(S, orc, 50, k, rp, ci, X, Y, W, T)
        assert err <= TOL_F32
    # kd = 0: every sampled product is the empty sum
    _, got, _ = sddmm_case(S, orc, 50, k, rp, ci, X[:, :0].copy(), Y[:, :0].copy(), 16, 512)
    assert (got == 0).all()


def test_sddmm_diagonal_closed_form(S, orc):
    # diagonal pattern with Y = X: squared row norms
    m, kd = 3000, 160
    X = synth.dense_f32_normal(m, kd, 85)
    rp = np.arange(m + 1, dtype=np.int64)
    ci = np.arange(m, dtype=np.int32)
    err, got, _ = sddmm_case(S, orc, m, m, rp, ci, X, X)
    np.testing.assert_allclose(got, (X.astype(np.float64) ** 2).sum(axis=1), rtol=1e-5)
    assert err <= TOL_F32


def test_sddmm_powerlaw_1m_sampled(S, orc):
    w = synth.WORKLOADS["sddmm_powerlaw_1m"]
    a = synth.make_a(w)
    X, Y = synth.make_xy(w)
    lens = np.diff(a["row_ptr"])
    r = np.random.default_rng(20)
    rows = np.unique(np.concatenate([np.argsort(lens)[-200:], r.choice(w.m, 2000, replace=False),
                                     np.arange(50), np.arange(w.m - 50, w.m)])).astype(np.int64)
    err, _, P = sddmm_case(S, orc, w.m, w.k, a["row_ptr"], a["col_idx"], X, Y, rows=rows)
    _say(f"sddmm_powerlaw_1m rows={len(rows)} grid={P.info()['grid']} rel_frob={err:.3e}")
    assert err <= TOL_F32


def test_sddmm_deterministic_and_plan_kinds(S, orc):
    torch = pytest.importorskip("torch")
    w = synth.SMALL["sddmm_small"]
    a = synth.make_a(w)
    X, Y = synth.make_xy(w)
    _, x1, P = sddmm_case(S, orc, w.m, w.k, a["row_ptr"], a["col_idx"], X, Y, 16, 64)
    _, x2, _ = sddmm_case(S, orc, w.m, w.k, a["row_ptr"], a["col_idx"], X, Y, 16, 64)
    np.testing.assert_array_equal(x1.view(np.uint32), x2.view(np.uint32))
    # an SDDMM plan is refused by spmm_execute, and an SpMM plan by the SDDMM call
    Bt, Ct = to_dev(np.zeros((w.k, 16), np.float32)), empty_out(w.m, 16, "f32")
    with pytest.raises(S.SpmmError) as ei:
        S.spmm_execute(P, Bt, Ct)
    assert ei.value.name == "SPMM_ERR_INVALID_ARG"
    M = S.spmm_pack_wcsr(w.m, w.k, a["row_ptr"], a["col_idx"], a["vals"])
    P2 = S.spmm_plan(M, 16, S.F32, S.F32)
    out = torch.zeros(len(a["col_idx"]), dtype=torch.float32, device="cuda")
    with pytest.raises(S.SpmmError) as ei:
        S.spmm_execute_sddmm(P2, to_dev(X), to_dev(Y), out)
    assert ei.value.name == "SPMM_ERR_INVALID_ARG"
    # BCSR and 2:4 matrices have no SDDMM
    with pytest.raises(S.SpmmError) as ei:
        S.spmm_plan_sddmm(S.spmm_pack_bcsr(np.zeros((64, 64), np.uint16)), 32)
    assert ei.value.name == "SPMM_ERR_UNSUPPORTED"


# ---------------------------------------------------------------------------
# SDDMM on the CSR pattern with bf16 (-> bf16) and int8 (-> int32) operands
# ---------------------------------------------------------------------------

def sddmm_typed_case(S, orc, m, k, rp, ci, X, Y, elem, W=0, T=0, rows=None, extra=0):
    """bf16 (uint16 bits) or int8 X, Y.  The oracle gets their exact fp32
    images and sums in fp64 (exact for the int8 products).  Returns the
    sampled outputs (float64) and the reference."""
    torch = pytest.importorskip("torch")
    M = S.spmm_pack_wcsr(m, k, rp, ci, np.ones(len(ci), np.float32), W, T)
    kd = X.shape[1]
    P = S.spmm_plan_sddmm(M, kd, S.BF16 if elem == "bf16" else S.I8)
    nnz = len(ci)
    if elem == "bf16":
        out = torch.full((max(nnz, 1),), -1, dtype=torch.int16, device="cuda")   # NaN bits
        pad = (-kd) % 8 + extra
    else:
        out = torch.full((max(nnz, 1),), I32_SENTINEL, dtype=torch.int32, device="cuda")
        pad = (-kd) % 16 + extra
    S.spmm_execute_sddmm(P, to_dev(X, pad), to_dev(Y, pad), out)
    torch.cuda.synchronize()
    raw = out.cpu().numpy()[:nnz]
    if elem == "bf16":
        got = bf16_to_f64(raw.view(np.uint16))
        assert np.isfinite(got).all(), "unwritten or non-finite outputs"
        Xf, Yf = synth.bf16_bits_to_f32(X), synth.bf16_bits_to_f32(Y)
    else:
        assert (raw != I32_SENTINEL).all(), "unwritten outputs"
        got = raw.astype(np.float64)
        Xf, Yf = X.astype(np.float32), Y.astype(np.float32)
    ref = orc.sddmm(rp, ci, Xf, Yf, rows=rows)
    sel = got if rows is None else (np.concatenate([got[rp[i]:rp[i + 1]] for i in rows])
                                    if len(rows) else got[:0])
    return sel, ref, raw, P


@pytest.mark.parametrize("elem", ["bf16", "i8"])
@pytest.mark.parametrize("kd", [1, 8, 16, 63, 64, 96, 128, 200, 256, 1000])
def test_sddmm_csr_typed_small(S, orc, elem, kd):
    w = synth.SMALL["sddmm_small"]          # 20000 x 20000 power-law pattern
    a = synth.make_a(w)
    X, Y = synth.make_xy(w, kd, elem)
    for W, T, extra in ((0, 0, 0), (16, 64, 16), (1, 5, 0)):
        got, ref, _, P = sddmm_typed_case(S, orc, w.m, w.k, a["row_ptr"], a["col_idx"], X, Y, elem,
                                          W, T, extra=extra)
        if elem == "bf16":
            err = orc.rel_frobenius(got, ref)
            assert err <= TOL_BF16, err
        else:
            np.testing.assert_array_equal(got, ref)
    _say(f"sddmm_small {elem} kd={kd} grid={P.info()['grid']} ok")


def test_sddmm_csr_bf16_integer_values_exact(S, orc):
    # small integers: the fp32 sums are exact, so each output is exactly the
    # round-to-nearest-even bf16 of the exact sum
    w = synth.SMALL["sddmm_small"]
    a = synth.make_a(w)
    r = np.random.default_rng(26)
    kd = 200
    X = synth.f32_to_bf16_bits(r.integers(-3, 4, size=(w.m, kd)).astype(np.float32))
    Y = synth.f32_to_bf16_bits(r.integers(-3, 4, size=(w.k, kd)).astype(np.float32))
    _, ref, raw, _ = sddmm_typed_case(S, orc, w.m, w.k, a["row_ptr"], a["col_idx"], X, Y, "bf16")
    exp = synth.f32_to_bf16_bits(ref.astype(np.float32))
    nz = ref != 0
    np.testing.assert_array_equal(raw.view(np.uint16)[nz], exp[nz])
    assert (raw.view(np.uint16)[~nz] & 0x7FFF == 0).all()


def test_sddmm_csr_typed_extremes_and_kd0(S, orc):
    # int8 extremes: -128 * -128 summed over a long row stays exact
    k, kd = 5000, 1024
    rp = np.array([0, 3, 3, 5000], np.int64)
    ci = np.concatenate([[0, 7, 4999], np.arange(4997)]).astype(np.int32)
    X = np.full((3, kd), -128, np.int8)
    Y = synth.int8_uniform(np.random.default_rng(27), (k, kd))
    Y[0] = -128
    got, ref, _, _ = sddmm_typed_case(S, orc, 3, k, rp, ci, X, Y, "i8", 1, 300)
    np.testing.assert_array_equal(got, ref)
    assert got[0] == 128 * 128 * kd
    # kd = 0: empty sums
    for elem in ("bf16", "i8"):
        Xe = np.zeros((3, 0), np.uint16 if elem == "bf16" else np.int8)
        Ye = np.zeros((k, 0), Xe.dtype)
        got, _, _, _ = sddmm_typed_case(S, orc, 3, k, rp, ci, Xe, Ye, elem, 16, 512)
        assert (got == 0).all()


@pytest.mark.parametrize("name", ["sddmm_bf16_powerlaw_1m", "sddmm_i8_powerlaw_1m"])
def test_sddmm_csr_typed_1m_sampled(S, orc, name):
    w = synth.WORKLOADS[name]
    a = synth.make_a(w)
    X, Y = synth.make_xy(w)
    lens = np.diff(a["row_ptr"])
    r = np.random.default_rng(28)
    rows = np.unique(np.concatenate([np.argsort(lens)[-100:], r.choice(w.m, 1000, replace=False),
                                     np.arange(20), np.arange(w.m - 20, w.m)])).astype(np.int64)
    got, ref, _, P = sddmm_typed_case(S, orc, w.m, w.k, a["row_ptr"], a["col_idx"], X, Y, w.elem,
                                      rows=rows)
    if w.elem == "bf16":
        err = orc.rel_frobenius(got, ref)
        _say(f"{name} rows={len(rows)} rel_frob={err:.3e}")
        assert err <= TOL_BF16
    else:
        np.testing.assert_array_equal(got, ref)
        _say(f"{name} rows={len(rows)} exact")


# ---------------------------------------------------------------------------
# SDDMM on a BCSR block pattern: bf16 -> bf16 and int8 -> int32
# ---------------------------------------------------------------------------

def sddmm_bcsr_case(S, orc, a_bits, X, Y, elem, blocks=None, extra=0):
    """Run the block-pattern SDDMM and return (got [nnzb, 64, 64], ref for
    `blocks` (all by default), plan).  X and Y go to the device as column
    slices with whole 16-byte rows plus `extra` padding columns."""
    torch = pytest.importorskip("torch")
    M = S.spmm_pack_bcsr(a_bits)
    kd = X.shape[1]
    P = S.spmm_plan_sddmm(M, kd, S.BF16 if elem == "bf16" else S.I8)
    rp, ci, _ = orc.pack_bcsr(a_bits, 64, 64)
    nnzb = len(ci)
    if elem == "bf16":
        out = torch.full((max(nnzb, 1), 64, 64), -1, dtype=torch.int16, device="cuda")   # 0xFFFF
        pad = (-kd) % 8 + extra
    else:
        out = torch.full((max(nnzb, 1), 64, 64), I32_SENTINEL, dtype=torch.int32, device="cuda")
        pad = (-kd) % 16 + extra
    S.spmm_execute_sddmm(P, to_dev(X, pad), to_dev(Y, pad), out)
    got = out.cpu().numpy()[:nnzb]
    if elem == "bf16":
        got = got.view(np.uint16)
        assert (got != 0xFFFF).all(), "some output element was not written"
    ref = orc.sddmm_bcsr(64, 64, rp, ci, X, Y, blocks=blocks)
    return got, ref, P


def _check_sddmm_bcsr(orc, got, ref, elem, blocks=None):
    g = got if blocks is None else got[blocks]
    if elem == "bf16":
        err = orc.rel_frobenius(bf16_to_f64(g), ref)
        assert err <= TOL_BF16, err
        return err
    np.testing.assert_array_equal(g, ref)
    return 0.0


@pytest.mark.parametrize("elem,kd", [("bf16", 8), ("bf16", 64), ("bf16", 1000), ("bf16", 4104),
                                     ("i8", 16), ("i8", 128), ("i8", 1000), ("i8", 8200)])
def test_sddmm_bcsr_small(S, orc, elem, kd):
    w = synth.SMALL["sddmm_bcsr_small"]       # 640 x 512, 24 of 80 blocks stored
    a = synth.make_a(w)["dense"]
    X, Y = synth.make_xy(w, kd, elem)
    got, ref, P = sddmm_bcsr_case(S, orc, a, X, Y, elem)
    err = _check_sddmm_bcsr(orc, got, ref, elem)
    _say(f"sddmm_bcsr_small {elem} kd={kd} grid={P.info()['grid']} "
         f"ws={P.info()['workspace_bytes']} rel_frob={err:.3e}")


@pytest.mark.parametrize("elem", ["bf16", "i8"])
def test_sddmm_bcsr_ld_kd0_and_repeat(S, orc, elem):
    w = synth.SMALL["sddmm_bcsr_small"]
    a = synth.make_a(w)["dense"]
    X, Y = synth.make_xy(w, 200, elem)
    g1, ref, _ = sddmm_bcsr_case(S, orc, a, X, Y, elem, extra=32)      # ld > kd
    _check_sddmm_bcsr(orc, g1, ref, elem)
    g2, _, _ = sddmm_bcsr_case(S, orc, a, X, Y, elem)
    np.testing.assert_array_equal(g1, g2)                              # bitwise repeatable
    gz, _, _ = sddmm_bcsr_case(S, orc, a, X[:, :0].copy(), Y[:, :0].copy(), elem)
    assert (gz & (0x7FFF if elem == "bf16" else -1) == 0).all()        # kd = 0: zeros


def test_sddmm_bcsr_dense_row_and_empty(S, orc):
    # one block row stored in full (8 blocks: two groups of four), the rest
    # empty; and an all-zero pattern, which has nothing to compute
    torch = pytest.importorskip("torch")
    a = np.zeros((256, 512), np.uint16)
    a[64:128, :] = 0x3F80
    X = synth.dense_bf16_normal(256, 320, 91)
    Y = synth.dense_bf16_normal(512, 320, 92)
    got, ref, _ = sddmm_bcsr_case(S, orc, a, X, Y, "bf16")
    assert got.shape == (8, 64, 64)
    _check_sddmm_bcsr(orc, got, ref, "bf16")
    M = S.spmm_pack_bcsr(np.zeros((128, 128), np.uint16))
    P = S.spmm_plan_sddmm(M, 64, S.BF16)
    out = torch.zeros(16, dtype=torch.int16, device="cuda")
    S.spmm_execute_sddmm(P, to_dev(X[:128, :64]), to_dev(Y[:128, :64]), out)


@pytest.mark.parametrize("name", ["sddmm_bcsr_prefill_kd8192", "sddmm_i8_prefill_kd8192"])
def test_sddmm_bcsr_prefill_sampled(S, orc, name):
    w = synth.WORKLOADS[name]
    a = synth.make_a(w)["dense"]
    X, Y = synth.make_xy(w)
    nnzb = w.nblocks
    r = np.random.default_rng(21)
    blocks = np.unique(np.concatenate([[0, nnzb - 1], r.choice(nnzb, 14, replace=False)])).astype(np.int64)
    got, ref, P = sddmm_bcsr_case(S, orc, a, X, Y, w.elem, blocks=blocks)
    err = _check_sddmm_bcsr(orc, got, ref, w.elem, blocks)
    _say(f"{name} blocks={len(blocks)} grid={P.info()['grid']} ws={P.info()['workspace_bytes']} "
         f"rel_frob={err:.3e}")


# ---------------------------------------------------------------------------
# BCSR of a CSR matrix after the row/column reordering
# ---------------------------------------------------------------------------

def _reordered_case(S, orc, w, rows=None):
    a = synth.make_a(w)
    B = synth.make_b(w)
    M = S.spmm_pack_bcsr_csr(w.m, w.k, a["row_ptr"], a["col_idx"], a["vals_bf16"],
                             reorder=w.reorder)
    P = S.spmm_plan(M, w.n, S.BF16, S.BF16)
    got = run(S, P, B, w.m, w.n, "bf16")
    assert (got != 0xFFFF).all(), "some C element was not written"
    ref = orc.csr_spmm(a["row_ptr"], a["col_idx"], a["vals"], synth.bf16_bits_to_f32(B), rows=rows)
    g = got if rows is None else got[rows]
    return orc.rel_frobenius(bf16_to_f64(g), ref), M, P


def test_reordered_bcsr_many_blocks_per_row(S, orc):
    # 24 of 32 blocks per block row: the reordering still pays (the scrambled
    # pattern touches nearly every block) and the rows stay long, so the
    # kernel reads B through the row map with whole-block stages at 256
    # columns
    w = synth.Workload("scrambled_dense_rows", "bcsr_csr", 512, 2048, 264, 90, nblocks=192,
                       scramble=91, reorder=True)
    err, M, P = _reordered_case(S, orc, w)
    info = S.spmm_matrix_info(M)
    _say(f"reordered dense rows: blocks={info['nnzb']} tile_n={P.info()['tile_n']} rel_frob={err:.3e}")
    assert S.spmm_matrix_array(M, S.ARRAY_COL_PERM).size == w.k
    assert 192 <= info["nnzb"] < 256 and info["nnzb"] > 16 * (w.m // 64)
    assert P.info()["tile_n"] == 256
    assert err <= TOL_BF16


@pytest.mark.parametrize("reorder", [True, False])
def test_reordered_bcsr_small(S, orc, reorder):
    import dataclasses
    w = dataclasses.replace(synth.SMALL["scrambled_small"], reorder=reorder)   # 1024 x 768, n = 520
    err, M, P = _reordered_case(S, orc, w)
    info = S.spmm_matrix_info(M)
    _say(f"scrambled_small reorder={reorder} nnzb={info['nnzb']} ws={P.info()['workspace_bytes']} "
         f"rel_frob={err:.3e}")
    assert err <= TOL_BF16
    assert P.info()["workspace_bytes"] == 0      # B is read through the permutation
    if reorder:
        assert info["nnzb"] == w.nblocks          # the hidden blocks, found again
        assert len(S.spmm_matrix_array(M, S.ARRAY_ROW_PERM)) == w.m


def test_reordered_bcsr_wide_n(S, orc):
    # n >= 8192 takes the 512-column tiles; a ragged last tile
    import dataclasses
    w = dataclasses.replace(synth.SMALL["scrambled_small"], n=8192 + 72)
    r = np.random.default_rng(25)
    rows = np.unique(np.concatenate([np.arange(8), r.choice(w.m, 40, replace=False)])).astype(np.int64)
    err, M, P = _reordered_case(S, orc, w, rows=rows)
    _say(f"scrambled_small n={w.n} tile_n={P.info()['tile_n']} rel_frob={err:.3e}")
    assert P.info()["tile_n"] == 512
    assert err <= TOL_BF16


def test_reordered_bcsr_4096_sampled(S, orc):
    w = synth.WORKLOADS["scrambled_4096_bcsr_reordered"]
    r = np.random.default_rng(22)
    rows = np.unique(np.concatenate([np.arange(32), r.choice(w.m, 200, replace=False)])).astype(np.int64)
    err, M, _ = _reordered_case(S, orc, w, rows=rows)
    _say(f"scrambled_4096 nnzb={S.spmm_matrix_info(M)['nnzb']} rel_frob={err:.3e}")
    assert err <= TOL_BF16
    assert S.spmm_matrix_info(M)["nnzb"] == w.nblocks


def test_reordered_pattern_has_no_sddmm(S, orc):
    w = synth.SMALL["scrambled_small"]
    a = synth.make_a(w)
    M = S.spmm_pack_bcsr_csr(w.m, w.k, a["row_ptr"], a["col_idx"], a["vals_bf16"], reorder=True)
    with pytest.raises(S.SpmmError) as ei:
        S.spmm_plan_sddmm(M, 64, S.BF16)
    assert ei.value.name == "SPMM_ERR_UNSUPPORTED"


# ---------------------------------------------------------------------------
# tile-vector-wise int8: the 2:4 kernel walking only the stored tiles
# ---------------------------------------------------------------------------

def tvw_case(S, orc, a, B, rows=None, pad=0):
    m, n = a.shape[0], B.shape[1]
    M = S.spmm_pack_tvw(a, 256, 128)
    P = S.spmm_plan(M, n, S.I8, S.I32)
    got = run(S, P, B, m, n, "i32", pad)
    assert_all_written(got, "i32")
    v, mt = orc.pack24(a)
    ref = orc.sp24_spmm(v, mt, B, rows=rows)
    np.testing.assert_array_equal(got if rows is None else got[rows], ref)
    return M


def test_tvw_small(S, orc):
    w = synth.SMALL["tvw_small"]        # 512 x 1024, 6 of 16 tiles stored, n = 272
    a = synth.make_a(w)["dense"]
    B = synth.make_b(w)
    for pad in (0, 16):
        M = tvw_case(S, orc, a, B, pad=pad)
    assert S.spmm_matrix_info(M)["nnzb"] == w.nblocks


def test_tvw_empty_rows_full_rows_and_extremes(S, orc):
    # tile row 0 empty, tile row 1 full, tile row 2 a single tile of -128s
    a = np.zeros((768, 512), np.int8)
    a[256:512] = synth.int8_uniform(np.random.default_rng(4), (256, 512))
    a[512:768, 128:256] = -128
    B = np.full((512, 64), -128, np.int8)
    B[:, 32:] = synth.int8_uniform(np.random.default_rng(5), (512, 32))
    tvw_case(S, orc, a, B)
    # no stored tile at all: C is zero
    Z = np.zeros((256, 256), np.int8)
    M = S.spmm_pack_tvw(Z, 256, 128)
    P = S.spmm_plan(M, 32, S.I8, S.I32)
    got = run(S, P, synth.int8_uniform(np.random.default_rng(6), (256, 32)), 256, 32, "i32")
    assert (got == 0).all()


def test_tvw_unsupported_tile(S, orc):
    M = S.spmm_pack_tvw(np.ones((128, 128), np.int8), 64, 64)
    with pytest.raises(S.SpmmError) as ei:
        S.spmm_plan(M, 32, S.I8, S.I32)
    assert ei.value.name == "SPMM_ERR_UNSUPPORTED"


@pytest.mark.parametrize("name", ["tvw_i8_8192_t50", "tvw_i8_8192_t75"])
def test_tvw_8192_sampled(S, orc, name):
    w = synth.WORKLOADS[name]
    a = synth.make_a(w)["dense"]
    B = synth.make_b(w)
    r = np.random.default_rng(23)
    rows = np.unique(np.concatenate([np.arange(16), np.arange(w.m - 16, w.m),
                                     r.choice(w.m, 96, replace=False)])).astype(np.int64)
    M = tvw_case(S, orc, a, B, rows=rows)
    _say(f"{name} tiles={S.spmm_matrix_info(M)['nnzb']} rows={len(rows)} exact")


def test_tvw_i8_wide_tiles(S, orc):
    # 256 x 256 tiles: each stored tile is two consecutive k-steps of the kernel
    a = synth.tile_sparse_i8(768, 1024, 256, 256, 5, 41)
    B = synth.int8_uniform(np.random.default_rng(42), (1024, 144))
    M = S.spmm_pack_tvw(a, 256, 256)
    P = S.spmm_plan(M, 144, S.I8, S.I32)
    got = run(S, P, B, 768, 144, "i32")
    v, mt = orc.pack24(a)
    np.testing.assert_array_equal(got, orc.sp24_spmm(v, mt, B))


# ---------------------------------------------------------------------------
# tile-vector-wise bf16: the 2:4 kernel on the bf16 sparse MFMA
# ---------------------------------------------------------------------------

def tvw_bf16_case(S, orc, a_bits, B_bits, tk=128, rows=None, pad=0):
    """GPU result (uint16 bits) and the oracle's fp64 product of the 2:4-pruned
    A (its pruning, then its BCSR product over tiles of 256 x tk)."""
    m, n = a_bits.shape[0], B_bits.shape[1]
    M = S.spmm_pack_tvw(a_bits, 256, tk)
    P = S.spmm_plan(M, n, S.BF16, S.BF16)
    got = run(S, P, B_bits, m, n, "bf16", pad)
    assert_all_written(got, "bf16")
    pruned = orc.prune_nm(a_bits, 2, 4)
    rp, ci, v = orc.pack_bcsr(pruned, 256, tk)
    ref = orc.bcsr_spmm(256, tk, rp, ci, v, B_bits, rows=rows)
    g = bf16_to_f64(got if rows is None else got[rows])
    assert np.isfinite(g).all(), "unwritten or non-finite outputs"
    return g, ref, got, M


@pytest.mark.parametrize("tk", [128, 64])
def test_tvw_bf16_small(S, orc, tk):
    w = synth.SMALL["tvw_bf16_small"]   # 512 x 1024, 6 of 16 tiles of 256 x 128, n = 272
    a = synth.make_a(w)["dense"]
    B = synth.make_b(w)
    for pad in (0, 16):
        g, ref, _, M = tvw_bf16_case(S, orc, a, B, tk=tk, pad=pad)
        err = orc.rel_frobenius(g, ref)
        assert err <= TOL_BF16, err
    _say(f"tvw_bf16_small tk={tk} tiles={S.spmm_matrix_info(M)['nnzb']} rel={err:.2e}")


def test_tvw_bf16_integer_values_are_exact(S, orc):
    # small integers: every fp32 partial sum is exact, so C must be exactly
    # the round-to-nearest-even bf16 of the exact sum; pins the index words,
    # the k order of B and the epilogue bit for bit
    r = np.random.default_rng(43)
    m, k, n = 768, 512, 336
    a = r.integers(-3, 4, size=(m, k)).astype(np.float32)
    a[0:256, 128:384] = 0                       # tile row 0: two zero tiles
    a[512:768] = 0
    a[600, 77] = -2.0                           # tile row 2: one tile, one entry
    a_bits = synth.f32_to_bf16_bits(a)
    B = synth.f32_to_bf16_bits(r.integers(-4, 5, size=(k, n)).astype(np.float32))
    _, ref, got, M = tvw_bf16_case(S, orc, a_bits, B)
    assert np.abs(ref).max() < 2 ** 24
    np.testing.assert_array_equal(got & 0x7FFF, synth.f32_to_bf16_bits(ref.astype(np.float32)) & 0x7FFF)
    nz = ref != 0
    np.testing.assert_array_equal(got[nz], synth.f32_to_bf16_bits(ref[nz].astype(np.float32)))
    assert S.spmm_matrix_info(M)["nnzb"] == 4 + 2 + 1


def test_tvw_bf16_identity_and_no_tiles(S, orc):
    m = 512
    eye = synth.f32_to_bf16_bits(np.eye(m, dtype=np.float32))   # one nonzero per group: kept
    B = synth.dense_bf16_normal(m, 272, 44)
    _, _, got, _ = tvw_bf16_case(S, orc, eye, B, tk=64)
    np.testing.assert_array_equal(got, B)
    Z = np.zeros((256, 256), np.uint16)
    M = S.spmm_pack_tvw(Z, 256, 128)
    P = S.spmm_plan(M, 32, S.BF16, S.BF16)
    got = run(S, P, synth.dense_bf16_normal(256, 32, 45), 256, 32, "bf16")
    assert (got & 0x7FFF == 0).all()


def test_tvw_bf16_plan_checks(S, orc):
    a = synth.f32_to_bf16_bits(np.ones((256, 96), np.float32))
    M = S.spmm_pack_tvw(a, 256, 96)              # 96 is not a multiple of the k-step
    with pytest.raises(S.SpmmError) as ei:
        S.spmm_plan(M, 32, S.BF16, S.BF16)
    assert ei.value.name == "SPMM_ERR_UNSUPPORTED"
    M = S.spmm_pack_tvw(synth.f32_to_bf16_bits(np.ones((256, 128), np.float32)), 256, 128)
    for types in ((S.I8, S.I32), (S.BF16, S.F32)):
        with pytest.raises(S.SpmmError) as ei:
            S.spmm_plan(M, 32, *types)
        assert ei.value.name == "SPMM_ERR_UNSUPPORTED"


@pytest.mark.parametrize("name", ["tvw_bf16_8192_t50", "tvw_bf16_8192_t75"])
def test_tvw_bf16_8192_sampled(S, orc, name):
    w = synth.WORKLOADS[name]
    a = synth.make_a(w)["dense"]
    B = synth.make_b(w)
    r = np.random.default_rng(24)
    rows = np.unique(np.concatenate([np.arange(16), np.arange(w.m - 16, w.m),
                                     r.choice(w.m, 64, replace=False)])).astype(np.int64)
    g, ref, _, M = tvw_bf16_case(S, orc, a, B, rows=rows)
    err = orc.rel_frobenius(g, ref)
    assert err <= TOL_BF16, err
    _say(f"{name} tiles={S.spmm_matrix_info(M)['nnzb']} rows={len(rows)} rel={err:.2e}")


# ---------------------------------------------------------------------------
# (2N-2):2N weights as overlapping 2:4 windows, on the 2:4 kernel
# ---------------------------------------------------------------------------

def slide_case(S, orc, a, B, group, rows=None, pad=0):
    m, n = a.shape[0], B.shape[1]
    M = S.spmm_pack_slide(a, group)
    P = S.spmm_plan(M, n, S.I8, S.I32)
    got = run(S, P, B, m, n, "i32", pad)
    assert_all_written(got, "i32")
    pruned = orc.prune_nm(a, group - 2, group)
    ref = orc.gemm_i8(pruned if rows is None else pruned[rows], B)
    g = got if rows is None else got[rows]
    np.testing.assert_array_equal(g.astype(np.int64), ref)
    return P


@pytest.mark.parametrize("group", [8, 6, 16, 4])
def test_slide_small(S, orc, group):
    w = synth.SMALL["slide_small"]       # 320 x 512 (k = 528 for 6 and 16), n = 400
    k = w.k if (w.k // group * 4 * (group // 2 - 1)) % 8 == 0 and w.k % group == 0 else 528
    a = synth.int8_uniform(np.random.default_rng(40 + group), (w.m, k))
    B = synth.int8_uniform(np.random.default_rng(41 + group), (k, w.n))
    for pad in (0, 16):
        P = slide_case(S, orc, a, B, group, pad=pad)
    _say(f"slide {group - 2}:{group} ws={P.info()['workspace_bytes']} exact")


def test_slide_extremes(S, orc):
    # all -128: every kept product is 16384, a row sums 6/8 of k of them
    k = 4096
    a = np.full((256, k), -128, np.int8)
    B = np.full((k, 32), -128, np.int8)
    slide_case(S, orc, a, B, 8)


def test_slide68_8192_sampled(S, orc):
    w = synth.WORKLOADS["slide68_i8_8192"]
    a = synth.make_a(w)["dense"]
    B = synth.make_b(w)
    r = np.random.default_rng(24)
    rows = np.unique(np.concatenate([np.arange(8), r.choice(w.m, 56, replace=False)])).astype(np.int64)
    slide_case(S, orc, a, B, w.nm_group, rows=rows)

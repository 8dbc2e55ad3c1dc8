"""spmm_execute_noalloc, the entry point that allocates nothing, against
spmm_execute on the same plans.

The two run the same kernels; the no-allocation call keeps a WCSR plan's
partial rows (rows split across chunks, the AsyncSparse page's row-window
splitting) in the library's fixed per-GPU scratch array instead of the
plan's workspace.  C must be bit-identical to spmm_execute's and within the
fp32 tolerance of the oracle, on two calls in a row, the second one on a
smaller input, so partial rows left in the array by the first call would
show in the second."""
import numpy as np
import pytest

import synth
from gpu_helpers import TOL_F32, assert_all_written, empty_out, from_dev, run, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def S():
    import sparse_dense_matrix_amd as S
    import torch
    assert torch.cuda.is_available()
    return S


def _wcsr_both(S, orc, w, W, T, n):
    a = synth.make_a(w)
    B = synth.dense_f32_normal(w.k, n, 95)
    M = S.spmm_pack_wcsr(w.m, w.k, a["row_ptr"], a["col_idx"], a["vals"], W, T)
    P = S.spmm_plan(M, n, S.F32, S.F32)
    info = P.info()
    assert info["num_slots"] > 0, "the case must split rows"
    pad = (-n) % 4
    want = run(S, P, B, w.m, n, "f32", pad)
    Bt = to_dev(B, pad)
    Ct = empty_out(w.m, n, "f32", pad)
    S.spmm_execute_noalloc(P, Bt, Ct)
    got = from_dev(Ct, "f32")
    assert_all_written(got, "f32")
    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))
    ref = orc.csr_spmm(a["row_ptr"], a["col_idx"], a["vals"], B)
    err = orc.rel_frobenius(got, ref)
    print(f"noalloc {w.name} W={W} T={T} n={n} slots={info['num_slots']} "
          f"scratch={info['num_slots'] * n * 4} B rel_frob={err:.3e}", flush=True)
    assert err <= TOL_F32


def test_noalloc_wcsr_two_calls_second_smaller(S, orc):
    # first call: many split rows at n = 128; second: fewer slots, ragged n
    _wcsr_both(S, orc, synth.SMALL["csr_powerlaw_small"], 16, 64, 128)
    _wcsr_both(S, orc, synth.SMALL["csr_uniform_small"], 3, 7, 65)


def test_noalloc_other_formats_match(S, orc):
    # formats without partial rows: the same call as spmm_execute
    w = synth.SMALL["bcsr_small"]
    a, B = synth.make_a(w)["dense"], synth.make_b(w)
    P = S.spmm_plan(S.spmm_pack_bcsr(a), w.n, S.BF16, S.BF16)
    want = run(S, P, B, w.m, w.n, "bf16")
    Ct = empty_out(w.m, w.n, "bf16")
    S.spmm_execute_noalloc(P, to_dev(B), Ct)
    np.testing.assert_array_equal(from_dev(Ct, "bf16"), want)


def test_noalloc_rejects_plans_beyond_the_scratch(S, orc):
    # 1000 rows of 100 entries, one row per window, one entry per chunk:
    # 100,000 partial rows of 128 fp32 = 51 MB, above the 32 MiB array
    m, k, n = 1000, 4096, 128
    r = np.random.default_rng(96)
    rp = np.arange(0, 100 * (m + 1), 100, dtype=np.int64)
    ci = np.concatenate([np.sort(r.choice(k, 100, replace=False)) for _ in range(m)]).astype(np.int32)
    v = r.uniform(-1, 1, len(ci)).astype(np.float32)
    P = S.spmm_plan(S.spmm_pack_wcsr(m, k, rp, ci, v, 1, 1), n, S.F32, S.F32)
    assert P.info()["num_slots"] * n * 4 > 32 << 20
    Bt = to_dev(synth.dense_f32_normal(k, n, 97))
    Ct = empty_out(m, n, "f32")
    with pytest.raises(S.SpmmError) as ei:
        S.spmm_execute_noalloc(P, Bt, Ct)
    assert ei.value.name == "SPMM_ERR_UNSUPPORTED"
    assert "scratch" in ei.value.message

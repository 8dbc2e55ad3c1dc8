"""Out-of-memory handling of spmm_plan / spmm_plan_sddmm on the GPU.

With SPMM_TEST_FAIL_ALLOC = n the n-th host or device allocation of the call
fails.  Walking n = 1, 2, ... until a plan is made, every failing call must
return SPMM_ERR_OUT_OF_MEMORY with *out NULL, and the device memory it had
taken must all be returned (free device memory is back where it started).
The successful plan must still give the oracle's result (C = A * B, the
AsyncSparse page's product)."""
import ctypes
import os

import numpy as np
import pytest

import synth
from gpu_helpers import TOL_BF16, TOL_F32, bf16_to_f64, run

pytestmark = pytest.mark.gpu
OOM = 3


@pytest.fixture(scope="module")
def S():
    import sparse_dense_matrix_amd as S
    import torch
    assert torch.cuda.is_available()
    return S


def walk_plan(S, call, limit=200):
    import torch
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    n = 0
    try:
        while True:
            n += 1
            assert n < limit, "no successful plan"
            os.environ["SPMM_TEST_FAIL_ALLOC"] = str(n)
            out = ctypes.c_void_p(0xDEAD)
            st = call(ctypes.byref(out))
            if st == 0:
                break
            assert st == OOM, (n, S.spmm_status_str(st), S.spmm_last_error())
            assert out.value is None, f"allocation {n}: *out not NULL on failure"
            torch.cuda.synchronize()
            free = torch.cuda.mem_get_info()[0]
            assert free >= free0 - (2 << 20), f"allocation {n}: {free0 - free} device bytes kept"
    finally:
        os.environ.pop("SPMM_TEST_FAIL_ALLOC", None)
    print(f"plan: {n - 1} allocation points failed cleanly", flush=True)
    assert n - 1 >= 3
    return S.Plan(out)


def test_plan_oom_bcsr_wcsr_24(S, orc):
    # warm the runtime (code objects, kernel attributes) before measuring
    w = synth.SMALL["bcsr_small"]
    a, B = synth.make_a(w)["dense"], synth.make_b(w)
    M = S.spmm_pack_bcsr(a)
    S.spmm_plan(M, w.n, S.BF16, S.BF16)
    P = walk_plan(S, lambda o: S._lib.spmm_plan(M.handle, w.n, S.BF16, S.BF16, 0, o))
    rp, ci, v = orc.pack_bcsr(a, 64, 64)
    got = run(S, P, B, w.m, w.n, "bf16")
    assert orc.rel_frobenius(bf16_to_f64(got), orc.bcsr_spmm(64, 64, rp, ci, v, B)) <= TOL_BF16

    w = synth.SMALL["csr_powerlaw_small"]
    x, B = synth.make_a(w), synth.make_b(w)
    M = S.spmm_pack_wcsr(w.m, w.k, x["row_ptr"], x["col_idx"], x["vals"], 16, 64)
    P = walk_plan(S, lambda o: S._lib.spmm_plan(M.handle, w.n, S.F32, S.F32, 0, o))
    assert P.info()["workspace_bytes"] > 0
    got = run(S, P, B, w.m, w.n, "f32")
    assert orc.rel_frobenius(got, orc.csr_spmm(x["row_ptr"], x["col_idx"], x["vals"], B)) <= TOL_F32

    w = synth.SMALL["sp24_small"]
    a, B = synth.make_a(w)["dense"], synth.make_b(w)
    M = S.spmm_pack_24(a)
    P = walk_plan(S, lambda o: S._lib.spmm_plan(M.handle, w.n, S.I8, S.I32, 0, o))
    vals, meta = orc.pack24(a)
    np.testing.assert_array_equal(run(S, P, B, w.m, w.n, "i32"), orc.sp24_spmm(vals, meta, B))


def test_plan_sddmm_oom(S, orc):
    w = synth.SMALL["bcsr_small"]
    a = synth.make_a(w)["dense"]
    M = S.spmm_pack_bcsr(a)
    S.spmm_plan_sddmm(M, 4096, S.BF16)
    P = walk_plan(S, lambda o: S._lib.spmm_plan_sddmm(M.handle, 4096, S.BF16, 0, o))
    assert P.info()["grid"] > 0

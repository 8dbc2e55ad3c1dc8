"""HIP graph capture of the execute calls (GPU).

Each execute path is only kernel launches on the caller's stream (no
allocation, copy, memset or synchronisation), so it can be recorded into a
HIP graph and replayed.  Every format is captured once, then replayed three
times with eager work (clearing the output) and a synchronisation between
replays, and every replay must reproduce the eager result bit for bit (the
kernels are deterministic)."""
import numpy as np
import pytest

import synth
from gpu_helpers import to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def S():
    import sparse_dense_matrix_amd as S
    import torch
    assert torch.cuda.is_available()
    return S


def _graph_case(fn, out):
    """fn(stream) launches into `out`; compare 3 graph replays with eager."""
    import torch
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        fn(s)
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fn(torch.cuda.current_stream())
    torch.cuda.synchronize()
    for rep in range(3):
        out.zero_()                     # eager work between replays
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs from the eager result"
    return eager


def _spmm_case(S, M, types, B, m, n, cdt):
    import torch
    P = S.spmm_plan(M, n, *types)
    Bt = to_dev(B)
    Ct = torch.empty((m, n), dtype=cdt, device="cuda")
    eager = _graph_case(lambda st: S.spmm_execute(P, Bt, Ct, stream=st), Ct)
    assert eager.abs().sum().item() > 0


def test_graph_bcsr_and_reordered(S):
    import torch
    w = synth.SMALL["bcsr_small"]
    _spmm_case(S, S.spmm_pack_bcsr(synth.make_a(w)["dense"]), (S.BF16, S.BF16), synth.make_b(w),
               w.m, w.n, torch.int16)
    w = synth.SMALL["scrambled_small"]
    a = synth.make_a(w)
    M = S.spmm_pack_bcsr_csr(w.m, w.k, a["row_ptr"], a["col_idx"], a["vals_bf16"], reorder=True)
    _spmm_case(S, M, (S.BF16, S.BF16), synth.make_b(w), w.m, w.n, torch.int16)


def test_graph_bcsr_paired_rows(S):
    # the prefill layer's block pattern at n = 4288: two block rows per tile
    import torch
    w = synth.SMALL["bcsr_prefill_slice"]
    M = S.spmm_pack_bcsr(synth.make_a(w)["dense"])
    assert S.spmm_plan(M, w.n, S.BF16, S.BF16).info()["tile_m"] == 128
    _spmm_case(S, M, (S.BF16, S.BF16), synth.make_b(w), w.m, w.n, torch.int16)


def test_graph_wcsr_with_split_rows(S):
    import torch
    w = synth.SMALL["csr_powerlaw_small"]
    a = synth.make_a(w)
    M = S.spmm_pack_wcsr(w.m, w.k, a["row_ptr"], a["col_idx"], a["vals"], 16, 256)
    _spmm_case(S, M, (S.F32, S.F32), synth.make_b(w), w.m, w.n, torch.float32)


def test_graph_24_tvw_and_slide(S):
    import torch
    w = synth.SMALL["sp24_small"]
    _spmm_case(S, S.spmm_pack_24(synth.make_a(w)["dense"]), (S.I8, S.I32), synth.make_b(w),
               w.m, w.n, torch.int32)
    w = synth.SMALL["sp24_bf16_small"]
    _spmm_case(S, S.spmm_pack_24(synth.make_a(w)["dense"]), (S.BF16, S.BF16), synth.make_b(w),
               w.m, w.n, torch.int16)
    w = synth.SMALL["tvw_bf16_small"]
    _spmm_case(S, S.spmm_pack_tvw(synth.make_a(w)["dense"], 256, 128), (S.BF16, S.BF16),
               synth.make_b(w), w.m, w.n, torch.int16)
    w = synth.SMALL["slide_small"]
    _spmm_case(S, S.spmm_pack_slide(synth.make_a(w)["dense"], w.nm_group), (S.I8, S.I32),
               synth.make_b(w), w.m, w.n, torch.int32)


def test_graph_sddmm(S):
    import torch
    w = synth.SMALL["sddmm_small"]
    a = synth.make_a(w)
    M = S.spmm_pack_wcsr(w.m, w.k, a["row_ptr"], a["col_idx"], a["vals"], 0, 0)
    P = S.spmm_plan_sddmm(M, w.n)
    X, Y = synth.make_xy(w)
    Xt, Yt = to_dev(X), to_dev(Y)
    out = torch.empty(S.spmm_matrix_info(M)["nnz"], dtype=torch.float32, device="cuda")
    _graph_case(lambda st: S.spmm_execute_sddmm(P, Xt, Yt, out, stream=st), out)
    w = synth.SMALL["sddmm_bcsr_small"]
    M = S.spmm_pack_bcsr(synth.make_a(w)["dense"], 64, 64)
    P = S.spmm_plan_sddmm(M, 4096, S.BF16)            # long enough to split into ranges
    X = synth.dense_bf16_normal(w.m, 4096, 81)
    Y = synth.dense_bf16_normal(w.k, 4096, 82)
    out = torch.empty((S.spmm_matrix_info(M)["nnzb"], 64, 64), dtype=torch.int16, device="cuda")
    Xt, Yt = to_dev(X), to_dev(Y)
    _graph_case(lambda st: S.spmm_execute_sddmm(P, Xt, Yt, out, stream=st), out)
    assert P.info()["workspace_bytes"] > 0             # the range-merge path is in the graph

"""SPMM_LOG: with the variable set (anything but empty or "0"), every plan
that succeeds prints one line of its decisions on stderr; unset or "0", the
library prints nothing.  The line must agree with spmm_plan_info."""
import contextlib
import os
import sys
import tempfile

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def S():
    import sparse_dense_matrix_amd as S
    import torch
    assert torch.cuda.is_available()
    return S


@contextlib.contextmanager
def log_env(value):
    old = os.environ.get("SPMM_LOG")
    if value is None:
        os.environ.pop("SPMM_LOG", None)
    else:
        os.environ["SPMM_LOG"] = value
    try:
        yield
    finally:
        if old is None:
            os.environ.pop("SPMM_LOG", None)
        else:
            os.environ["SPMM_LOG"] = old


def stderr_of(fn, value="1"):
    """Run fn with SPMM_LOG=value; return (its result, what file descriptor 2 received)."""
    sys.stderr.flush()
    saved = os.dup(2)
    with tempfile.TemporaryFile() as f:
        os.dup2(f.fileno(), 2)
        try:
            with log_env(value):
                out = fn()
        finally:
            os.dup2(saved, 2)
            os.close(saved)
        f.seek(0)
        text = f.read().decode()
    return out, text


def the_line(text, fn):
    lines = [ln for ln in text.splitlines() if ln.startswith(f"[spmm] {fn}:")]
    assert len(lines) == 1, text
    return lines[0]


def fields(line):
    return dict(tok.split("=", 1) for tok in line.split() if "=" in tok)


def test_bcsr_plans_name_their_kernel(S):
    for name, kernel in (("bcsr_small", None), ("bcsr_prefill_slice", "bcsr_bf16_pair")):
        w = synth.SMALL[name]
        M = S.spmm_pack_bcsr(synth.make_a(w)["dense"])
        P, text = stderr_of(lambda: S.spmm_plan(M, w.n, S.BF16, S.BF16))
        info = P.info()
        f = fields(the_line(text, "spmm_plan"))
        want = "bcsr_bf16_pair" if info["tile_m"] == 128 else "bcsr_bf16_mfma"
        if kernel:
            assert want == kernel
        assert f["format"] == "bcsr" and f["kernel"] == want
        assert (f["m"], f["k"], f["n"]) == (str(w.m), str(w.k), str(w.n))
        assert f["tile"] == f"{info['tile_m']}x{info['tile_n']}" and f["grid"] == str(info["grid"])
        assert f["device_bytes"] == str(info["device_bytes"]) and f["workspace_bytes"] == "0"


def test_wcsr_and_sp24_and_sddmm_plans(S):
    w = synth.SMALL["csr_powerlaw_small"]
    a = synth.make_a(w)
    M = S.spmm_pack_wcsr(w.m, w.k, a["row_ptr"], a["col_idx"], a["vals"], 16, 64)
    P, text = stderr_of(lambda: S.spmm_plan(M, w.n, S.F32, S.F32))
    info = P.info()
    f = fields(the_line(text, "spmm_plan"))
    assert info["num_split_rows"] > 0, "the case should split rows"
    assert f["format"] == "wcsr" and f["kernel"] == "wcsr_stream+wcsr_merge"
    assert f["window_rows"] == "16" and f["max_chunk_nnz"] == "64"
    assert f["split_rows"] == str(info["num_split_rows"]) and f["slots"] == str(info["num_slots"])
    assert f["workspace_bytes"] == str(info["workspace_bytes"])

    Q, text = stderr_of(lambda: S.spmm_plan_sddmm(M, 32))
    f = fields(the_line(text, "spmm_plan_sddmm"))
    assert f["format"] == "wcsr" and f["kernel"] == "sddmm_csr" and f["n"] == "32"

    w = synth.SMALL["sp24_small"]
    M = S.spmm_pack_24(synth.make_a(w)["dense"])
    P, text = stderr_of(lambda: S.spmm_plan(M, w.n, S.I8, S.I32))
    f = fields(the_line(text, "spmm_plan"))
    assert f["format"] == "24" and f["kernel"] == "sp24_i8_smfmac"
    assert int(f["k_pad"]) % 128 == 0 and int(f["k_pad"]) >= w.k


@pytest.mark.parametrize("value", [None, "0", ""])
def test_quiet_unless_set(S, value):
    w = synth.SMALL["bcsr_small"]
    M = S.spmm_pack_bcsr(synth.make_a(w)["dense"])
    _, text = stderr_of(lambda: S.spmm_plan(M, w.n, S.BF16, S.BF16), value)
    assert "[spmm]" not in text

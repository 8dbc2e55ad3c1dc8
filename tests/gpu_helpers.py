"""Helpers for the GPU tests: run the library through its C ABI on torch
device memory, and compare with the oracle."""
import numpy as np

# tolerances: relative Frobenius error of the fp32 and the bf16-in /
# fp32-accumulate / bf16-out paths; int8 is compared bit for bit
TOL_F32 = 1e-5
TOL_BF16 = 2e-3


def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    return torch


def to_dev(x: np.ndarray, pad_cols: int = 0):
    """Host array -> device tensor (bf16 bits travel as int16).  With pad_cols
    the tensor is a column slice of a wider allocation (ld > n)."""
    torch = torch_dev()
    x = np.ascontiguousarray(x)
    view = {np.dtype(np.uint16): np.int16}.get(x.dtype, None)
    host = x.view(view) if view is not None else x
    t = torch.from_numpy(host)
    if pad_cols:
        wide = torch.zeros((x.shape[0], x.shape[1] + pad_cols), dtype=t.dtype)
        wide[:, : x.shape[1]] = t
        return wide.cuda()[:, : x.shape[1]]
    return t.cuda()


def empty_out(m: int, n: int, kind: str, pad_cols: int = 0):
    """Output buffer pre-filled with a sentinel no result can take."""
    torch = torch_dev()
    dt = {"bf16": torch.int16, "f32": torch.float32, "i32": torch.int32}[kind]
    fill = {"bf16": -1, "f32": float("nan"), "i32": -(2 ** 31)}[kind]
    t = torch.full((m, n + pad_cols), fill, dtype=dt, device="cuda")
    return t[:, :n] if pad_cols else t


def from_dev(t, kind: str) -> np.ndarray:
    torch = torch_dev()
    torch.cuda.synchronize()
    a = t.cpu().numpy()
    return a.view(np.uint16) if kind == "bf16" else a


def run(S, plan, B: np.ndarray, m: int, n: int, kind: str, pad: int = 0):
    Bt = to_dev(B, pad)
    Ct = empty_out(m, n, kind, pad)
    S.spmm_execute(plan, Bt, Ct)
    return from_dev(Ct, kind)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def assert_all_written(got: np.ndarray, kind: str):
    """Every element of C was written: none still holds empty_out's sentinel
    (bf16 0xFFFF is a NaN, fp32 NaN, int32 -2^31; no finite product of the
    tested inputs takes them)."""
    if kind == "bf16":
        bad = int(np.count_nonzero(np.asarray(got).view(np.uint16) == 0xFFFF))
    elif kind == "f32":
        bad = int(np.count_nonzero(~np.isfinite(got)))
    else:
        bad = int(np.count_nonzero(np.asarray(got) == -(2 ** 31)))
    assert bad == 0, f"{bad} elements of C were not written"

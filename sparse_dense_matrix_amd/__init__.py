"""Python binding of libspmm.so: sparse x dense matrix multiplication on
MI355X (gfx950).

The functions carry the C ABI's names (include/spmm.h) and only marshal
arguments: packing runs in the library's host code and every multiplication
step runs in its HIP kernels.  PyTorch is used for device memory and streams
only (spmm_execute takes torch tensors or raw device pointers).

There is no fallback: if libspmm.so is missing or fails to load, importing
this package raises.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

__all__ = [
    "SpmmError", "Matrix", "Plan", "F32", "BF16", "I8", "I32",
    "FORMAT_BCSR", "FORMAT_WCSR", "FORMAT_24", "FORMAT_TVW", "FORMAT_SLIDE",
    "ARRAY_ROW_PTR", "ARRAY_COL_IDX", "ARRAY_VALS", "ARRAY_META",
    "ARRAY_CHUNK_WINDOW", "ARRAY_CHUNK_BEGIN", "ARRAY_ROW_PERM", "ARRAY_COL_PERM",
    "spmm_pack_bcsr", "spmm_pack_bcsr_csr", "spmm_pack_wcsr", "spmm_pack_24", "spmm_pack_tvw", "spmm_pack_slide",
    "spmm_matrix_info",
    "spmm_matrix_array", "spmm_plan", "spmm_plan_info", "spmm_execute", "spmm_execute_noalloc",
    "spmm_plan_sddmm", "spmm_execute_sddmm",
    "spmm_status_str", "spmm_last_error", "LIB_PATH", "EXPORTS",
]

HERE = os.path.dirname(os.path.abspath(__file__))
# SPMM_LIBRARY may point at another build of the same library
LIB_PATH = os.environ.get("SPMM_LIBRARY") or os.path.join(HERE, "libspmm.so")

F32, BF16, I8, I32 = 0, 1, 2, 3
_ELEM = {F32: 4, BF16: 2, I8: 1, I32: 4}  # bytes per element of each type
FORMAT_BCSR, FORMAT_WCSR, FORMAT_24, FORMAT_TVW, FORMAT_SLIDE = 0, 1, 2, 3, 4
(ARRAY_ROW_PTR, ARRAY_COL_IDX, ARRAY_VALS, ARRAY_META, ARRAY_CHUNK_WINDOW,
 ARRAY_CHUNK_BEGIN, ARRAY_ROW_PERM, ARRAY_COL_PERM) = range(8)

# Default row-window shape for WCSR: 0 lets the library choose (W rows per
# window, at most T stored entries per chunk; one wavefront reduces one chunk).
DEFAULT_WINDOW_ROWS = 0
DEFAULT_MAX_CHUNK_NNZ = 0

# every symbol include/spmm.h declares
EXPORTS = (
    "spmm_pack_bcsr", "spmm_pack_bcsr_csr", "spmm_pack_wcsr", "spmm_pack_24", "spmm_pack_tvw", "spmm_pack_slide",
    "spmm_matrix_info",
    "spmm_matrix_array", "spmm_matrix_destroy", "spmm_plan", "spmm_plan_info",
    "spmm_plan_destroy", "spmm_execute", "spmm_execute_noalloc", "spmm_plan_sddmm",
    "spmm_execute_sddmm",
    "spmm_status_str", "spmm_last_error",
)


class MatrixInfo(C.Structure):
    _fields_ = [("format", C.c_int32), ("dtype", C.c_int32), ("m", C.c_int64),
                ("k", C.c_int64), ("nnz", C.c_int64), ("nnzb", C.c_int64),
                ("block_m", C.c_int32), ("block_k", C.c_int32),
                ("window_rows", C.c_int32), ("max_chunk_nnz", C.c_int64),
                ("num_windows", C.c_int64), ("num_chunks", C.c_int64)]


class PlanInfo(C.Structure):
    _fields_ = [("format", C.c_int32), ("device", C.c_int32), ("m", C.c_int64),
                ("k", C.c_int64), ("n", C.c_int64), ("device_bytes", C.c_int64),
                ("workspace_bytes", C.c_int64), ("num_split_rows", C.c_int64),
                ("num_slots", C.c_int64), ("tile_m", C.c_int32), ("tile_n", C.c_int32),
                ("grid", C.c_int64)]


def _load():
    # One HIP runtime per process: torch ships its own libamdhip64 with the
    # same soname as the system one libspmm.so links.  Loading torch first
    # makes libspmm.so bind to that already-loaded runtime; two runtimes in
    # one process do not share devices.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built (run __graft_entry__.build() or "
                          f"python sparse_dense_matrix_amd/build.py)")
    L = C.CDLL(LIB_PATH)
    P, i64, i32, st = C.c_void_p, C.c_int64, C.c_int32, C.c_int
    sig = {
        "spmm_pack_bcsr": (st, [i64, i64, i32, i32, st, P, i64, C.POINTER(P)]),
        "spmm_pack_wcsr": (st, [i64, i64, st, P, P, P, i32, i64, C.POINTER(P)]),
        "spmm_pack_bcsr_csr": (st, [i64, i64, st, P, P, P, i32, i32, i32, C.POINTER(P)]),
        "spmm_pack_24": (st, [i64, i64, i32, P, i64, C.POINTER(P)]),
        "spmm_pack_tvw": (st, [i64, i64, i32, P, i64, i32, i32, C.POINTER(P)]),
        "spmm_pack_slide": (st, [i64, i64, P, i64, i32, C.POINTER(P)]),
        "spmm_matrix_info": (st, [P, C.POINTER(MatrixInfo)]),
        "spmm_matrix_array": (st, [P, i32, C.POINTER(P), C.POINTER(i64)]),
        "spmm_matrix_destroy": (None, [P]),
        "spmm_plan": (st, [P, i64, st, st, i32, C.POINTER(P)]),
        "spmm_plan_info": (st, [P, C.POINTER(PlanInfo)]),
        "spmm_plan_destroy": (None, [P]),
        "spmm_execute": (st, [P, P, i64, P, i64, P]),
        "spmm_execute_noalloc": (st, [P, P, i64, P, i64, P]),
        "spmm_plan_sddmm": (st, [P, i64, st, i32, C.POINTER(P)]),
        "spmm_execute_sddmm": (st, [P, P, i64, P, i64, P, P]),
        "spmm_status_str": (C.c_char_p, [st]),
        "spmm_last_error": (C.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    return L


_lib = _load()


def lib():
    return _lib


class SpmmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        self.name = spmm_status_str(status)
        self.message = spmm_last_error()
        super().__init__(f"{where}: {self.name}: {self.message}")


def spmm_status_str(status: int) -> str:
    return _lib.spmm_status_str(status).decode()


def spmm_last_error() -> str:
    return _lib.spmm_last_error().decode()


def _check(status: int, where: str):
    if status != 0:
        raise SpmmError(status, where)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


class Matrix:
    """Owns one reference to a packed sparse operand."""

    def __init__(self, handle):
        self.handle = handle

    def __del__(self):
        h, self.handle = getattr(self, "handle", None), None
        if h and _lib is not None:
            _lib.spmm_matrix_destroy(h)

    def info(self) -> dict:
        return spmm_matrix_info(self)


class Plan:
    """Owns a device plan (and through it a reference to its matrix).

    `expect` maps each dense operand of an execute call to (rows, cols,
    bytes per element), or ("count", n, bytes) for the SDDMM output, plus
    "device"; torch tensors handed to execute are checked against it so that
    a kernel never reads or writes past them."""

    def __init__(self, handle, expect=None):
        self.handle = handle
        self.expect = expect or {}

    def __del__(self):
        h, self.handle = getattr(self, "handle", None), None
        if h and _lib is not None:
            _lib.spmm_plan_destroy(h)

    def info(self) -> dict:
        return spmm_plan_info(self)


def spmm_pack_bcsr(a_bits: np.ndarray, block_m: int = 64, block_k: int = 64,
                   dtype: int = BF16) -> Matrix:
    """BCSR from a dense row-major bf16 matrix given as uint16 bit patterns."""
    a = np.ascontiguousarray(a_bits)
    if a.ndim != 2:
        raise ValueError("a must be 2-D")
    h = C.c_void_p()
    _check(_lib.spmm_pack_bcsr(a.shape[0], a.shape[1], block_m, block_k, dtype, _ptr(a),
                               a.shape[1], C.byref(h)), "spmm_pack_bcsr")
    return Matrix(h)


def spmm_pack_slide(a: np.ndarray, group: int = 8) -> Matrix:
    """(group-2):group weights (group = 2N) as N-1 overlapping 2:4 windows per
    group, from a dense int8 matrix."""
    a = np.ascontiguousarray(a, dtype=np.int8)
    if a.ndim != 2:
        raise ValueError("a must be 2-D")
    h = C.c_void_p()
    _check(_lib.spmm_pack_slide(a.shape[0], a.shape[1], _ptr(a), a.shape[1], group, C.byref(h)),
           "spmm_pack_slide")
    return Matrix(h)


def spmm_pack_tvw(a: np.ndarray, tile_m: int = 256, tile_k: int = 128) -> Matrix:
    """Tile-vector-wise from a dense matrix: int8, or bf16 given as uint16
    bit patterns.  Tiles with a nonzero are stored, 2:4-pruned along k."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        dtype = BF16
    elif a.dtype == np.int8:
        dtype = I8
    else:
        raise TypeError("spmm_pack_tvw takes int8 or uint16 (bf16 bits) values")
    a = np.ascontiguousarray(a)
    if a.ndim != 2:
        raise ValueError("a must be 2-D")
    h = C.c_void_p()
    _check(_lib.spmm_pack_tvw(a.shape[0], a.shape[1], dtype, _ptr(a), a.shape[1], tile_m, tile_k,
                              C.byref(h)), "spmm_pack_tvw")
    return Matrix(h)


def spmm_pack_bcsr_csr(m: int, k: int, row_ptr, col_idx, vals_bits, reorder: bool = False,
                       block_m: int = 64, block_k: int = 64, dtype: int = BF16) -> Matrix:
    """BCSR from a canonical CSR with bf16 values (uint16 bit patterns),
    optionally after the row/column permutation that clusters entries into
    fewer blocks (read back with ARRAY_ROW_PERM / ARRAY_COL_PERM)."""
    rp = np.ascontiguousarray(row_ptr, dtype=np.int64)
    ci = np.ascontiguousarray(col_idx, dtype=np.int32)
    v = np.ascontiguousarray(vals_bits, dtype=np.uint16)
    if len(rp) != m + 1:
        raise ValueError("row_ptr must have m + 1 entries")
    h = C.c_void_p()
    _check(_lib.spmm_pack_bcsr_csr(m, k, dtype, _ptr(rp), _ptr(ci), _ptr(v), block_m, block_k,
                                   int(bool(reorder)), C.byref(h)), "spmm_pack_bcsr_csr")
    return Matrix(h)


def spmm_pack_wcsr(m: int, k: int, row_ptr, col_idx, vals,
                   window_rows: int = DEFAULT_WINDOW_ROWS,
                   max_chunk_nnz: int = DEFAULT_MAX_CHUNK_NNZ, dtype: int = F32) -> Matrix:
    rp = np.ascontiguousarray(row_ptr, dtype=np.int64)
    ci = np.ascontiguousarray(col_idx, dtype=np.int32)
    v = np.ascontiguousarray(vals, dtype=np.float32)
    if len(rp) != m + 1:
        raise ValueError("row_ptr must have m + 1 entries")
    h = C.c_void_p()
    _check(_lib.spmm_pack_wcsr(m, k, dtype, _ptr(rp), _ptr(ci), _ptr(v), window_rows,
                               max_chunk_nnz, C.byref(h)), "spmm_pack_wcsr")
    return Matrix(h)


def spmm_pack_24(a: np.ndarray) -> Matrix:
    """2:4 from a dense matrix: int8, or bf16 given as uint16 bit patterns."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        dtype = BF16
    elif a.dtype == np.int8:
        dtype = I8
    else:
        raise TypeError("spmm_pack_24 takes int8 or uint16 (bf16 bits) values")
    a = np.ascontiguousarray(a)
    if a.ndim != 2:
        raise ValueError("a must be 2-D")
    h = C.c_void_p()
    _check(_lib.spmm_pack_24(a.shape[0], a.shape[1], dtype, _ptr(a), a.shape[1], C.byref(h)),
           "spmm_pack_24")
    return Matrix(h)


def spmm_matrix_info(mat: Matrix) -> dict:
    info = MatrixInfo()
    _check(_lib.spmm_matrix_info(mat.handle, C.byref(info)), "spmm_matrix_info")
    return {f: getattr(info, f) for f, _ in MatrixInfo._fields_}


_ARRAY_DTYPES = {
    (FORMAT_BCSR, ARRAY_ROW_PTR): np.int32, (FORMAT_BCSR, ARRAY_COL_IDX): np.int32,
    (FORMAT_BCSR, ARRAY_VALS): np.uint16, (FORMAT_BCSR, ARRAY_ROW_PERM): np.int32,
    (FORMAT_BCSR, ARRAY_COL_PERM): np.int32,
    (FORMAT_WCSR, ARRAY_ROW_PTR): np.int64, (FORMAT_WCSR, ARRAY_COL_IDX): np.int32,
    (FORMAT_WCSR, ARRAY_VALS): np.float32, (FORMAT_WCSR, ARRAY_CHUNK_WINDOW): np.int32,
    (FORMAT_WCSR, ARRAY_CHUNK_BEGIN): np.int64,
    (FORMAT_24, ARRAY_VALS): np.int8, (FORMAT_24, ARRAY_META): np.uint8,
    (FORMAT_TVW, ARRAY_ROW_PTR): np.int32, (FORMAT_TVW, ARRAY_COL_IDX): np.int32,
    (FORMAT_TVW, ARRAY_VALS): np.int8, (FORMAT_TVW, ARRAY_META): np.uint8,
    (FORMAT_SLIDE, ARRAY_VALS): np.int8, (FORMAT_SLIDE, ARRAY_META): np.uint8,
}


def spmm_matrix_array(mat: Matrix, which: int) -> np.ndarray:
    """Copy of a canonical array (see include/spmm.h)."""
    data, count = C.c_void_p(), C.c_int64()
    _check(_lib.spmm_matrix_array(mat.handle, which, C.byref(data), C.byref(count)),
           "spmm_matrix_array")
    info = spmm_matrix_info(mat)
    fmt = info["format"]
    dt = np.dtype(_ARRAY_DTYPES[(fmt, which)])
    if fmt in (FORMAT_TVW, FORMAT_24) and which == ARRAY_VALS and info["dtype"] == BF16:
        dt = np.dtype(np.uint16)
    if count.value == 0:
        return np.zeros(0, dtype=dt)
    buf = (C.c_char * (count.value * dt.itemsize)).from_address(data.value)
    return np.frombuffer(buf, dtype=dt).copy()


def spmm_plan(mat: Matrix, n: int, b_dtype: int, c_dtype: int, device: int = 0) -> Plan:
    h = C.c_void_p()
    _check(_lib.spmm_plan(mat.handle, n, b_dtype, c_dtype, device, C.byref(h)), "spmm_plan")
    mi = spmm_matrix_info(mat)
    return Plan(h, {"b": (mi["k"], n, _ELEM[b_dtype]), "c": (mi["m"], n, _ELEM[c_dtype]),
                    "device": device})


def spmm_plan_info(plan: Plan) -> dict:
    info = PlanInfo()
    _check(_lib.spmm_plan_info(plan.handle, C.byref(info)), "spmm_plan_info")
    return {f: getattr(info, f) for f, _ in PlanInfo._fields_}


def _dev_ptr_ld(t):
    """(pointer, leading dimension) of a 2-D row-major torch tensor.  A tensor
    with no columns has no meaningful strides: its leading dimension is 0."""
    if t.dim() == 2 and t.shape[1] == 0:
        return t.data_ptr(), 0
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("dense operands must be 2-D row-major (stride(1) == 1)")
    return t.data_ptr(), t.stride(0)


def _check_tensor(plan: Plan, name: str, t):
    """Shape, element size and device of a torch tensor against the plan."""
    want = plan.expect.get(name)
    if want is None:
        return
    dev = plan.expect["device"]
    if not t.is_cuda or (t.device.index if t.device.index is not None else 0) != dev:
        raise ValueError(f"{name} must be on cuda:{dev}")
    rows, cols, elem = want
    if t.element_size() != elem:
        raise ValueError(f"{name} has {t.element_size()}-byte elements; the plan takes {elem}")
    if rows == "count":
        if t.numel() < cols or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous with at least {cols} elements")
    elif tuple(t.shape) != (rows, cols):
        raise ValueError(f"{name} has shape {tuple(t.shape)}; the plan takes ({rows}, {cols})")


def _execute(fn: str, plan: Plan, b, c, stream, ldb, ldc):
    if isinstance(b, int) or isinstance(c, int):
        bp, cp = int(b), int(c)
        if ldb is None or ldc is None:
            raise ValueError("raw pointers need ldb and ldc")
    else:
        _check_tensor(plan, "b", b)
        _check_tensor(plan, "c", c)
        bp, ldb = _dev_ptr_ld(b)
        cp, ldc = _dev_ptr_ld(c)
    if stream is None:
        import torch
        dev = c.device if hasattr(c, "device") else None
        stream = torch.cuda.current_stream(dev).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    _check(getattr(_lib, fn)(plan.handle, C.c_void_p(bp), ldb, C.c_void_p(cp), ldc,
                             C.c_void_p(stream)), fn)


def spmm_execute(plan: Plan, b, c, stream=None, ldb: int | None = None,
                 ldc: int | None = None):
    """C = A * B on `stream` (default: torch's current stream on C's device).

    b and c are torch tensors on the plan's device, or raw device pointers
    with ldb / ldc given."""
    _execute("spmm_execute", plan, b, c, stream, ldb, ldc)


def spmm_execute_noalloc(plan: Plan, b, c, stream=None, ldb: int | None = None,
                         ldc: int | None = None):
    """spmm_execute that allocates nothing: a WCSR plan's partial rows live in
    the library's fixed per-GPU scratch array (calls that overlap on one GPU
    race).  Arguments as for spmm_execute."""
    _execute("spmm_execute_noalloc", plan, b, c, stream, ldb, ldc)


def spmm_plan_sddmm(mat: Matrix, kd: int, dtype: int = F32, device: int = 0) -> Plan:
    """Plan the sampled product out[p] = X[i] . Y[j] over the stored entries
    (i, j) of a WCSR (dtype F32, BF16 or I8) or 64 x 64 BCSR (BF16 or I8)
    matrix, inner dimension kd."""
    h = C.c_void_p()
    _check(_lib.spmm_plan_sddmm(mat.handle, kd, dtype, device, C.byref(h)), "spmm_plan_sddmm")
    mi = spmm_matrix_info(mat)
    count = mi["nnzb"] * 64 * 64 if mi["format"] == 0 else mi["nnz"]
    out_elem = {F32: 4, BF16: 2, I8: 4}[dtype]
    return Plan(h, {"x": (mi["m"], kd, _ELEM[dtype]), "y": (mi["k"], kd, _ELEM[dtype]),
                    "out": ("count", count, out_elem), "device": device})


def spmm_execute_sddmm(plan: Plan, x, y, out, stream=None, ldx: int | None = None,
                       ldy: int | None = None):
    """out[p] for every stored entry on `stream` (default: torch's current
    stream).  x [m, kd] and y [k, kd] are 2-D row-major torch tensors (or raw
    device pointers with ldx / ldy); out (tensor or raw pointer) holds the
    plan's output type: fp32, bf16 bits or int32, one per stored entry (WCSR)
    or [nnzb, 64, 64] (BCSR)."""
    if isinstance(x, int) or isinstance(y, int):
        xp, yp = int(x), int(y)
        if ldx is None or ldy is None:
            raise ValueError("raw pointers need ldx and ldy")
    else:
        _check_tensor(plan, "x", x)
        _check_tensor(plan, "y", y)
        xp, ldx = _dev_ptr_ld(x)
        yp, ldy = _dev_ptr_ld(y)
    if not isinstance(out, int):
        _check_tensor(plan, "out", out)
    op = int(out) if isinstance(out, int) else out.data_ptr()
    if stream is None:
        import torch
        dev = out.device if hasattr(out, "device") else None
        stream = torch.cuda.current_stream(dev).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    _check(_lib.spmm_execute_sddmm(plan.handle, C.c_void_p(xp), ldx, C.c_void_p(yp), ldy,
                                   C.c_void_p(op), C.c_void_p(stream)), "spmm_execute_sddmm")

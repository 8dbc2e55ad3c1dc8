"""Python view of the CPU oracle (oracle.c) for C = A_sparse * B_dense.

TEST INFRASTRUCTURE: only the test suite, the smoke check and the benchmark's
CPU-baseline leg import this package.  It never imports the HIP library, and
the HIP library never imports it.

Sources are cited per function in oracle.h (AsyncSparse abstract and Figure 2;
Magicube abstract, for SpMM on low-precision integers and for SDDMM; tiled-GEMM /
tile-wise abstract; the N:M and SpMM entries of the search-results page).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_LIBRARY may point at another build of the same source (the sanitized one)
LIB_PATH = os.environ.get("ORACLE_LIBRARY") or os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "oracle.c")
SANITIZED_LIB = os.path.join(os.path.dirname(_HERE), "_build", "sanitize", "liboracle.so")


def build(verbose: bool = False) -> str:
    """Compile liboracle.so with gcc (no -ffast-math; OpenMP over rows)."""
    tmp = LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", tmp, _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def build_sanitized(verbose: bool = False) -> str:
    """The same source under AddressSanitizer and UndefinedBehaviorSanitizer,
    built with clang so that one ASan runtime serves it and the library."""
    os.makedirs(os.path.dirname(SANITIZED_LIB), exist_ok=True)
    tmp = SANITIZED_LIB + ".tmp"
    cmd = ["/opt/rocm/llvm/bin/clang", "-O1", "-g", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-Wl,-rpath,/opt/rocm/llvm/lib", "-o", tmp, _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, SANITIZED_LIB)
    return SANITIZED_LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run oracle.build()")
        L = C.CDLL(LIB_PATH)
        P = C.c_void_p
        i64, i32 = C.c_int64, C.c_int32
        sig = {
            "orc_bf16_to_double": (C.c_double, [C.c_uint16]),
            "orc_bcsr_count": (i64, [i64, i64, i32, i32, P, i64]),
            "orc_bcsr_fill": (None, [i64, i64, i32, i32, P, i64, P, P, P]),
            "orc_bcsr_densify": (None, [i64, i64, i32, i32, P, P, P, P]),
            "orc_csr_check": (C.c_int, [i64, i64, i64, P, P]),
            "orc_wcsr_num_chunks": (i64, [i64, P, i32, i64]),
            "orc_wcsr_chunks": (None, [i64, P, i32, i64, P, P]),
            "orc_csr_densify": (None, [i64, i64, P, P, P, P]),
            "orc_pack24": (C.c_int, [i64, i64, P, i64, P, P]),
            "orc_densify24": (None, [i64, i64, P, P, P]),
            "orc_prune_nm": (C.c_int, [i64, i64, P, i64, C.c_int, C.c_int, P]),
            "orc_prune_nm_bf16": (C.c_int, [i64, i64, P, i64, C.c_int, C.c_int, P]),
            "orc_csr_spmm_rows": (None, [P, P, P, P, i64, i64, P, i64, i64, P]),
            "orc_bcsr_spmm_rows": (None, [i32, i32, P, P, P, P, i64, i64, P, i64, i64, P]),
            "orc_sp24_spmm_rows": (i64, [i64, P, P, P, i64, i64, P, i64, i64, P]),
            "orc_sddmm_rows": (None, [P, P, P, i64, P, i64, i64, i64, P, P]),
            "orc_sddmm_bcsr_bf16": (None, [i32, i32, P, P, i64, P, i64, P, i64, i64, i64, P, P]),
            "orc_sddmm_bcsr_i8": (i64, [i32, i32, P, P, i64, P, i64, P, i64, i64, i64, P, P]),
            "orc_gemm_f64": (None, [i64, i64, i64, P, P, P]),
            "orc_gemm_i8": (None, [i64, i64, i64, P, P, P]),
            "orc_num_threads": (C.c_int, []),
            "orc_reorder_perms": (C.c_int, [i64, i64, P, P, i32, i32, P, P, P, P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return lib().orc_num_threads()


def bf16_to_double(h: int) -> float:
    return lib().orc_bf16_to_double(h)


# ---- BCSR ------------------------------------------------------------------
def pack_bcsr(a_bits: np.ndarray, bm: int, bk: int):
    """Dense bf16 bits [m, k] -> (row_ptr int32, col_idx int32, vals uint16[nnzb, bm, bk])."""
    a = _c(a_bits, np.uint16)
    m, k = a.shape
    nnzb = lib().orc_bcsr_count(m, k, bm, bk, _p(a), k)
    if nnzb < 0:
        raise ValueError("shape not divisible by the block")
    row_ptr = np.zeros(m // bm + 1, dtype=np.int32)
    col_idx = np.zeros(nnzb, dtype=np.int32)
    vals = np.zeros((nnzb, bm, bk), dtype=np.uint16)
    lib().orc_bcsr_fill(m, k, bm, bk, _p(a), k, _p(row_ptr), _p(col_idx), _p(vals))
    return row_ptr, col_idx, vals


def bcsr_densify(m, k, bm, bk, row_ptr, col_idx, vals) -> np.ndarray:
    out = np.empty((m, k), dtype=np.float64)
    rp, ci, v = _c(row_ptr, np.int32), _c(col_idx, np.int32), _c(vals, np.uint16)
    lib().orc_bcsr_densify(m, k, bm, bk, _p(rp), _p(ci), _p(v), _p(out))
    return out


def bcsr_spmm(bm, bk, row_ptr, col_idx, vals, B_bits, rows=None, j0=0, j1=None):
    """Reference C rows (float64) of BCSR(bf16) x B(bf16 bits [k, n])."""
    B = _c(B_bits, np.uint16)
    n = B.shape[1]
    j1 = n if j1 is None else j1
    if rows is None:
        rows = np.arange((len(row_ptr) - 1) * bm, dtype=np.int64)
    rows = _c(rows, np.int64)
    out = np.empty((len(rows), j1 - j0), dtype=np.float64)
    rp, ci, v = _c(row_ptr, np.int32), _c(col_idx, np.int32), _c(vals, np.uint16)
    lib().orc_bcsr_spmm_rows(bm, bk, _p(rp), _p(ci), _p(v), _p(B), n, len(rows), _p(rows),
                             j0, j1, _p(out))
    return out


# ---- CSR / WCSR ----------------------------------------------------------------
def csr_check(m, k, row_ptr, col_idx) -> int:
    rp, ci = _c(row_ptr, np.int64), _c(col_idx, np.int32)
    return lib().orc_csr_check(m, k, len(ci), _p(rp), _p(ci))


def wcsr_chunks(m, row_ptr, W, T):
    """(chunk_window int32[C], chunk_begin int64[C+1])."""
    rp = _c(row_ptr, np.int64)
    nc = lib().orc_wcsr_num_chunks(m, _p(rp), W, T)
    cw = np.zeros(nc, dtype=np.int32)
    cb = np.zeros(nc + 1, dtype=np.int64)
    lib().orc_wcsr_chunks(m, _p(rp), W, T, _p(cw), _p(cb))
    return cw, cb


def csr_densify(m, k, row_ptr, col_idx, vals) -> np.ndarray:
    out = np.empty((m, k), dtype=np.float64)
    rp, ci, v = _c(row_ptr, np.int64), _c(col_idx, np.int32), _c(vals, np.float32)
    lib().orc_csr_densify(m, k, _p(rp), _p(ci), _p(v), _p(out))
    return out


def csr_spmm(row_ptr, col_idx, vals, B, rows=None, j0=0, j1=None):
    """Reference C rows (float64) of CSR(float32) x B(float32 [k, n])."""
    B = _c(B, np.float32)
    n = B.shape[1]
    j1 = n if j1 is None else j1
    if rows is None:
        rows = np.arange(len(row_ptr) - 1, dtype=np.int64)
    rows = _c(rows, np.int64)
    out = np.empty((len(rows), j1 - j0), dtype=np.float64)
    rp, ci, v = _c(row_ptr, np.int64), _c(col_idx, np.int32), _c(vals, np.float32)
    lib().orc_csr_spmm_rows(_p(rp), _p(ci), _p(v), _p(B), n, len(rows), _p(rows), j0, j1,
                            _p(out))
    return out


# ---- 2:4 -----------------------------------------------------------------------
def pack24(a: np.ndarray):
    """Dense int8 [m, k] -> (vals int8 [m, k/2], meta uint8 [m, k/8])."""
    a = _c(a, np.int8)
    m, k = a.shape
    vals = np.zeros((m, k // 2), dtype=np.int8)
    meta = np.zeros((m, k // 8), dtype=np.uint8)
    if lib().orc_pack24(m, k, _p(a), k, _p(vals), _p(meta)) != 0:
        raise ValueError("k must be a multiple of 8")
    return vals, meta


def densify24(vals, meta) -> np.ndarray:
    v, mt = _c(vals, np.int8), _c(meta, np.uint8)
    m, k = v.shape[0], v.shape[1] * 2
    out = np.empty((m, k), dtype=np.int8)
    lib().orc_densify24(m, k, _p(v), _p(mt), _p(out))
    return out


def prune_nm(a: np.ndarray, keep: int, group: int) -> np.ndarray:
    """Dense int8, or bf16 bit patterns (uint16), with only the `keep` largest
    |a| of every `group` consecutive elements of a row kept (ties to the lower
    position; for bf16 NaN ranks above every number)."""
    a = np.asarray(a)
    bf16 = a.dtype == np.uint16
    a = _c(a, np.uint16 if bf16 else np.int8)
    m, k = a.shape
    out = np.empty((m, k), dtype=a.dtype)
    fn = lib().orc_prune_nm_bf16 if bf16 else lib().orc_prune_nm
    if fn(m, k, _p(a), k, keep, group, _p(out)) != 0:
        raise ValueError("k must be a multiple of the group, group <= 64")
    return out


def sp24_spmm(vals, meta, B, rows=None, j0=0, j1=None):
    """Reference C rows (int32) of 2:4(int8) x B(int8 [k, n]); raises on overflow."""
    v, mt, B = _c(vals, np.int8), _c(meta, np.uint8), _c(B, np.int8)
    m, k = v.shape[0], v.shape[1] * 2
    n = B.shape[1]
    j1 = n if j1 is None else j1
    if rows is None:
        rows = np.arange(m, dtype=np.int64)
    rows = _c(rows, np.int64)
    out = np.empty((len(rows), j1 - j0), dtype=np.int32)
    ov = lib().orc_sp24_spmm_rows(k, _p(v), _p(mt), _p(B), n, len(rows), _p(rows), j0, j1,
                                  _p(out))
    if ov:
        raise OverflowError(f"{ov} int32 sums overflowed")
    return out


# ---- sampled dense-dense product (SDDMM) ------------------------------------------
def sddmm(row_ptr, col_idx, X, Y, rows=None):
    """Reference out (float64) of the CSR pattern sampled from X (float32
    [m, kd]) times Y^T (Y float32 [k, kd]): the entries of `rows` (all rows
    by default) in stored order."""
    rp, ci = _c(row_ptr, np.int64), _c(col_idx, np.int32)
    X, Y = _c(X, np.float32), _c(Y, np.float32)
    if rows is None:
        rows = np.arange(len(rp) - 1, dtype=np.int64)
    rows = _c(rows, np.int64)
    count = int((rp[rows + 1] - rp[rows]).sum())
    out = np.empty(count, dtype=np.float64)
    lib().orc_sddmm_rows(_p(rp), _p(ci), _p(X), X.shape[1], _p(Y), Y.shape[1], X.shape[1],
                         len(rows), _p(rows), _p(out))
    return out


def sddmm_bcsr(bm, bk, row_ptr, col_idx, X, Y, blocks=None):
    """Reference block values of the BCSR pattern (row_ptr, col_idx) sampled
    from X [m, kd] times Y^T (Y [k, kd]): float64 [nsel, bm, bk] for bf16 bits
    (uint16) operands, int32 for int8 operands (raises on int32 overflow).
    `blocks` selects stored blocks (all by default)."""
    rp, ci = _c(row_ptr, np.int32), _c(col_idx, np.int32)
    nbrows = len(rp) - 1
    if blocks is None:
        blocks = np.arange(int(rp[-1]), dtype=np.int64)
    blocks = _c(blocks, np.int64)
    X = np.ascontiguousarray(X)
    Y = np.ascontiguousarray(Y)
    kd = X.shape[1]
    if X.dtype == np.int8:
        out = np.empty((len(blocks), bm, bk), dtype=np.int32)
        ov = lib().orc_sddmm_bcsr_i8(bm, bk, _p(rp), _p(ci), nbrows, _p(X), X.shape[1], _p(Y),
                                     Y.shape[1], kd, len(blocks), _p(blocks), _p(out))
        if ov:
            raise OverflowError(f"{ov} int32 sums overflowed")
        return out
    X, Y = _c(X, np.uint16), _c(Y, np.uint16)
    out = np.empty((len(blocks), bm, bk), dtype=np.float64)
    lib().orc_sddmm_bcsr_bf16(bm, bk, _p(rp), _p(ci), nbrows, _p(X), X.shape[1], _p(Y),
                              Y.shape[1], kd, len(blocks), _p(blocks), _p(out))
    return out


# ---- row/column permutation before BCSR --------------------------------------
def reorder_perms(m, k, row_ptr, col_idx, bm, bk):
    """(kept, row_perm int32[m], col_perm int32[k], blocks_before, blocks_after)
    of the permutation read in oracle.h (identity arrays when not kept)."""
    rp, ci = _c(row_ptr, np.int64), _c(col_idx, np.int32)
    rperm = np.zeros(max(m, 1), np.int32)
    cperm = np.zeros(max(k, 1), np.int32)
    before, after = C.c_int64(), C.c_int64()
    kept = lib().orc_reorder_perms(m, k, _p(rp), _p(ci), bm, bk, _p(rperm), _p(cperm),
                                   C.byref(before), C.byref(after))
    return bool(kept), rperm[:m], cperm[:k], before.value, after.value


# ---- brute force -------------------------------------------------------------
def gemm_f64(A, B) -> np.ndarray:
    A, B = _c(A, np.float64), _c(B, np.float64)
    out = np.empty((A.shape[0], B.shape[1]), dtype=np.float64)
    lib().orc_gemm_f64(A.shape[0], A.shape[1], B.shape[1], _p(A), _p(B), _p(out))
    return out


def gemm_i8(A, B) -> np.ndarray:
    A, B = _c(A, np.int8), _c(B, np.int8)
    out = np.empty((A.shape[0], B.shape[1]), dtype=np.int64)
    lib().orc_gemm_i8(A.shape[0], A.shape[1], B.shape[1], _p(A), _p(B), _p(out))
    return out


# ---- comparison ----------------------------------------------------------------
def rel_frobenius(got, ref) -> float:
    """||got - ref||_F / ||ref||_F in float64 (0 when both are zero; inf when
    only ref is zero)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = float(np.sqrt(np.sum((got - ref) ** 2)))
    den = float(np.sqrt(np.sum(ref ** 2)))
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / den

"""Seeded synthetic inputs for sparse x dense multiplication (C = A_sparse * B_dense).

This module only *draws* inputs: sparsity patterns, values and dense operands.
It holds none of the multiplication's arithmetic and none of the packing rules,
so both the CPU oracle and the HIP path can be fed from it without sharing any
of the method.

Random streams come from numpy's Philox bit generator (the counter-based
Philox4x64-10 of Salmon et al., "Parallel random numbers: as easy as 1, 2, 3",
SC'11).  Every stream is keyed by (seed, stream id), so each operand of a
workload is reproducible on its own.

Workloads follow the shapes the AsyncSparse page (abstract) benchmarks on --
block-structured sparsity at 90% for a 7B-model MLP weight with 64K tokens, and
irregular matrices from a public sparse-matrix collection -- and the 2:4 int8
case of the tile-wise / Magicube pages.  The public matrix collection and the
model weights are not available; the power-law CSR and the uniform block masks
stand in for them.
"""
from __future__ import annotations

import dataclasses
from typing import Dict

import numpy as np

# stream ids: one independent Philox key per random quantity of a workload
S_PATTERN, S_AVAL, S_BVAL, S_ROWLEN, S_COLS, S_BAND, S_YVAL, S_PERM = 0, 1, 2, 3, 4, 5, 6, 7


def rng(seed: int, stream: int) -> np.random.Generator:
    """Philox generator for (seed, stream)."""
    return np.random.Generator(np.random.Philox(key=(int(seed) << 16) | int(stream)))


# ---------------------------------------------------------------------------
# value formatting (input preparation only)
# ---------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16, round-to-nearest-even, returned as uint16 bits.

    Inputs are finite (nothing here draws NaN or Inf)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits to float32."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_f32(g: np.random.Generator, shape, sigma: float = 1.0) -> np.ndarray:
    x = g.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return x


def uniform_pm1_f32(g: np.random.Generator, shape) -> np.ndarray:
    """U[-1, 1) in float32."""
    x = g.random(size=shape, dtype=np.float32)
    return x * np.float32(2.0) - np.float32(1.0)


def int8_uniform(g: np.random.Generator, shape) -> np.ndarray:
    """Integers uniform on {-127 ... 127}."""
    return g.integers(-127, 128, size=shape, dtype=np.int8)


# ---------------------------------------------------------------------------
# sparse patterns
# ---------------------------------------------------------------------------
def csr_uniform(m: int, k: int, density: float, seed: int):
    """CSR with exactly round(density*m*k) nonzeros at uniform random positions
    (chosen without replacement), values U[-1,1) float32.

    Returns (row_ptr int64[m+1], col_idx int32[nnz], vals float32[nnz])."""
    total = m * k
    nnz = int(round(density * total))
    pos = np.sort(rng(seed, S_PATTERN).choice(total, size=nnz, replace=False))
    rows = pos // k
    cols = (pos % k).astype(np.int32)
    vals = uniform_pm1_f32(rng(seed, S_AVAL), nnz)
    row_ptr = np.zeros(m + 1, dtype=np.int64)
    np.cumsum(np.bincount(rows, minlength=m), out=row_ptr[1:])
    return row_ptr, cols, vals


def zipf_lengths(m: int, exponent: float, cap: int, seed: int) -> np.ndarray:
    """Row lengths L with P(L = j) proportional to j^-exponent on {1..cap}."""
    j = np.arange(1, cap + 1, dtype=np.float64)
    p = j ** (-exponent)
    cdf = np.cumsum(p)
    cdf /= cdf[-1]
    u = rng(seed, S_ROWLEN).random(m)
    return (np.searchsorted(cdf, u, side="right") + 1).astype(np.int64)


def csr_powerlaw(m: int, k: int, exponent: float, cap: int, band_frac: float,
                 band_half: int, seed: int):
    """Irregular CSR: power-law row lengths, a fraction of the columns drawn
    within +/-band_half of the diagonal and the rest uniform on [0, k).

    Per draw: with probability band_frac the column is uniform on
    [max(0, i-band_half), min(k-1, i+band_half)], else uniform on [0, k).
    Duplicate (row, col) draws are collapsed keeping the first drawn value,
    so a row can end up shorter than its drawn length.  Values U[-1,1).
    """
    lens = np.minimum(zipf_lengths(m, exponent, cap, seed), k)
    total = int(lens.sum())
    rows = np.repeat(np.arange(m, dtype=np.int64), lens)
    banded = rng(seed, S_BAND).random(total) < band_frac
    lo = np.maximum(rows - band_half, 0)
    width = np.where(banded, np.minimum(rows + band_half, k - 1) - lo + 1, k)
    lo[~banded] = 0
    del banded
    u = rng(seed, S_COLS).random(total)
    u *= width
    cols = lo + u.astype(np.int64)
    del lo, width, u
    np.minimum(cols, k - 1, out=cols)
    vals = uniform_pm1_f32(rng(seed, S_AVAL), total)
    # rows are already grouped; order each row by (col, draw order) and keep
    # the first draw of every (row, col)
    cols += rows * np.int64(k)
    order = np.argsort(cols, kind="stable")
    key = cols[order]
    del cols
    keep = np.empty(total, dtype=bool)
    keep[0] = True
    np.not_equal(key[1:], key[:-1], out=keep[1:])
    order = order[keep]
    key = key[keep]
    col_idx = (key % np.int64(k)).astype(np.int32)
    vals = vals[order]
    row_ptr = np.zeros(m + 1, dtype=np.int64)
    np.cumsum(np.bincount(key // np.int64(k), minlength=m), out=row_ptr[1:])
    return row_ptr, col_idx, vals


def block_sparse_dense_bf16(m: int, k: int, bm: int, bk: int, nblocks: int,
                            sigma: float, seed: int):
    """Dense row-major bf16 matrix (uint16 bits) that is zero except on exactly
    `nblocks` bm x bk blocks chosen uniformly without replacement; values in
    those blocks N(0, sigma) rounded to bf16.  Returns (a, block_ids)."""
    mb, kb = m // bm, k // bk
    ids = np.sort(rng(seed, S_PATTERN).choice(mb * kb, size=nblocks, replace=False))
    a = np.zeros((m, k), dtype=np.uint16)
    vals = f32_to_bf16_bits(normal_f32(rng(seed, S_AVAL), (nblocks, bm, bk), sigma))
    for t, b in enumerate(ids):
        r, c = divmod(int(b), kb)
        a[r * bm:(r + 1) * bm, c * bk:(c + 1) * bk] = vals[t]
    return a, ids


def tile_sparse_i8(m: int, k: int, tm: int, tk: int, ntiles: int, seed: int) -> np.ndarray:
    """Dense int8 [m x k] that is zero except on exactly `ntiles` tm x tk
    tiles chosen uniformly without replacement, whose values are uniform on
    {-127 ... 127}.  (The 2:4 pruning inside the tiles is the packer's job.)"""
    mt, kt = m // tm, k // tk
    ids = np.sort(rng(seed, S_PATTERN).choice(mt * kt, size=ntiles, replace=False))
    vals = int8_uniform(rng(seed, S_AVAL), (ntiles, tm, tk))
    a = np.zeros((m, k), dtype=np.int8)
    for t, b in enumerate(ids):
        r, c = divmod(int(b), kt)
        a[r * tm:(r + 1) * tm, c * tk:(c + 1) * tk] = vals[t]
    return a


def scrambled_csr_bf16(a_bits: np.ndarray, seed: int):
    """A dense bf16 matrix (uint16 bits) with its rows and columns shuffled by
    seeded random permutations, as a canonical CSR (row_ptr int64, col_idx
    int32, vals uint16 bits): block structure that is there but not visible.
    Also returns the two permutations (new -> original)."""
    m, k = a_bits.shape
    g = rng(seed, S_PERM)
    rperm = g.permutation(m)
    cperm = g.permutation(k)
    a = a_bits[rperm][:, cperm]
    nz = (a & 0x7FFF) != 0
    row_ptr = np.zeros(m + 1, dtype=np.int64)
    np.cumsum(nz.sum(axis=1), out=row_ptr[1:])
    rows, cols = np.nonzero(nz)
    return row_ptr, cols.astype(np.int32), a[rows, cols].astype(np.uint16), rperm, cperm


def dense_bf16_normal(rows: int, cols: int, seed: int, stream: int = S_BVAL,
                      sigma: float = 1.0, chunk_rows: int = 256) -> np.ndarray:
    """Dense row-major bf16 (uint16 bits) N(0, sigma), drawn in row slabs to
    bound the float32 temporary."""
    out = np.empty((rows, cols), dtype=np.uint16)
    g = rng(seed, stream)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        out[r0:r1] = f32_to_bf16_bits(normal_f32(g, (r1 - r0, cols), sigma))
    return out


def dense_f32_normal(rows: int, cols: int, seed: int, stream: int = S_BVAL) -> np.ndarray:
    return normal_f32(rng(seed, stream), (rows, cols))


# ---------------------------------------------------------------------------
# workload catalogue
# ---------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    fmt: str            # "wcsr" | "bcsr" | "bcsr_csr" | "sp24" | "tvw" | "slide" | "sddmm" | "sddmm_bcsr"
    m: int
    k: int
    n: int
    seed: int
    density: float = 0.0          # wcsr uniform
    powerlaw: bool = False        # wcsr power-law
    zipf: float = 1.8
    cap: int = 20000
    band_frac: float = 0.3
    band_half: int = 512
    block: int = 64               # bcsr
    nblocks: int = 0
    sigma: float = 0.02
    elem: str = ""                # sddmm, sddmm_bcsr: "bf16" | "i8" operands X, Y (sddmm
                                  # default fp32); sp24, tvw: "bf16" A and B (default int8)
    scramble: int = 0             # > 0: a block-sparse matrix with rows and columns
                                  # shuffled (this seed), given as CSR
    reorder: bool = False         # bcsr_csr: pack after the row/column reordering
    nm_group: int = 0             # slide: group width 2N of the (2N-2):2N pattern

    @property
    def describe(self) -> str:
        return f"{self.name} ({self.fmt}, m={self.m}, k={self.k}, n={self.n})"


def _bcsr(name, m, k, n, zero_frac, seed, block=64, fmt="bcsr", elem=""):
    total = (m // block) * (k // block)
    return Workload(name, fmt, m, k, n, seed, block=block,
                    nblocks=int(round((1.0 - zero_frac) * total)), elem=elem)


# tile shape of the tile-vector-wise workloads (the 2:4 kernel's A tile)
TVW_TILE_M, TVW_TILE_K = 256, 128

# The five benchmark shapes (seed 20260000 + index) ...
WORKLOADS: Dict[str, Workload] = {
    "csr_tiny_256": Workload("csr_tiny_256", "wcsr", 256, 256, 64, 20260001, density=0.05),
    "bcsr_4096_b64_90": _bcsr("bcsr_4096_b64_90", 4096, 4096, 4096, 0.90, 20260002),
    "csr_powerlaw_1m": Workload("csr_powerlaw_1m", "wcsr", 1_000_000, 1_000_000, 128, 20260003,
                                powerlaw=True),
    "sp24_i8_8192": Workload("sp24_i8_8192", "sp24", 8192, 8192, 2048, 20260004),
    # the same shapes in bf16: weights N(0, 0.02), B N(0, 1)
    "sp24_bf16_8192": Workload("sp24_bf16_8192", "sp24", 8192, 8192, 2048, 20260014, elem="bf16"),
    "bcsr_prefill_18944x3584": _bcsr("bcsr_prefill_18944x3584", 18944, 3584, 65536, 0.90, 20260005),
    # the same layer at milder block sparsity (50% and 70% of the blocks zero)
    "bcsr_prefill_18944x3584_z50": _bcsr("bcsr_prefill_18944x3584_z50", 18944, 3584, 65536, 0.50,
                                         20260006),
    "bcsr_prefill_18944x3584_z70": _bcsr("bcsr_prefill_18944x3584_z70", 18944, 3584, 65536, 0.70,
                                         20260007),
    # tile-vector-wise: the 8192 x 8192 int8 weight with half / three quarters
    # of its 256 x 128 tiles zero (2:4 inside the rest), same B as the 2:4 case
    "tvw_i8_8192_t50": Workload("tvw_i8_8192_t50", "tvw", 8192, 8192, 2048, 20260009, nblocks=1024),
    "tvw_i8_8192_t75": Workload("tvw_i8_8192_t75", "tvw", 8192, 8192, 2048, 20260010, nblocks=512),
    # the same shapes and tile counts in bf16 (weights N(0, 0.02), B N(0, 1))
    "tvw_bf16_8192_t50": Workload("tvw_bf16_8192_t50", "tvw", 8192, 8192, 2048, 20260012,
                                  nblocks=1024, elem="bf16"),
    "tvw_bf16_8192_t75": Workload("tvw_bf16_8192_t75", "tvw", 8192, 8192, 2048, 20260013,
                                  nblocks=512, elem="bf16"),
    # the 2:4 case's shapes with a milder pattern: 6 of every 8 kept, as
    # overlapping 2:4 windows
    "slide68_i8_8192": Workload("slide68_i8_8192", "slide", 8192, 8192, 2048, 20260011, nm_group=8),
    # the 4096 block-sparse matrix with rows and columns shuffled, given as
    # CSR: packed as BCSR with and without the reordering, and as WCSR
    "scrambled_4096_bcsr_reordered": Workload("scrambled_4096_bcsr_reordered", "bcsr_csr", 4096,
                                              4096, 4096, 20260002, nblocks=410,
                                              scramble=20260008, reorder=True),
    "scrambled_4096_bcsr_plain": Workload("scrambled_4096_bcsr_plain", "bcsr_csr", 4096, 4096,
                                          4096, 20260002, nblocks=410, scramble=20260008),
    "scrambled_4096_wcsr": Workload("scrambled_4096_wcsr", "wcsr", 4096, 4096, 4096, 20260002,
                                    nblocks=410, scramble=20260008),
    # the sampled dense-dense product on the power-law pattern, inner dimension 128
    "sddmm_powerlaw_1m": Workload("sddmm_powerlaw_1m", "sddmm", 1_000_000, 1_000_000, 128, 20260003,
                                  powerlaw=True),
    # the same pattern with bf16 and int8 X, Y
    "sddmm_bf16_powerlaw_1m": Workload("sddmm_bf16_powerlaw_1m", "sddmm", 1_000_000, 1_000_000, 128,
                                       20260003, powerlaw=True, elem="bf16"),
    "sddmm_i8_powerlaw_1m": Workload("sddmm_i8_powerlaw_1m", "sddmm", 1_000_000, 1_000_000, 128,
                                     20260003, powerlaw=True, elem="i8"),
    # the same product on the block pattern of the 18944 x 3584 layer: the
    # layer's weight gradient over one GPU's share (8192) of 65536 tokens
    "sddmm_bcsr_prefill_kd8192": _bcsr("sddmm_bcsr_prefill_kd8192", 18944, 3584, 8192, 0.90,
                                       20260005, fmt="sddmm_bcsr", elem="bf16"),
    "sddmm_i8_prefill_kd8192": _bcsr("sddmm_i8_prefill_kd8192", 18944, 3584, 8192, 0.90,
                                     20260005, fmt="sddmm_bcsr", elem="i8"),
}

# ... and smaller cases of the same construction for element-wise parity
# (several tiles plus a ragged tail in every dimension the kernels tile).
SMALL: Dict[str, Workload] = {
    "csr_uniform_small": Workload("csr_uniform_small", "wcsr", 1000, 777, 200, 31, density=0.03),
    "csr_powerlaw_small": Workload("csr_powerlaw_small", "wcsr", 20000, 20000, 128, 32,
                                   powerlaw=True, cap=3000, band_half=64),
    "bcsr_small": _bcsr("bcsr_small", 640, 512, 1000, 0.7, 33),
    "sp24_small": Workload("sp24_small", "sp24", 320, 512, 400, 34),
    "sp24_bf16_small": Workload("sp24_bf16_small", "sp24", 320, 512, 400, 41, elem="bf16"),
    "bcsr_prefill_slice": _bcsr("bcsr_prefill_slice", 18944, 3584, 4096 + 64 * 3, 0.90, 20260005),
    "sddmm_small": Workload("sddmm_small", "sddmm", 20000, 20000, 96, 32, powerlaw=True, cap=3000,
                            band_half=64),
    "sddmm_bcsr_small": _bcsr("sddmm_bcsr_small", 640, 512, 1000, 0.7, 35, fmt="sddmm_bcsr",
                              elem="bf16"),
    "tvw_small": Workload("tvw_small", "tvw", 512, 1024, 272, 38, nblocks=6),
    "tvw_bf16_small": Workload("tvw_bf16_small", "tvw", 512, 1024, 272, 40, nblocks=6, elem="bf16"),
    "slide_small": Workload("slide_small", "slide", 320, 512, 400, 39, nm_group=8),
    "scrambled_small": Workload("scrambled_small", "bcsr_csr", 1024, 768, 520, 36, nblocks=30,
                                scramble=37, reorder=True),
}


def make_a(w: Workload) -> dict:
    """Draw the sparse operand.  wcsr -> CSR arrays; bcsr -> dense bf16 bits;
    sp24 -> dense int8 (not yet pruned: pruning is the packer's job)."""
    if w.scramble:
        dense, _ = block_sparse_dense_bf16(w.m, w.k, w.block, w.block, w.nblocks, w.sigma, w.seed)
        rp, ci, v, rperm, cperm = scrambled_csr_bf16(dense, w.scramble)
        out = {"row_ptr": rp, "col_idx": ci, "vals_bf16": v, "row_shuffle": rperm,
               "col_shuffle": cperm}
        out["vals"] = bf16_bits_to_f32(v)            # the same values, for fp32 paths
        return out
    if w.fmt in ("wcsr", "sddmm"):
        if w.powerlaw:
            rp, ci, v = csr_powerlaw(w.m, w.k, w.zipf, w.cap, w.band_frac, w.band_half, w.seed)
        else:
            rp, ci, v = csr_uniform(w.m, w.k, w.density, w.seed)
        return {"row_ptr": rp, "col_idx": ci, "vals": v}
    if w.fmt in ("bcsr", "sddmm_bcsr"):
        a, ids = block_sparse_dense_bf16(w.m, w.k, w.block, w.block, w.nblocks, w.sigma, w.seed)
        return {"dense": a, "block_ids": ids}
    if w.fmt == "sp24" and w.elem == "bf16":
        return {"dense": f32_to_bf16_bits(normal_f32(rng(w.seed, S_AVAL), (w.m, w.k), w.sigma))}
    if w.fmt in ("sp24", "slide"):
        return {"dense": int8_uniform(rng(w.seed, S_AVAL), (w.m, w.k))}
    if w.fmt == "tvw" and w.elem == "bf16":
        a, _ = block_sparse_dense_bf16(w.m, w.k, TVW_TILE_M, TVW_TILE_K, w.nblocks, w.sigma, w.seed)
        return {"dense": a}
    if w.fmt == "tvw":
        return {"dense": tile_sparse_i8(w.m, w.k, TVW_TILE_M, TVW_TILE_K, w.nblocks, w.seed)}
    raise ValueError(w.fmt)


def make_xy(w: Workload, kd: int | None = None, elem: str | None = None):
    """Draw the dense operands of the sampled product: X [m x kd] and
    Y [k x kd], row-major; float32 N(0, 1) (the CSR pattern's default), bf16
    bits N(0, 1) or int8 uniform on {-127 ... 127}."""
    kd = w.n if kd is None else kd
    elem = w.elem if elem is None else elem
    if elem == "bf16":
        return (dense_bf16_normal(w.m, kd, w.seed, S_BVAL),
                dense_bf16_normal(w.k, kd, w.seed, S_YVAL))
    if elem == "i8":
        return (int8_uniform(rng(w.seed, S_BVAL), (w.m, kd)),
                int8_uniform(rng(w.seed, S_YVAL), (w.k, kd)))
    return dense_f32_normal(w.m, kd, w.seed, S_BVAL), dense_f32_normal(w.k, kd, w.seed, S_YVAL)


def make_b(w: Workload, n: int | None = None) -> np.ndarray:
    """Draw the dense operand B [k x n] row-major."""
    n = w.n if n is None else n
    if w.scramble:
        bits = dense_bf16_normal(w.k, n, w.seed)
        return bf16_bits_to_f32(bits) if w.fmt == "wcsr" else bits   # the same values
    if w.fmt == "wcsr":
        return dense_f32_normal(w.k, n, w.seed)
    if w.fmt == "bcsr" or (w.fmt in ("tvw", "sp24") and w.elem == "bf16"):
        return dense_bf16_normal(w.k, n, w.seed)
    if w.fmt in ("sp24", "tvw", "slide"):
        return int8_uniform(rng(w.seed, S_BVAL), (w.k, n))
    raise ValueError(w.fmt)

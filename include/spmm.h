/*
 * spmm.h -- C ABI of the MI355X (gfx950) sparse x dense multiplication library.
 *
 * The library computes C = A * B, A sparse, B and C dense, for these sparse
 * encodings:
 *
 *   BCSR  block compressed sparse row, bf16 A and B, fp32 accumulation,
 *         bf16 C.  Block-structured sparsity: "AsyncSparse: Accelerating
 *         Sparse Matrix-Matrix Multiplication on Asynchronous GPU
 *         Architectures", abstract and Figure 2 caption.
 *   WCSR  CSR processed in windows of consecutive rows whose stored entries
 *         are cut into bounded chunks, so one long window is spread over many
 *         workgroups; fp32 A, B, C.  Irregular sparsity: same page, abstract
 *         and the summary's "What carries the argument" paragraph
 *         (row-window splitting across thread blocks for load balance).
 *   2:4   int8 A pruned so that every group of 4 consecutive elements along k
 *         holds at most 2 nonzeros, stored compressed with 2-bit positions;
 *         int8 B, exact int32 C.  "Accelerating Sparse DNNs Based on Tiled
 *         GEMM", abstract (2:4 pattern); "Efficient Quantized Sparse Matrix
 *         Operations on Tensor Cores", abstract (SpMM on low-precision
 *         integers); the N:M entry of the "Daily Papers" search page.
 *   TVW   tile-vector-wise: tiles of A that hold a nonzero are stored, 2:4
 *         inside; int8 (int32 C) or bf16 (bf16 C).  "Accelerating Sparse
 *         DNNs Based on Tiled GEMM", abstract.
 *   SLIDE (2N-2):2N weights as N-1 overlapping 2:4 windows per group, int8;
 *         the (2N-2):2N entry of the "Daily Papers" search page.
 *
 * and the sampled dense-dense product (SDDMM) on a WCSR or BCSR pattern, the
 * companion of SpMM on the Magicube page ("Efficient Quantized Sparse Matrix
 * Operations on Tensor Cores", abstract).
 *
 * Usage: pack A once on the host (spmm_pack_*), build a device plan for a
 * given number of columns n (spmm_plan), then multiply any number of dense B
 * by it (spmm_execute) on the caller's HIP stream.
 *
 * Conventions for every call:
 *   - Each call returns a status.  On failure any out-parameter is set to
 *     NULL, nothing leaks, and spmm_last_error() returns a message (per
 *     thread).  No exception or abort crosses the ABI.
 *   - Dense matrices are row-major with a leading dimension (elements between
 *     consecutive rows).
 *   - Integers in the ABI are signed 64-bit unless stated; row and column
 *     counts must fit in int32.
 */
#ifndef SPMM_H
#define SPMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* HIP stream handle, as in hip_runtime_api.h (NULL = the legacy default stream). */
typedef struct ihipStream_t *hipStream_t;

typedef enum {
  SPMM_OK = 0,
  SPMM_ERR_INVALID_ARG = 1,   /* bad pointer, size, layout or non-canonical input   */
  SPMM_ERR_UNSUPPORTED = 2,   /* valid request outside what the kernels implement   */
  SPMM_ERR_OUT_OF_MEMORY = 3, /* host or device allocation failed                   */
  SPMM_ERR_HIP = 4,           /* a HIP runtime call failed; message holds its text  */
  SPMM_ERR_INTERNAL = 5
} spmm_status_t;

typedef enum { SPMM_F32 = 0, SPMM_BF16 = 1, SPMM_I8 = 2, SPMM_I32 = 3 } spmm_dtype_t;

typedef enum {
  SPMM_FORMAT_BCSR = 0,
  SPMM_FORMAT_WCSR = 1,
  SPMM_FORMAT_24 = 2,
  SPMM_FORMAT_TVW = 3,   /* tile-vector-wise: 2:4 inside the stored tiles of a tile grid */
  SPMM_FORMAT_SLIDE = 4  /* (2N-2):2N as overlapping 2:4 windows                        */
} spmm_format_t;

/* Packed sparse operand: immutable host arrays in the canonical layout below,
 * reference counted (a plan holds a reference). */
typedef struct spmm_matrix_s *spmm_matrix_t;
/* Device copy of a packed operand plus kernel choice and workspace, for one n. */
typedef struct spmm_plan_s *spmm_plan_t;

typedef struct {
  int32_t format;        /* spmm_format_t                                      */
  int32_t dtype;         /* element type of A                                  */
  int64_t m, k;          /* logical shape of A                                 */
  int64_t nnz;           /* stored entries: nnzb*bm*bk (BCSR), CSR nnz, m*k/2   */
                         /* (2:4), nnzb*bm*bk/2 (TVW), m*k_lift/2 (SLIDE)      */
  int64_t nnzb;          /* BCSR: stored blocks; TVW: stored tiles; else 0    */
  int32_t block_m, block_k;        /* BCSR block / TVW tile shape; SLIDE: 0 and */
                                   /* the group width 2N; otherwise 0          */
  int32_t window_rows;             /* WCSR: rows per window W; otherwise 0     */
  int64_t max_chunk_nnz;           /* WCSR: chunk bound T; otherwise 0         */
  int64_t num_windows, num_chunks; /* WCSR; otherwise 0                        */
} spmm_matrix_info_t;

/* Canonical arrays, read with spmm_matrix_array(which):
 *  BCSR (nnzb blocks, mb = m / block_m block rows)
 *    SPMM_ARRAY_ROW_PTR   int32[mb + 1]   blocks of block row r: [row_ptr[r], row_ptr[r+1])
 *    SPMM_ARRAY_COL_IDX   int32[nnzb]     block column, ascending within a block row
 *    SPMM_ARRAY_VALS      bf16 bits, uint16[nnzb * bm * bk], each block row-major
 *    SPMM_ARRAY_ROW_PERM  int32[m]        (spmm_pack_bcsr_csr with reordering) original
 *                                         row of each row of the packed matrix; count 0
 *                                         when rows keep their order
 *    SPMM_ARRAY_COL_PERM  int32[k]        original column of each packed column; count 0
 *                                         when columns keep their order
 *  WCSR
 *    SPMM_ARRAY_ROW_PTR   int64[m + 1]
 *    SPMM_ARRAY_COL_IDX   int32[nnz]      strictly ascending within a row
 *    SPMM_ARRAY_VALS      float[nnz]
 *    SPMM_ARRAY_CHUNK_WINDOW  int32[num_chunks]    window of each chunk
 *    SPMM_ARRAY_CHUNK_BEGIN   int64[num_chunks+1]  first stored entry; last = nnz
 *  2:4
 *    SPMM_ARRAY_VALS      int8 or bf16 (uint16)[m * k/2]  the two kept values of group g
 *                                         of row i at
 *                                         [i*k/2 + 2g], [i*k/2 + 2g + 1], ascending position
 *    SPMM_ARRAY_META      uint8[m * k/8]  nibble (i0 | i1 << 2) of group g in byte
 *                                         i*k/8 + g/2, low nibble for even g
 *  SLIDE ((2N-2):2N as overlapping 2:4 windows, group = 2N, k_lift = 4(N-1) k / 2N)
 *    SPMM_ARRAY_VALS      int8[m * k_lift/2]   the lifted 2:4 matrix, layout as for 2:4
 *    SPMM_ARRAY_META      uint8[m * k_lift/8]  its nibbles
 *  TVW (nt stored tiles of tm x tk, mt = m / tm tile rows)
 *    SPMM_ARRAY_ROW_PTR   int32[mt + 1]   stored tiles of tile row T: [row_ptr[T], row_ptr[T+1])
 *    SPMM_ARRAY_COL_IDX   int32[nt]       tile column (k / tk units), ascending in a tile row
 *    SPMM_ARRAY_VALS      int8 or bf16 (uint16)[nt * tm * tk/2]  each stored tile in the
 *                                         2:4 layout above, tile row-major, rows of tk/2
 *                                         kept values
 *    SPMM_ARRAY_META      uint8[nt * tm * tk/8] each stored tile's nibbles, rows of tk/8 */
typedef enum {
  SPMM_ARRAY_ROW_PTR = 0,
  SPMM_ARRAY_COL_IDX = 1,
  SPMM_ARRAY_VALS = 2,
  SPMM_ARRAY_META = 3,
  SPMM_ARRAY_CHUNK_WINDOW = 4,
  SPMM_ARRAY_CHUNK_BEGIN = 5,
  SPMM_ARRAY_ROW_PERM = 6,
  SPMM_ARRAY_COL_PERM = 7
} spmm_array_t;

/* ---- packing (host only; inputs are borrowed for the call and copied) ---- */

/* Defining passage: "AsyncSparse: Accelerating Sparse Matrix-Matrix
 * Multiplication on Asynchronous GPU Architectures", abstract (BCSR for
 * structured sparsity) and the caption of Figure 2 (BCSR and WCSR compared
 * on one matrix); the block size is not given there, the kernels take 64.
 * BCSR from a dense row-major bf16 matrix a_host [m x k] (uint16 bit patterns,
 * leading dimension lda >= k).  A block_m x block_k block is stored when any
 * element is numerically nonzero (+0 and -0 are zero, NaN is not); block rows
 * ascending, block columns ascending, values row-major within the block.
 * Requires dtype == SPMM_BF16 (else UNSUPPORTED), m % block_m == 0 and
 * k % block_k == 0 (else INVALID_ARG).  The kernels take 64 x 64 blocks. */
spmm_status_t spmm_pack_bcsr(int64_t m, int64_t k, int32_t block_m, int32_t block_k,
                             spmm_dtype_t dtype, const void *a_host, int64_t lda,
                             spmm_matrix_t *out);

/* (2N-2):2N weights as overlapping 2:4 windows (the sliding-window
 * decomposition of the (2N-2):2N family on the "Daily Papers" search page):
 * from a dense int8 a_host [m x k], every group of `group` = 2N consecutive
 * elements of a row keeps its 2N-2 largest |a| (as integers, ties to the
 * lower position; the rest are dropped) and the kept elements are dealt, in
 * ascending position, to the lowest of the N-1 windows of four (window w
 * covers positions 2w .. 2w+3) that covers them and has room; each window is
 * then one 2:4 group.  The product is that of the pruned A.  Lifted column
 * 4w + j of group g multiplies B's row 2N g + 2w + j; the kernel reads B's
 * rows through that map (no workspace).  Requires
 * group even in [4, 64], k % group == 0 and k_lift % 8 == 0 (else
 * INVALID_ARG); spmm_matrix_info reports group as block_k. */
spmm_status_t spmm_pack_slide(int64_t m, int64_t k, const int8_t *a_host, int64_t lda, int32_t group,
                              spmm_matrix_t *out);

/* Tile-vector-wise (the tile-wise pattern combined with 2:4 of "Accelerating
 * Sparse DNNs Based on Tiled GEMM", abstract) from a dense row-major matrix
 * a_host [m x k] (lda >= k) of dtype SPMM_I8 (int8) or SPMM_BF16 (uint16 bit
 * patterns; else UNSUPPORTED): A is cut into tile_m x tile_k tiles, a tile is
 * stored when any element is nonzero (bf16: +0 and -0 are zero, NaN is not),
 * and a stored tile is pruned 2:4 along k by the rule of spmm_pack_24 (for
 * bf16, |a| in magnitude order, every NaN above infinity and NaNs equal).  The product is
 * therefore the 2:4 product of the pruned A with the zero tiles skipped.
 * Requires m % tile_m == 0, k % tile_k == 0 and tile_k % 8 == 0 (else
 * INVALID_ARG); the kernels take tile_m = 256 and tile_k a multiple of 128
 * (int8) or 64 (bf16) (spmm_plan returns UNSUPPORTED for others). */
spmm_status_t spmm_pack_tvw(int64_t m, int64_t k, spmm_dtype_t dtype, const void *a_host,
                            int64_t lda, int32_t tile_m, int32_t tile_k, spmm_matrix_t *out);

/* BCSR from a canonical CSR on the host (row_ptr, col_idx as for
 * spmm_pack_wcsr; vals bf16 bit patterns, uint16[nnz]).  A block is stored
 * when a CSR entry falls in it (structural: an explicit zero still makes a
 * block).  reorder = 0 keeps rows and columns in place; reorder = 1 first
 * permutes rows and columns so the entries fall into fewer blocks, the
 * row/column permutation before BCSR named on the "Daily Papers" search page
 * (entry on block-sparse SpMM on tensor cores for unstructured matrices):
 * columns ordered by their sorted row lists, then rows by their sorted lists
 * of block columns, both lexicographically; the original order is kept when
 * the permutation does not reduce the block count.  The packed matrix is
 * P_r A P_c^T; the permutations are readable as SPMM_ARRAY_ROW_PERM /
 * SPMM_ARRAY_COL_PERM, and spmm_execute applies them, so C = A * B in the
 * original row and column order.  dtype must be SPMM_BF16; m % block_m == 0
 * and k % block_k == 0; reorder must be 0 or 1 (else INVALID_ARG). */
spmm_status_t spmm_pack_bcsr_csr(int64_t m, int64_t k, spmm_dtype_t dtype,
                                 const int64_t *row_ptr, const int32_t *col_idx,
                                 const void *vals, int32_t block_m, int32_t block_k,
                                 int32_t reorder, spmm_matrix_t *out);

/* Defining passage: the AsyncSparse page, abstract (WCSR for irregular
 * sparsity, large row windows split across thread blocks for load balance)
 * and the summary's "What carries the argument" (windowed irregular
 * sparsity with cross-block row splitting).  The pages give neither window
 * height nor split size; both are arguments here.
 * WCSR from a canonical CSR on the host: row_ptr int64[m+1] with row_ptr[0] = 0,
 * non-decreasing; col_idx int32[nnz] strictly ascending within each row and in
 * [0, k); vals float[nnz] (explicit zeros are kept).  Anything else is
 * INVALID_ARG, never silently fixed.  Rows are grouped into windows of
 * window_rows rows; a window holding at most max_chunk_nnz entries is one
 * chunk (even when empty), a longer one is cut into ceil(nnz_w / T) chunks of
 * T consecutive entries (the last one shorter).  window_rows = 0 picks
 * min(16, max(1, m / 16384)) rows and max_chunk_nnz = 0 picks 512;
 * spmm_matrix_info reports the values used.  dtype must be SPMM_F32. */
spmm_status_t spmm_pack_wcsr(int64_t m, int64_t k, spmm_dtype_t dtype,
                             const int64_t *row_ptr, const int32_t *col_idx,
                             const void *vals, int32_t window_rows,
                             int64_t max_chunk_nnz, spmm_matrix_t *out);

/* Defining passage: "Accelerating Sparse DNNs Based on Tiled GEMM",
 * abstract (the 2:4 pattern the sparse tensor core runs at the register
 * level); "Efficient Quantized Sparse Matrix Operations on Tensor Cores",
 * abstract (SpMM on low-precision integers); the N:M entry of the "Daily
 * Papers" search page (definition of N:M).  The dtype argument goes beyond
 * the int8 case: the same pattern in bf16.
 * 2:4 from a dense row-major matrix a_host [m x k] (lda >= k) of dtype SPMM_I8
 * (int8) or SPMM_BF16 (uint16 bit patterns; else UNSUPPORTED): in every group
 * of 4 consecutive elements of a row keep the two of largest |a| (int8 as
 * integers: |-128| = 128; bf16 in magnitude order, every NaN above infinity
 * and NaNs equal), ties to the lower position, and store them with their
 * 2-bit positions as described above.  Packing an already 2:4 matrix is
 * lossless.  Requires k % 8 == 0. */
spmm_status_t spmm_pack_24(int64_t m, int64_t k, spmm_dtype_t dtype, const void *a_host,
                           int64_t lda, spmm_matrix_t *out);

spmm_status_t spmm_matrix_info(spmm_matrix_t a, spmm_matrix_info_t *info);
/* Read-only view of a canonical array, valid while the matrix lives.
 * *count receives the number of elements.  INVALID_ARG if the format has no
 * such array. */
spmm_status_t spmm_matrix_array(spmm_matrix_t a, int32_t which, const void **data,
                                int64_t *count);
/* Drop the caller's reference (plans keep their own); NULL is ignored. */
void spmm_matrix_destroy(spmm_matrix_t a);

/* ---- plan (host -> device, synchronous) ---- */

/* The pages give no planning step; the plan is where the per-format kernel
 * choice of the AsyncSparse page (abstract: one kernel for block-structured,
 * one for irregular sparsity) and the 2:4 kernel of "Accelerating Sparse
 * DNNs Based on Tiled GEMM" (abstract) are made, once per (A, n).
 * Copy the packed operand to device `device`, choose the kernel and tiles
 * for n columns, and allocate the workspace.  Supported (b_dtype, c_dtype):
 *   BCSR (64 x 64 blocks): (BF16, BF16), n % 8 == 0
 *   WCSR:                  (F32, F32), any n >= 1
 *   2:4, int8:             (I8, I32), n % 16 == 0
 *   2:4, bf16:             (BF16, BF16), n % 16 == 0; fp32 sums rounded to nearest even
 *   TVW, int8 (256 x 128j tiles):  (I8, I32), n % 16 == 0
 *   TVW, bf16 (256 x 64j tiles):   (BF16, BF16), n % 16 == 0; fp32 sums rounded to
 *                                  nearest even
 *   SLIDE:                 (I8, I32), n % 16 == 0 (no workspace)
 * A BCSR matrix packed with reordering reads B's rows through its column
 * permutation (no workspace; spmm_execute then needs k * ldb * 2 < 2^32).
 * Otherwise a BCSR plan may pair block rows that share block columns, so
 * that a workgroup computes two block rows and loads a slab of B they both
 * use once (spmm_plan_info then reports tile_m = 128); the result is the
 * same product.
 * Anything else is UNSUPPORTED.  n = 0 is allowed (execute does nothing).
 * With the environment variable SPMM_LOG set to anything but "" or "0"
 * (read at each call), a plan that succeeds (this call or spmm_plan_sddmm)
 * prints one line of its decisions on stderr: format, kernel(s), tile,
 * grid, schedule, device and workspace bytes. */
spmm_status_t spmm_plan(spmm_matrix_t a, int64_t n, spmm_dtype_t b_dtype,
                        spmm_dtype_t c_dtype, int32_t device, spmm_plan_t *out);

typedef struct {
  int32_t format;
  int32_t device;
  int64_t m, k, n;           /* n: columns of B and C; kd for an SDDMM plan    */
  int64_t device_bytes;     /* packed operand + tables on the device          */
  int64_t workspace_bytes;  /* WCSR partial rows of split windows             */
  int64_t num_split_rows;   /* WCSR rows whose entries span several chunks    */
  int64_t num_slots;        /* WCSR partial rows                              */
  int32_t tile_m, tile_n;   /* output tile of one workgroup                   */
  int64_t grid;             /* workgroups of the main kernel                  */
} spmm_plan_info_t;
spmm_status_t spmm_plan_info(spmm_plan_t p, spmm_plan_info_t *info);
void spmm_plan_destroy(spmm_plan_t p);

/* ---- execute (asynchronous on the caller's stream) ---- */

/* Defining passage: the product SpMM computes, sparse A times dense B, as
 * stated in the AsyncSparse page's abstract (SpMM as a kernel of scientific
 * computing and machine learning) and in the Magicube page's abstract
 * ("Efficient Quantized Sparse Matrix Operations on Tensor Cores").
 * C = A * B on `stream`; every element of C[m x n] is overwritten (rows of A
 * without entries give zeros).  b_dev [k x n] and c_dev [m x n] are device
 * pointers on the plan's device, 16-byte aligned, with ldb >= n, ldc >= n and
 * ldb * elem, ldc * elem multiples of 16 bytes.  Allocates nothing and does
 * not synchronise; launch errors are returned, faults surface at the caller's
 * next synchronisation.  A plan's workspace allows one execute in flight at a
 * time: concurrent streams need separate plans.  B and C must not overlap.
 * The kernels address B with 32-bit byte offsets: BCSR needs ldb <= 2^24
 * (and k * ldb * 2 < 2^32 when packed with reordering); 2:4, TVW and SLIDE
 * need k_pad * ldb * elem < 2^32, k_pad being k (k_lift for SLIDE) rounded up
 * to the k-step of 128 (int8) or 64 (bf16).  Larger ldb returns UNSUPPORTED
 * before anything is launched. */
spmm_status_t spmm_execute(spmm_plan_t p, const void *b_dev, int64_t ldb, void *c_dev,
                           int64_t ldc, hipStream_t stream);

/* For callers that cannot allocate device memory while they run: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same as spmm_execute (same checks, kernels and results), except that the
 * partial rows of a WCSR plan's split rows (num_slots * n * 4 bytes, see
 * spmm_plan_info) are kept in a fixed scratch array of 32 MiB per GPU inside
 * the library instead of the plan's workspace; other formats use no scratch.
 * Allocates nothing: the array is part of the library's device image, held
 * by every GPU the library runs on until the process ends.  A plan needing
 * more than 32 MiB returns UNSUPPORTED before anything is launched.  Every
 * call on one GPU shares that GPU's array, and a call leaves its partial rows
 * there: calls that overlap on one GPU (concurrent streams, or host threads
 * launching at once) race and give wrong results; order them on one stream
 * or use spmm_execute with separate plans. */
spmm_status_t spmm_execute_noalloc(spmm_plan_t p, const void *b_dev, int64_t ldb, void *c_dev,
                                   int64_t ldc, hipStream_t stream);

/* ---- sampled dense-dense product (SDDMM) ---- */

/* Plan out[p] = sum over t < kd of X[i][t] * Y[j][t] for every stored entry
 * p = (i, j) of the matrix a: its stored pattern is the sample mask and its
 * values play no part.  SDDMM is the companion of SpMM on the Magicube page
 * ("Efficient Quantized Sparse Matrix Operations on Tensor Cores",
 * abstract), which runs both on low-precision integers.  Two patterns:
 *   - WCSR with dtype SPMM_F32 (X, Y and out fp32), SPMM_BF16 (X, Y bf16;
 *     fp32 sums; out bf16, rounded to nearest even) or SPMM_I8 (X, Y int8;
 *     out int32, exact while |sum| < 2^31): out holds one value per stored
 *     entry in stored order ([nnz]); work is split by a's chunks;
 *   - BCSR of 64 x 64 blocks with dtype SPMM_BF16 (X, Y bf16; fp32 sums;
 *     out bf16, rounded to nearest even) or SPMM_I8 (X, Y int8; out int32,
 *     exact while |sum| < 2^31): every element of every stored block is
 *     sampled and out has the layout of the block values, [nnzb][64][64]
 *     row-major inside a block, in stored block order.  The plan may hold a
 *     workspace of fp32 / int32 partial blocks (workspace_bytes).
 * Anything else is UNSUPPORTED.  Synchronous; the plan holds a reference on
 * a.  kd = 0 is allowed (out becomes zeros). */
spmm_status_t spmm_plan_sddmm(spmm_matrix_t a, int64_t kd, spmm_dtype_t dtype, int32_t device,
                              spmm_plan_t *out);

/* out_dev for every stored entry of the plan's pattern, on `stream`.
 * x_dev [m x kd] and y_dev [k x kd] are row-major device arrays of the plan's
 * element type on the plan's device, 16-byte aligned, with ldx, ldy >= kd
 * (elements) and ldx * elem, ldy * elem multiples of 16 bytes (with kd = 0
 * X, Y and their ld are not read); for a BCSR pattern 64 * ldx * elem and
 * 64 * ldy * elem must stay below 4 GiB (else UNSUPPORTED).  out_dev is aligned to its
 * element (WCSR: 4 bytes for fp32 and int32, 2 for bf16) or to 16 bytes (BCSR).  Allocates nothing and does not synchronise; one
 * execute in flight per plan (the workspace).  Plans of spmm_plan are
 * refused here and SDDMM plans by spmm_execute (INVALID_ARG). */
spmm_status_t spmm_execute_sddmm(spmm_plan_t p, const void *x_dev, int64_t ldx, const void *y_dev,
                                 int64_t ldy, void *out_dev, hipStream_t stream);

/* ---- errors ---- */
const char *spmm_status_str(spmm_status_t s);
/* Message of the last failing call on this thread ("" if none). */
const char *spmm_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* SPMM_H */

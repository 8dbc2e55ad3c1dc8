/*
 * oracle.h -- CPU reference for C = A_sparse * B_dense.
 *
 * TEST INFRASTRUCTURE.  This library exists to check the HIP path; only the
 * test suite, the smoke check and the benchmark's CPU-baseline leg may load
 * it.  It shares no code, header, table or helper with the HIP library, and
 * the HIP library never calls it.
 *
 * Everything here is a plain loop, in the order the definition states:
 *   - floating point is widened exactly to double and summed in double, over
 *     the stored entries of a row in ascending column order;
 *   - int8 products are formed in int32 and summed in int64.
 * OpenMP splits work over output rows only, so no element's summation order
 * depends on the thread count.
 *
 * Sources (cited by page title and the part of the page):
 *   [AS]  "AsyncSparse: Accelerating Sparse Matrix-Matrix Multiplication on
 *         Asynchronous GPU Architectures" -- abstract; Figure 2 caption
 *         (BCSR vs WCSR formats); summary paragraph "What carries the
 *         argument" (row-window splitting across thread blocks).
 *   [MC]  "Efficient Quantized Sparse Matrix Operations on Tensor Cores" --
 *         abstract (SpMM on low-precision integers; SDDMM, the sampled
 *         dense-dense product, as its companion operation).
 *   [TW]  "Accelerating Sparse DNNs Based on Tiled GEMM" -- abstract (the 2:4
 *         pattern of the sparse tensor core; tile-wise sparsity).
 *   [DP]  "Daily Papers" search page for sparse FP4 GEMM -- the entry on
 *         block-sparse SpMM for Transformer inference on CPUs (SpMM as sparse
 *         matrix times dense matrix) and the entry on N:M sparse training
 *         (N of every M consecutive elements nonzero).
 */
#ifndef SDM_ORACLE_H
#define SDM_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- exact conversions ------------------------------------------------- */
double orc_bf16_to_double(uint16_t h);

/* ---- BCSR packing [AS abstract, Fig. 2] -------------------------------- */
/* Count the bm x bk blocks of the dense row-major bf16 matrix that hold at
 * least one nonzero (bits & 0x7FFF != 0: +0 and -0 are zero, NaN is not).
 * Returns the count, or -1 when m % bm or k % bk is nonzero or lda < k. */
int64_t orc_bcsr_count(int64_t m, int64_t k, int32_t bm, int32_t bk,
                       const uint16_t *a, int64_t lda);
/* Fill row_ptr[m/bm + 1], col_idx[nnzb], vals[nnzb * bm * bk] (each block
 * row-major), block rows ascending, block columns ascending. */
void orc_bcsr_fill(int64_t m, int64_t k, int32_t bm, int32_t bk,
                   const uint16_t *a, int64_t lda,
                   int32_t *row_ptr, int32_t *col_idx, uint16_t *vals);
/* Dense double image of a BCSR matrix (for brute-force checks). */
void orc_bcsr_densify(int64_t m, int64_t k, int32_t bm, int32_t bk,
                      const int32_t *row_ptr, const int32_t *col_idx,
                      const uint16_t *vals, double *out);

/* ---- CSR validation and row windows [AS abstract, Fig. 2] --------------- */
/* 0 if canonical; otherwise a positive code:
 *   1 row_ptr[0] != 0     2 row_ptr decreasing     3 row_ptr[m] != nnz
 *   4 column out of [0,k) 5 columns not strictly ascending in a row */
int orc_csr_check(int64_t m, int64_t k, int64_t nnz,
                  const int64_t *row_ptr, const int32_t *col_idx);
/* Number of chunks when windows of W rows are cut into pieces of at most T
 * stored entries: each window contributes max(1, ceil(nnz_w / T)). */
int64_t orc_wcsr_num_chunks(int64_t m, const int64_t *row_ptr, int32_t W, int64_t T);
/* chunk_window[C] and chunk_begin[C + 1] (last entry = nnz). */
void orc_wcsr_chunks(int64_t m, const int64_t *row_ptr, int32_t W, int64_t T,
                     int32_t *chunk_window, int64_t *chunk_begin);
void orc_csr_densify(int64_t m, int64_t k, const int64_t *row_ptr,
                     const int32_t *col_idx, const float *vals, double *out);

/* ---- 2:4 packing [TW abstract; DP N:M entry] ---------------------------- */
/* For every group of 4 consecutive elements along k keep the two of largest
 * |a| (as int, so -128 -> 128), ties to the lower index, stored in ascending
 * index order: vals[i*(k/2) + 2g + {0,1}], and the two 2-bit positions as the
 * nibble (i0 | i1 << 2) of meta[i*(k/8) + g/2], low nibble for even g.
 * Returns 0, or -1 when k % 8 != 0 or lda < k. */
int orc_pack24(int64_t m, int64_t k, const int8_t *a, int64_t lda,
               int8_t *vals, uint8_t *meta);
void orc_densify24(int64_t m, int64_t k, const int8_t *vals, const uint8_t *meta,
                   int8_t *out);

/* N:M pruning: keep the `keep` largest |a| of every `group` consecutive
 * elements of a row (ties to the lower position), zero the rest; out is
 * dense int8 [m][k].  Returns -1 for a bad group (k % group != 0, group > 64). */
int orc_prune_nm(int64_t m, int64_t k, const int8_t *a, int64_t lda, int keep, int group,
                 int8_t *out);

/* The same rule for bf16 bit patterns [TW abstract; DP N:M entry]: rank by
 * |a| as a real number, NaN above every number and NaNs equal, ties to the
 * lower position; dropped elements become +0 (bits 0).  Same return codes. */
int orc_prune_nm_bf16(int64_t m, int64_t k, const uint16_t *a, int64_t lda, int keep, int group,
                      uint16_t *out);

/* ---- reference products [AS abstract; MC abstract; DP SpMM entry] ------- */
/* out[r][j - j0] = sum over stored (rows[r], c) in ascending c of
 * A[rows[r]][c] * B[c][j], for j in [j0, j1).  out is row-major with
 * (j1 - j0) columns. */
void orc_csr_spmm_rows(const int64_t *row_ptr, const int32_t *col_idx, const float *vals,
                       const float *B, int64_t ldb,
                       int64_t nrows, const int64_t *rows, int64_t j0, int64_t j1,
                       double *out);
void orc_bcsr_spmm_rows(int32_t bm, int32_t bk, const int32_t *row_ptr,
                        const int32_t *col_idx, const uint16_t *vals,
                        const uint16_t *B, int64_t ldb,
                        int64_t nrows, const int64_t *rows, int64_t j0, int64_t j1,
                        double *out);
/* int8 2:4: returns the number of sums with |sum| >= 2^31 (0 when exact). */
int64_t orc_sp24_spmm_rows(int64_t k, const int8_t *vals, const uint8_t *meta,
                           const int8_t *B, int64_t ldb,
                           int64_t nrows, const int64_t *rows, int64_t j0, int64_t j1,
                           int32_t *out);

/* ---- sampled dense-dense product [MC abstract: SDDMM] ---------------------- */
/* out[p] = sum over t ascending of X[i][t] * Y[j][t] (fp64), for every stored
 * entry p = (i, j) of the CSR pattern (row_ptr, col_idx) whose row i is in
 * rows[0 .. nrows); out holds the entries of those rows in stored order.
 * The pattern's values play no part: it is the sample mask. */
void orc_sddmm_rows(const int64_t *row_ptr, const int32_t *col_idx,
                    const float *X, int64_t ldx, const float *Y, int64_t ldy, int64_t kd,
                    int64_t nrows, const int64_t *rows, double *out);

/* The same product with a BCSR block pattern (row_ptr over nbrows block rows,
 * col_idx block columns) as the mask: for each block b in blocks[0 .. nsel),
 * out[q][i][j] = sum over t ascending of X[I*bm + i][t] * Y[J*bk + j][t],
 * with (I, J) the block's block row and column.  bf16 operands are widened
 * exactly and summed in fp64; int8 products are formed in int32 and summed in
 * int64 (the return value counts sums with |sum| >= 2^31; 0 when exact). */
void orc_sddmm_bcsr_bf16(int32_t bm, int32_t bk, const int32_t *row_ptr, const int32_t *col_idx,
                         int64_t nbrows, const uint16_t *X, int64_t ldx, const uint16_t *Y,
                         int64_t ldy, int64_t kd, int64_t nsel, const int64_t *blocks,
                         double *out);
int64_t orc_sddmm_bcsr_i8(int32_t bm, int32_t bk, const int32_t *row_ptr, const int32_t *col_idx,
                          int64_t nbrows, const int8_t *X, int64_t ldx, const int8_t *Y,
                          int64_t ldy, int64_t kd, int64_t nsel, const int64_t *blocks,
                          int32_t *out);

/* ---- brute force (dense, naive triple loops) ---------------------------- */
void orc_gemm_f64(int64_t m, int64_t k, int64_t n, const double *A, const double *B,
                  double *C);
void orc_gemm_i8(int64_t m, int64_t k, int64_t n, const int8_t *A, const int8_t *B,
                 int64_t *C);

/* Number of OpenMP threads the reference loops use. */
int orc_num_threads(void);

/* ---- row/column permutation before BCSR [DP: block-sparse SpMM on tensor
 * cores for unstructured matrices; the goal named there is fewer nonzero
 * blocks, the method below is this build's reading of it] ----------------
 * For a CSR pattern (m x k): every column's list of rows, ascending; columns
 * ordered by those lists compared lexicographically (a list that is a prefix
 * of another comes first, so empty columns lead; equal lists by column
 * index).  Then every row's list of distinct block columns (bk wide) under the
 * new column order, ascending; rows ordered the same way.  The permutation is
 * kept only when the permuted matrix occupies fewer bm x bk blocks than the
 * original.  Outputs: row_perm[i'] = original row of row i', col_perm[j'] =
 * original column of column j' (the identity when not kept), and the block
 * counts before and after.  Returns 1 when kept, 0 when not (and for a
 * matrix with no entries). */
int orc_reorder_perms(int64_t m, int64_t k, const int64_t *row_ptr, const int32_t *col_idx,
                      int32_t bm, int32_t bk, int32_t *row_perm, int32_t *col_perm,
                      int64_t *blocks_before, int64_t *blocks_after);

#ifdef __cplusplus
}
#endif
#endif

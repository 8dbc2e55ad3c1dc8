/*
 * oracle.c -- plain CPU reference for C = A_sparse * B_dense.
 *
 * TEST INFRASTRUCTURE: loaded only by the test suite, the smoke check and the
 * benchmark's CPU-baseline leg.  Nothing in the HIP library links or calls it.
 * See oracle.h for the sources each function follows.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

double orc_bf16_to_double(uint16_t h) {
  /* bf16 is the top half of an IEEE binary32: widening is a shift. */
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* ------------------------------------------------------------------------ */
/* BCSR: block compressed sparse row [AS abstract, Fig. 2].  A block is kept  */
/* when any of its elements is numerically nonzero.                           */
/* ------------------------------------------------------------------------ */
static int block_is_nonzero(const uint16_t *a, int64_t lda, int64_t r0, int64_t c0,
                            int32_t bm, int32_t bk) {
  for (int64_t i = 0; i < bm; ++i)
    for (int64_t j = 0; j < bk; ++j)
      if ((a[(r0 + i) * lda + c0 + j] & 0x7FFFu) != 0) return 1;
  return 0;
}

int64_t orc_bcsr_count(int64_t m, int64_t k, int32_t bm, int32_t bk,
                       const uint16_t *a, int64_t lda) {
  if (bm <= 0 || bk <= 0 || m % bm != 0 || k % bk != 0 || lda < k) return -1;
  int64_t count = 0;
  for (int64_t br = 0; br < m / bm; ++br)
    for (int64_t bc = 0; bc < k / bk; ++bc)
      count += block_is_nonzero(a, lda, br * bm, bc * bk, bm, bk);
  return count;
}

void orc_bcsr_fill(int64_t m, int64_t k, int32_t bm, int32_t bk,
                   const uint16_t *a, int64_t lda,
                   int32_t *row_ptr, int32_t *col_idx, uint16_t *vals) {
  int64_t nb = 0;
  row_ptr[0] = 0;
  for (int64_t br = 0; br < m / bm; ++br) {
    for (int64_t bc = 0; bc < k / bk; ++bc) {
      if (!block_is_nonzero(a, lda, br * bm, bc * bk, bm, bk)) continue;
      col_idx[nb] = (int32_t)bc;
      uint16_t *dst = vals + nb * (int64_t)bm * bk;
      for (int64_t i = 0; i < bm; ++i)
        for (int64_t j = 0; j < bk; ++j)
          dst[i * bk + j] = a[(br * bm + i) * lda + bc * bk + j];
      ++nb;
    }
    row_ptr[br + 1] = (int32_t)nb;
  }
}

void orc_bcsr_densify(int64_t m, int64_t k, int32_t bm, int32_t bk,
                      const int32_t *row_ptr, const int32_t *col_idx,
                      const uint16_t *vals, double *out) {
  for (int64_t i = 0; i < m * k; ++i) out[i] = 0.0;
  for (int64_t br = 0; br < m / bm; ++br)
    for (int64_t p = row_ptr[br]; p < row_ptr[br + 1]; ++p) {
      const uint16_t *blk = vals + p * (int64_t)bm * bk;
      for (int64_t i = 0; i < bm; ++i)
        for (int64_t j = 0; j < bk; ++j)
          out[(br * bm + i) * k + (int64_t)col_idx[p] * bk + j] =
              orc_bf16_to_double(blk[i * bk + j]);
    }
}

/* ------------------------------------------------------------------------ */
/* CSR and row windows [AS abstract, Fig. 2, "What carries the argument"].   */
/* Windows are W consecutive rows; a window whose stored entries exceed T is */
/* cut into consecutive pieces of T entries so separate workgroups can take  */
/* them.                                                                      */
/* ------------------------------------------------------------------------ */
int orc_csr_check(int64_t m, int64_t k, int64_t nnz,
                  const int64_t *row_ptr, const int32_t *col_idx) {
  if (row_ptr[0] != 0) return 1;
  for (int64_t i = 0; i < m; ++i)
    if (row_ptr[i + 1] < row_ptr[i]) return 2;
  if (row_ptr[m] != nnz) return 3;
  for (int64_t i = 0; i < m; ++i)
    for (int64_t p = row_ptr[i]; p < row_ptr[i + 1]; ++p) {
      if (col_idx[p] < 0 || col_idx[p] >= k) return 4;
      if (p > row_ptr[i] && col_idx[p] <= col_idx[p - 1]) return 5;
    }
  return 0;
}

static int64_t window_chunks(int64_t e_minus_s, int64_t T) {
  if (e_minus_s <= T) return 1;
  return (e_minus_s + T - 1) / T;
}

int64_t orc_wcsr_num_chunks(int64_t m, const int64_t *row_ptr, int32_t W, int64_t T) {
  int64_t total = 0;
  for (int64_t r0 = 0; r0 < m; r0 += W) {
    int64_t r1 = r0 + W < m ? r0 + W : m;
    total += window_chunks(row_ptr[r1] - row_ptr[r0], T);
  }
  return total;
}

void orc_wcsr_chunks(int64_t m, const int64_t *row_ptr, int32_t W, int64_t T,
                     int32_t *chunk_window, int64_t *chunk_begin) {
  int64_t c = 0;
  int64_t w = 0;
  for (int64_t r0 = 0; r0 < m; r0 += W, ++w) {
    int64_t r1 = r0 + W < m ? r0 + W : m;
    int64_t s = row_ptr[r0], e = row_ptr[r1];
    int64_t pieces = window_chunks(e - s, T);
    for (int64_t q = 0; q < pieces; ++q) {
      chunk_window[c] = (int32_t)w;
      chunk_begin[c] = s + q * T;
      ++c;
    }
  }
  chunk_begin[c] = row_ptr[m];
}

void orc_csr_densify(int64_t m, int64_t k, const int64_t *row_ptr,
                     const int32_t *col_idx, const float *vals, double *out) {
  for (int64_t i = 0; i < m * k; ++i) out[i] = 0.0;
  for (int64_t i = 0; i < m; ++i)
    for (int64_t p = row_ptr[i]; p < row_ptr[i + 1]; ++p)
      out[i * k + col_idx[p]] = (double)vals[p];
}

/* ------------------------------------------------------------------------ */
/* 2:4 structured sparsity [TW abstract; DP N:M entry]: in every 4          */
/* consecutive elements along k at most 2 are nonzero.  Pruning keeps the two */
/* largest magnitudes of each group.                                          */
/* ------------------------------------------------------------------------ */
int orc_pack24(int64_t m, int64_t k, const int8_t *a, int64_t lda,
               int8_t *vals, uint8_t *meta) {
  if (k % 8 != 0 || lda < k) return -1;
  for (int64_t i = 0; i < m; ++i) {
    for (int64_t i8 = 0; i8 < k / 8; ++i8) meta[i * (k / 8) + i8] = 0;
    for (int64_t g = 0; g < k / 4; ++g) {
      const int8_t *grp = a + i * lda + 4 * g;
      /* rank the four positions by (larger |a| first, then lower index) */
      int order[4] = {0, 1, 2, 3};
      for (int x = 0; x < 4; ++x)
        for (int y = x + 1; y < 4; ++y) {
          int ax = abs((int)grp[order[x]]), ay = abs((int)grp[order[y]]);
          int y_first = ay > ax || (ay == ax && order[y] < order[x]);
          if (y_first) {
            int t = order[x];
            order[x] = order[y];
            order[y] = t;
          }
        }
      int i0 = order[0] < order[1] ? order[0] : order[1];
      int i1 = order[0] < order[1] ? order[1] : order[0];
      vals[i * (k / 2) + 2 * g] = grp[i0];
      vals[i * (k / 2) + 2 * g + 1] = grp[i1];
      uint8_t nib = (uint8_t)(i0 | (i1 << 2));
      meta[i * (k / 8) + g / 2] |= (uint8_t)((g % 2 == 0) ? nib : (nib << 4));
    }
  }
  return 0;
}

void orc_densify24(int64_t m, int64_t k, const int8_t *vals, const uint8_t *meta,
                   int8_t *out) {
  for (int64_t i = 0; i < m; ++i)
    for (int64_t g = 0; g < k / 4; ++g) {
      uint8_t byte = meta[i * (k / 8) + g / 2];
      uint8_t nib = (g % 2 == 0) ? (byte & 0xF) : (byte >> 4);
      int i0 = nib & 3, i1 = (nib >> 2) & 3;
      for (int t = 0; t < 4; ++t) out[i * k + 4 * g + t] = 0;
      out[i * k + 4 * g + i0] = vals[i * (k / 2) + 2 * g];
      out[i * k + 4 * g + i1] = vals[i * (k / 2) + 2 * g + 1];
    }
}

/* ------------------------------------------------------------------------ */
/* Reference products: C = A * B for the A each format stores              */
/* [AS abstract; MC abstract; DP SpMM entry].                                */
/* ------------------------------------------------------------------------ */
void orc_csr_spmm_rows(const int64_t *row_ptr, const int32_t *col_idx, const float *vals,
                       const float *B, int64_t ldb,
                       int64_t nrows, const int64_t *rows, int64_t j0, int64_t j1,
                       double *out) {
  const int64_t w = j1 - j0;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t r = 0; r < nrows; ++r) {
    double *o = out + r * w;
    for (int64_t j = 0; j < w; ++j) o[j] = 0.0;
    const int64_t i = rows[r];
    for (int64_t p = row_ptr[i]; p < row_ptr[i + 1]; ++p) {
      const double a = (double)vals[p];
      const float *b = B + (int64_t)col_idx[p] * ldb + j0;
      for (int64_t j = 0; j < w; ++j) o[j] += a * (double)b[j];
    }
  }
}

void orc_bcsr_spmm_rows(int32_t bm, int32_t bk, const int32_t *row_ptr,
                        const int32_t *col_idx, const uint16_t *vals,
                        const uint16_t *B, int64_t ldb,
                        int64_t nrows, const int64_t *rows, int64_t j0, int64_t j1,
                        double *out) {
  const int64_t w = j1 - j0;
#pragma omp parallel
  {
    double *brow = (double *)malloc(sizeof(double) * (size_t)(w > 0 ? w : 1));
#pragma omp for schedule(dynamic, 4)
    for (int64_t r = 0; r < nrows; ++r) {
      double *o = out + r * w;
      for (int64_t j = 0; j < w; ++j) o[j] = 0.0;
      const int64_t i = rows[r];
      const int64_t br = i / bm, ii = i % bm;
      /* blocks of the block row in ascending block column, then the block's
       * columns ascending: stored entries in ascending column order */
      for (int64_t p = row_ptr[br]; p < row_ptr[br + 1]; ++p) {
        const uint16_t *arow = vals + p * (int64_t)bm * bk + ii * bk;
        for (int64_t t = 0; t < bk; ++t) {
          const double a = orc_bf16_to_double(arow[t]);
          const uint16_t *b = B + ((int64_t)col_idx[p] * bk + t) * ldb + j0;
          for (int64_t j = 0; j < w; ++j) brow[j] = orc_bf16_to_double(b[j]);
          for (int64_t j = 0; j < w; ++j) o[j] += a * brow[j];
        }
      }
    }
    free(brow);
  }
}

int64_t orc_sp24_spmm_rows(int64_t k, const int8_t *vals, const uint8_t *meta,
                           const int8_t *B, int64_t ldb,
                           int64_t nrows, const int64_t *rows, int64_t j0, int64_t j1,
                           int32_t *out) {
  const int64_t w = j1 - j0;
  int64_t overflow = 0;
#pragma omp parallel
  {
    int64_t *acc = (int64_t *)malloc(sizeof(int64_t) * (size_t)(w > 0 ? w : 1));
#pragma omp for schedule(dynamic, 4) reduction(+ : overflow)
    for (int64_t r = 0; r < nrows; ++r) {
      for (int64_t j = 0; j < w; ++j) acc[j] = 0;
      const int64_t i = rows[r];
      for (int64_t g = 0; g < k / 4; ++g) {
        const uint8_t byte = meta[i * (k / 8) + g / 2];
        const uint8_t nib = (g % 2 == 0) ? (byte & 0xF) : (byte >> 4);
        const int64_t kk[2] = {4 * g + (nib & 3), 4 * g + ((nib >> 2) & 3)};
        for (int s = 0; s < 2; ++s) {
          const int32_t a = vals[i * (k / 2) + 2 * g + s];
          const int8_t *b = B + kk[s] * ldb + j0;
          for (int64_t j = 0; j < w; ++j) acc[j] += (int64_t)(a * (int32_t)b[j]);
        }
      }
      for (int64_t j = 0; j < w; ++j) {
        if (acc[j] >= 2147483648LL || acc[j] < -2147483648LL) ++overflow;
        out[r * w + j] = (int32_t)acc[j];
      }
    }
    free(acc);
  }
  return overflow;
}

/* ------------------------------------------------------------------------ */
/* Sampled dense-dense product [MC abstract]: the dense product X * Y^T is   */
/* evaluated only where the sparse pattern stores an entry.                  */
/* ------------------------------------------------------------------------ */
void orc_sddmm_rows(const int64_t *row_ptr, const int32_t *col_idx,
                    const float *X, int64_t ldx, const float *Y, int64_t ldy, int64_t kd,
                    int64_t nrows, const int64_t *rows, double *out) {
  /* output offset of each requested row */
  int64_t *off = (int64_t *)malloc(sizeof(int64_t) * (size_t)(nrows + 1));
  off[0] = 0;
  for (int64_t r = 0; r < nrows; ++r)
    off[r + 1] = off[r] + (row_ptr[rows[r] + 1] - row_ptr[rows[r]]);
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t i = rows[r];
    const float *x = X + i * ldx;
    for (int64_t p = row_ptr[i]; p < row_ptr[i + 1]; ++p) {
      const float *y = Y + (int64_t)col_idx[p] * ldy;
      double s = 0.0;
      for (int64_t t = 0; t < kd; ++t) s += (double)x[t] * (double)y[t];
      out[off[r] + (p - row_ptr[i])] = s;
    }
  }
  free(off);
}

/* Block-pattern SDDMM: the sample mask is a BCSR pattern, every element of */
/* every stored block is sampled, and the result has the layout of the       */
/* block values (block by block, row-major inside a block).                  */
static int64_t *block_rows(const int32_t *row_ptr, int64_t nbrows) {
  const int64_t nnzb = row_ptr[nbrows];
  int64_t *br = (int64_t *)malloc(sizeof(int64_t) * (size_t)(nnzb > 0 ? nnzb : 1));
  for (int64_t r = 0; r < nbrows; ++r)
    for (int64_t b = row_ptr[r]; b < row_ptr[r + 1]; ++b) br[b] = r;
  return br;
}

void orc_sddmm_bcsr_bf16(int32_t bm, int32_t bk, const int32_t *row_ptr, const int32_t *col_idx,
                         int64_t nbrows, const uint16_t *X, int64_t ldx, const uint16_t *Y,
                         int64_t ldy, int64_t kd, int64_t nsel, const int64_t *blocks,
                         double *out) {
  int64_t *br = block_rows(row_ptr, nbrows);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t q = 0; q < nsel; ++q) {
    const int64_t b = blocks[q];
    for (int64_t i = 0; i < bm; ++i) {
      const uint16_t *x = X + (br[b] * bm + i) * ldx;
      for (int64_t j = 0; j < bk; ++j) {
        const uint16_t *y = Y + ((int64_t)col_idx[b] * bk + j) * ldy;
        double s = 0.0;
        for (int64_t t = 0; t < kd; ++t) s += orc_bf16_to_double(x[t]) * orc_bf16_to_double(y[t]);
        out[(q * bm + i) * bk + j] = s;
      }
    }
  }
  free(br);
}

int64_t orc_sddmm_bcsr_i8(int32_t bm, int32_t bk, const int32_t *row_ptr, const int32_t *col_idx,
                          int64_t nbrows, const int8_t *X, int64_t ldx, const int8_t *Y,
                          int64_t ldy, int64_t kd, int64_t nsel, const int64_t *blocks,
                          int32_t *out) {
  int64_t *br = block_rows(row_ptr, nbrows);
  int64_t overflow = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : overflow)
  for (int64_t q = 0; q < nsel; ++q) {
    const int64_t b = blocks[q];
    for (int64_t i = 0; i < bm; ++i) {
      const int8_t *x = X + (br[b] * bm + i) * ldx;
      for (int64_t j = 0; j < bk; ++j) {
        const int8_t *y = Y + ((int64_t)col_idx[b] * bk + j) * ldy;
        int64_t s = 0;
        for (int64_t t = 0; t < kd; ++t) s += (int64_t)((int32_t)x[t] * (int32_t)y[t]);
        if (s >= 2147483648LL || s < -2147483648LL) ++overflow;
        out[(q * bm + i) * bk + j] = (int32_t)s;
      }
    }
  }
  free(br);
  return overflow;
}

/* N:M pruning [DP N:M entry; the (2N-2):2N family on the same page]: in    */
/* every group of `group` consecutive elements of a row keep the `keep` of   */
/* largest |a| (as integers: |-128| = 128), ties to the lower position; the  */
/* others become zero.  keep = 2, group = 4 is the 2:4 rule above.            */
int orc_prune_nm(int64_t m, int64_t k, const int8_t *a, int64_t lda, int keep, int group,
                 int8_t *out) {
  if (group <= 0 || group > 64 || keep < 0 || keep > group || k % group != 0 || lda < k) return -1;
  for (int64_t i = 0; i < m; ++i)
    for (int64_t g = 0; g < k / group; ++g) {
      const int8_t *grp = a + i * lda + g * group;
      int8_t *dst = out + i * k + g * group;
      /* position t is kept iff fewer than `keep` positions rank before it,
         where u ranks before t when |a_u| > |a_t|, or equal and u < t */
      for (int t = 0; t < group; ++t) {
        int before = 0;
        const int at = abs((int)grp[t]);
        for (int u = 0; u < group; ++u) {
          const int au = abs((int)grp[u]);
          if (au > at || (au == at && u < t)) ++before;
        }
        dst[t] = before < keep ? grp[t] : 0;
      }
    }
  return 0;
}

/* 1 when bf16 u has the larger magnitude than bf16 t: compared as real
 * numbers in double, a NaN above every number, two NaNs equal */
static int bf16_mag_above(uint16_t u, uint16_t t) {
  const double du = orc_bf16_to_double(u), dt = orc_bf16_to_double(t);
  const int nu = du != du, nt = dt != dt;
  if (nu || nt) return nu && !nt;
  return fabs(du) > fabs(dt);
}

int orc_prune_nm_bf16(int64_t m, int64_t k, const uint16_t *a, int64_t lda, int keep, int group,
                      uint16_t *out) {
  if (group <= 0 || group > 64 || keep < 0 || keep > group || k % group != 0 || lda < k) return -1;
#pragma omp parallel for
  for (int64_t i = 0; i < m; ++i)
    for (int64_t g = 0; g < k / group; ++g) {
      const uint16_t *grp = a + i * lda + g * group;
      uint16_t *dst = out + i * k + g * group;
      /* as for int8: t is kept iff fewer than `keep` positions rank before it */
      for (int t = 0; t < group; ++t) {
        int before = 0;
        for (int u = 0; u < group; ++u)
          if (bf16_mag_above(grp[u], grp[t]) || (!bf16_mag_above(grp[t], grp[u]) && u < t))
            ++before;
        dst[t] = before < keep ? grp[t] : (uint16_t)0;
      }
    }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Brute force: dense naive triple loops, i then j then k.                   */
/* ------------------------------------------------------------------------ */
void orc_gemm_f64(int64_t m, int64_t k, int64_t n, const double *A, const double *B,
                  double *C) {
#pragma omp parallel for
  for (int64_t i = 0; i < m; ++i)
    for (int64_t j = 0; j < n; ++j) {
      double s = 0.0;
      for (int64_t t = 0; t < k; ++t) s += A[i * k + t] * B[t * n + j];
      C[i * n + j] = s;
    }
}

void orc_gemm_i8(int64_t m, int64_t k, int64_t n, const int8_t *A, const int8_t *B,
                 int64_t *C) {
#pragma omp parallel for
  for (int64_t i = 0; i < m; ++i)
    for (int64_t j = 0; j < n; ++j) {
      int64_t s = 0;
      for (int64_t t = 0; t < k; ++t) s += (int64_t)A[i * k + t] * (int64_t)B[t * n + j];
      C[i * n + j] = s;
    }
}

/* ---- row/column permutation before BCSR (see oracle.h) ----------------- */

/* lexicographic comparison of two ascending lists; a prefix comes first */
static int orc_list_less(const int32_t *a, int64_t na, const int32_t *b, int64_t nb) {
  for (int64_t t = 0; t < na && t < nb; ++t)
    if (a[t] != b[t]) return a[t] < b[t];
  return na < nb;
}

/* stable insertion sort of ids 0..n-1 by their lists (list of id i:
 * val[ptr[i] .. ptr[i+1])); equal lists keep ascending id */
static void orc_order_by_lists(int64_t n, const int64_t *ptr, const int32_t *val, int32_t *order) {
  for (int64_t i = 0; i < n; ++i) {
    int64_t j = i;
    while (j > 0 && orc_list_less(val + ptr[i], ptr[i + 1] - ptr[i], val + ptr[order[j - 1]],
                                  ptr[order[j - 1] + 1] - ptr[order[j - 1]])) {
      order[j] = order[j - 1];
      --j;
    }
    order[j] = (int32_t)i;
  }
}

/* distinct (block row, block column) pairs of the pattern with row i placed
 * at rowpos[i] and column j at colpos[j] */
static int64_t orc_count_blocks(int64_t m, int64_t k, const int64_t *row_ptr, const int32_t *col_idx,
                                const int32_t *rowpos, const int32_t *colpos, int32_t bm, int32_t bk) {
  const int64_t mb = (m + bm - 1) / bm, kb = (k + bk - 1) / bk;
  unsigned char *mask = (unsigned char *)calloc((size_t)(mb * kb > 0 ? mb * kb : 1), 1);
  int64_t count = 0;
  for (int64_t i = 0; i < m; ++i)
    for (int64_t p = row_ptr[i]; p < row_ptr[i + 1]; ++p) {
      const int64_t cell = (rowpos[i] / bm) * kb + colpos[col_idx[p]] / bk;
      if (!mask[cell]) {
        mask[cell] = 1;
        ++count;
      }
    }
  free(mask);
  return count;
}

int orc_reorder_perms(int64_t m, int64_t k, const int64_t *row_ptr, const int32_t *col_idx,
                      int32_t bm, int32_t bk, int32_t *row_perm, int32_t *col_perm,
                      int64_t *blocks_before, int64_t *blocks_after) {
  const int64_t nnz = row_ptr[m];
  int32_t *ident_r = (int32_t *)calloc((size_t)(m > 0 ? m : 1), sizeof(int32_t));
  int32_t *ident_c = (int32_t *)calloc((size_t)(k > 0 ? k : 1), sizeof(int32_t));
  for (int64_t i = 0; i < m; ++i) ident_r[i] = (int32_t)i;
  for (int64_t j = 0; j < k; ++j) ident_c[j] = (int32_t)j;
  *blocks_before = orc_count_blocks(m, k, row_ptr, col_idx, ident_r, ident_c, bm, bk);
  *blocks_after = *blocks_before;
  int kept = 0;
  for (int64_t i = 0; i < m; ++i) row_perm[i] = (int32_t)i;
  for (int64_t j = 0; j < k; ++j) col_perm[j] = (int32_t)j;
  if (nnz > 0) {
    /* 1. each column's rows, ascending: scan the rows in order */
    int64_t *cptr = (int64_t *)calloc((size_t)(k + 1), sizeof(int64_t));
    int32_t *crow = (int32_t *)calloc((size_t)nnz, sizeof(int32_t));
    for (int64_t j = 0; j < k; ++j) {
      cptr[j + 1] = cptr[j];
      for (int64_t i = 0; i < m; ++i)
        for (int64_t p = row_ptr[i]; p < row_ptr[i + 1]; ++p)
          if (col_idx[p] == j) crow[cptr[j + 1]++] = (int32_t)i;
    }
    int32_t *corder = (int32_t *)malloc(sizeof(int32_t) * (size_t)k);
    orc_order_by_lists(k, cptr, crow, corder);
    int32_t *colpos = (int32_t *)malloc(sizeof(int32_t) * (size_t)k);
    for (int64_t jn = 0; jn < k; ++jn) colpos[corder[jn]] = (int32_t)jn;
    /* 2. each row's distinct block columns under the new column order,
     * ascending: walk the block columns in order and keep those the row
     * touches */
    const int64_t kb = (k + bk - 1) / bk;
    int64_t *rptr = (int64_t *)calloc((size_t)(m + 1), sizeof(int64_t));
    int32_t *rblk = (int32_t *)calloc((size_t)nnz, sizeof(int32_t));
    for (int64_t i = 0; i < m; ++i) {
      rptr[i + 1] = rptr[i];
      for (int64_t c = 0; c < kb; ++c) {
        int touches = 0;
        for (int64_t p = row_ptr[i]; p < row_ptr[i + 1]; ++p)
          if (colpos[col_idx[p]] / bk == c) touches = 1;
        if (touches) rblk[rptr[i + 1]++] = (int32_t)c;
      }
    }
    int32_t *rorder = (int32_t *)malloc(sizeof(int32_t) * (size_t)m);
    orc_order_by_lists(m, rptr, rblk, rorder);
    int32_t *rowpos = (int32_t *)malloc(sizeof(int32_t) * (size_t)m);
    for (int64_t in = 0; in < m; ++in) rowpos[rorder[in]] = (int32_t)in;
    const int64_t after = orc_count_blocks(m, k, row_ptr, col_idx, rowpos, colpos, bm, bk);
    if (after < *blocks_before) {
      kept = 1;
      *blocks_after = after;
      for (int64_t i = 0; i < m; ++i) row_perm[i] = rorder[i];
      for (int64_t j = 0; j < k; ++j) col_perm[j] = corder[j];
    }
    free(cptr); free(crow); free(corder); free(colpos);
    free(rptr); free(rblk); free(rorder); free(rowpos);
  }
  free(ident_r);
  free(ident_c);
  return kept;
}

/* Leak check of the packers' failure paths, run under AddressSanitizer's
 * leak detector by tests/test_sanitizers.py (a C program, so every report is
 * the library's own).  For each packer it walks SPMM_TEST_FAIL_ALLOC = 1, 2,
 * ... until the call succeeds, checks that every failure returns
 * SPMM_ERR_OUT_OF_MEMORY with *out NULL, then destroys the packed matrix;
 * bad arguments are rejected without allocating.  At exit the detector reports
 * any block the library still holds.  Packing rules: BCSR, WCSR (AsyncSparse
 * page), 2:4 and tile-vector-wise (tiled-GEMM page), (2N-2):2N and the
 * reordered BCSR (search page). */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "spmm.h"

static uint64_t lcg = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) {
  lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
  return (uint32_t)(lcg >> 33);
}

typedef spmm_status_t (*pack_fn)(void *ctx, spmm_matrix_t *out);

static int walk(const char *name, pack_fn f, void *ctx) {
  char buf[32];
  for (int n = 1; n < 1000; ++n) {
    snprintf(buf, sizeof buf, "%d", n);
    setenv("SPMM_TEST_FAIL_ALLOC", buf, 1);
    spmm_matrix_t m = (spmm_matrix_t)(uintptr_t)0xDEAD;
    spmm_status_t s = f(ctx, &m);
    if (s == SPMM_OK) {
      unsetenv("SPMM_TEST_FAIL_ALLOC");
      spmm_matrix_info_t info;
      if (spmm_matrix_info(m, &info) != SPMM_OK) return 1;
      spmm_matrix_destroy(m);
      printf("%s: %d failing allocations, then ok\n", name, n - 1);
      return n > 1 ? 0 : 1;
    }
    if (s != SPMM_ERR_OUT_OF_MEMORY || m != NULL) {
      printf("%s: allocation %d gave %s, out %p\n", name, n, spmm_status_str(s), (void *)m);
      return 1;
    }
  }
  printf("%s: never succeeded\n", name);
  return 1;
}

enum { M = 128, K = 256 };
static uint16_t bf[M * K];
static int8_t i8[M * K];
static int64_t rp[M + 1];
static int32_t ci[M * K];
static float fv[M * K];
static uint16_t bv[M * K];

static spmm_status_t p_bcsr(void *c, spmm_matrix_t *o) { (void)c; return spmm_pack_bcsr(M, K, 64, 64, SPMM_BF16, bf, K, o); }
static spmm_status_t p_wcsr(void *c, spmm_matrix_t *o) { (void)c; return spmm_pack_wcsr(M, K, SPMM_F32, rp, ci, fv, 3, 5, o); }
static spmm_status_t p_24i(void *c, spmm_matrix_t *o) { (void)c; return spmm_pack_24(M, K, SPMM_I8, i8, K, o); }
static spmm_status_t p_24b(void *c, spmm_matrix_t *o) { (void)c; return spmm_pack_24(M, K, SPMM_BF16, bf, K, o); }
static spmm_status_t p_tvw(void *c, spmm_matrix_t *o) { (void)c; return spmm_pack_tvw(M, K, SPMM_I8, i8, K, 64, 64, o); }
static spmm_status_t p_slide(void *c, spmm_matrix_t *o) { (void)c; return spmm_pack_slide(M, K, i8, K, 8, o); }
static spmm_status_t p_bcsr_csr(void *c, spmm_matrix_t *o) {
  return spmm_pack_bcsr_csr(M, K, SPMM_BF16, rp, ci, bv, 64, 64, *(int *)c, o);
}

int main(void) {
  /* dense operands with a zero block row and a zero tile column */
  for (int i = 0; i < M; ++i)
    for (int j = 0; j < K; ++j) {
      const int zero = (i >= 64) || (j >= 64 && j < 128) || (next_u32() % 3 == 0);
      const uint32_t r = next_u32();
      bf[i * K + j] = zero ? 0 : (uint16_t)(0x3C00 + (r & 0x7F) + ((r >> 8) & 1) * 0x8000);
      i8[i * K + j] = zero ? 0 : (int8_t)(r % 255 - 127);
    }
  /* canonical CSR: strictly ascending columns, some empty rows */
  int64_t nnz = 0;
  rp[0] = 0;
  for (int i = 0; i < M; ++i) {
    if (i % 7 != 3)
      for (int j = 0; j < K; ++j)
        if (next_u32() % 10 == 0) {
          ci[nnz] = j;
          fv[nnz] = (float)(next_u32() % 2001) / 1000.0f - 1.0f;
          bv[nnz] = (uint16_t)(0x3F80 + (next_u32() & 0x7F));
          ++nnz;
        }
    rp[i + 1] = nnz;
  }
  int bad = 0, zero = 0, one = 1;
  bad |= walk("pack_bcsr", p_bcsr, NULL);
  bad |= walk("pack_wcsr", p_wcsr, NULL);
  bad |= walk("pack_24 int8", p_24i, NULL);
  bad |= walk("pack_24 bf16", p_24b, NULL);
  bad |= walk("pack_tvw", p_tvw, NULL);
  bad |= walk("pack_slide", p_slide, NULL);
  bad |= walk("pack_bcsr_csr", p_bcsr_csr, &zero);
  bad |= walk("pack_bcsr_csr reordered", p_bcsr_csr, &one);
  /* rejected inputs allocate nothing and leave *out NULL */
  spmm_matrix_t m = (spmm_matrix_t)(uintptr_t)0xDEAD;
  int32_t ci_bad[2] = {5, 5};
  int64_t rp_bad[3] = {0, 2, 2};
  if (spmm_pack_wcsr(2, 8, SPMM_F32, rp_bad, ci_bad, fv, 1, 1, &m) != SPMM_ERR_INVALID_ARG || m) bad = 1;
  m = (spmm_matrix_t)(uintptr_t)0xDEAD;
  if (spmm_pack_bcsr(M, 100, 64, 64, SPMM_BF16, bf, K, &m) != SPMM_ERR_INVALID_ARG || m) bad = 1;
  printf(bad ? "FAILED\n" : "driver ok\n");
  return bad;
}

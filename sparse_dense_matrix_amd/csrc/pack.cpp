// pack.cpp -- host packers into the canonical arrays of spmm.h.
//
// BCSR and the row-window CSR follow the AsyncSparse page (abstract; Figure 2
// caption compares the two formats; the summary describes splitting long row
// windows across thread blocks).  The 2:4 packer follows the tiled-GEMM page
// (abstract: the 2:4 pattern of the sparse tensor core) and the N:M entry of
// the search-results page.
#include <algorithm>
#include <cstdlib>
#include <cstring>

#include "internal.h"

namespace sdm {

// ---------------------------------------------------------------------------
// BCSR: one pass over each block row marks the block columns that hold a
// nonzero (bf16 bits other than +0 / -0), then the marked blocks are copied.
// ---------------------------------------------------------------------------
spmm_status_t pack_bcsr_bf16(int64_t m, int64_t k, int32_t bm, int32_t bk,
                             const uint16_t *a, int64_t lda, Matrix &out) {
  const int64_t mb = m / bm, kb = k / bk;
  out.format = SPMM_FORMAT_BCSR;
  out.dtype = SPMM_BF16;
  out.m = m;
  out.k = k;
  out.bm = bm;
  out.bk = bk;
  out.brow_ptr.assign(mb + 1, 0);
  out.bcol_idx.clear();
  vec<uint8_t> marked(kb);
  for (int64_t br = 0; br < mb; ++br) {
    std::fill(marked.begin(), marked.end(), 0);
    for (int64_t i = br * bm; i < (br + 1) * bm; ++i) {
      const uint16_t *row = a + i * lda;
      for (int64_t j = 0; j < k; ++j)
        if (row[j] & 0x7FFFu) marked[j / bk] = 1;
    }
    for (int64_t bc = 0; bc < kb; ++bc)
      if (marked[bc]) out.bcol_idx.push_back(static_cast<int32_t>(bc));
    if (out.bcol_idx.size() > static_cast<size_t>(INT32_MAX))
      return fail(SPMM_ERR_UNSUPPORTED, "spmm_pack_bcsr: more than 2^31-1 blocks");
    out.brow_ptr[br + 1] = static_cast<int32_t>(out.bcol_idx.size());
  }
  const int64_t nnzb = static_cast<int64_t>(out.bcol_idx.size());
  const int64_t belems = static_cast<int64_t>(bm) * bk;
  out.bvals.resize(static_cast<size_t>(nnzb * belems));
  for (int64_t br = 0; br < mb; ++br)
    for (int32_t p = out.brow_ptr[br]; p < out.brow_ptr[br + 1]; ++p) {
      uint16_t *dst = out.bvals.data() + p * belems;
      const uint16_t *src = a + br * bm * lda + static_cast<int64_t>(out.bcol_idx[p]) * bk;
      for (int32_t i = 0; i < bm; ++i) std::memcpy(dst + i * bk, src + i * lda, bk * sizeof(uint16_t));
    }
  out.nnz = nnzb * belems;
  return SPMM_OK;
}

// ---------------------------------------------------------------------------
// WCSR: validate the CSR, copy it, and cut each window of W rows into chunks
// of at most T stored entries.
// ---------------------------------------------------------------------------
// A canonical CSR: row_ptr starts at 0 and never decreases, columns lie in
// [0, k) and strictly ascend within a row.  Nothing is ever fixed silently.
static spmm_status_t check_csr(const char *who, int64_t m, int64_t k, const int64_t *row_ptr,
                               const int32_t *col_idx, const void *vals) {
  const std::string w(who);
  if (row_ptr[0] != 0) return fail(SPMM_ERR_INVALID_ARG, w + ": row_ptr[0] != 0");
  for (int64_t i = 0; i < m; ++i)
    if (row_ptr[i + 1] < row_ptr[i])
      return fail(SPMM_ERR_INVALID_ARG, w + ": row_ptr decreases at row " + std::to_string(i));
  const int64_t nnz = row_ptr[m];
  if (nnz > 0 && (col_idx == nullptr || vals == nullptr))
    return fail(SPMM_ERR_INVALID_ARG, w + ": col_idx / vals is NULL");
  for (int64_t i = 0; i < m; ++i) {
    int64_t prev = -1;
    for (int64_t p = row_ptr[i]; p < row_ptr[i + 1]; ++p) {
      const int64_t c = col_idx[p];
      if (c < 0 || c >= k)
        return fail(SPMM_ERR_INVALID_ARG, w + ": column out of range in row " + std::to_string(i));
      if (c <= prev)
        return fail(SPMM_ERR_INVALID_ARG,
                    w + ": columns not strictly ascending in row " + std::to_string(i));
      prev = c;
    }
  }
  return SPMM_OK;
}

spmm_status_t pack_wcsr_f32(int64_t m, int64_t k, const int64_t *row_ptr,
                            const int32_t *col_idx, const float *vals, int32_t W,
                            int64_t T, Matrix &out) {
  spmm_status_t st = check_csr("spmm_pack_wcsr", m, k, row_ptr, col_idx, vals);
  if (st != SPMM_OK) return st;
  const int64_t nnz = row_ptr[m];
  out.format = SPMM_FORMAT_WCSR;
  out.dtype = SPMM_F32;
  out.m = m;
  out.k = k;
  out.nnz = nnz;
  out.window_rows = W;
  out.max_chunk_nnz = T;
  out.row_ptr.assign(row_ptr, row_ptr + m + 1);
  out.col_idx.assign(col_idx, col_idx + nnz);
  out.vals.assign(vals, vals + nnz);
  out.chunk_window.clear();
  out.chunk_begin.clear();
  const int64_t nwin = (m + W - 1) / W;
  for (int64_t w = 0; w < nwin; ++w) {
    const int64_t s = row_ptr[w * W];
    const int64_t e = row_ptr[std::min<int64_t>(m, (w + 1) * W)];
    const int64_t pieces = std::max<int64_t>(1, (e - s + T - 1) / T);
    for (int64_t q = 0; q < pieces; ++q) {
      out.chunk_window.push_back(static_cast<int32_t>(w));
      out.chunk_begin.push_back(s + q * T);
    }
  }
  out.chunk_begin.push_back(nnz);
  return SPMM_OK;
}

// ---------------------------------------------------------------------------
// BCSR from a CSR matrix, optionally after permuting rows and columns so the
// entries fall into fewer blocks (the row/column permutation that minimises
// nonzero blocks, on the search page's entry about block-sparse SpMM on
// tensor cores for unstructured matrices).  The permutation used here:
//   1. columns are ordered by their sorted lists of rows, compared
//      lexicographically (ties by column index), so columns used by the same
//      rows become neighbours and land in the same block columns;
//   2. rows are then ordered by their sorted lists of block columns under the
//      new column order (ties by row index), so rows touching the same block
//      columns share block rows.
// When the permuted matrix needs no fewer blocks than the original, the
// original order is kept.  row_perm[i'] is the original row of row i',
// col_perm[j'] the original column of column j'; both are empty when the
// order is the original one.
// ---------------------------------------------------------------------------
namespace {

// lexicographic order of variable-length sorted lists, ties by index
struct ListOrder {
  const vec<int64_t> &ptr;
  const vec<int32_t> &val;
  bool operator()(int32_t a, int32_t b) const {
    const int32_t *pa = val.data() + ptr[a], *ea = val.data() + ptr[a + 1];
    const int32_t *pb = val.data() + ptr[b], *eb = val.data() + ptr[b + 1];
    for (; pa != ea && pb != eb; ++pa, ++pb)
      if (*pa != *pb) return *pa < *pb;
    if (pa != ea || pb != eb) return pa == ea;  // the shorter (prefix) list first
    return a < b;
  }
};

// blocks a permuted CSR pattern occupies (newcol[c]: position of column c)
int64_t count_blocks(int64_t m, const int64_t *row_ptr, const int32_t *col_idx,
                     const vec<int32_t> &row_perm, const vec<int32_t> &newcol,
                     int32_t bm, int32_t bk, int64_t kb) {
  vec<int64_t> seen(kb, -1);
  int64_t blocks = 0;
  for (int64_t ip = 0; ip < m; ++ip) {
    const int64_t i = row_perm.empty() ? ip : row_perm[ip];
    const int64_t br = ip / bm;
    for (int64_t p = row_ptr[i]; p < row_ptr[i + 1]; ++p) {
      const int64_t bc = (newcol.empty() ? col_idx[p] : newcol[col_idx[p]]) / bk;
      if (seen[bc] != br) {
        seen[bc] = br;
        ++blocks;
      }
    }
  }
  return blocks;
}

void cluster_order(int64_t m, int64_t k, const int64_t *row_ptr, const int32_t *col_idx,
                   int32_t bk, vec<int32_t> &row_perm, vec<int32_t> &col_perm) {
  const int64_t nnz = row_ptr[m];
  // 1. columns by their row lists (a CSC view; rows come out ascending)
  vec<int64_t> cptr(k + 1, 0);
  for (int64_t p = 0; p < nnz; ++p) ++cptr[col_idx[p] + 1];
  for (int64_t c = 0; c < k; ++c) cptr[c + 1] += cptr[c];
  vec<int32_t> crow(nnz);
  {
    vec<int64_t> fill(cptr.begin(), cptr.end() - 1);
    for (int64_t i = 0; i < m; ++i)
      for (int64_t p = row_ptr[i]; p < row_ptr[i + 1]; ++p) crow[fill[col_idx[p]]++] = static_cast<int32_t>(i);
  }
  col_perm.resize(k);
  for (int64_t c = 0; c < k; ++c) col_perm[c] = static_cast<int32_t>(c);
  std::sort(col_perm.begin(), col_perm.end(), ListOrder{cptr, crow});
  vec<int32_t> newcol(k);
  for (int64_t j = 0; j < k; ++j) newcol[col_perm[j]] = static_cast<int32_t>(j);
  // 2. rows by their sorted, distinct block columns under the new order
  vec<int64_t> rptr(m + 1, 0);
  vec<int32_t> rblk;
  rblk.reserve(nnz);
  vec<int32_t> tmp;
  for (int64_t i = 0; i < m; ++i) {
    tmp.clear();
    for (int64_t p = row_ptr[i]; p < row_ptr[i + 1]; ++p) tmp.push_back(newcol[col_idx[p]] / bk);
    std::sort(tmp.begin(), tmp.end());
    tmp.erase(std::unique(tmp.begin(), tmp.end()), tmp.end());
    rblk.insert(rblk.end(), tmp.begin(), tmp.end());
    rptr[i + 1] = static_cast<int64_t>(rblk.size());
  }
  row_perm.resize(m);
  for (int64_t i = 0; i < m; ++i) row_perm[i] = static_cast<int32_t>(i);
  std::sort(row_perm.begin(), row_perm.end(), ListOrder{rptr, rblk});
}

}  // namespace

spmm_status_t pack_bcsr_csr_bf16(int64_t m, int64_t k, const int64_t *row_ptr,
                                 const int32_t *col_idx, const uint16_t *vals, int32_t bm,
                                 int32_t bk, bool reorder, Matrix &out) {
  spmm_status_t st = check_csr("spmm_pack_bcsr_csr", m, k, row_ptr, col_idx, vals);
  if (st != SPMM_OK) return st;
  const int64_t mb = m / bm, kb = k / bk;
  vec<int32_t> row_perm, col_perm, newcol;
  if (reorder && row_ptr[m] > 0) {
    cluster_order(m, k, row_ptr, col_idx, bk, row_perm, col_perm);
    newcol.resize(k);
    for (int64_t j = 0; j < k; ++j) newcol[col_perm[j]] = static_cast<int32_t>(j);
    const int64_t before = count_blocks(m, row_ptr, col_idx, {}, {}, bm, bk, kb);
    const int64_t after = count_blocks(m, row_ptr, col_idx, row_perm, newcol, bm, bk, kb);
    if (after >= before) {
      row_perm.clear();
      col_perm.clear();
      newcol.clear();
    }
  }
  out.format = SPMM_FORMAT_BCSR;
  out.dtype = SPMM_BF16;
  out.m = m;
  out.k = k;
  out.bm = bm;
  out.bk = bk;
  out.row_perm = row_perm;
  out.col_perm = col_perm;
  out.brow_ptr.assign(mb + 1, 0);
  out.bcol_idx.clear();
  out.bvals.clear();
  const int64_t belems = static_cast<int64_t>(bm) * bk;
  vec<int32_t> slot(kb, -1);  // block column -> block index within the block row
  vec<int32_t> cols;
  for (int64_t br = 0; br < mb; ++br) {
    cols.clear();
    for (int64_t ip = br * bm; ip < (br + 1) * bm; ++ip) {
      const int64_t i = row_perm.empty() ? ip : row_perm[ip];
      for (int64_t p = row_ptr[i]; p < row_ptr[i + 1]; ++p) {
        const int32_t bc = (newcol.empty() ? col_idx[p] : newcol[col_idx[p]]) / bk;
        if (slot[bc] < 0) {
          slot[bc] = 0;
          cols.push_back(bc);
        }
      }
    }
    std::sort(cols.begin(), cols.end());
    const int64_t first = static_cast<int64_t>(out.bcol_idx.size());
    if (first + static_cast<int64_t>(cols.size()) > INT32_MAX)
      return fail(SPMM_ERR_UNSUPPORTED, "spmm_pack_bcsr_csr: more than 2^31-1 blocks");
    for (size_t q = 0; q < cols.size(); ++q) {
      slot[cols[q]] = static_cast<int32_t>(q);
      out.bcol_idx.push_back(cols[q]);
    }
    out.bvals.resize(static_cast<size_t>((first + static_cast<int64_t>(cols.size())) * belems), 0);
    for (int64_t ip = br * bm; ip < (br + 1) * bm; ++ip) {
      const int64_t i = row_perm.empty() ? ip : row_perm[ip];
      for (int64_t p = row_ptr[i]; p < row_ptr[i + 1]; ++p) {
        const int64_t jn = newcol.empty() ? col_idx[p] : newcol[col_idx[p]];
        const int64_t b = first + slot[jn / bk];
        out.bvals[static_cast<size_t>(b * belems + (ip - br * bm) * bk + jn % bk)] = vals[p];
      }
    }
    for (int32_t bc : cols) slot[bc] = -1;
    out.brow_ptr[br + 1] = static_cast<int32_t>(out.bcol_idx.size());
  }
  out.nnz = static_cast<int64_t>(out.bcol_idx.size()) * belems;
  return SPMM_OK;
}

// ---------------------------------------------------------------------------
// 2:4: in every group of four, the two largest of key = mag(a) * 4 + (3 - pos)
// are kept (larger magnitude first, ties to the lower position), then stored
// in ascending position.  mag is |a| for int8 (|-128| = 128); for bf16 it is
// the bit pattern with the sign cleared, which orders finite values and
// infinities by magnitude, with every NaN mapped to one rank above infinity
// (so NaNs tie with each other).
// ---------------------------------------------------------------------------
static inline int mag(int8_t x) { return x < 0 ? -x : x; }
static inline int mag(uint16_t x) {
  const int v = x & 0x7fff;
  return v > 0x7f80 ? 0x7f81 : v;
}

template <class T>
static inline void prune_group(const T *grp, T *kept, uint8_t &nibble) {
  int key[4];
  for (int t = 0; t < 4; ++t) key[t] = mag(grp[t]) * 4 + (3 - t);
  int first = 0;
  for (int t = 1; t < 4; ++t)
    if (key[t] > key[first]) first = t;
  int second = first == 0 ? 1 : 0;
  for (int t = 0; t < 4; ++t)
    if (t != first && key[t] > key[second]) second = t;
  const int lo = std::min(first, second), hi = std::max(first, second);
  kept[0] = grp[lo];
  kept[1] = grp[hi];
  nibble = static_cast<uint8_t>(lo | (hi << 2));
}

// one row of `len` elements (len % 8 == 0) into len/2 values and len/8 bytes
template <class T>
static void prune_row(const T *row, int64_t len, T *v, uint8_t *mt) {
  for (int64_t g = 0; g < len / 4; ++g) {
    uint8_t nibble;
    prune_group(row + 4 * g, v + 2 * g, nibble);
    mt[g >> 1] = static_cast<uint8_t>(mt[g >> 1] | (nibble << ((g & 1) * 4)));
  }
}

template <class V>
static void pack_24_t(int64_t m, int64_t k, const V *a, int64_t lda, vec<V> &vals,
                      Matrix &out) {
  vals.assign(static_cast<size_t>(m * (k / 2)), 0);
  out.meta24.assign(static_cast<size_t>(m * (k / 8)), 0);
  for (int64_t i = 0; i < m; ++i)
    prune_row(a + i * lda, k, vals.data() + i * (k / 2), out.meta24.data() + i * (k / 8));
}

spmm_status_t pack_24(int64_t m, int64_t k, spmm_dtype_t dtype, const void *a, int64_t lda,
                      Matrix &out) {
  out.format = SPMM_FORMAT_24;
  out.dtype = dtype;
  out.m = m;
  out.k = k;
  out.nnz = m * (k / 2);
  out.vals24.clear();
  out.vals24_bf16.clear();
  if (dtype == SPMM_BF16)
    pack_24_t(m, k, static_cast<const uint16_t *>(a), lda, out.vals24_bf16, out);
  else
    pack_24_t(m, k, static_cast<const int8_t *>(a), lda, out.vals24, out);
  return SPMM_OK;
}

// ---------------------------------------------------------------------------
// Sliding-window decomposition of (2N-2):2N weights (the search page's entry
// on the (2N-2):2N family): every group of 2N elements keeps its 2N-2 largest
// |a| (ties to the lower position), and the kept elements are dealt to N-1
// overlapping windows of four (window w covers positions 2w .. 2w+3), two per
// window, so the group becomes N-1 2:4 groups.  The lifted row has 4(N-1)
// columns per group; lifted column 4w + j of group g multiplies B's row
// 2N g + 2w + j.  Kept positions are dealt in ascending order to the lower
// window while it has room: positions 2w and 2w+1 belong to windows w-1 and
// w, the two ends to one window only.
// ---------------------------------------------------------------------------
int64_t slide_source_row(int64_t j, int32_t group) {
  const int64_t per = 2 * (group - 2);  // lifted columns per group: 4 (N - 1)
  const int64_t g = j / per, o = j % per;
  return g * group + 2 * (o / 4) + (o % 4);
}

spmm_status_t pack_slide_i8(int64_t m, int64_t k, const int8_t *a, int64_t lda, int32_t group,
                            Matrix &out) {
  const int32_t N = group / 2, keep = group - 2, windows = N - 1;
  const int64_t groups = k / group;
  const int64_t k_lift = groups * 4 * windows;
  out.format = SPMM_FORMAT_SLIDE;
  out.dtype = SPMM_I8;
  out.m = m;
  out.k = k;
  out.slide_group = group;
  out.k_lift = k_lift;
  out.nnz = m * (k_lift / 2);
  out.vals24.assign(static_cast<size_t>(m * (k_lift / 2)), 0);
  out.meta24.assign(static_cast<size_t>(m * (k_lift / 8)), 0);
  vec<int> rank_key(group);
  vec<int8_t> lifted(static_cast<size_t>(4 * windows));
  vec<int> wcount(windows);
  vec<uint8_t> taken(4 * windows);
  for (int64_t i = 0; i < m; ++i) {
    const int8_t *row = a + i * lda;
    int8_t *v = out.vals24.data() + i * (k_lift / 2);
    uint8_t *mt = out.meta24.data() + i * (k_lift / 8);
    for (int64_t g = 0; g < groups; ++g) {
      const int8_t *grp = row + g * group;
      std::fill(wcount.begin(), wcount.end(), 0);
      std::fill(taken.begin(), taken.end(), 0);
      std::fill(lifted.begin(), lifted.end(), 0);
      for (int32_t p = 0; p < group; ++p) {
        // kept iff fewer than `keep` positions rank before p
        int before = 0;
        const int ap = std::abs(static_cast<int>(grp[p]));
        for (int32_t u = 0; u < group; ++u) {
          const int au = std::abs(static_cast<int>(grp[u]));
          if (au > ap || (au == ap && u < p)) ++before;
        }
        if (before >= keep) continue;
        const int w_lo = p / 2 - 1, w_hi = p / 2;
        int w = -1;
        if (w_lo >= 0 && w_lo < windows && wcount[w_lo] < 2) w = w_lo;
        else if (w_hi < windows && wcount[w_hi] < 2) w = w_hi;
        if (w < 0) return fail(SPMM_ERR_INTERNAL, "spmm_pack_slide: window assignment failed");
        ++wcount[w];
        const int j = p - 2 * w;
        taken[4 * w + j] = 1;
        lifted[4 * w + j] = grp[p];
      }
      // every window is a 2:4 group: its two taken positions (every window
      // is full, since 2N-2 elements fill N-1 windows of two)
      for (int32_t w = 0; w < windows; ++w) {
        int pos[2], q = 0;
        for (int j = 0; j < 4 && q < 2; ++j)
          if (taken[4 * w + j]) pos[q++] = j;
        for (int j = 0; j < 4 && q < 2; ++j)  // (unreachable) pad with an untaken slot
          if (!taken[4 * w + j] && (q == 0 || j > pos[0])) pos[q++] = j;
        const int64_t lg = g * windows + w;  // 2:4 group index in the lifted row
        v[2 * lg] = lifted[4 * w + pos[0]];
        v[2 * lg + 1] = lifted[4 * w + pos[1]];
        const uint8_t nibble = static_cast<uint8_t>(pos[0] | (pos[1] << 2));
        mt[lg >> 1] = static_cast<uint8_t>(mt[lg >> 1] | (nibble << ((lg & 1) * 4)));
      }
    }
  }
  return SPMM_OK;
}

// ---------------------------------------------------------------------------
// Tile-vector-wise (the tiled-GEMM page, abstract): A is cut into tm x tk
// tiles; a tile is stored when any element is nonzero (for bf16, +0 and -0
// are zero and NaN is not), and a stored tile is pruned 2:4 along k exactly
// as above.  Since 2:4 pruning maps a zero tile to zero and keeps a nonzero
// in every nonzero group, the stored product is the 2:4 product of A with
// the zero tiles skipped.
// ---------------------------------------------------------------------------
template <class V>
static spmm_status_t pack_tvw_t(int64_t m, int64_t k, const V *a, int64_t lda, int32_t tm,
                                int32_t tk, vec<V> &vals, Matrix &out) {
  const int64_t mt = m / tm, kt = k / tk;
  out.format = SPMM_FORMAT_TVW;
  out.m = m;
  out.k = k;
  out.bm = tm;
  out.bk = tk;
  out.brow_ptr.assign(mt + 1, 0);
  out.bcol_idx.clear();
  vals.clear();
  out.meta24.clear();
  const int64_t tv = static_cast<int64_t>(tm) * (tk / 2), tmeta = static_cast<int64_t>(tm) * (tk / 8);
  for (int64_t T = 0; T < mt; ++T) {
    for (int64_t s = 0; s < kt; ++s) {
      bool any = false;
      for (int64_t i = T * tm; i < (T + 1) * tm && !any; ++i) {
        const V *row = a + i * lda + s * tk;
        for (int32_t j = 0; j < tk; ++j)
          if (mag(row[j]) != 0) {
            any = true;
            break;
          }
      }
      if (!any) continue;
      if (out.bcol_idx.size() >= static_cast<size_t>(INT32_MAX))
        return fail(SPMM_ERR_UNSUPPORTED, "spmm_pack_tvw: more than 2^31-1 tiles");
      const size_t v0 = vals.size(), m0 = out.meta24.size();
      vals.resize(v0 + static_cast<size_t>(tv), 0);
      out.meta24.resize(m0 + static_cast<size_t>(tmeta), 0);
      for (int32_t r = 0; r < tm; ++r)
        prune_row(a + (T * tm + r) * lda + s * tk, tk, vals.data() + v0 + r * (tk / 2),
                  out.meta24.data() + m0 + r * (tk / 8));
      out.bcol_idx.push_back(static_cast<int32_t>(s));
    }
    out.brow_ptr[T + 1] = static_cast<int32_t>(out.bcol_idx.size());
  }
  out.nnz = static_cast<int64_t>(out.bcol_idx.size()) * tv;
  return SPMM_OK;
}

spmm_status_t pack_tvw(int64_t m, int64_t k, spmm_dtype_t dtype, const void *a, int64_t lda,
                       int32_t tm, int32_t tk, Matrix &out) {
  out.dtype = dtype;
  out.vals24.clear();
  out.vals24_bf16.clear();
  if (dtype == SPMM_BF16)
    return pack_tvw_t(m, k, static_cast<const uint16_t *>(a), lda, tm, tk, out.vals24_bf16, out);
  return pack_tvw_t(m, k, static_cast<const int8_t *>(a), lda, tm, tk, out.vals24, out);
}

}  // namespace sdm

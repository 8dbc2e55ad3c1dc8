// internal.h -- objects behind the C ABI and the kernel launch interfaces.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <memory>
#include <new>
#include <string>
#include <vector>

#include "../../include/spmm.h"

namespace sdm {

// ---------------------------------------------------------------------------
// errors
// ---------------------------------------------------------------------------
spmm_status_t fail(spmm_status_t s, const std::string &msg);
spmm_status_t hip_fail(hipError_t e, const char *what);
void clear_error();

// ---------------------------------------------------------------------------
// forced allocation failures (tests)
// ---------------------------------------------------------------------------
// When the environment variable SPMM_TEST_FAIL_ALLOC holds n > 0 at the start
// of an ABI call that allocates (packing, planning), the n-th allocation of
// that call fails as it would when memory runs out: a host allocation throws
// std::bad_alloc, a device allocation reports hipErrorOutOfMemory.  Tests walk
// n = 1, 2, ... to check that every failure returns SPMM_ERR_OUT_OF_MEMORY,
// leaves *out NULL and leaks nothing.  Unset or 0: no effect.
void alloc_hook_begin();
bool alloc_hook_fail();  // true when this allocation is the one to fail

// Allocator of every host array the library owns: std::allocator behind the
// failure hook.
template <class T>
struct HostAlloc {
  using value_type = T;
  HostAlloc() = default;
  template <class U>
  HostAlloc(const HostAlloc<U> &) {}
  T *allocate(size_t n) {
    if (alloc_hook_fail()) throw std::bad_alloc();
    return std::allocator<T>().allocate(n);
  }
  void deallocate(T *p, size_t n) { std::allocator<T>().deallocate(p, n); }
  template <class U>
  bool operator==(const HostAlloc<U> &) const { return true; }
  template <class U>
  bool operator!=(const HostAlloc<U> &) const { return false; }
};
template <class T>
using vec = std::vector<T, HostAlloc<T>>;

// ---------------------------------------------------------------------------
// packed operand (host, canonical arrays)
// ---------------------------------------------------------------------------
struct Matrix {
  std::atomic<int> refs{1};
  spmm_format_t format = SPMM_FORMAT_BCSR;
  spmm_dtype_t dtype = SPMM_F32;
  int64_t m = 0, k = 0, nnz = 0;
  // BCSR
  int32_t bm = 0, bk = 0;
  vec<int32_t> brow_ptr, bcol_idx;
  vec<uint16_t> bvals;
  // BCSR of a permuted CSR matrix: original row of each row / original
  // column of each column of the packed matrix (empty: original order)
  vec<int32_t> row_perm, col_perm;
  // sliding-window 2:4 ((2N-2):2N weights): group width 2N; vals24 / meta24
  // hold the lifted 2:4 matrix of m x k_lift columns
  int32_t slide_group = 0;
  int64_t k_lift = 0;
  // WCSR
  int32_t window_rows = 0;
  int64_t max_chunk_nnz = 0;
  vec<int64_t> row_ptr;
  vec<int32_t> col_idx;
  vec<float> vals;
  vec<int32_t> chunk_window;
  vec<int64_t> chunk_begin;
  // 2:4 (and the stored tiles of tile-vector-wise: brow_ptr / bcol_idx over
  // tiles of bm x bk, vals24 / meta24 tile after tile); bf16 values go to
  // vals24_bf16 instead of vals24
  vec<int8_t> vals24;
  vec<uint16_t> vals24_bf16;
  vec<uint8_t> meta24;
};

void retain(Matrix *a);
void release(Matrix *a);

// packers (pack.cpp); they fill `a` and return a status (message set on error)
spmm_status_t pack_bcsr_bf16(int64_t m, int64_t k, int32_t bm, int32_t bk,
                             const uint16_t *a, int64_t lda, Matrix &out);
spmm_status_t pack_wcsr_f32(int64_t m, int64_t k, const int64_t *row_ptr,
                            const int32_t *col_idx, const float *vals, int32_t W,
                            int64_t T, Matrix &out);
// dtype SPMM_I8 (a: int8) or SPMM_BF16 (a: bf16 bit patterns)
spmm_status_t pack_24(int64_t m, int64_t k, spmm_dtype_t dtype, const void *a, int64_t lda,
                      Matrix &out);
spmm_status_t pack_slide_i8(int64_t m, int64_t k, const int8_t *a, int64_t lda, int32_t group,
                            Matrix &out);
// lifted row j of a sliding-window matrix -> row of B it multiplies
int64_t slide_source_row(int64_t j, int32_t group);
// dtype SPMM_I8 (a: int8) or SPMM_BF16 (a: bf16 bit patterns)
spmm_status_t pack_tvw(int64_t m, int64_t k, spmm_dtype_t dtype, const void *a, int64_t lda,
                       int32_t tm, int32_t tk, Matrix &out);
spmm_status_t pack_bcsr_csr_bf16(int64_t m, int64_t k, const int64_t *row_ptr,
                                 const int32_t *col_idx, const uint16_t *vals, int32_t bm,
                                 int32_t bk, bool reorder, Matrix &out);

// ---------------------------------------------------------------------------
// device-side descriptors (plan-private layouts)
// ---------------------------------------------------------------------------

// One chunk of a row window: the stored entries [nz_begin, nz_end) it reduces
// and the output rows [row_begin, row_end) it writes.  A row whose entries lie
// inside the chunk (or an empty row the chunk owns) goes straight to C; the
// first / last row may instead be a piece of a row split over several chunks
// and then goes to partial row slot_first / slot_last (-1 when not split).
struct WcsrChunk {
  int64_t nz_begin, nz_end;
  int32_t row_begin, row_end;
  int32_t slot_first, slot_last;
};
static_assert(sizeof(WcsrChunk) == 32, "WcsrChunk layout");

// Raise a kernel's dynamic LDS limit to `bytes` on the current device (once
// per kernel and device).
hipError_t allow_dynamic_lds(const void *kernel, size_t bytes);

// ---------------------------------------------------------------------------
// kernel launchers (one per format, in the .hip files)
// ---------------------------------------------------------------------------
struct BcsrLaunch {
  const int32_t *row_ptr;   // [mb + 1]
  const int32_t *col_idx;   // [nnzb]
  const uint16_t *frag;     // [nnzb][4096] in MFMA fragment order
  const int32_t *row_order; // [mb] block rows, row group by row group, each in dispatch order
  const int32_t *row_seg;   // [row_groups + 1] start of each row group in row_order
  int32_t row_groups;       // 1, 2, 4 or 8: XCD x serves row group x % row_groups
  int32_t tn;               // columns of C per workgroup: 256 or 512
  int32_t kh;               // k-rows per LDS stage: 64 (whole blocks) or 32 (tn 256 only)
  int64_t grid;             // workgroups (bcsr_grid)
  int32_t mb;               // block rows (64 rows each)
  int64_t n;
  const uint16_t *B;
  int64_t ldb;
  uint16_t *C;
  int64_t ldc;
  // A packed with its rows and columns permuted (spmm_pack_bcsr_csr): packed
  // column j multiplies B row col_perm[j] (the kernel reads B through the
  // map), and packed row i is written to C row c_rows[i]; null otherwise
  int64_t k_rows;           // k: rows of B
  const int32_t *col_perm;  // [k] original row of B for each packed column
  const int32_t *c_rows;    // [m] original row of C for each packed row
  // Paired block rows (bcsr_bf16_pair): a tile is two block rows that walk
  // the union of their block columns, so a B slab both use is loaded once.
  // row_order / row_seg then hold pairs instead of block rows.
  bool paired;
  const int32_t *pair_rows;  // [2 * npairs] block rows of each pair (second -1 when alone)
  const int32_t *pair_ptr;   // [npairs + 1] units of pair p: [pair_ptr[p], pair_ptr[p+1])
  const int4 *units;         // per unit: block column, block of the first row, of the second (-1: none)
  int32_t npairs;
};
// The paired kernel's tile (256 columns, half-block stages) and when the plan
// takes it: the pairing saves at least this fraction of B slab loads and
// leaves at least this many tiles.
constexpr int kBcsrPairTN = 256, kBcsrPairKH = 32;
constexpr double kBcsrPairMinSaving = 0.10;
constexpr int64_t kBcsrPairMinTiles = 8 * 256;
// a pair's units sit one per lane of a wave
constexpr int32_t kBcsrPairMaxUnits = 64;
// bound on the pairing search (row visits), which keeps plan time under a
// second or so; larger patterns are not paired
constexpr double kBcsrPairMaxWork = 1 << 28;
// Pairs of block rows for the paired kernel: greedy, largest rows first, each
// with the unpaired row sharing most block columns (ties: lowest index).
// Returns the fraction of B slab loads the pairing saves; 0 when a pair would
// exceed kBcsrPairMaxUnits or the search kBcsrPairMaxWork (the pairing is
// then not to be used).
double bcsr_pairing(const int32_t *row_ptr, const int32_t *col_idx, int32_t mb, int32_t kb,
                    vec<int32_t> &pair_rows, vec<int32_t> &pair_ptr, vec<int32_t> &units);
// Fragment order of one 64 x 64 block: [rb 2][s 4][lane 64][8 elements], lane l
// holding row 32*rb + l%32, columns 16*s + 8*(l/32) + 0..7.
void bcsr_fragment_order(const uint16_t *block_rowmajor, uint16_t *frag);
// Tile width and row groups for the XCD mapping of a plan (see the kernel),
// and the grid for a given split of row_order into groups.
struct BcsrSchedule {
  int tn;
  int row_groups;
  int kh;
};
BcsrSchedule bcsr_schedule(const int32_t *row_ptr, int32_t mb, int64_t n);
int64_t bcsr_grid(const int32_t *row_seg, const BcsrSchedule &sc, int64_t n);
hipError_t launch_bcsr_bf16(const BcsrLaunch &a, hipStream_t s);

struct WcsrLaunch {
  const WcsrChunk *chunks;
  int64_t num_chunks;
  const int64_t *row_ptr;
  const int32_t *col_idx;
  const float *vals;
  const int32_t *merge_row;   // [num_split_rows]
  const int32_t *merge_slot;  // [num_split_rows + 1]
  int64_t num_split_rows;
  float *partial;             // [num_slots][n]
  int64_t n;
  const float *B;
  int64_t ldb;
  float *C;
  int64_t ldc;
};
hipError_t launch_wcsr_f32(const WcsrLaunch &a, hipStream_t s);
int64_t wcsr_grid(int64_t num_chunks, int64_t n);
// Size of the per-GPU scratch array that holds a WCSR plan's partial rows in
// spmm_execute_noalloc, and its address on `device` (which must be the
// current device; looked up once per device, then cached).
constexpr int64_t kNoallocScratchBytes = int64_t(32) << 20;
hipError_t noalloc_scratch(int device, void **ptr);

// Chunk descriptors of a WCSR matrix (row range of each chunk, and the
// partial-row slots of rows split across chunks, slot_row[s] = row of slot
// s in slot order).  Fails only on an internal inconsistency.
spmm_status_t wcsr_chunk_descriptors(const Matrix &a, vec<WcsrChunk> &chunks,
                                     vec<int32_t> &slot_row);

struct SddmmLaunch {
  const WcsrChunk *chunks;
  int64_t num_chunks;
  const int64_t *row_ptr;
  const int32_t *col_idx;
  int64_t kd;         // inner dimension
  spmm_dtype_t dtype; // X and Y: F32 (out fp32), BF16 (out bf16) or I8 (out int32)
  const void *X;      // [m][ldx]
  int64_t ldx;
  const void *Y;      // [k][ldy]
  int64_t ldy;
  void *out;          // [nnz]
};
hipError_t launch_sddmm_csr(const SddmmLaunch &a, hipStream_t s);
int64_t sddmm_grid(int64_t num_chunks);

// SDDMM with a BCSR pattern of 64 x 64 blocks: a workgroup serves a group of
// up to sddmm_bcsr_group() stored blocks of one block row over one range of
// the inner dimension (ksplit elements, a multiple of sddmm_bcsr_chunk()).
struct SddmmBcsrLaunch {
  const int4 *groups;       // [ngroups] (block row, first block, block count, 0)
  int32_t ngroups;
  const int32_t *col_idx;   // [nnzb]
  int64_t nnzb;
  int64_t kd;               // inner dimension
  int64_t ksplit;           // elements per range
  int32_t nsplit;           // ranges; > 1 goes through `partial`
  bool int8;                // int8 X, Y -> int32 out; else bf16 -> bf16
  const void *X;            // [m][ldx]
  int64_t ldx;              // elements
  const void *Y;            // [k][ldy]
  int64_t ldy;
  void *out;                // [nnzb][64][64]
  void *partial;            // [nsplit][nnzb][64][64] fp32 / int32 when nsplit > 1
};
int sddmm_bcsr_chunk(bool int8);
int sddmm_bcsr_group();
hipError_t launch_sddmm_bcsr(const SddmmBcsrLaunch &a, hipStream_t s);

struct Sp24Launch {
  bool bf16;            // bf16 A, B and C (else int8 A, B and int32 C)
  const void *vals;     // tiled copy of the values (sp24_tile_layout / tvw_tile_layout)
  const uint8_t *meta;  // tiled copy of the index words
  // tile-vector-wise A: stored k-steps of row tile T are
  // tile_step[tile_ptr[T] .. tile_ptr[T+1]); null for a plain 2:4 A
  const int32_t *tile_ptr;
  const int32_t *tile_step;
  // sliding-window A: lifted k-row j multiplies B row b_rows[j] (k_pad
  // entries, row 0 past k); the kernel reads B through it; null otherwise
  const int32_t *b_rows;
  // tile-vector-wise A: the row tiles in dispatch order, groups of four per
  // XCD (mtiles entries); null otherwise
  const int32_t *row_order;
  int64_t m, k, n;
  int64_t m_pad, k_pad;
  int32_t tn;   // columns of C per workgroup (sp24_tile_n)
  const void *B;
  int64_t ldb;  // elements
  void *C;
  int64_t ldc;  // elements
};
// Dispatch order of the row tiles of a tile-vector-wise A (tile_ptr[T] ..
// tile_ptr[T+1] are row tile T's stored tiles; mtiles row tiles).  The
// kernel deals groups of four row tiles to an XCD, row slot slowest, so
// that with 16 column tiles (one round of workgroups) each CU holds slots 0
// and 2, or 1 and 3, of a group.  Groups are filled heaviest first in snake
// order (0 .. G-1, G-1 .. 0, ...), which evens out their totals, and each
// group of four is ordered heaviest, second, lightest, third, which puts a
// heavy and a light row tile on each CU.  Only the last group may hold
// fewer than four.
vec<int32_t> tvw_row_order(const int32_t *tile_ptr, int64_t mtiles);
// Plan-private copies of the canonical 2:4 arrays (values int8 or bf16),
// zero-padded to m_pad x k_pad and laid out per 256-row tile and k-step
// (sp24_tile_k) in the order the kernel's shared-memory stages hold them
// (vals_tiled: m_pad * k_pad / 2 elements, meta_tiled: m_pad * k_pad / 8
// bytes).
void sp24_tile_layout(const void *vals, const uint8_t *meta, int64_t m, int64_t k, int64_t m_pad,
                      int64_t k_pad, bool bf16, void *vals_tiled, uint8_t *meta_tiled);
// The same layout for the stored tiles of a tile-vector-wise matrix, given
// per tile as [256][tk/2] values and [256][tk/8] index bytes, tk a multiple
// of sp24_tile_k; every tile becomes tk / sp24_tile_k consecutive k-steps.
void tvw_tile_layout(const void *tile_vals, const uint8_t *tile_meta, int64_t ntiles, int32_t tk,
                     bool bf16, void *vals_tiled, uint8_t *meta_tiled);
int sp24_tile_m();
// columns of C per workgroup for n columns; mapped: B read through a row map
int sp24_tile_n(int64_t n, bool mapped);
int sp24_tile_k(bool bf16);  // dense k per step: 128 int8, 64 bf16
int64_t sp24_grid(int64_t m, int64_t n, int tn);
hipError_t launch_sp24(const Sp24Launch &a, hipStream_t s);

}  // namespace sdm

// ---------------------------------------------------------------------------
// plan object
// ---------------------------------------------------------------------------
struct spmm_plan_s {
  sdm::Matrix *a = nullptr;
  bool sddmm = false;  // plan of spmm_plan_sddmm rather than spmm_plan
  spmm_dtype_t sddmm_dtype = SPMM_F32;  // element type of X and Y
  int32_t device = 0;
  int64_t n = 0;
  spmm_plan_info_t info{};
  sdm::vec<void *> allocations;
  sdm::BcsrLaunch bcsr{};
  sdm::WcsrLaunch wcsr{};
  sdm::Sp24Launch sp24{};
  sdm::SddmmLaunch sdd{};
  sdm::SddmmBcsrLaunch sddb{};
};

struct spmm_matrix_s : sdm::Matrix {};

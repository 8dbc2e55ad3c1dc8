// api.cpp -- the C ABI of spmm.h: argument checks, object lifetimes, device
// upload and per-format launch dispatch.
#include <algorithm>
#include <cstdarg>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>

#include "internal.h"

namespace sdm {

static thread_local std::string g_last_error;
static thread_local int64_t g_alloc_countdown = 0;

void alloc_hook_begin() {
  const char *v = std::getenv("SPMM_TEST_FAIL_ALLOC");
  g_alloc_countdown = v ? std::max<int64_t>(0, std::atoll(v)) : 0;
}

bool alloc_hook_fail() { return g_alloc_countdown > 0 && --g_alloc_countdown == 0; }

spmm_status_t fail(spmm_status_t s, const std::string &msg) {
  g_last_error = msg;
  return s;
}

spmm_status_t hip_fail(hipError_t e, const char *what) {
  g_last_error = std::string(what) + ": " + hipGetErrorString(e);
  return e == hipErrorOutOfMemory ? SPMM_ERR_OUT_OF_MEMORY : SPMM_ERR_HIP;
}

void clear_error() { g_last_error.clear(); }

hipError_t allow_dynamic_lds(const void *kernel, size_t bytes) {
  struct Entry {
    const void *kernel;
    int device;
  };
  static std::mutex mu;
  static std::vector<Entry> done;  // not a library array: no failure hook
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  for (const Entry &x : done)
    if (x.kernel == kernel && x.device == dev) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes));
  if (e == hipSuccess) done.push_back({kernel, dev});
  return e;
}

void retain(Matrix *a) { a->refs.fetch_add(1, std::memory_order_relaxed); }

void release(Matrix *a) {
  if (a && a->refs.fetch_sub(1, std::memory_order_acq_rel) == 1)
    delete static_cast<spmm_matrix_s *>(a);
}

namespace {

template <class F>
spmm_status_t guarded(F &&f) {
  try {
    return f();
  } catch (const std::bad_alloc &) {
    return fail(SPMM_ERR_OUT_OF_MEMORY, "host allocation failed");
  } catch (const std::exception &e) {
    return fail(SPMM_ERR_INTERNAL, e.what());
  } catch (...) {
    return fail(SPMM_ERR_INTERNAL, "unknown exception");
  }
}

// A new packed operand, owned until it is handed to the caller.
std::unique_ptr<spmm_matrix_s> new_matrix() {
  if (alloc_hook_fail()) throw std::bad_alloc();
  return std::unique_ptr<spmm_matrix_s>(new spmm_matrix_s());
}

// Restores the caller's current device on scope exit.
struct DeviceScope {
  int prev = -1;
  hipError_t err = hipSuccess;
  explicit DeviceScope(int dev) {
    err = hipGetDevice(&prev);
    if (err == hipSuccess && prev != dev) err = hipSetDevice(dev);
  }
  ~DeviceScope() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

void free_plan(spmm_plan_s *p) {
  if (!p) return;
  if (!p->allocations.empty()) {
    DeviceScope ds(p->device);
    for (void *ptr : p->allocations) (void)hipFree(ptr);
  }
  release(p->a);
  delete p;
}

// hipMalloc + copy; the pointer is owned by the plan.
spmm_status_t upload(spmm_plan_s *p, const void *src, size_t bytes, void **dst) {
  *dst = nullptr;
  if (bytes == 0) bytes = 16;  // keep every table pointer valid
  p->allocations.push_back(nullptr);  // may throw; nothing is allocated yet
  void *d = nullptr;
  hipError_t e = alloc_hook_fail() ? hipErrorOutOfMemory : hipMalloc(&d, bytes);
  if (e != hipSuccess) {
    p->allocations.pop_back();
    return hip_fail(e, "hipMalloc");
  }
  p->allocations.back() = d;
  p->info.device_bytes += static_cast<int64_t>(bytes);
  if (src) {
    e = hipMemcpy(d, src, bytes, hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpy");
  }
  *dst = d;
  return SPMM_OK;
}

template <class T>
spmm_status_t upload_vec(spmm_plan_s *p, const vec<T> &v, T **dst) {
  void *d = nullptr;
  spmm_status_t s = upload(p, v.empty() ? nullptr : v.data(), v.size() * sizeof(T), &d);
  *dst = static_cast<T *>(d);
  return s;
}

// ---- BCSR plan ---------------------------------------------------------------
spmm_status_t plan_bcsr(spmm_plan_s *p) {
  const Matrix &a = *p->a;
  if (a.bm != 64 || a.bk != 64)
    return fail(SPMM_ERR_UNSUPPORTED, "spmm_plan: BCSR kernels take 64 x 64 blocks");
  if (p->n % 8 != 0) return fail(SPMM_ERR_UNSUPPORTED, "spmm_plan: BCSR needs n % 8 == 0");
  const int64_t nnzb = static_cast<int64_t>(a.bcol_idx.size());
  vec<uint16_t> frag(a.bvals.size());
  for (int64_t b = 0; b < nnzb; ++b) bcsr_fragment_order(a.bvals.data() + b * 4096, frag.data() + b * 4096);
  BcsrLaunch &L = p->bcsr;
  int32_t *rp = nullptr, *ci = nullptr;
  uint16_t *fv = nullptr;
  spmm_status_t s;
  if ((s = upload_vec(p, a.brow_ptr, &rp)) != SPMM_OK) return s;
  if ((s = upload_vec(p, a.bcol_idx, &ci)) != SPMM_OK) return s;
  if ((s = upload_vec(p, frag, &fv)) != SPMM_OK) return s;
  const int32_t mb = static_cast<int32_t>(a.m / 64);
  BcsrSchedule sc = bcsr_schedule(a.brow_ptr.data(), mb, p->n);
  // Paired block rows (two rows per tile over the union of their block
  // columns, 256-wide half-block stages) when the pairing saves at least a
  // tenth of the B slab loads and the pairs still give every CU several
  // tiles; in place of the single-row schedules of 256-wide half-block
  // stages and of 512-wide whole-block stages (not of 256-wide whole-block
  // stages, which only rows of many blocks at small n take).  Not for
  // column-permuted A (the kernel reads B rows in place).
  vec<int32_t> pair_rows, pair_ptr, units;
  bool paired = false;
  const bool half_sched = sc.tn == kBcsrPairTN && sc.kh == kBcsrPairKH;
  if ((half_sched || sc.tn == 512) && a.col_perm.empty() && mb >= 2) {
    const double saving = bcsr_pairing(a.brow_ptr.data(), a.bcol_idx.data(), mb,
                                       static_cast<int32_t>((a.k + 63) / 64), pair_rows, pair_ptr, units);
    const int64_t tiles =
        static_cast<int64_t>(pair_ptr.size() - 1) * ((p->n + kBcsrPairTN - 1) / kBcsrPairTN);
    paired = saving >= kBcsrPairMinSaving && tiles >= kBcsrPairMinTiles;
    if (paired) {
      sc.tn = kBcsrPairTN;
      sc.kh = kBcsrPairKH;
    }
  }
  // tiles (block rows, or pairs) in dispatch order: most work first (ties by
  // index), so the longest tiles of a column tile start first and the short
  // ones fill in behind them.  A tile's work is its stages (blocks, or units
  // of a pair) plus one per C block row it writes.
  const int32_t ntiles = paired ? static_cast<int32_t>(pair_ptr.size() - 1) : mb;
  auto work = [&](int32_t r) -> int64_t {
    if (!paired) return a.brow_ptr[r + 1] - a.brow_ptr[r] + 1;
    return pair_ptr[r + 1] - pair_ptr[r] + 1 + (pair_rows[2 * r + 1] >= 0 ? 1 : 0);
  };
  vec<int32_t> sorted(static_cast<size_t>(ntiles));
  for (int32_t i = 0; i < ntiles; ++i) sorted[i] = i;
  std::stable_sort(sorted.begin(), sorted.end(), [&](int32_t x, int32_t y) { return work(x) > work(y); });
  // row groups of about equal work: longest first, each to the lightest
  // group (lowest on ties); every group keeps the longest-first order.  The
  // order array carries the groups' start offsets after its entries.
  const int groups = sc.row_groups;
  vec<vec<int32_t>> members(static_cast<size_t>(groups));
  vec<int64_t> load(static_cast<size_t>(groups), 0);
  for (int32_t r : sorted) {
    const size_t g = static_cast<size_t>(std::min_element(load.begin(), load.end()) - load.begin());
    members[g].push_back(r);
    load[g] += work(r);
  }
  vec<int32_t> order;
  order.reserve(static_cast<size_t>(ntiles) + 9);
  vec<int32_t> seg(1, 0);
  for (const auto &g : members) {
    order.insert(order.end(), g.begin(), g.end());
    seg.push_back(static_cast<int32_t>(order.size()));
  }
  order.insert(order.end(), seg.begin(), seg.end());
  int32_t *ro = nullptr;
  if ((s = upload_vec(p, order, &ro)) != SPMM_OK) return s;
  L.row_ptr = rp;
  L.col_idx = ci;
  L.frag = fv;
  L.row_order = ro;
  L.row_seg = ro + ntiles;
  L.paired = paired;
  L.pair_rows = nullptr;
  L.pair_ptr = nullptr;
  L.units = nullptr;
  L.npairs = 0;
  if (paired) {
    int32_t *prw = nullptr, *pp = nullptr, *un = nullptr;
    if ((s = upload_vec(p, pair_rows, &prw)) != SPMM_OK) return s;
    if ((s = upload_vec(p, pair_ptr, &pp)) != SPMM_OK) return s;
    if ((s = upload_vec(p, units, &un)) != SPMM_OK) return s;
    L.pair_rows = prw;
    L.pair_ptr = pp;
    L.units = reinterpret_cast<const int4 *>(un);
    L.npairs = ntiles;
  }
  L.row_groups = groups;
  L.tn = sc.tn;
  L.kh = sc.kh;
  L.grid = bcsr_grid(seg.data(), sc, p->n);
  L.mb = mb;
  L.n = p->n;
  L.k_rows = a.k;
  L.col_perm = nullptr;
  L.c_rows = nullptr;
  if (!a.col_perm.empty()) {
    int32_t *cp = nullptr;
    if ((s = upload_vec(p, a.col_perm, &cp)) != SPMM_OK) return s;
    L.col_perm = cp;
  }
  if (!a.row_perm.empty()) {
    int32_t *rows = nullptr;
    if ((s = upload_vec(p, a.row_perm, &rows)) != SPMM_OK) return s;
    L.c_rows = rows;
  }
  p->info.tile_m = paired ? 128 : 64;
  p->info.tile_n = L.tn;
  p->info.grid = L.grid;
  return SPMM_OK;
}

// ---- WCSR plan: chunk descriptors, split rows and their partial slots ------
}  // namespace

spmm_status_t wcsr_chunk_descriptors(const Matrix &a, vec<WcsrChunk> &chunks,
                                     vec<int32_t> &slot_row) {
  const int64_t m = a.m, W = a.window_rows;
  const int64_t C = static_cast<int64_t>(a.chunk_window.size());
  const int64_t *rp = a.row_ptr.data();
  chunks.assign(C, WcsrChunk{});
  slot_row.clear();
  for (int64_t c = 0; c < C; ++c) {
    const int64_t w = a.chunk_window[c];
    const int64_t r0 = w * W, r1 = std::min(m, r0 + W);
    const int64_t b = a.chunk_begin[c], e = a.chunk_begin[c + 1];
    const bool last_of_window = (e == rp[r1]);
    int64_t rb = -1, re = -1;
    for (int64_t r = r0; r < r1; ++r) {
      const int64_t s0 = rp[r], s1 = rp[r + 1];
      bool mine;
      if (s0 == s1)  // empty row: owned by the chunk whose range holds its position
        mine = (b <= s0 && s0 < e) || (s0 == e && last_of_window);
      else
        mine = s0 < e && s1 > b;
      if (mine) {
        if (rb < 0) rb = r;
        re = r + 1;
      }
    }
    if (rb < 0) return fail(SPMM_ERR_INTERNAL, "spmm_plan: chunk without rows");
    WcsrChunk &d = chunks[c];
    d.nz_begin = b;
    d.nz_end = e;
    d.row_begin = static_cast<int32_t>(rb);
    d.row_end = static_cast<int32_t>(re);
    d.slot_first = d.slot_last = -1;
    auto split = [&](int64_t r) { return rp[r] != rp[r + 1] && (rp[r] < b || rp[r + 1] > e); };
    if (split(rb)) {
      d.slot_first = static_cast<int32_t>(slot_row.size());
      slot_row.push_back(static_cast<int32_t>(rb));
    }
    if (re - 1 == rb) {
      d.slot_last = d.slot_first;
    } else if (split(re - 1)) {
      d.slot_last = static_cast<int32_t>(slot_row.size());
      slot_row.push_back(static_cast<int32_t>(re - 1));
    }
  }
  return SPMM_OK;
}

namespace {

spmm_status_t plan_wcsr(spmm_plan_s *p) {
  const Matrix &a = *p->a;
  const int64_t C = static_cast<int64_t>(a.chunk_window.size());
  vec<WcsrChunk> chunks;
  vec<int32_t> slot_row;  // row of each partial slot, in slot order
  spmm_status_t st = wcsr_chunk_descriptors(a, chunks, slot_row);
  if (st != SPMM_OK) return st;
  // slots of one split row are consecutive: group them
  vec<int32_t> merge_row, merge_slot;
  for (size_t s = 0; s < slot_row.size(); ++s) {
    if (s == 0 || slot_row[s] != slot_row[s - 1]) {
      merge_row.push_back(slot_row[s]);
      merge_slot.push_back(static_cast<int32_t>(s));
    }
  }
  merge_slot.push_back(static_cast<int32_t>(slot_row.size()));
  for (size_t q = 0; q + 1 < merge_slot.size(); ++q)
    if (merge_slot[q + 1] - merge_slot[q] < 2)
      return fail(SPMM_ERR_INTERNAL, "spmm_plan: split row with a single piece");

  WcsrLaunch &L = p->wcsr;
  spmm_status_t s;
  WcsrChunk *dchunks = nullptr;
  int64_t *drp = nullptr;
  int32_t *dci = nullptr, *dmr = nullptr, *dms = nullptr;
  float *dv = nullptr;
  if ((s = upload_vec(p, chunks, &dchunks)) != SPMM_OK) return s;
  if ((s = upload_vec(p, a.row_ptr, &drp)) != SPMM_OK) return s;
  if ((s = upload_vec(p, a.col_idx, &dci)) != SPMM_OK) return s;
  if ((s = upload_vec(p, a.vals, &dv)) != SPMM_OK) return s;
  if ((s = upload_vec(p, merge_row, &dmr)) != SPMM_OK) return s;
  if ((s = upload_vec(p, merge_slot, &dms)) != SPMM_OK) return s;
  const int64_t ws_bytes = static_cast<int64_t>(slot_row.size()) * p->n * 4;
  void *ws = nullptr;
  if ((s = upload(p, nullptr, static_cast<size_t>(ws_bytes), &ws)) != SPMM_OK) return s;
  p->info.device_bytes -= std::max<int64_t>(ws_bytes, 16);
  L.chunks = dchunks;
  L.num_chunks = C;
  L.row_ptr = drp;
  L.col_idx = dci;
  L.vals = dv;
  L.merge_row = dmr;
  L.merge_slot = dms;
  L.num_split_rows = static_cast<int64_t>(merge_row.size());
  L.partial = static_cast<float *>(ws);
  L.n = p->n;
  p->info.workspace_bytes = ws_bytes;
  p->info.num_split_rows = L.num_split_rows;
  p->info.num_slots = static_cast<int64_t>(slot_row.size());
  p->info.tile_m = 0;
  p->info.tile_n = 0;
  p->info.grid = wcsr_grid(C, p->n);
  return SPMM_OK;
}

// ---- SDDMM plan: the WCSR chunks, the pattern, no workspace ----------------
spmm_status_t plan_sddmm(spmm_plan_s *p, int64_t kd, spmm_dtype_t dtype) {
  const Matrix &a = *p->a;
  vec<WcsrChunk> chunks;
  vec<int32_t> slot_row;  // unused: sampled entries are independent
  spmm_status_t st = wcsr_chunk_descriptors(a, chunks, slot_row);
  if (st != SPMM_OK) return st;
  SddmmLaunch &L = p->sdd;
  WcsrChunk *dchunks = nullptr;
  int64_t *drp = nullptr;
  int32_t *dci = nullptr;
  if ((st = upload_vec(p, chunks, &dchunks)) != SPMM_OK) return st;
  if ((st = upload_vec(p, a.row_ptr, &drp)) != SPMM_OK) return st;
  if ((st = upload_vec(p, a.col_idx, &dci)) != SPMM_OK) return st;
  L.chunks = dchunks;
  L.num_chunks = static_cast<int64_t>(chunks.size());
  L.row_ptr = drp;
  L.col_idx = dci;
  L.kd = kd;
  L.dtype = dtype;
  p->info.grid = sddmm_grid(L.num_chunks);
  return SPMM_OK;
}

// ---- SDDMM plan on a BCSR pattern: block groups and inner-dimension ranges ---
// workgroups a block-SDDMM launch aims for (about eight per CU)
constexpr int64_t kSddmmUnits = 2048;
spmm_status_t plan_sddmm_bcsr(spmm_plan_s *p, int64_t kd, bool int8) {
  const Matrix &a = *p->a;
  const int64_t nnzb = static_cast<int64_t>(a.bcol_idx.size());
  const int G = sddmm_bcsr_group();
  // groups of up to G consecutive stored blocks of one block row
  vec<int32_t> groups;
  for (int64_t r = 0; r + 1 < static_cast<int64_t>(a.brow_ptr.size()); ++r)
    for (int32_t b = a.brow_ptr[r]; b < a.brow_ptr[r + 1]; b += G)
      groups.insert(groups.end(),
                    {static_cast<int32_t>(r), b, std::min<int32_t>(G, a.brow_ptr[r + 1] - b), 0});
  const int64_t ngroups = static_cast<int64_t>(groups.size() / 4);
  // ranges of the inner dimension: enough workgroups for the chip (about
  // kSddmmUnits), each range at least 16 chunks long
  const int64_t chunk = sddmm_bcsr_chunk(int8);
  const int64_t chunks = (kd + chunk - 1) / chunk;
  int64_t nsplit = 1;
  if (ngroups > 0 && chunks > 0) {
    nsplit = std::min<int64_t>((kSddmmUnits + ngroups - 1) / ngroups,
                               std::max<int64_t>(1, chunks / 16));
    nsplit = std::max<int64_t>(1, nsplit);
  }
  const int64_t ksplit = std::max<int64_t>(1, (chunks + nsplit - 1) / nsplit) * chunk;
  if (kd > 0) nsplit = (kd + ksplit - 1) / ksplit;
  if (ngroups * 8 * nsplit > INT32_MAX) return fail(SPMM_ERR_UNSUPPORTED, "spmm_plan_sddmm: too many blocks");

  SddmmBcsrLaunch &L = p->sddb;
  spmm_status_t st;
  int32_t *dg = nullptr, *dci = nullptr;
  if ((st = upload_vec(p, groups, &dg)) != SPMM_OK) return st;
  if ((st = upload_vec(p, a.bcol_idx, &dci)) != SPMM_OK) return st;
  const int64_t ws_bytes = nsplit > 1 ? nsplit * nnzb * 64 * 64 * 4 : 0;
  void *ws = nullptr;
  if (ws_bytes > 0) {
    if ((st = upload(p, nullptr, static_cast<size_t>(ws_bytes), &ws)) != SPMM_OK) return st;
    p->info.device_bytes -= ws_bytes;
  }
  L.groups = reinterpret_cast<const int4 *>(dg);
  L.ngroups = static_cast<int32_t>(ngroups);
  L.col_idx = dci;
  L.nnzb = nnzb;
  L.kd = kd;
  L.ksplit = ksplit;
  L.nsplit = static_cast<int32_t>(nsplit);
  L.int8 = int8;
  L.partial = ws;
  p->info.workspace_bytes = ws_bytes;
  p->info.tile_m = 64;
  p->info.tile_n = 64;
  p->info.grid = 8 * ((ngroups + 7) / 8) * nsplit;
  return SPMM_OK;
}

// ---- 2:4 plan: rows and k padded to whole tiles with zeros -----------------
spmm_status_t plan_24(spmm_plan_s *p) {
  const Matrix &a = *p->a;
  if (p->n % 16 != 0) return fail(SPMM_ERR_UNSUPPORTED, "spmm_plan: 2:4 needs n % 16 == 0");
  // a sliding-window matrix is the 2:4 matrix of its lifted columns
  const bool slide = a.format == SPMM_FORMAT_SLIDE;
  const bool bf16 = a.dtype == SPMM_BF16;
  const int64_t elem = bf16 ? 2 : 1;
  const int64_t k = slide ? a.k_lift : a.k;
  const int64_t TM = sp24_tile_m(), TK = sp24_tile_k(bf16);
  const int64_t m_pad = (a.m + TM - 1) / TM * TM;
  // k = 0 gives no k-steps: the kernel then writes zeros and never reads B
  const int64_t k_pad = (k + TK - 1) / TK * TK;
  vec<int8_t> v(static_cast<size_t>(m_pad * (k_pad / 2) * elem));
  vec<uint8_t> mt(static_cast<size_t>(m_pad * (k_pad / 8)));
  const void *src = bf16 ? static_cast<const void *>(a.vals24_bf16.data())
                         : static_cast<const void *>(a.vals24.data());
  sp24_tile_layout(src, a.meta24.data(), a.m, k, m_pad, k_pad, bf16, v.data(), mt.data());
  Sp24Launch &L = p->sp24;
  L.bf16 = bf16;
  spmm_status_t s;
  int8_t *dv = nullptr;
  uint8_t *dm = nullptr;
  if ((s = upload_vec(p, v, &dv)) != SPMM_OK) return s;
  if ((s = upload_vec(p, mt, &dm)) != SPMM_OK) return s;
  L.vals = dv;
  L.meta = dm;
  L.m = a.m;
  L.k = k;
  L.n = p->n;
  L.m_pad = m_pad;
  L.k_pad = k_pad;
  L.tile_ptr = nullptr;
  L.tile_step = nullptr;
  L.row_order = nullptr;
  L.b_rows = nullptr;
  if (slide) {
    // B row of every lifted k-row, padded with row 0 to whole k-steps (the
    // padded k-rows meet zero A values)
    vec<int32_t> rows(static_cast<size_t>(k_pad), 0);
    for (int64_t j = 0; j < k; ++j) rows[j] = static_cast<int32_t>(slide_source_row(j, a.slide_group));
    int32_t *dr = nullptr;
    if ((s = upload_vec(p, rows, &dr)) != SPMM_OK) return s;
    L.b_rows = dr;
  }
  p->info.tile_m = sp24_tile_m();
  L.tn = sp24_tile_n(p->n, L.b_rows != nullptr);
  p->info.tile_n = L.tn;
  p->info.grid = sp24_grid(a.m, p->n, L.tn);
  return SPMM_OK;
}

// ---- tile-vector-wise plan: the stored tiles in the 2:4 kernel's layout ------
// A stored tile of tk columns becomes tk / TK consecutive k-steps of the
// kernel (TK = 128 int8, 64 bf16).
spmm_status_t plan_tvw(spmm_plan_s *p) {
  const Matrix &a = *p->a;
  const bool bf16 = a.dtype == SPMM_BF16;
  const int64_t TK = sp24_tile_k(bf16), elem = bf16 ? 2 : 1;
  if (p->n % 16 != 0) return fail(SPMM_ERR_UNSUPPORTED, "spmm_plan: TVW needs n % 16 == 0");
  if (a.bm != sp24_tile_m() || a.bk % TK != 0)
    return fail(SPMM_ERR_UNSUPPORTED,
                "spmm_plan: TVW kernels take tiles of 256 rows and a multiple of 128 (int8) or "
                "64 (bf16) columns");
  const int64_t ntiles = static_cast<int64_t>(a.bcol_idx.size());
  const int64_t per = a.bk / TK;
  vec<int8_t> v(static_cast<size_t>(ntiles * a.bm * (a.bk / 2) * elem));
  vec<uint8_t> mt(static_cast<size_t>(ntiles * a.bm * (a.bk / 8)));
  const void *src = bf16 ? static_cast<const void *>(a.vals24_bf16.data())
                         : static_cast<const void *>(a.vals24.data());
  tvw_tile_layout(src, a.meta24.data(), ntiles, a.bk, bf16, v.data(), mt.data());
  vec<int32_t> ptr(a.brow_ptr.size()), step(static_cast<size_t>(ntiles * per));
  for (size_t T = 0; T < a.brow_ptr.size(); ++T) ptr[T] = static_cast<int32_t>(a.brow_ptr[T] * per);
  for (int64_t t = 0; t < ntiles; ++t)
    for (int64_t s = 0; s < per; ++s) step[t * per + s] = static_cast<int32_t>(a.bcol_idx[t] * per + s);
  const vec<int32_t> order = tvw_row_order(a.brow_ptr.data(), static_cast<int64_t>(a.brow_ptr.size()) - 1);
  Sp24Launch &L = p->sp24;
  spmm_status_t s;
  int8_t *dv = nullptr;
  uint8_t *dm = nullptr;
  int32_t *tp = nullptr, *ts = nullptr, *ro = nullptr;
  if ((s = upload_vec(p, v, &dv)) != SPMM_OK) return s;
  if ((s = upload_vec(p, mt, &dm)) != SPMM_OK) return s;
  if ((s = upload_vec(p, ptr, &tp)) != SPMM_OK) return s;
  if ((s = upload_vec(p, step, &ts)) != SPMM_OK) return s;
  if ((s = upload_vec(p, order, &ro)) != SPMM_OK) return s;
  L.row_order = ro;
  L.bf16 = bf16;
  L.vals = dv;
  L.meta = dm;
  L.tile_ptr = tp;
  L.tile_step = ts;
  L.b_rows = nullptr;
  L.m = a.m;
  L.k = a.k;
  L.n = p->n;
  L.m_pad = a.m;
  L.k_pad = a.k;
  p->info.tile_m = sp24_tile_m();
  L.tn = sp24_tile_n(p->n, L.b_rows != nullptr);
  p->info.tile_n = L.tn;
  p->info.grid = sp24_grid(a.m, p->n, L.tn);
  return SPMM_OK;
}

bool aligned16(const void *ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// SPMM_LOG set to anything but "" or "0": every plan that succeeds prints
// its decisions (kernel, tile, grid, schedule, device and workspace bytes)
// as one line on stderr.  Read at each call.
bool plan_log_on() {
  const char *v = std::getenv("SPMM_LOG");
  return v && v[0] && std::strcmp(v, "0") != 0;
}

void plan_log(const char *fn, const spmm_plan_s *p) {
  static const char *const kFormat[] = {"bcsr", "wcsr", "24", "tvw", "slide"};
  const Matrix &a = *p->a;
  const spmm_plan_info_t &i = p->info;
  const char *fmt = a.format >= 0 && a.format <= 4 ? kFormat[a.format] : "?";
  std::string what;
  if (p->sddmm && a.format == SPMM_FORMAT_WCSR) {
    what = "kernel=sddmm_csr chunks=" + std::to_string(p->sdd.num_chunks);
  } else if (p->sddmm) {
    what = std::string("kernel=sddmm_bcsr_mfma") + (p->sddb.nsplit > 1 ? "+sddmm_bcsr_merge" : "") +
           " groups=" + std::to_string(p->sddb.ngroups) + " ranges=" + std::to_string(p->sddb.nsplit);
  } else if (a.format == SPMM_FORMAT_BCSR) {
    const BcsrLaunch &L = p->bcsr;
    what = std::string("kernel=") + (L.paired ? "bcsr_bf16_pair" : "bcsr_bf16_mfma") +
           " row_groups=" + std::to_string(L.row_groups) + " stage_k=" + std::to_string(L.kh) +
           (L.paired ? " pairs=" + std::to_string(L.npairs) : "") + (L.col_perm ? " reordered" : "");
  } else if (a.format == SPMM_FORMAT_WCSR) {
    what = std::string("kernel=wcsr_stream") + (p->wcsr.num_split_rows > 0 ? "+wcsr_merge" : "") +
           " window_rows=" + std::to_string(a.window_rows) + " max_chunk_nnz=" +
           std::to_string(a.max_chunk_nnz) + " chunks=" + std::to_string(p->wcsr.num_chunks) +
           " split_rows=" + std::to_string(i.num_split_rows) + " slots=" + std::to_string(i.num_slots);
  } else {
    what = std::string("kernel=") + (p->sp24.bf16 ? "sp24_bf16_smfmac" : "sp24_i8_smfmac") +
           " k_pad=" + std::to_string(p->sp24.k_pad);
  }
  std::fprintf(stderr,
               "[spmm] %s: format=%s device=%d m=%lld k=%lld n=%lld %s tile=%dx%d grid=%lld "
               "device_bytes=%lld workspace_bytes=%lld\n",
               fn, fmt, static_cast<int>(i.device), static_cast<long long>(i.m),
               static_cast<long long>(i.k), static_cast<long long>(i.n), what.c_str(),
               static_cast<int>(i.tile_m), static_cast<int>(i.tile_n), static_cast<long long>(i.grid),
               static_cast<long long>(i.device_bytes), static_cast<long long>(i.workspace_bytes));
  std::fflush(stderr);
}

}  // namespace
}  // namespace sdm

using namespace sdm;

extern "C" {

const char *spmm_status_str(spmm_status_t s) {
  switch (s) {
    case SPMM_OK: return "SPMM_OK";
    case SPMM_ERR_INVALID_ARG: return "SPMM_ERR_INVALID_ARG";
    case SPMM_ERR_UNSUPPORTED: return "SPMM_ERR_UNSUPPORTED";
    case SPMM_ERR_OUT_OF_MEMORY: return "SPMM_ERR_OUT_OF_MEMORY";
    case SPMM_ERR_HIP: return "SPMM_ERR_HIP";
    case SPMM_ERR_INTERNAL: return "SPMM_ERR_INTERNAL";
  }
  return "SPMM_ERR_UNKNOWN";
}

const char *spmm_last_error(void) { return g_last_error.c_str(); }

spmm_status_t spmm_pack_bcsr(int64_t m, int64_t k, int32_t block_m, int32_t block_k,
                             spmm_dtype_t dtype, const void *a_host, int64_t lda,
                             spmm_matrix_t *out) {
  alloc_hook_begin();
  if (!out) return fail(SPMM_ERR_INVALID_ARG, "spmm_pack_bcsr: out is NULL");
  *out = nullptr;
  if (dtype != SPMM_BF16) return fail(SPMM_ERR_UNSUPPORTED, "spmm_pack_bcsr: only bf16 values");
  if (m < 0 || k < 0 || m > INT32_MAX || k > INT32_MAX || block_m <= 0 || block_k <= 0 ||
      m % block_m != 0 || k % block_k != 0 || lda < k || (m * k > 0 && !a_host))
    return fail(SPMM_ERR_INVALID_ARG, "spmm_pack_bcsr: bad shape, block, lda or pointer");
  return guarded([&]() -> spmm_status_t {
    auto a = new_matrix();
    spmm_status_t s = pack_bcsr_bf16(m, k, block_m, block_k,
                                     static_cast<const uint16_t *>(a_host), lda, *a);
    if (s != SPMM_OK) return s;
    *out = a.release();
    return SPMM_OK;
  });
}

spmm_status_t spmm_pack_slide(int64_t m, int64_t k, const int8_t *a_host, int64_t lda, int32_t group,
                              spmm_matrix_t *out) {
  alloc_hook_begin();
  if (!out) return fail(SPMM_ERR_INVALID_ARG, "spmm_pack_slide: out is NULL");
  *out = nullptr;
  // group = 2N with N >= 2; the lifted row (4(N-1) columns per group) must
  // hold whole bytes of 2:4 metadata
  if (m < 0 || k < 0 || m > INT32_MAX || k > INT32_MAX || group < 4 || group > 64 || group % 2 != 0 ||
      k % group != 0 || ((k / group) * 4 * (group / 2 - 1)) % 8 != 0 || lda < k ||
      (m * k > 0 && !a_host))
    return fail(SPMM_ERR_INVALID_ARG, "spmm_pack_slide: bad shape, group, lda or pointer");
  return guarded([&]() -> spmm_status_t {
    auto a = new_matrix();
    spmm_status_t s = pack_slide_i8(m, k, a_host, lda, group, *a);
    if (s != SPMM_OK) return s;
    *out = a.release();
    return SPMM_OK;
  });
}

spmm_status_t spmm_pack_tvw(int64_t m, int64_t k, spmm_dtype_t dtype, const void *a_host,
                            int64_t lda, int32_t tile_m, int32_t tile_k, spmm_matrix_t *out) {
  alloc_hook_begin();
  if (!out) return fail(SPMM_ERR_INVALID_ARG, "spmm_pack_tvw: out is NULL");
  *out = nullptr;
  if (dtype != SPMM_I8 && dtype != SPMM_BF16)
    return fail(SPMM_ERR_UNSUPPORTED, "spmm_pack_tvw: int8 or bf16 values only");
  if (m < 0 || k < 0 || m > INT32_MAX || k > INT32_MAX || tile_m <= 0 || tile_k <= 0 ||
      tile_k % 8 != 0 || m % tile_m != 0 || k % tile_k != 0 || lda < k || (m * k > 0 && !a_host))
    return fail(SPMM_ERR_INVALID_ARG, "spmm_pack_tvw: bad shape, tile, lda or pointer");
  return guarded([&]() -> spmm_status_t {
    auto a = new_matrix();
    spmm_status_t s = pack_tvw(m, k, dtype, a_host, lda, tile_m, tile_k, *a);
    if (s != SPMM_OK) return s;
    *out = a.release();
    return SPMM_OK;
  });
}

spmm_status_t spmm_pack_bcsr_csr(int64_t m, int64_t k, spmm_dtype_t dtype,
                                 const int64_t *row_ptr, const int32_t *col_idx,
                                 const void *vals, int32_t block_m, int32_t block_k,
                                 int32_t reorder, spmm_matrix_t *out) {
  alloc_hook_begin();
  if (!out) return fail(SPMM_ERR_INVALID_ARG, "spmm_pack_bcsr_csr: out is NULL");
  *out = nullptr;
  if (dtype != SPMM_BF16) return fail(SPMM_ERR_UNSUPPORTED, "spmm_pack_bcsr_csr: only bf16 values");
  if (m < 0 || k < 0 || m > INT32_MAX || k > INT32_MAX || !row_ptr || block_m <= 0 ||
      block_k <= 0 || m % block_m != 0 || k % block_k != 0 || (reorder != 0 && reorder != 1))
    return fail(SPMM_ERR_INVALID_ARG, "spmm_pack_bcsr_csr: bad shape, block, reorder or pointer");
  return guarded([&]() -> spmm_status_t {
    auto a = new_matrix();
    spmm_status_t s = pack_bcsr_csr_bf16(m, k, row_ptr, col_idx, static_cast<const uint16_t *>(vals),
                                         block_m, block_k, reorder == 1, *a);
    if (s != SPMM_OK) return s;
    *out = a.release();
    return SPMM_OK;
  });
}

spmm_status_t spmm_pack_wcsr(int64_t m, int64_t k, spmm_dtype_t dtype,
                             const int64_t *row_ptr, const int32_t *col_idx,
                             const void *vals, int32_t window_rows,
                             int64_t max_chunk_nnz, spmm_matrix_t *out) {
  alloc_hook_begin();
  if (!out) return fail(SPMM_ERR_INVALID_ARG, "spmm_pack_wcsr: out is NULL");
  *out = nullptr;
  if (dtype != SPMM_F32) return fail(SPMM_ERR_UNSUPPORTED, "spmm_pack_wcsr: only fp32 values");
  if (m < 0 || k < 0 || m > INT32_MAX - 1 || k > INT32_MAX || !row_ptr || window_rows < 0 ||
      max_chunk_nnz < 0)
    return fail(SPMM_ERR_INVALID_ARG, "spmm_pack_wcsr: bad shape, window, chunk bound or pointer");
  // 0 selects the defaults: windows of 16 rows for large matrices, fewer
  // (down to one row) below 16 x 16384 rows so that a small matrix still
  // gives each CU several windows; chunks of at most 512 entries
  if (window_rows == 0)
    window_rows = static_cast<int32_t>(std::max<int64_t>(1, std::min<int64_t>(16, m / 16384)));
  if (max_chunk_nnz == 0) max_chunk_nnz = 512;
  return guarded([&]() -> spmm_status_t {
    auto a = new_matrix();
    spmm_status_t s = pack_wcsr_f32(m, k, row_ptr, col_idx, static_cast<const float *>(vals),
                                    window_rows, max_chunk_nnz, *a);
    if (s != SPMM_OK) return s;
    *out = a.release();
    return SPMM_OK;
  });
}

spmm_status_t spmm_pack_24(int64_t m, int64_t k, spmm_dtype_t dtype, const void *a_host,
                           int64_t lda, spmm_matrix_t *out) {
  alloc_hook_begin();
  if (!out) return fail(SPMM_ERR_INVALID_ARG, "spmm_pack_24: out is NULL");
  *out = nullptr;
  if (dtype != SPMM_I8 && dtype != SPMM_BF16)
    return fail(SPMM_ERR_UNSUPPORTED, "spmm_pack_24: int8 or bf16 values only");
  if (m < 0 || k < 0 || m > INT32_MAX || k > INT32_MAX || k % 8 != 0 || lda < k ||
      (m * k > 0 && !a_host))
    return fail(SPMM_ERR_INVALID_ARG, "spmm_pack_24: bad shape (k % 8 == 0 needed), lda or pointer");
  return guarded([&]() -> spmm_status_t {
    auto a = new_matrix();
    spmm_status_t s = pack_24(m, k, dtype, a_host, lda, *a);
    if (s != SPMM_OK) return s;
    *out = a.release();
    return SPMM_OK;
  });
}

spmm_status_t spmm_matrix_info(spmm_matrix_t a, spmm_matrix_info_t *info) {
  if (!a || !info) return fail(SPMM_ERR_INVALID_ARG, "spmm_matrix_info: NULL argument");
  std::memset(info, 0, sizeof(*info));
  info->format = a->format;
  info->dtype = a->dtype;
  info->m = a->m;
  info->k = a->k;
  info->nnz = a->nnz;
  if (a->format == SPMM_FORMAT_BCSR || a->format == SPMM_FORMAT_TVW) {
    info->nnzb = static_cast<int64_t>(a->bcol_idx.size());
    info->block_m = a->bm;
    info->block_k = a->bk;
  } else if (a->format == SPMM_FORMAT_SLIDE) {
    info->block_k = a->slide_group;
  } else if (a->format == SPMM_FORMAT_WCSR) {
    info->window_rows = a->window_rows;
    info->max_chunk_nnz = a->max_chunk_nnz;
    info->num_windows = (a->m + a->window_rows - 1) / a->window_rows;
    info->num_chunks = static_cast<int64_t>(a->chunk_window.size());
  }
  return SPMM_OK;
}

spmm_status_t spmm_matrix_array(spmm_matrix_t a, int32_t which, const void **data,
                                int64_t *count) {
  if (!a || !data || !count) return fail(SPMM_ERR_INVALID_ARG, "spmm_matrix_array: NULL argument");
  *data = nullptr;
  *count = 0;
  auto give = [&](const auto &v) {
    *data = v.data();
    *count = static_cast<int64_t>(v.size());
    return SPMM_OK;
  };
  switch (a->format) {
    case SPMM_FORMAT_BCSR:
      if (which == SPMM_ARRAY_ROW_PTR) return give(a->brow_ptr);
      if (which == SPMM_ARRAY_COL_IDX) return give(a->bcol_idx);
      if (which == SPMM_ARRAY_VALS) return give(a->bvals);
      if (which == SPMM_ARRAY_ROW_PERM) return give(a->row_perm);
      if (which == SPMM_ARRAY_COL_PERM) return give(a->col_perm);
      break;
    case SPMM_FORMAT_WCSR:
      if (which == SPMM_ARRAY_ROW_PTR) return give(a->row_ptr);
      if (which == SPMM_ARRAY_COL_IDX) return give(a->col_idx);
      if (which == SPMM_ARRAY_VALS) return give(a->vals);
      if (which == SPMM_ARRAY_CHUNK_WINDOW) return give(a->chunk_window);
      if (which == SPMM_ARRAY_CHUNK_BEGIN) return give(a->chunk_begin);
      break;
    case SPMM_FORMAT_24:
      if (which == SPMM_ARRAY_VALS)
        return a->dtype == SPMM_BF16 ? give(a->vals24_bf16) : give(a->vals24);
      if (which == SPMM_ARRAY_META) return give(a->meta24);
      break;
    case SPMM_FORMAT_SLIDE:
      if (which == SPMM_ARRAY_VALS) return give(a->vals24);
      if (which == SPMM_ARRAY_META) return give(a->meta24);
      break;
    case SPMM_FORMAT_TVW:
      if (which == SPMM_ARRAY_ROW_PTR) return give(a->brow_ptr);
      if (which == SPMM_ARRAY_COL_IDX) return give(a->bcol_idx);
      if (which == SPMM_ARRAY_VALS)
        return a->dtype == SPMM_BF16 ? give(a->vals24_bf16) : give(a->vals24);
      if (which == SPMM_ARRAY_META) return give(a->meta24);
      break;
  }
  return fail(SPMM_ERR_INVALID_ARG, "spmm_matrix_array: no such array for this format");
}

void spmm_matrix_destroy(spmm_matrix_t a) { release(a); }

spmm_status_t spmm_plan(spmm_matrix_t a, int64_t n, spmm_dtype_t b_dtype, spmm_dtype_t c_dtype,
                        int32_t device, spmm_plan_t *out) {
  alloc_hook_begin();
  if (!out) return fail(SPMM_ERR_INVALID_ARG, "spmm_plan: out is NULL");
  *out = nullptr;
  if (!a || n < 0 || n > INT32_MAX) return fail(SPMM_ERR_INVALID_ARG, "spmm_plan: bad matrix or n");
  const bool ok_types =
      (a->format == SPMM_FORMAT_BCSR && b_dtype == SPMM_BF16 && c_dtype == SPMM_BF16) ||
      (a->format == SPMM_FORMAT_WCSR && b_dtype == SPMM_F32 && c_dtype == SPMM_F32) ||
      ((a->format == SPMM_FORMAT_24 || a->format == SPMM_FORMAT_TVW ||
        a->format == SPMM_FORMAT_SLIDE) &&
       a->dtype == SPMM_I8 && b_dtype == SPMM_I8 && c_dtype == SPMM_I32) ||
      ((a->format == SPMM_FORMAT_TVW || a->format == SPMM_FORMAT_24) && a->dtype == SPMM_BF16 &&
       b_dtype == SPMM_BF16 && c_dtype == SPMM_BF16);
  if (!ok_types) return fail(SPMM_ERR_UNSUPPORTED, "spmm_plan: unsupported (format, B, C) types");
  int ndev = 0;
  hipError_t e = hipGetDeviceCount(&ndev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceCount");
  if (device < 0 || device >= ndev) return fail(SPMM_ERR_INVALID_ARG, "spmm_plan: no such device");
  return guarded([&]() -> spmm_status_t {
    DeviceScope ds(device);
    if (ds.err != hipSuccess) return hip_fail(ds.err, "hipSetDevice");
    if (alloc_hook_fail()) throw std::bad_alloc();
    auto *p = new spmm_plan_s();
    retain(a);
    p->a = a;
    p->device = device;
    p->n = n;
    p->info.format = a->format;
    p->info.device = device;
    p->info.m = a->m;
    p->info.k = a->k;
    p->info.n = n;
    spmm_status_t s = SPMM_ERR_INTERNAL;
    try {
      if (a->format == SPMM_FORMAT_BCSR) s = plan_bcsr(p);
      else if (a->format == SPMM_FORMAT_WCSR) s = plan_wcsr(p);
      else if (a->format == SPMM_FORMAT_TVW) s = plan_tvw(p);
      else s = plan_24(p);  // 2:4 and sliding-window
    } catch (...) {
      free_plan(p);
      throw;
    }
    if (s == SPMM_OK) {
      e = hipDeviceSynchronize();
      if (e != hipSuccess) s = hip_fail(e, "hipDeviceSynchronize");
    }
    if (s != SPMM_OK) {
      free_plan(p);
      return s;
    }
    *out = p;
    if (plan_log_on()) plan_log("spmm_plan", p);
    return SPMM_OK;
  });
}

spmm_status_t spmm_plan_info(spmm_plan_t p, spmm_plan_info_t *info) {
  if (!p || !info) return fail(SPMM_ERR_INVALID_ARG, "spmm_plan_info: NULL argument");
  *info = p->info;
  return SPMM_OK;
}

void spmm_plan_destroy(spmm_plan_t p) { free_plan(p); }

}  // extern "C"

namespace {

// spmm_execute and spmm_execute_noalloc: the same checks and kernels; with
// noalloc, a WCSR plan's partial rows go to the library's per-GPU scratch
// array instead of the plan's workspace.
spmm_status_t execute(const char *fn, spmm_plan_t p, const void *b_dev, int64_t ldb, void *c_dev,
                      int64_t ldc, hipStream_t stream, bool noalloc) {
  const std::string name(fn);
  if (!p) return fail(SPMM_ERR_INVALID_ARG, name + ": plan is NULL");
  if (p->sddmm) return fail(SPMM_ERR_INVALID_ARG, name + ": plan is an SDDMM plan");
  const Matrix &a = *p->a;
  const int64_t n = p->n;
  if (n == 0 || a.m == 0) return SPMM_OK;
  const bool bf16 = a.format == SPMM_FORMAT_BCSR || a.dtype == SPMM_BF16;
  const bool i8 = a.dtype == SPMM_I8;
  const int64_t eb = bf16 ? 2 : (i8 ? 1 : 4);  // B: bf16, int8 or fp32
  const int64_t ec = bf16 ? 2 : 4;              // C: bf16, int32 or fp32
  if (!c_dev || (!b_dev && a.k > 0))
    return fail(SPMM_ERR_INVALID_ARG, name + ": B or C is NULL");
  if (!aligned16(b_dev) || !aligned16(c_dev) || ldb < n || ldc < n || (ldb * eb) % 16 != 0 ||
      (ldc * ec) % 16 != 0)
    return fail(SPMM_ERR_INVALID_ARG,
                name + ": B/C must be 16-byte aligned with ld >= n and ld*elem % 16 == 0");
  // the kernels address B with 32-bit byte offsets from its start (BCSR:
  // from the first row of a block; through a row map: from row 0)
  if (a.format == SPMM_FORMAT_BCSR) {
    if (ldb > (int64_t(1) << 24) || (p->bcsr.col_perm && a.k * ldb * 2 > int64_t(UINT32_MAX)))
      return fail(SPMM_ERR_UNSUPPORTED, name + ": ldb too large for this BCSR plan");
  } else if (a.format != SPMM_FORMAT_WCSR && p->sp24.k_pad * ldb * eb > int64_t(UINT32_MAX)) {
    return fail(SPMM_ERR_UNSUPPORTED, name + ": k_pad * ldb * elem must be below 2^32");
  }
  const int64_t scratch_bytes = p->info.num_slots * n * 4;
  if (noalloc && a.format == SPMM_FORMAT_WCSR && scratch_bytes > kNoallocScratchBytes)
    return fail(SPMM_ERR_UNSUPPORTED,
                name + ": the plan's partial rows need " + std::to_string(scratch_bytes) +
                    " bytes of scratch, more than the " + std::to_string(kNoallocScratchBytes) +
                    " the library holds per GPU; use spmm_execute");
  DeviceScope ds(p->device);
  if (ds.err != hipSuccess) return hip_fail(ds.err, "hipSetDevice");
  hipError_t e = hipSuccess;
  if (a.format == SPMM_FORMAT_BCSR) {
    BcsrLaunch L = p->bcsr;
    L.B = static_cast<const uint16_t *>(b_dev);
    L.ldb = ldb;
    L.C = static_cast<uint16_t *>(c_dev);
    L.ldc = ldc;
    e = launch_bcsr_bf16(L, stream);
  } else if (a.format == SPMM_FORMAT_WCSR) {
    WcsrLaunch L = p->wcsr;
    L.B = static_cast<const float *>(b_dev);
    L.ldb = ldb;
    L.C = static_cast<float *>(c_dev);
    L.ldc = ldc;
    if (noalloc && scratch_bytes > 0) {
      void *ptr = nullptr;
      e = noalloc_scratch(p->device, &ptr);
      if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress");
      L.partial = static_cast<float *>(ptr);
    }
    e = launch_wcsr_f32(L, stream);
  } else {
    Sp24Launch L = p->sp24;
    L.B = b_dev;
    L.ldb = ldb;
    L.C = c_dev;
    L.ldc = ldc;
    e = launch_sp24(L, stream);
  }
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  return SPMM_OK;
}

}  // namespace

extern "C" {

spmm_status_t spmm_execute(spmm_plan_t p, const void *b_dev, int64_t ldb, void *c_dev,
                           int64_t ldc, hipStream_t stream) {
  return execute("spmm_execute", p, b_dev, ldb, c_dev, ldc, stream, false);
}

spmm_status_t spmm_execute_noalloc(spmm_plan_t p, const void *b_dev, int64_t ldb, void *c_dev,
                                   int64_t ldc, hipStream_t stream) {
  return execute("spmm_execute_noalloc", p, b_dev, ldb, c_dev, ldc, stream, true);
}

spmm_status_t spmm_plan_sddmm(spmm_matrix_t a, int64_t kd, spmm_dtype_t dtype, int32_t device,
                              spmm_plan_t *out) {
  alloc_hook_begin();
  if (!out) return fail(SPMM_ERR_INVALID_ARG, "spmm_plan_sddmm: out is NULL");
  *out = nullptr;
  if (!a || kd < 0 || kd > INT32_MAX) return fail(SPMM_ERR_INVALID_ARG, "spmm_plan_sddmm: bad matrix or kd");
  const bool wcsr = a->format == SPMM_FORMAT_WCSR &&
                    (dtype == SPMM_F32 || dtype == SPMM_BF16 || dtype == SPMM_I8);
  const bool bcsr = a->format == SPMM_FORMAT_BCSR && (dtype == SPMM_BF16 || dtype == SPMM_I8);
  if (!wcsr && !bcsr)
    return fail(SPMM_ERR_UNSUPPORTED,
                "spmm_plan_sddmm: needs a WCSR pattern (fp32, bf16 or int8 X, Y) or a BCSR pattern "
                "(bf16 or int8 X, Y)");
  if (bcsr && (a->bm != 64 || a->bk != 64))
    return fail(SPMM_ERR_UNSUPPORTED, "spmm_plan_sddmm: BCSR patterns take 64 x 64 blocks");
  if (bcsr && (!a->row_perm.empty() || !a->col_perm.empty()))
    return fail(SPMM_ERR_UNSUPPORTED, "spmm_plan_sddmm: not for a reordered BCSR pattern");
  int ndev = 0;
  hipError_t e = hipGetDeviceCount(&ndev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceCount");
  if (device < 0 || device >= ndev) return fail(SPMM_ERR_INVALID_ARG, "spmm_plan_sddmm: no such device");
  return guarded([&]() -> spmm_status_t {
    DeviceScope ds(device);
    if (ds.err != hipSuccess) return hip_fail(ds.err, "hipSetDevice");
    if (alloc_hook_fail()) throw std::bad_alloc();
    auto *p = new spmm_plan_s();
    retain(a);
    p->a = a;
    p->sddmm = true;
    p->sddmm_dtype = dtype;
    p->device = device;
    p->n = kd;
    p->info.format = a->format;
    p->info.device = device;
    p->info.m = a->m;
    p->info.k = a->k;
    p->info.n = kd;
    spmm_status_t s = SPMM_ERR_INTERNAL;
    try {
      s = wcsr ? plan_sddmm(p, kd, dtype) : plan_sddmm_bcsr(p, kd, dtype == SPMM_I8);
    } catch (...) {
      free_plan(p);
      throw;
    }
    if (s == SPMM_OK) {
      e = hipDeviceSynchronize();
      if (e != hipSuccess) s = hip_fail(e, "hipDeviceSynchronize");
    }
    if (s != SPMM_OK) {
      free_plan(p);
      return s;
    }
    *out = p;
    if (plan_log_on()) plan_log("spmm_plan_sddmm", p);
    return SPMM_OK;
  });
}

spmm_status_t spmm_execute_sddmm(spmm_plan_t p, const void *x_dev, int64_t ldx, const void *y_dev,
                                 int64_t ldy, void *out_dev, hipStream_t stream) {
  if (!p) return fail(SPMM_ERR_INVALID_ARG, "spmm_execute_sddmm: plan is NULL");
  if (!p->sddmm) return fail(SPMM_ERR_INVALID_ARG, "spmm_execute_sddmm: plan is not an SDDMM plan");
  const Matrix &a = *p->a;
  const int64_t kd = p->n;
  const bool bcsr = a.format == SPMM_FORMAT_BCSR;
  const int64_t elem = p->sddmm_dtype == SPMM_F32 ? 4 : (p->sddmm_dtype == SPMM_BF16 ? 2 : 1);
  if (bcsr ? a.bcol_idx.empty() : a.nnz == 0) return SPMM_OK;
  if (!out_dev || (kd > 0 && (!x_dev || !y_dev)))
    return fail(SPMM_ERR_INVALID_ARG, "spmm_execute_sddmm: X, Y or out is NULL");
  // out: 16-byte pieces of blocks (BCSR), else one element per entry
  const uintptr_t out_align = bcsr ? 15u : (p->sddmm_dtype == SPMM_BF16 ? 1u : 3u);
  if ((reinterpret_cast<uintptr_t>(out_dev) & out_align) ||
      (kd > 0 && (!aligned16(x_dev) || !aligned16(y_dev) || ldx < kd || ldy < kd ||
                  (ldx * elem) % 16 != 0 || (ldy * elem) % 16 != 0)))
    return fail(SPMM_ERR_INVALID_ARG,
                "spmm_execute_sddmm: X/Y must be 16-byte aligned with ld >= kd and ld*elem % 16 "
                "== 0; out aligned to 16 bytes (BCSR) or to its element (WCSR)");
  // a BCSR workgroup addresses its 64 rows of X and of Y with 32-bit byte offsets
  if (bcsr && kd > 0 && 64 * std::max(ldx, ldy) * elem >= (int64_t(1) << 32))
    return fail(SPMM_ERR_UNSUPPORTED, "spmm_execute_sddmm: rows of X or Y longer than 64 MiB");
  DeviceScope ds(p->device);
  if (ds.err != hipSuccess) return hip_fail(ds.err, "hipSetDevice");
  hipError_t e;
  if (bcsr) {
    SddmmBcsrLaunch L = p->sddb;
    L.X = x_dev;
    L.ldx = ldx;
    L.Y = y_dev;
    L.ldy = ldy;
    L.out = out_dev;
    e = launch_sddmm_bcsr(L, stream);
  } else {
    SddmmLaunch L = p->sdd;
    L.X = x_dev;
    L.ldx = ldx;
    L.Y = y_dev;
    L.ldy = ldy;
    L.out = out_dev;
    e = launch_sddmm_csr(L, stream);
  }
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  return SPMM_OK;
}

}  // extern "C"

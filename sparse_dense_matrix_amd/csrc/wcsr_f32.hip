// wcsr_f32.hip -- C = A * B with A in row-window CSR (fp32), B and C dense
// row-major fp32.
//
// Irregular SpMM of the AsyncSparse page (abstract: WCSR kernel; summary:
// long row windows split across thread blocks for load balance).  The pages
// stream the sparse operand with TMA; here one wavefront owns one chunk (at
// most T stored entries of one window) and:
//   - streams the chunk's (column, value) pairs with coalesced 64-wide vector
//     loads, then broadcasts them lane by lane (v_readlane) so each pair's
//     B-row gather is a wave-uniform address plus lane offset;
//   - keeps U B-row gathers in flight before consuming them, independent of
//     row boundaries (the row-boundary test is scalar control flow);
//   - reduces each row in registers in stored order (a segmented reduction
//     over the chunk's entry stream) and writes finished rows straight to C;
//     a row cut by a chunk boundary is written as a partial row, and a second
//     kernel adds the partial rows of each split row in chunk order.
// No floating-point atomics: results are bitwise reproducible.
#include <mutex>
#include <vector>

#include "internal.h"

// Partial rows of split rows for spmm_execute_noalloc, which allocates
// nothing: one fixed array per GPU, held until the process ends.  Host code
// reaches a GPU's copy only through the address hipGetSymbolAddress returns
// with that GPU current (the array's name on the host is not a device
// address).  Every slot is written by wcsr_stream before wcsr_merge reads
// it, so nothing has to be cleared between calls.
static __device__ __align__(256) char scratch[sdm::kNoallocScratchBytes];

namespace sdm {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kUnroll = 16;

template <int V>
struct Vec;
template <>
struct Vec<1> {
  float v[1];
};
template <>
struct Vec<2> {
  float v[2];
};
template <>
struct Vec<4> {
  float v[4];
};

// Lane's V consecutive columns [c, c+V) of a row; `full` means all inside n.
template <int V>
__device__ __forceinline__ Vec<V> load_row(const float *__restrict__ row, int64_t c, int64_t n,
                                           bool full) {
  Vec<V> r;
  if (full) {
    if constexpr (V == 4) {
      const float4 x = *reinterpret_cast<const float4 *>(row + c);
      r.v[0] = x.x; r.v[1] = x.y; r.v[2] = x.z; r.v[3] = x.w;
    } else if constexpr (V == 2) {
      const float2 x = *reinterpret_cast<const float2 *>(row + c);
      r.v[0] = x.x; r.v[1] = x.y;
    } else {
      r.v[0] = row[c];
    }
  } else {
#pragma unroll
    for (int i = 0; i < V; ++i) r.v[i] = (c + i < n) ? row[c + i] : 0.0f;
  }
  return r;
}

template <int V>
__device__ __forceinline__ void store_row(float *__restrict__ row, int64_t c, int64_t n, bool full,
                                          const Vec<V> &x) {
  if (full) {
    if constexpr (V == 4) {
      *reinterpret_cast<float4 *>(row + c) = make_float4(x.v[0], x.v[1], x.v[2], x.v[3]);
    } else if constexpr (V == 2) {
      *reinterpret_cast<float2 *>(row + c) = make_float2(x.v[0], x.v[1]);
    } else {
      row[c] = x.v[0];
    }
  } else {
#pragma unroll
    for (int i = 0; i < V; ++i)
      if (c + i < n) row[c + i] = x.v[i];
  }
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

template <int V>
__global__ __launch_bounds__(64 * kWavesPerBlock) void wcsr_stream(
    const WcsrChunk *__restrict__ chunks, int64_t num_chunks, const int64_t *__restrict__ row_ptr,
    const int32_t *__restrict__ col_idx, const float *__restrict__ vals,
    const float *__restrict__ B, int64_t ldb, float *__restrict__ C, int64_t ldc,
    float *__restrict__ partial, int64_t n, int64_t per_xcd) {
  const int lane = threadIdx.x & 63;
  // workgroup b runs on XCD b % 8: give each XCD a contiguous range of
  // chunks, so the rows in flight on one XCD are neighbours and B rows that
  // nearby rows share can be found in that XCD's L2
  const int64_t lb = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  const int64_t c = lb * kWavesPerBlock + uniform(threadIdx.x >> 6);
  if (c >= num_chunks) return;
  const WcsrChunk d = chunks[c];
  const int64_t col = static_cast<int64_t>(blockIdx.y) * 64 * V + lane * V;
  const bool full = col + V <= n;
  const bool any = col < n;

  const int64_t b = d.nz_begin, e = d.nz_end;
  int row = d.row_begin;
  int64_t rs = row_ptr[row], re = row_ptr[row + 1];
  Vec<V> acc;
#pragma unroll
  for (int i = 0; i < V; ++i) acc.v[i] = 0.0f;

  // write the finished row and move to the next one
  auto flush = [&]() {
    float *dst;
    if (rs >= b && re <= e) {
      dst = C + static_cast<int64_t>(row) * ldc;
    } else {
      const int slot = (row == d.row_begin) ? d.slot_first : d.slot_last;
      dst = partial + static_cast<int64_t>(slot) * n;
    }
    if (any) store_row<V>(dst, col, n, full, acc);
#pragma unroll
    for (int i = 0; i < V; ++i) acc.v[i] = 0.0f;
    ++row;
    rs = re;
    if (row < d.row_end) re = row_ptr[row + 1];
  };

  for (int64_t j0 = b; j0 < e; j0 += 64) {
    const int cnt = static_cast<int>(e - j0 < 64 ? e - j0 : 64);
    const int cv = lane < cnt ? col_idx[j0 + lane] : 0;
    const float vv = lane < cnt ? vals[j0 + lane] : 0.0f;
    for (int u0 = 0; u0 < cnt; u0 += kUnroll) {
      Vec<V> bv[kUnroll];
      float av[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (u0 + u < cnt) {
          const int bc = __builtin_amdgcn_readlane(cv, u0 + u);
          av[u] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, vv), u0 + u));
          if (any) bv[u] = load_row<V>(B + static_cast<int64_t>(bc) * ldb, col, n, full);
        }
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (u0 + u < cnt) {
          const int64_t jj = j0 + u0 + u;
          while (jj >= re && row < d.row_end) flush();
          if (any) {
#pragma unroll
            for (int i = 0; i < V; ++i) acc.v[i] = __builtin_fmaf(av[u], bv[u].v[i], acc.v[i]);
          }
        }
      }
    }
  }
  while (row < d.row_end) flush();
}

// Sum the partial rows of each split row in slot (= chunk) order.
template <int V>
__global__ __launch_bounds__(64 * kWavesPerBlock) void wcsr_merge(
    const int32_t *__restrict__ merge_row, const int32_t *__restrict__ merge_slot,
    int64_t num_split_rows, const float *__restrict__ partial, int64_t n, float *__restrict__ C,
    int64_t ldc) {
  const int lane = threadIdx.x & 63;
  const int64_t q = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + uniform(threadIdx.x >> 6);
  if (q >= num_split_rows) return;
  const int64_t col = static_cast<int64_t>(blockIdx.y) * 64 * V + lane * V;
  if (col >= n) return;
  const bool full = col + V <= n;
  const int s0 = merge_slot[q], s1 = merge_slot[q + 1];
  Vec<V> acc = load_row<V>(partial + static_cast<int64_t>(s0) * n, col, n, full);
  for (int s = s0 + 1; s < s1; ++s) {
    const Vec<V> x = load_row<V>(partial + static_cast<int64_t>(s) * n, col, n, full);
#pragma unroll
    for (int i = 0; i < V; ++i) acc.v[i] += x.v[i];
  }
  store_row<V>(C + static_cast<int64_t>(merge_row[q]) * ldc, col, n, full, acc);
}

int pick_v(int64_t n) { return n <= 64 ? 1 : (n <= 128 ? 2 : 4); }

template <int V>
hipError_t launch_v(const WcsrLaunch &a, hipStream_t s) {
  const int64_t tiles = (a.n + 64 * V - 1) / (64 * V);
  const int64_t blocks = (a.num_chunks + kWavesPerBlock - 1) / kWavesPerBlock;
  const int64_t per_xcd = (blocks + 7) / 8;
  const int64_t grid = 8 * per_xcd;
  if (grid > 0x7fffffff || tiles > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(wcsr_stream<V>, dim3(static_cast<unsigned>(grid), static_cast<unsigned>(tiles)),
                     dim3(64 * kWavesPerBlock), 0, s, a.chunks, a.num_chunks, a.row_ptr, a.col_idx,
                     a.vals, a.B, a.ldb, a.C, a.ldc, a.partial, a.n, per_xcd);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.num_split_rows == 0) return e;
  const int64_t mgrid = (a.num_split_rows + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL(wcsr_merge<V>, dim3(static_cast<unsigned>(mgrid), static_cast<unsigned>(tiles)),
                     dim3(64 * kWavesPerBlock), 0, s, a.merge_row, a.merge_slot, a.num_split_rows,
                     a.partial, a.n, a.C, a.ldc);
  return hipGetLastError();
}

}  // namespace

hipError_t noalloc_scratch(int device, void **ptr) {
  static std::mutex mu;
  static std::vector<void *> addr;  // per device, filled on first use
  *ptr = nullptr;
  if (device < 0) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr.size() <= static_cast<size_t>(device)) addr.resize(static_cast<size_t>(device) + 1, nullptr);
  if (!addr[device]) {
    void *a = nullptr;
    const hipError_t e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[device] = a;
  }
  *ptr = addr[device];
  return hipSuccess;
}

int64_t wcsr_grid(int64_t num_chunks, int64_t n) {
  const int V = pick_v(n);
  return ((num_chunks + kWavesPerBlock - 1) / kWavesPerBlock) * ((n + 64 * V - 1) / (64 * V));
}

hipError_t launch_wcsr_f32(const WcsrLaunch &a, hipStream_t s) {
  if (a.num_chunks == 0 || a.n == 0) return hipSuccess;
  switch (pick_v(a.n)) {
    case 1: return launch_v<1>(a, s);
    case 2: return launch_v<2>(a, s);
    default: return launch_v<4>(a, s);
  }
}

}  // namespace sdm

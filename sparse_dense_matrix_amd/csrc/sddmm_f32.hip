// sddmm_f32.hip -- sampled dense-dense product on a row-window CSR pattern:
// out[p] = sum over t of X[i][t] * Y[j][t] for every stored entry p = (i, j),
// fp32 in and out.
//
// SDDMM is the companion of SpMM named on the Magicube page (abstract); the
// stored pattern is the sample mask.  It is the transpose of the irregular
// SpMM's access pattern: every stored entry gathers one row of Y (the dense
// operand indexed by the sparse column) and reads the row of X of its own
// row, so the work is split exactly like the irregular SpMM -- one wavefront
// per chunk of at most T stored entries of one row window -- and each output
// entry is independent (no split rows, no merge).
//   - a group of G lanes serves one entry: lane q of the group holds V
//     consecutive elements of every G*V-wide step of the inner dimension, so
//     one load instruction fetches a contiguous G*V*4-byte piece of each of
//     the wavefront's 64/G entries' rows (identical X rows of neighbouring
//     entries coalesce inside the instruction);
//   - two rounds of 64/G entries and four steps are loaded before any
//     product is formed: 16 loads of V floats in flight per lane, no branch
//     between them;
//   - each entry's sum is reduced inside its lane group with log2(G)
//     butterfly exchanges (DPP within 16 lanes), in a fixed order, so
//     results are bitwise reproducible;
//   - each entry's row comes from one wave-wide compare against the row end
//     offsets the lanes hold, not from a search through row_ptr.
#include "internal.h"

namespace sdm {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kRounds = 2;  // rounds of 64/G entries per iteration
constexpr int kSteps = 4;   // G*V-wide steps of the inner dimension loaded together

template <int V>
struct Vec {
  float v[V];
};

// V consecutive floats of a row starting at element c, or zeros when c is
// past the row's n elements.  V divides n and c is a multiple of V, so a
// segment is either wholly inside the row or wholly past it; the load is
// unconditional (from element 0 when past), which keeps every gather of an
// iteration free of branches and so in flight together.
template <int V>
__device__ __forceinline__ Vec<V> load_seg(const float *__restrict__ row, int64_t c, int64_t n) {
  const bool in = c < n;
  const float *src = row + (in ? c : 0);
  Vec<V> r;
  if constexpr (V == 4) {
    const float4 x = *reinterpret_cast<const float4 *>(src);
    r.v[0] = x.x; r.v[1] = x.y; r.v[2] = x.z; r.v[3] = x.w;
  } else {
    r.v[0] = *src;
  }
#pragma unroll
  for (int i = 0; i < V; ++i) r.v[i] = in ? r.v[i] : 0.0f;
  return r;
}

// the value lane 63 holds, wave-uniform
__device__ __forceinline__ int64_t lane63(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(v), 63);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(v >> 32), 63);
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// v plus the value of a partner lane; after the exchanges for 1, 2, ..., G/2
// every lane of an aligned group of G lanes holds the group's sum.  Below 16
// the partner is picked by DPP: the other lane of the pair / pair of the quad
// (quad permutations), then the mirror image within 8 and within 16 lanes,
// which pairs each lane with one of the other half (all lanes of a half
// already hold the same value there).
template <int M>
__device__ __forceinline__ float add_partner(float v) {
  int o;
  const int x = __float_as_int(v);
  if constexpr (M == 1) o = __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);        // quad 1,0,3,2
  else if constexpr (M == 2) o = __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);   // quad 2,3,0,1
  else if constexpr (M == 4) o = __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false);  // half-row mirror
  else if constexpr (M == 8) o = __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, false);  // row mirror
  else o = __shfl_xor(x, M);
  return v + __int_as_float(o);
}

template <int G>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (G > 1) v = add_partner<1>(v);
  if constexpr (G > 2) v = add_partner<2>(v);
  if constexpr (G > 4) v = add_partner<4>(v);
  if constexpr (G > 8) v = add_partner<8>(v);
  if constexpr (G > 16) v = add_partner<16>(v);
  if constexpr (G > 32) v = add_partner<32>(v);
  return v;
}

template <int V, int G>
__global__ __launch_bounds__(64 * kWavesPerBlock) void sddmm_f32(
    const WcsrChunk *__restrict__ chunks, int64_t num_chunks, const int64_t *__restrict__ row_ptr,
    const int32_t *__restrict__ col_idx, const float *__restrict__ X, int64_t ldx,
    const float *__restrict__ Y, int64_t ldy, int64_t kd, float *__restrict__ out,
    int64_t per_xcd) {
  constexpr int E = 64 / G;            // entries per round
  constexpr int B = kRounds * E;       // entries per iteration
  const int lane = threadIdx.x & 63;
  const int slot = lane / G, q = lane % G;
  // workgroup b runs on XCD b % 8: contiguous chunk ranges per XCD, so the
  // rows of X in flight on one XCD are neighbours
  const int64_t lb = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  const int64_t c = lb * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (c >= num_chunks) return;
  const WcsrChunk d = chunks[c];

  // Row lookup without dependent loads: the lanes hold the end offsets of a
  // group of 64 consecutive rows of the chunk (lane j: row_ptr[g0 + j + 1],
  // past the chunk's last row a value no entry reaches).  The row of entry
  // p is g0 plus the number of those ends at or before p; entries are
  // visited in increasing order, so the group only moves forward.
  int g0 = d.row_begin;
  int64_t end_l = (g0 + lane < d.row_end) ? row_ptr[g0 + lane + 1] : INT64_MAX;
  int64_t g_last = lane63(end_l);
  const int64_t step = static_cast<int64_t>(G) * V;

  for (int64_t p0 = d.nz_begin; p0 < d.nz_end; p0 += B) {
    // places past the chunk's last entry repeat it, so every lane loads
    // valid rows; their sums are never stored
    const int64_t last = d.nz_end - 1;
    int my_row[kRounds], my_col[kRounds];
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      const int64_t pe = p0 + r * E + slot;
      my_col[r] = col_idx[pe < last ? pe : last];
      my_row[r] = 0;
    }
#pragma unroll
    for (int o = 0; o < B; ++o) {
      const int64_t p = (p0 + o < last) ? p0 + o : last;
      while (p >= g_last) {  // entry lies past this group of rows
        g0 += 64;
        end_l = (g0 + lane < d.row_end) ? row_ptr[g0 + lane + 1] : INT64_MAX;
        g_last = lane63(end_l);
      }
      const int row = g0 + __builtin_popcountll(__ballot(end_l <= p));
      if (slot == o % E) my_row[o / E] = row;
    }
    const float *xr[kRounds], *yr[kRounds];
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      xr[r] = X + static_cast<int64_t>(my_row[r]) * ldx;
      yr[r] = Y + static_cast<int64_t>(my_col[r]) * ldy;
    }

    float acc[kRounds];
#pragma unroll
    for (int r = 0; r < kRounds; ++r) acc[r] = 0.0f;
    for (int64_t k0 = static_cast<int64_t>(q) * V; k0 < kd; k0 += kSteps * step) {
      Vec<V> xs[kRounds][kSteps], ys[kRounds][kSteps];
#pragma unroll
      for (int u = 0; u < kSteps; ++u) {
#pragma unroll
        for (int r = 0; r < kRounds; ++r) {
          xs[r][u] = load_seg<V>(xr[r], k0 + u * step, kd);
          ys[r][u] = load_seg<V>(yr[r], k0 + u * step, kd);
        }
      }
#pragma unroll
      for (int u = 0; u < kSteps; ++u) {
#pragma unroll
        for (int r = 0; r < kRounds; ++r) {
#pragma unroll
          for (int i = 0; i < V; ++i) acc[r] = __builtin_fmaf(xs[r][u].v[i], ys[r][u].v[i], acc[r]);
        }
      }
    }

#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      const float tot = group_sum<G>(acc[r]);
      const int64_t pe = p0 + r * E + slot;
      if (q == 0 && pe < d.nz_end) out[pe] = tot;
    }
  }
}

// floats per lane per load: 4 when they divide the inner dimension (so a
// segment never straddles the end of a row), else 1
int pick_v(int64_t kd) { return kd % 4 == 0 ? 4 : 1; }

// lanes per entry: enough that four steps cover the inner dimension, at
// least 4 and at most the wavefront
int pick_g(int64_t kd, int v) {
  const int64_t need = (kd + 4 * v - 1) / (4 * v);
  int g = 4;
  while (g < 64 && g < need) g *= 2;
  return g;
}

template <int V, int G>
hipError_t launch_vg(const SddmmLaunch &a, hipStream_t s) {
  const int64_t blocks = (a.num_chunks + kWavesPerBlock - 1) / kWavesPerBlock;
  const int64_t per_xcd = (blocks + 7) / 8;
  if (8 * per_xcd > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((sddmm_f32<V, G>), dim3(static_cast<unsigned>(8 * per_xcd)),
                     dim3(64 * kWavesPerBlock), 0, s, a.chunks, a.num_chunks, a.row_ptr, a.col_idx,
                     a.X, a.ldx, a.Y, a.ldy, a.kd, a.out, per_xcd);
  return hipGetLastError();
}

template <int V>
hipError_t launch_v(const SddmmLaunch &a, hipStream_t s) {
  switch (pick_g(a.kd, V)) {
    case 4: return launch_vg<V, 4>(a, s);
    case 8: return launch_vg<V, 8>(a, s);
    case 16: return launch_vg<V, 16>(a, s);
    case 32: return launch_vg<V, 32>(a, s);
    default: return launch_vg<V, 64>(a, s);
  }
}

}  // namespace

int64_t sddmm_grid(int64_t num_chunks) {
  const int64_t blocks = (num_chunks + kWavesPerBlock - 1) / kWavesPerBlock;
  return 8 * ((blocks + 7) / 8);
}

hipError_t launch_sddmm_f32(const SddmmLaunch &a, hipStream_t s) {
  if (a.num_chunks == 0) return hipSuccess;
  return pick_v(a.kd) == 4 ? launch_v<4>(a, s) : launch_v<1>(a, s);
}

}  // namespace sdm

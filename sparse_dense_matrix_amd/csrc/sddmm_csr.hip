// sddmm_csr.hip -- sampled dense-dense product on a row-window CSR pattern:
// out[p] = sum over t of X[i][t] * Y[j][t] for every stored entry p = (i, j).
// X and Y are fp32 (fp32 out), bf16 (fp32 sums, bf16 out rounded to nearest
// even) or int8 (exact int32 out).
//
// SDDMM is the companion of SpMM named on the Magicube page (abstract), which
// runs both on low-precision integers; the stored pattern is the sample mask.
// It is the transpose of the irregular SpMM's access pattern: every stored
// entry gathers one row of Y (the dense operand indexed by the sparse column)
// and reads the row of X of its own row, so the work is split exactly like
// the irregular SpMM -- one wavefront per chunk of at most T stored entries
// of one row window -- and each output entry is independent (no split rows,
// no merge).
//   - a group of G lanes serves one entry: lane q of the group holds V
//     consecutive elements of every G*V-wide step of the inner dimension, so
//     one load instruction fetches a contiguous piece of each of the
//     wavefront's 64/G entries' rows (identical X rows of neighbouring
//     entries coalesce inside the instruction); a piece is 16 bytes when V
//     elements of 16 bytes divide the inner dimension;
//   - two rounds of 64/G entries and four steps are loaded before any
//     product is formed: 16 loads per lane in flight, no branch between them;
//   - each entry's sum is reduced inside its lane group with log2(G)
//     butterfly exchanges (DPP within 16 lanes), in a fixed order, so
//     results are bitwise reproducible;
//   - each entry's row comes from one wave-wide compare against the row end
//     offsets the lanes hold, not from a search through row_ptr.
#include "internal.h"

#include <type_traits>

namespace sdm {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kRounds = 2;  // rounds of 64/G entries per iteration
constexpr int kSteps = 4;   // G*V-wide steps of the inner dimension loaded together

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Element types: storage T, accumulator Acc.  fma takes one element of X
// and Y; dot takes one 32-bit word of each (1 fp32, 2 bf16 or 4 int8
// elements) and adds their products with one instruction (v_dot2c_f32_bf16,
// v_dot4c_i32_i8), so 16-byte pieces are used packed, as loaded.
struct F32 {
  using T = float;
  using Acc = float;
  static constexpr int kWide = 4;  // elements per 16-byte piece
  __device__ static Acc fma(T a, T b, Acc c) { return __builtin_fmaf(a, b, c); }
  __device__ static Acc dot(uint32_t a, uint32_t b, Acc c) {
    return __builtin_fmaf(__uint_as_float(a), __uint_as_float(b), c);
  }
  __device__ static void store(void *out, int64_t p, Acc v) { static_cast<float *>(out)[p] = v; }
};
struct Bf16 {
  using T = uint16_t;
  using Acc = float;
  static constexpr int kWide = 8;
  // bf16 -> fp32 is exact: the bits are the top half of the float
  __device__ static float widen(T x) { return __uint_as_float(static_cast<uint32_t>(x) << 16); }
  __device__ static Acc fma(T a, T b, Acc c) { return __builtin_fmaf(widen(a), widen(b), c); }
  __device__ static Acc dot(uint32_t a, uint32_t b, Acc c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
  }
  __device__ static void store(void *out, int64_t p, Acc v) {
    // float -> bf16 rounds to nearest even
    static_cast<uint16_t *>(out)[p] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
  }
};
struct I8 {
  using T = int8_t;
  using Acc = int32_t;
  static constexpr int kWide = 16;
  __device__ static Acc fma(T a, T b, Acc c) {
    return c + static_cast<int32_t>(a) * static_cast<int32_t>(b);
  }
  __device__ static Acc dot(uint32_t a, uint32_t b, Acc c) {
    return __builtin_amdgcn_sdot4(static_cast<int>(a), static_cast<int>(b), c, false);
  }
  __device__ static void store(void *out, int64_t p, Acc v) { static_cast<int32_t *>(out)[p] = v; }
};

// one element, or one 16-byte piece kept as four 32-bit words
template <class E>
struct One {
  typename E::T v[1];
};
struct Piece {
  uint32_t w[4];
};
template <class E, int V>
using Vec = std::conditional_t<V == E::kWide, Piece, One<E>>;

// V consecutive elements of a row starting at element c, or zeros when c is
// past the row's n elements.  V divides n and c is a multiple of V, so a
// segment is either wholly inside the row or wholly past it; the load is
// unconditional (from element 0 when past), which keeps every gather of an
// iteration free of branches and so in flight together.
template <class E, int V>
__device__ __forceinline__ Vec<E, V> load_seg(const typename E::T *__restrict__ row, int64_t c,
                                              int64_t n) {
  using T = typename E::T;
  const bool in = c < n;
  const T *src = row + (in ? c : 0);
  Vec<E, V> r;
  if constexpr (V == E::kWide) {
    r = *reinterpret_cast<const Vec<E, V> *>(src);
#pragma unroll
    for (int i = 0; i < 4; ++i) r.w[i] = in ? r.w[i] : 0u;
  } else {
    static_assert(V == 1, "one element or one 16-byte piece");
    r.v[0] = in ? *src : T(0);
  }
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
template <int M, class A>
__device__ __forceinline__ A add_partner(A v) {
  int o;
  const int x = __builtin_bit_cast(int, v);
  if constexpr (M == 1) o = __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);        // quad 1,0,3,2
  else if constexpr (M == 2) o = __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);   // quad 2,3,0,1
  else if constexpr (M == 4) o = __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false);  // half-row mirror
  else if constexpr (M == 8) o = __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, false);  // row mirror
  else o = __shfl_xor(x, M);
  return v + __builtin_bit_cast(A, o);
}

template <int G, class A>
__device__ __forceinline__ A group_sum(A v) {
  if constexpr (G > 1) v = add_partner<1>(v);
  if constexpr (G > 2) v = add_partner<2>(v);
  if constexpr (G > 4) v = add_partner<4>(v);
  if constexpr (G > 8) v = add_partner<8>(v);
  if constexpr (G > 16) v = add_partner<16>(v);
  if constexpr (G > 32) v = add_partner<32>(v);
  return v;
}

template <class Ty, int V, int G>
__global__ __launch_bounds__(64 * kWavesPerBlock) void sddmm_csr(
    const WcsrChunk *__restrict__ chunks, int64_t num_chunks, const int64_t *__restrict__ row_ptr,
    const int32_t *__restrict__ col_idx, const typename Ty::T *__restrict__ X, int64_t ldx,
    const typename Ty::T *__restrict__ Y, int64_t ldy, int64_t kd, void *__restrict__ out,
    int64_t per_xcd) {
  using T = typename Ty::T;
  using Acc = typename Ty::Acc;
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
    const T *xr[kRounds], *yr[kRounds];
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      xr[r] = X + static_cast<int64_t>(my_row[r]) * ldx;
      yr[r] = Y + static_cast<int64_t>(my_col[r]) * ldy;
    }

    Acc acc[kRounds];
#pragma unroll
    for (int r = 0; r < kRounds; ++r) acc[r] = Acc(0);
    for (int64_t k0 = static_cast<int64_t>(q) * V; k0 < kd; k0 += kSteps * step) {
      Vec<Ty, V> xs[kRounds][kSteps], ys[kRounds][kSteps];
#pragma unroll
      for (int u = 0; u < kSteps; ++u) {
#pragma unroll
        for (int r = 0; r < kRounds; ++r) {
          xs[r][u] = load_seg<Ty, V>(xr[r], k0 + u * step, kd);
          ys[r][u] = load_seg<Ty, V>(yr[r], k0 + u * step, kd);
        }
      }
#pragma unroll
      for (int u = 0; u < kSteps; ++u) {
#pragma unroll
        for (int r = 0; r < kRounds; ++r) {
          if constexpr (V == Ty::kWide) {
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[r] = Ty::dot(xs[r][u].w[i], ys[r][u].w[i], acc[r]);
          } else {
            acc[r] = Ty::fma(xs[r][u].v[0], ys[r][u].v[0], acc[r]);
          }
        }
      }
    }

#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      const Acc tot = group_sum<G>(acc[r]);
      const int64_t pe = p0 + r * E + slot;
      if (q == 0 && pe < d.nz_end) Ty::store(out, pe, tot);
    }
  }
}

// elements per lane per load: one 16-byte piece when those divide the inner
// dimension (so a piece never straddles the end of a row), else one element
template <class Ty>
bool wide_loads(int64_t kd) { return kd % Ty::kWide == 0; }

// lanes per entry: enough that four steps cover the inner dimension, at
// least 2 and at most the wavefront
int pick_g(int64_t kd, int v) {
  const int64_t need = (kd + 4 * v - 1) / (4 * v);
  int g = 2;
  while (g < 64 && g < need) g *= 2;
  return g;
}

template <class Ty, int V, int G>
hipError_t launch_vg(const SddmmLaunch &a, hipStream_t s) {
  const int64_t blocks = (a.num_chunks + kWavesPerBlock - 1) / kWavesPerBlock;
  const int64_t per_xcd = (blocks + 7) / 8;
  if (8 * per_xcd > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((sddmm_csr<Ty, V, G>), dim3(static_cast<unsigned>(8 * per_xcd)),
                     dim3(64 * kWavesPerBlock), 0, s, a.chunks, a.num_chunks, a.row_ptr, a.col_idx,
                     static_cast<const typename Ty::T *>(a.X), a.ldx,
                     static_cast<const typename Ty::T *>(a.Y), a.ldy, a.kd, a.out, per_xcd);
  return hipGetLastError();
}

template <class Ty, int V>
hipError_t launch_v(const SddmmLaunch &a, hipStream_t s) {
  switch (pick_g(a.kd, V)) {
    case 2: return launch_vg<Ty, V, 2>(a, s);
    case 4: return launch_vg<Ty, V, 4>(a, s);
    case 8: return launch_vg<Ty, V, 8>(a, s);
    case 16: return launch_vg<Ty, V, 16>(a, s);
    case 32: return launch_vg<Ty, V, 32>(a, s);
    default: return launch_vg<Ty, V, 64>(a, s);
  }
}

template <class Ty>
hipError_t launch_t(const SddmmLaunch &a, hipStream_t s) {
  return wide_loads<Ty>(a.kd) ? launch_v<Ty, Ty::kWide>(a, s) : launch_v<Ty, 1>(a, s);
}

}  // namespace

int64_t sddmm_grid(int64_t num_chunks) {
  const int64_t blocks = (num_chunks + kWavesPerBlock - 1) / kWavesPerBlock;
  return 8 * ((blocks + 7) / 8);
}

hipError_t launch_sddmm_csr(const SddmmLaunch &a, hipStream_t s) {
  if (a.num_chunks == 0) return hipSuccess;
  switch (a.dtype) {
    case SPMM_F32: return launch_t<F32>(a, s);
    case SPMM_BF16: return launch_t<Bf16>(a, s);
    case SPMM_I8: return launch_t<I8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sdm

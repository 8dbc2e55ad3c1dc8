// sddmm_bcsr.hip -- sampled dense-dense product with a BCSR block pattern as
// the mask: for every stored 64 x 64 block b = (I, J),
//   out[b][i][j] = sum over t of X[64 I + i][t] * Y[64 J + j][t],
// with bf16 operands, fp32 accumulation and bf16 round-to-nearest-even
// output, or int8 operands and exact int32 output.
//
// SDDMM is the companion of SpMM on the Magicube page (abstract), which
// runs both on low-precision integers.  Each stored block is a small dense
// product X_I . Y_J^T contracted over the whole inner dimension, so it goes
// on the MFMA units:
//   - both operands are contiguous along the inner dimension, which is what
//     the MFMA operand registers want: a lane's 16 bytes of a row are one
//     operand fragment, with no transpose.  The contraction order is free,
//     so a lane takes a contiguous 64-byte half of each 128-byte row chunk
//     and the same byte positions of X and Y meet in one MFMA;
//   - a workgroup of four waves serves up to four stored blocks of one
//     block row.  Per 128-byte chunk of the inner dimension the X_I rows they
//     share and each block's Y_J rows are copied into LDS by direct
//     global->LDS loads, whole 128-byte lines at a time (fragment-shaped
//     loads straight into registers would touch 32 lines per instruction and
//     stall the address unit); the copies are XOR-swizzled so the fragment
//     reads are free of bank conflicts;
//   - two LDS stages: the next chunk loads while this one is multiplied,
//     and the two workgroups sharing a CU cover each other's waits;
//   - the inner dimension is split into ranges when the blocks alone would
//     not fill the chip; each range writes fp32 / int32 partial blocks and a
//     second kernel adds them in range order, so results are reproducible;
//   - workgroups are dealt range-major, so the workgroups resident together
//     stream the same range of Y and share it in cache.
// With a random block pattern a block row holds few blocks, so the bound is
// the rate at which the L2 feeds operand chunks: about 52 flop per byte for
// four blocks per X_I chunk (bf16), twice that for int8.
#include <type_traits>

#include "internal.h"

// load_lds16 below names m0 as clobbered on purpose (it sets m0 for the
// LDS-DMA instruction); clang warns about clobbering a reserved register.
#pragma clang diagnostic ignored "-Winline-asm"

namespace sdm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlk = 64;                        // block edge
constexpr int kWaves = 4;                       // one stored block per wave
constexpr int kChunkBytes = 128;               // bytes of a row per pipeline step
constexpr int kPieces = kChunkBytes / 16;       // 16-byte pieces per chunk row
constexpr int kSteps = kPieces / 2;             // MFMA k-steps per chunk (a lane takes half a row)
constexpr int kTileBytes = kBlk * kChunkBytes;  // one 64-row chunk
constexpr int kStages = 2;                     // LDS ring: kStages - 1 chunks load ahead
constexpr int kAhead = kStages - 1;
constexpr int kStageBytes = (1 + kWaves) * kTileBytes;  // X_I, then Y_J of each wave
constexpr int kLdsBytes = kStages * kStageBytes;
constexpr int kXLoads = kTileBytes / 1024 / kWaves;     // 1 KB direct loads of X_I per wave
constexpr int kYLoads = kTileBytes / 1024;              // ... of its own Y_J
static_assert(kXLoads >= 1 && kXLoads * kWaves * 1024 == kTileBytes, "X_I split");
static_assert(kLdsBytes <= 80 * 1024, "two workgroups per CU");
static_assert(kAhead >= 1 && kAhead <= 3, "wait counts below cover up to three chunks ahead");

// bf16: MFMA 32x32x16, 8 elements per lane and step
struct Bf16Op {
  using Acc = f32x16;
  static constexpr int kElem = 2;
  __device__ static Acc mma(u32x4 a, u32x4 b, Acc c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};
// int8: MFMA 32x32x32, 16 elements per lane and step, exact int32 sums
struct I8Op {
  using Acc = i32x16;
  static constexpr int kElem = 1;
  __device__ static Acc mma(u32x4 a, u32x4 b, Acc c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a),
                                                 __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
  }
};

// physical 16-byte piece of logical piece c in row r of a staged chunk:
// sixteen consecutive rows at one logical piece land on sixteen distinct
// 16-byte bank groups (256 / kChunkBytes rows share a 256-byte bank row)
__device__ __forceinline__ int swz(int r, int c) {
  constexpr int kShift = kChunkBytes == 128 ? 1 : 2;
  return c ^ ((r >> kShift) & (kPieces - 1));
}

// s_waitcnt vmcnt(n), leaving the other counters alone
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Direct global->LDS load of 16 bytes per lane: LDS[lds + 16 * lane] =
// global[base + voff].  Inline asm, so the compiler neither waits on it (the
// kernel counts vmcnt itself) nor assumes later LDS reads depend on it.
__device__ __forceinline__ void load_lds16(uint32_t lds, const void *base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds), "v"(voff), "s"(base)
               : "memory", "m0");
}

// Workgroup barrier after this wave's LDS reads have completed (so no read
// of a stage can still be in flight when another wave refills it), without
// waiting for the global loads in flight (their vmcnt waits are explicit).
__device__ __forceinline__ void barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char *)(p)));
}

__device__ __forceinline__ unsigned short to_bf16_rne(float f) {
  return __builtin_bit_cast(unsigned short, static_cast<__bf16>(f));
}

// 16 bytes of a row starting at element e, zero past element `end` (the
// slow path of the last, partial chunk)
template <int kElem>
__device__ __forceinline__ u32x4 load_masked(const char *row, int64_t e, int64_t end) {
  constexpr int kPer = 16 / kElem;
  if (e + kPer <= end) return *reinterpret_cast<const u32x4 *>(row + e * kElem);
  u32x4 v = {0u, 0u, 0u, 0u};
  if (e >= end) return v;
  unsigned char bytes[16] = {};
  for (int i = 0; i < kPer; ++i)
    if (e + i < end)
      for (int b = 0; b < kElem; ++b) bytes[i * kElem + b] = row[(e + i) * kElem + b];
  return __builtin_bit_cast(u32x4, bytes);
}


template <typename Op>
__global__ __launch_bounds__(64 * kWaves) void sddmm_bcsr_mfma(
    const int4 *__restrict__ groups, int32_t ngroups, int32_t per_xcd,
    const int32_t *__restrict__ col_idx, int64_t nnzb, int64_t kd, int64_t ksplit,
    int32_t nsplit, const char *__restrict__ X, int64_t ldxb, const char *__restrict__ Y,
    int64_t ldyb, void *__restrict__ out, void *__restrict__ partial) {
  constexpr int E = Op::kElem;
  constexpr int kChunk = kChunkBytes / E;  // elements per chunk
  extern __shared__ __attribute__((aligned(1024))) char lds[];

  // range-major, XCD-contiguous: workgroup b runs on XCD b % 8
  const int32_t gp = 8 * per_xcd;
  const int32_t s = blockIdx.x / gp;
  const int32_t r = blockIdx.x % gp;
  const int32_t g = (r & 7) * per_xcd + (r >> 3);
  if (g >= ngroups) return;
  const int4 grp = groups[g];  // block row, first block, block count
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool active = wave < grp.z;
  const int64_t blk = grp.y + (active ? wave : 0);
  const int64_t J = col_idx[blk];
  const int64_t kbeg = static_cast<int64_t>(s) * ksplit;
  const int64_t kend = kbeg + ksplit < kd ? kbeg + ksplit : kd;
  const int64_t nfull = (kend - kbeg) / kChunk;
  const int64_t tail = (kend - kbeg) % kChunk;
  const int h = lane >> 5;  // which half of a chunk row the lane's fragments take

  const char *xb = X + static_cast<int64_t>(grp.x) * kBlk * ldxb;
  const char *yb = Y + J * kBlk * ldyb;
  // this lane's 16-byte piece of a 1 KB direct load (1024 / kChunkBytes
  // rows): physical piece pp of row prow holds logical piece swz(prow, pp)
  auto piece = [&](int i, int64_t ld) {
    const int o = i * 1024 + lane * 16;
    const int prow = o / kChunkBytes, pp = (o % kChunkBytes) / 16;
    return static_cast<uint32_t>(prow * ld + swz(prow, pp) * 16);
  };
  uint32_t xoff[kXLoads], yoff[kYLoads];
#pragma unroll
  for (int i = 0; i < kXLoads; ++i) xoff[i] = piece(wave * kXLoads + i, ldxb);
#pragma unroll
  for (int i = 0; i < kYLoads; ++i) yoff[i] = piece(i, ldyb);
  const uint32_t lds0 = lds_addr(lds);

  typename Op::Acc acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0;

  // MFMAs of one chunk from an LDS stage: X_I tile, then this wave's Y_J tile
  auto compute = [&](const char *stage) {
    const char *yt = stage + (1 + wave) * kTileBytes;
#pragma unroll
    for (int u = 0; u < kSteps; ++u) {
      u32x4 xf[2], yf[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int row = t * 32 + (lane & 31);
        const int off = row * kChunkBytes + swz(row, h * kSteps + u) * 16;
        xf[t] = *reinterpret_cast<const u32x4 *>(stage + off);
        yf[t] = *reinterpret_cast<const u32x4 *>(yt + off);
      }
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) acc[rt][ct] = Op::mma(xf[rt], yf[ct], acc[rt][ct]);
    }
  };

  // The pipeline, written once for a wave that owns a block (kActive: it
  // loads a share of X_I and its Y_J) and once for a wave that only helps
  // with X_I (a group of fewer than four blocks), so every wait count is a
  // constant.
  auto run = [&](auto act) {
    constexpr bool kActive = decltype(act)::value;
    // issue chunk c into LDS stage c % kStages
    auto issue = [&](int64_t c) {
      const int64_t kb = (kbeg + c * kChunk) * E;  // byte offset along the rows
      const uint32_t st = lds0 + static_cast<uint32_t>(c % kStages) * kStageBytes;
#pragma unroll
      for (int i = 0; i < kXLoads; ++i)
        load_lds16(__builtin_amdgcn_readfirstlane(st + (wave * kXLoads + i) * 1024), xb + kb,
                   xoff[i]);
      if constexpr (kActive) {
        const uint32_t yt = st + (1 + wave) * kTileBytes;
#pragma unroll
        for (int i = 0; i < kYLoads; ++i)
          load_lds16(__builtin_amdgcn_readfirstlane(yt + i * 1024), yb + kb, yoff[i]);
      }
    };
    constexpr int kPerChunk = kXLoads + (kActive ? kYLoads : 0);
#pragma unroll
    for (int c = 0; c < kAhead; ++c)
      if (c < nfull) issue(c);
    for (int64_t c = 0; c < nfull; ++c) {
      // this wave's part of chunk c has landed: the loads still allowed in
      // flight are those of the chunks issued after it (up to kAhead - 1)
      const int64_t later = nfull - 1 - c;
      if (later >= 2 && kAhead >= 3) wait_vm<2 * kPerChunk>();
      else if (later >= 1 && kAhead >= 2) wait_vm<kPerChunk>();
      else wait_vm<0>();
      barrier();  // ... every wave's; and the stage of chunk c - 1 is no longer read
      if (c + kAhead < nfull) issue(c + kAhead);
      if constexpr (kActive) compute(lds + (c % kStages) * kStageBytes);
    }
    if (tail > 0) {
      // last, partial chunk: masked loads through registers into stage 0
      wait_vm<0>();
      barrier();
      const int64_t kc = kbeg + nfull * kChunk;
#pragma unroll
      for (int i = 0; i < kXLoads; ++i) {
        const int o = (wave * kXLoads + i) * 1024 + lane * 16;
        const int prow = o / kChunkBytes, pp = (o % kChunkBytes) / 16;
        const int lp = swz(prow, pp);  // swz is its own inverse
        *reinterpret_cast<u32x4 *>(lds + o) =
            load_masked<E>(xb + prow * ldxb, kc + lp * (16 / E), kend);
      }
      if constexpr (kActive) {
#pragma unroll
        for (int i = 0; i < kYLoads; ++i) {
          const int o = i * 1024 + lane * 16;
          const int prow = o / kChunkBytes, pp = (o % kChunkBytes) / 16;
          const int lp = swz(prow, pp);
          *reinterpret_cast<u32x4 *>(lds + (1 + wave) * kTileBytes + o) =
              load_masked<E>(yb + prow * ldyb, kc + lp * (16 / E), kend);
        }
      }
      __syncthreads();
      if constexpr (kActive) compute(lds);
    }
  };
  if (active)
    run(std::true_type{});
  else
    run(std::false_type{});

  if (!active) return;
  // acc element e of tile (rt, ct): row 32 rt + 8 (e / 4) + 4 h + e % 4,
  // column 32 ct + lane % 32
  if (nsplit == 1) {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = rt * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
          const int col = ct * 32 + (lane & 31);
          const int64_t idx = blk * (kBlk * kBlk) + row * kBlk + col;
          if constexpr (E == 2)
            static_cast<unsigned short *>(out)[idx] = to_bf16_rne(acc[rt][ct][e]);
          else
            static_cast<int32_t *>(out)[idx] = acc[rt][ct][e];
        }
  } else {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = rt * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
          const int col = ct * 32 + (lane & 31);
          const int64_t idx = (s * nnzb + blk) * (kBlk * kBlk) + row * kBlk + col;
          if constexpr (E == 2)
            static_cast<float *>(partial)[idx] = acc[rt][ct][e];
          else
            static_cast<int32_t *>(partial)[idx] = acc[rt][ct][e];
        }
  }
}

// out[i] = sum over ranges s ascending of partial[s][i]; four elements per
// thread
template <typename Op>
__global__ __launch_bounds__(256) void sddmm_bcsr_merge(const void *__restrict__ partial,
                                                        int64_t count, int32_t nsplit,
                                                        void *__restrict__ out) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i >= count) return;
  if constexpr (Op::kElem == 2) {
    const float4 *p = static_cast<const float4 *>(partial);
    float4 t = p[i / 4];
    for (int s = 1; s < nsplit; ++s) {
      const float4 v = p[(s * count + i) / 4];
      t.x += v.x; t.y += v.y; t.z += v.z; t.w += v.w;
    }
    ushort4 o;
    o.x = to_bf16_rne(t.x); o.y = to_bf16_rne(t.y); o.z = to_bf16_rne(t.z); o.w = to_bf16_rne(t.w);
    static_cast<ushort4 *>(out)[i / 4] = o;
  } else {
    const int4 *p = static_cast<const int4 *>(partial);
    int4 t = p[i / 4];
    for (int s = 1; s < nsplit; ++s) {
      const int4 v = p[(s * count + i) / 4];
      t.x += v.x; t.y += v.y; t.z += v.z; t.w += v.w;
    }
    static_cast<int4 *>(out)[i / 4] = t;
  }
}

template <typename Op>
hipError_t launch(const SddmmBcsrLaunch &a, hipStream_t st) {
  const int32_t per_xcd = (a.ngroups + 7) / 8;
  const int64_t grid = static_cast<int64_t>(8) * per_xcd * a.nsplit;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipError_t e = allow_dynamic_lds(reinterpret_cast<const void *>(&sddmm_bcsr_mfma<Op>), kLdsBytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sddmm_bcsr_mfma<Op>, dim3(static_cast<unsigned>(grid)), dim3(64 * kWaves),
                     kLdsBytes, st, a.groups, a.ngroups, per_xcd, a.col_idx, a.nnzb, a.kd, a.ksplit, a.nsplit,
                     static_cast<const char *>(a.X), a.ldx * Op::kElem,
                     static_cast<const char *>(a.Y), a.ldy * Op::kElem, a.out, a.partial);
  e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;
  const int64_t count = a.nnzb * kBlk * kBlk;
  const int64_t blocks = (count / 4 + 255) / 256;
  hipLaunchKernelGGL(sddmm_bcsr_merge<Op>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st,
                     a.partial, count, a.nsplit, a.out);
  return hipGetLastError();
}

}  // namespace

int sddmm_bcsr_chunk(bool int8) { return kChunkBytes / (int8 ? 1 : 2); }
int sddmm_bcsr_group() { return kWaves; }

hipError_t launch_sddmm_bcsr(const SddmmBcsrLaunch &a, hipStream_t s) {
  if (a.ngroups == 0) return hipSuccess;
  return a.int8 ? launch<I8Op>(a, s) : launch<Bf16Op>(a, s);
}

}  // namespace sdm

// sp24_i8.hip -- C = A * B with A int8 in 2:4 compressed form (two kept
// values and their 2-bit positions per group of four along k), B int8 dense
// row-major, C int32 exact.
//
// The 2:4 pattern is the one the tiled-GEMM page (abstract) describes for the
// sparse tensor core; the Magicube page (abstract) motivates SpMM on
// low-precision integers.  On gfx950 the sparse MFMA
// v_smfmac_i32_16x16x128_i8 consumes the compressed operand directly:
//   - A operand, lane l: row l%16 of the 16-row tile, the 16 kept bytes of
//     dense k in [32*(l/16), 32*(l/16) + 32) of the 128-wide step, and one
//     32-bit index word whose bits [2j, 2j+2) give kept byte j's position in
//     its group of four -- bit for bit the canonical metadata nibbles, so the
//     plan uploads the canonical arrays unchanged (only zero-padded);
//   - B operand, lane l: column l%16, 32 bytes = dense k rows 16*(l/16)+0..15
//     and 64+16*(l/16)+0..15, read out of the row-major LDS slab with the
//     gfx950 transpose read ds_read_b64_tr_b8 (8 k-values per read);
//   - D: 4 int32 per lane, rows 4*(l/16)+0..3, column l%16.
// A workgroup of 8 waves computes a 256 x 256 tile of C (each wave 128 x 64,
// 8 x 4 sparse MFMA tiles).  Operands go global -> LDS with direct loads
// into a three-stage ring (two k-steps in flight).  The plan stores the
// compressed values and the index words tiled: for each 256-row tile and
// 128-deep k-step, one contiguous 16 KB piece of values already in MFMA
// fragment order and one contiguous 4 KB piece of index words, so every
// direct load reads 1 KB of consecutive bytes.  The B slab's 16-byte pieces
// are XOR-swizzled by k-row so the transpose reads are bank-conflict free.
// The tile order groups 4 row tiles with every column tile on one XCD, so A
// panels are shared 8-fold and B panels 4-fold in that XCD's L2.
//
// The same kernel runs the tile-vector-wise pattern of the tiled-GEMM page
// (abstract: tile-wise sparsity at the global-memory level combined with 2:4
// at the register level): A is cut into tiles of one row tile (256 rows) by
// one k-step (128), only the tiles holding a nonzero are stored (2:4 inside),
// and a per-row-tile table lists their k-steps; the kernel walks that list
// instead of every k-step, so a zero tile is never loaded.
#include "internal.h"

// load_lds below names m0 as clobbered on purpose (it sets m0 for the
// LDS-DMA instruction); clang warns about clobbering a reserved register.
#pragma clang diagnostic ignored "-Winline-asm"

namespace sdm {
namespace {

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr int kTM = 256, kTN = 256, kTK = 128;  // dense k per step
constexpr int kWaves = 8;                       // 2 (rows) x 4 (columns)
constexpr int kThreads = 64 * kWaves;
constexpr int kMG = 4;                          // row tiles grouped on one XCD
constexpr int kAVBytes = kTM * kTK / 2;         // 16 KB compressed values
constexpr int kAMBytes = kTM * kTK / 8;         // 4 KB metadata
constexpr int kBBytes = kTK * kTN;              // 32 KB
constexpr int kStageBytes = kAVBytes + kAMBytes + kBBytes;
constexpr int kStages = 3;                      // two k-steps in flight
constexpr int kLdsBytes = kStages * kStageBytes;  // 156 KB
constexpr int kLoads = 7;                       // direct loads per wave per k-step
constexpr int kMLanes = kAMBytes / kWaves / 16;  // lanes of a wave that load index words
static_assert(kLdsBytes <= 160 * 1024, "LDS");

// physical 16-byte piece of logical piece c in k-row r of the B slab: the 16
// rows one transpose read touches land in 16 distinct bank groups
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r & 7) | (((r >> 4) & 1) << 3)); }

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Direct global->LDS load of 16 bytes per lane: LDS[lds + 16 * lane] =
// global[base + voff].  Inline asm so the compiler neither drains it at
// barriers nor makes later LDS reads wait on it; the kernel counts vmcnt.
__device__ __forceinline__ void load_lds16(uint32_t lds, const void *base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds), "v"(voff), "s"(base)
               : "memory", "m0");
}

// Workgroup barrier without a memory fence.  Every LDS read of a k-step
// feeds that step's MFMAs, so its wait comes before the loop's back edge
// and no read of a stage is in flight when the next step refills it.
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char *)(p)));
}

// exchange with the lane `xor` away inside a quad (DPP quad permutation)
template <int kXor>
__device__ __forceinline__ int quad_swap(int v) {
  constexpr int perm = kXor == 1 ? 0xB1 : 0x4E;  // [1,0,3,2] or [2,3,0,1]
  return __builtin_amdgcn_mov_dpp(v, perm, 0xF, 0xF, false);
}

// kTiles: A is tile-vector-wise; row tile T holds the stored k-steps
// tile_step[tile_ptr[T] .. tile_ptr[T+1]), their values and index words in
// that order.  Otherwise every k-step of every row tile is stored.
template <bool kTiles>
__global__ __launch_bounds__(kThreads) void sp24_i8_smfmac(
    const int8_t *__restrict__ vals, const uint8_t *__restrict__ meta,
    const int32_t *__restrict__ tile_ptr, const int32_t *__restrict__ tile_step, int64_t m,
    int64_t k, int64_t n, int64_t k_pad, int32_t mtiles, int32_t ntiles, int32_t tiles,
    int32_t per_xcd, const int8_t *__restrict__ B, int64_t ldb, int32_t *__restrict__ C,
    int64_t ldc) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];

  // logical tile t: groups of kMG row tiles x every column tile, contiguous
  // per XCD (workgroup b runs on XCD b % 8)
  const int t = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (t >= tiles) return;
  const int grp = t / (kMG * ntiles), rem = t % (kMG * ntiles);
  const int gsize = min(kMG, mtiles - grp * kMG);
  const int64_t m0 = static_cast<int64_t>(grp * kMG + rem % gsize) * kTM;
  const int64_t n0 = static_cast<int64_t>(rem / gsize) * kTN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  // this row tile's stored k-steps and their tiled values and index words
  int64_t first, ksteps;
  if constexpr (kTiles) {
    first = tile_ptr[m0 / kTM];
    ksteps = tile_ptr[m0 / kTM + 1] - first;
  } else {
    ksteps = k_pad / kTK;
    first = (m0 / kTM) * ksteps;
  }
  const int8_t *vt = vals + first * kAVBytes;
  const uint8_t *mtl = meta + first * kAMBytes;
  // k-step of B for the ks-th stored step
  auto kstep = [&](int64_t ks) -> int64_t {
    if constexpr (kTiles) return tile_step[first + ks];
    else return ks;
  };

  // Loads of one k-step, per wave: A values 2 x 1 KB and half a KB of index
  // words, all consecutive bytes of the tiled copies; B 4 x 1 KB (4 k-rows x
  // 256 B each).
  const uint32_t lds_base = lds_addr(lds);
  uint32_t b_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (wave * 4 + i) * 4 + (lane >> 4);  // k-row of the slab
    const int c = swz(r, lane & 15);                 // logical 16-byte piece
    const int64_t col = (n0 + c * 16 < n) ? n0 + c * 16 : n0;
    b_off[i] = static_cast<uint32_t>(r * ldb + col);
  }
  // load `part` (0..6) of k-step ks into stage `stage`: A values 0..1,
  // index words 2, B 3..6.  Every wave issues all kLoads parts per step (the
  // vmcnt waits count them).
  auto issue_part = [&](int64_t ks, int stage, int part) {
    const uint32_t sb = lds_base + stage * kStageBytes;
    if (part < 2) {
      const uint32_t o = (wave * 2 + part) * 1024;
      load_lds16(sb + o, vt + ks * kAVBytes, o + lane * 16);
    } else if (part == 2) {
      const uint32_t o = wave * kMLanes * 16;
      if (lane < kMLanes) load_lds16(sb + kAVBytes + o, mtl + ks * kAMBytes, o + lane * 16);
    } else {
      // k-rows past k (the last step when k % 128 != 0) are read from row 0:
      // the matching A values are zero-padded, so they add nothing
      const int i = part - 3;
      const int64_t krow0 = kstep(ks) * kTK;
      const int r = (wave * 4 + i) * 4 + (lane >> 4);
      const uint32_t off = krow0 + r < k ? static_cast<uint32_t>(krow0 * ldb) + b_off[i]
                                         : b_off[i] - static_cast<uint32_t>(r * ldb);
      load_lds16(sb + kAVBytes + kAMBytes + (wave * 4 + i) * 1024, B, off);
    }
  };
  auto issue = [&](int64_t ks, int stage) {
#pragma unroll
    for (int part = 0; part < kLoads; ++part) issue_part(ks, stage, part);
  };

  i32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = i32x4{0, 0, 0, 0};

  // transpose-read addressing: in a 16-lane group, lane p supplies the 8
  // columns 8*(p%2).. of k-row p/2; lane i then holds k-rows 0..7 of column i
  const int g = lane >> 4;
  const int pl = lane & 15;
  const int tr_row = 16 * g + (pl >> 1);  // + 0, 8, 64, 72
  const int tr_colb = wn * 64 + 8 * (pl & 1);

  for (int s = 0; s < kStages - 1; ++s)
    if (s < ksteps) issue(s, s);
  for (int64_t ks = 0; ks < ksteps; ++ks) {
    // this step's loads have landed (the next step's may still be in flight)
    if (ks + 1 < ksteps) wait_vm<kLoads>();
    else wait_vm<0>();
    barrier();  // ... for every wave; and the stage of step ks-1 is free
    // the loads of step ks+2 are issued between this step's MFMAs, so the
    // address unit works through them while the matrix cores run
    const bool more = ks + kStages - 1 < ksteps;
    const int64_t kn = ks + kStages - 1;
    const int sn = static_cast<int>(kn % kStages);
    const char *sb = lds + (ks % kStages) * kStageBytes;
    const char *sbb = sb + kAVBytes + kAMBytes;
    i32x8 bop[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      i32x2 q[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int r = tr_row + (h & 1) * 8 + (h >> 1) * 64;
        const int c = tr_colb + 16 * j;  // byte column
        q[h] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (lds_i32x2 *)(sbb + r * kTN + swz(r, c >> 4) * 16 + (c & 15)));
      }
      bop[j] = i32x8{q[0][0], q[0][1], q[1][0], q[1][1], q[2][0], q[2][1], q[3][0], q[3][1]};
    }
    // The index words of a wave's 8 row tiles sit together per lane (two
    // 16-byte reads); the A fragments of the first four row tiles are read
    // with them, those of the last four behind the first 16 sparse MFMAs.
    const i32x4 *afr = reinterpret_cast<const i32x4 *>(sb);
    const i32x4 *mfr = reinterpret_cast<const i32x4 *>(sb + kAVBytes) + (wm * 64 + lane) * 2;
    i32x4 aop[8];
    const i32x4 idx_lo = mfr[0], idx_hi = mfr[1];
    const int idx[8] = {idx_lo[0], idx_lo[1], idx_lo[2], idx_lo[3],
                        idx_hi[0], idx_hi[1], idx_hi[2], idx_hi[3]};
#pragma unroll
    for (int i = 0; i < 4; ++i) aop[i] = afr[(wm * 8 + i) * 64 + lane];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 4; i < 8; ++i) aop[i] = afr[(wm * 8 + i) * 64 + lane];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_smfmac_i32_16x16x128_i8(aop[i], bop[j], acc[i][j], idx[i], 0, 0);
      if (more && i < kLoads) issue_part(kn, sn, i);
    }
  }

  // D element r of lane l is row 4*(l/16) + r, column l%16 of its 16 x 16
  // tile.  A 4 x 4 transpose inside each quad of lanes gives lane q of the
  // quad row 4*(l/16) + q and the quad's 4 columns: one 16-byte store.
  const int q = lane & 3;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
      {  // exchange with lane ^ 1: elements 1,3 <-> 0,2
        const bool hi = q & 1;
        const int s0 = quad_swap<1>(hi ? v[0] : v[1]);
        const int s1 = quad_swap<1>(hi ? v[2] : v[3]);
        if (hi) { v[0] = s0; v[2] = s1; } else { v[1] = s0; v[3] = s1; }
      }
      {  // exchange with lane ^ 2: elements 2,3 <-> 0,1
        const bool hi = q & 2;
        const int s0 = quad_swap<2>(hi ? v[0] : v[2]);
        const int s1 = quad_swap<2>(hi ? v[1] : v[3]);
        if (hi) { v[0] = s0; v[1] = s1; } else { v[2] = s0; v[3] = s1; }
      }
      const int64_t row = m0 + wm * 128 + i * 16 + 4 * g + q;
      const int64_t col = n0 + wn * 64 + j * 16 + (lane & 12);
      if (row < m && col < n)
        __builtin_nontemporal_store(i32x4{v[0], v[1], v[2], v[3]},
                                    reinterpret_cast<i32x4 *>(C + row * ldc + col));
    }
}

}  // namespace

// One (row tile, k-step) piece of the plan layout.  v points at the piece's
// first compressed value (row stride vs bytes), mt at its first index byte
// (row stride ms); rows >= rows_ok and value / index columns >= vcols /
// mcols read as zero.
static void sp24_piece(const int8_t *v, int64_t vs, const uint8_t *mt, int64_t ms, int64_t rows_ok,
                       int64_t vcols, int64_t mcols, int8_t *vdst, uint8_t *mdst) {
  // values: [16-row tile][lane][16 bytes], lane l holding row l%16 and
  // bytes 16*(l/16).. of the step's 64 compressed bytes
  for (int t16 = 0; t16 < kTM / 16; ++t16)
    for (int l = 0; l < 64; ++l) {
      const int64_t row = t16 * 16 + (l & 15);
      const int64_t c0 = (l >> 4) * 16;
      for (int b = 0; b < 16; ++b)
        vdst[(t16 * 64 + l) * 16 + b] =
            (row < rows_ok && c0 + b < vcols) ? v[row * vs + c0 + b] : int8_t(0);
    }
  // index words: [row half wm 2][lane 64][row tile i 8][4 bytes]; lane l of
  // row half wm gets, for its 8 row tiles, word l/16 of row (8*wm + i)*16 + l%16
  for (int wm = 0; wm < 2; ++wm)
    for (int l = 0; l < 64; ++l)
      for (int i = 0; i < 8; ++i) {
        const int64_t row = (wm * 8 + i) * 16 + (l & 15);
        const int64_t c0 = (l >> 4) * 4;
        for (int b = 0; b < 4; ++b)
          mdst[((wm * 64 + l) * 8 + i) * 4 + b] =
              (row < rows_ok && c0 + b < mcols) ? mt[row * ms + c0 + b] : uint8_t(0);
      }
}

void sp24_tile_layout(const int8_t *vals, const uint8_t *meta, int64_t m, int64_t k,
                      int64_t m_pad, int64_t k_pad, int8_t *vals_tiled, uint8_t *meta_tiled) {
  const int64_t ksteps = k_pad / kTK;
  for (int64_t t = 0; t < m_pad / kTM; ++t)
    for (int64_t s = 0; s < ksteps; ++s)
      sp24_piece(vals + t * kTM * (k / 2) + s * (kTK / 2), k / 2,
                 meta + t * kTM * (k / 8) + s * (kTK / 8), k / 8, m - t * kTM,
                 k / 2 - s * (kTK / 2), k / 8 - s * (kTK / 8),
                 vals_tiled + (t * ksteps + s) * kAVBytes, meta_tiled + (t * ksteps + s) * kAMBytes);
}

void tvw_tile_layout(const int8_t *tile_vals, const uint8_t *tile_meta, int64_t ntiles,
                     int8_t *vals_tiled, uint8_t *meta_tiled) {
  for (int64_t t = 0; t < ntiles; ++t)
    sp24_piece(tile_vals + t * kTM * (kTK / 2), kTK / 2, tile_meta + t * kTM * (kTK / 8), kTK / 8,
               kTM, kTK / 2, kTK / 8, vals_tiled + t * kAVBytes, meta_tiled + t * kAMBytes);
}

int sp24_tile_m() { return kTM; }
int sp24_tile_n() { return kTN; }
int sp24_tile_k() { return kTK; }

int64_t sp24_grid(int64_t m, int64_t n) {
  const int64_t tiles = ((m + kTM - 1) / kTM) * ((n + kTN - 1) / kTN);
  return 8 * ((tiles + 7) / 8);
}

template <bool kTiles>
hipError_t launch(const Sp24Launch &a, hipStream_t s) {
  const int64_t mtiles = (a.m + kTM - 1) / kTM;
  const int64_t ntiles = (a.n + kTN - 1) / kTN;
  const int64_t tiles = mtiles * ntiles;
  if (tiles == 0) return hipSuccess;
  if (tiles > INT32_MAX / 2 || a.k_pad * a.ldb > UINT32_MAX)
    return hipErrorInvalidValue;
  hipError_t e =
      allow_dynamic_lds(reinterpret_cast<const void *>(&sp24_i8_smfmac<kTiles>), kLdsBytes);
  if (e != hipSuccess) return e;
  const int64_t per_xcd = (tiles + 7) / 8;
  hipLaunchKernelGGL(sp24_i8_smfmac<kTiles>, dim3(static_cast<unsigned>(8 * per_xcd)),
                     dim3(kThreads), kLdsBytes, s, a.vals, a.meta, a.tile_ptr, a.tile_step, a.m,
                     a.k, a.n, a.k_pad, static_cast<int32_t>(mtiles), static_cast<int32_t>(ntiles),
                     static_cast<int32_t>(tiles), static_cast<int32_t>(per_xcd), a.B, a.ldb, a.C,
                     a.ldc);
  return hipGetLastError();
}

hipError_t launch_sp24_i8(const Sp24Launch &a0, hipStream_t s) {
  Sp24Launch a = a0;
  if (a.b_rows) {
    // sliding-window A: B's rows in lifted order first (a.k lifted rows)
    hipError_t e = launch_gather_rows(a.B, a.ldb, a.b_rows, a.k, a.n, a.b_lift, a.n, s);
    if (e != hipSuccess) return e;
    a.B = a.b_lift;
    a.ldb = a.n;
  }
  return a.tile_ptr ? launch<true>(a, s) : launch<false>(a, s);
}

}  // namespace sdm

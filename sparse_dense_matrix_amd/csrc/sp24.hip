// sp24.hip -- C = A * B with A in 2:4 compressed form (two kept values and
// their 2-bit positions per group of four along k) and B dense row-major:
// int8 A and B with exact int32 C, or bf16 A and B with fp32 sums rounded to
// bf16 C (round to nearest even).
//
// The 2:4 pattern is the one the tiled-GEMM page (abstract) describes for the
// sparse tensor core; the Magicube page (abstract) motivates SpMM on
// low-precision integers.  On gfx950 the sparse MFMAs
// v_smfmac_i32_16x16x128_i8 and v_smfmac_f32_16x16x64_bf16 consume the
// compressed operand directly.  Both take, per lane, 16 bytes of kept values,
// 32 bytes of B and one index word, and give 4 accumulators; one covers a
// k-step of 128 (int8) or 64 (bf16) dense positions, a quarter of it per
// group of 16 lanes:
//   - A operand, lane l: row l%16 of the 16-row tile, the kept values of the
//     quarter l/16 of the step, and an index word whose bits [2j, 2j+2) give
//     kept value j's position in its group of four -- bit for bit the
//     canonical metadata nibbles of those groups (4 bytes for int8, the low 2
//     bytes for bf16), so the plan uploads the canonical arrays unchanged
//     (only zero-padded and reordered);
//   - B operand, lane l: column l%16; int8: dense k rows 16*(l/16)+0..15 and
//     64+16*(l/16)+0..15, read out of the row-major LDS slab with the gfx950
//     transpose read ds_read_b64_tr_b8 (8 k-values per read); bf16: rows
//     8*(l/16)+0..7 and 32+8*(l/16)+0..7 with ds_read_b64_tr_b16 (4 per read);
//   - D: rows 4*(l/16)+0..3, column l%16.
// A workgroup computes a 256 x 128 tile of C with 4 waves (each 128 x 64,
// 8 x 4 sparse MFMA tiles).  Operands go global -> LDS with direct loads
// into a two-stage ring (72 KB), so two workgroups share a CU and one
// covers the other's barriers and epilogue; each step's loads go out at its
// start, before its LDS reads.  The plan stores the
// compressed values and the index words tiled: for each 256-row tile and
// k-step, one contiguous 16 KB piece of values already in MFMA fragment
// order and one contiguous piece of index words (4 KB int8, 2 KB bf16), so
// every direct load reads 1 KB of consecutive bytes.  The B slab (16 KB at
// 128 columns: 128 k-rows of 128 bytes, or 64 of 256) has its 16-byte
// pieces XOR-swizzled by k-row so the transpose reads are bank-conflict
// free.  The tile order
// groups 4 row tiles with every column tile on one XCD, so each A panel is
// shared by all column tiles and each B panel 4-fold in that XCD's L2.
//
// The same kernel runs the tile-vector-wise pattern of the tiled-GEMM page
// (abstract: tile-wise sparsity at the global-memory level combined with 2:4
// at the register level): A is cut into tiles of 256 rows by a multiple of
// the k-step, only the tiles holding a nonzero are stored (2:4 inside), and
// a per-row-tile table lists their k-steps; the kernel walks that list
// instead of every k-step, so a zero tile is never loaded.
#include <algorithm>

#include "internal.h"

// load_lds16 below names m0 as clobbered on purpose (it sets m0 for the
// LDS-DMA instruction); clang warns about clobbering a reserved register.
#pragma clang diagnostic ignored "-Winline-asm"

namespace sdm {
namespace {

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kTM = 256;
constexpr int kMG = 4;                          // row tiles grouped on one XCD

// Workgroup tile: 256 rows x kN columns of C, waves of 128 x 64 (2 x kN/64).
// kN = 128: 4 waves and a two-stage ring (72 KB), so two workgroups share a
// CU and one covers the other's barriers and epilogue.  (256 x 256 tiles of
// 8 waves with a three-stage ring, one workgroup per CU, were 11-16% slower.)
template <int kN>
struct Tile {
  static_assert(kN == 128, "tile width");
  static constexpr int kWaves = kN / 32;
  static constexpr int kWN = kWaves / 2;        // waves along n
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kStages = 2;
  static constexpr int kAL = 16 / kWaves;       // 1 KB loads of A values per wave per k-step
  static constexpr int kBL = 4;                 // ... of the B slab
  static constexpr int kLoads = kAL + 1 + kBL;  // direct loads per wave per k-step
};

// Element types.  kTK: dense k per step (one sparse MFMA deep); kElem:
// bytes per element; kIdx: index bytes per lane and 16-row tile.
struct I8 {
  static constexpr int kTK = 128, kElem = 1, kIdx = 4;
  using Acc = i32x4;
};
struct Bf16 {
  static constexpr int kTK = 64, kElem = 2, kIdx = 2;
  using Acc = f32x4;
};

template <class E, int kN>
struct Geo {
  using T = Tile<kN>;
  static constexpr int kTK = E::kTK;
  static constexpr int kBRow = kN * E::kElem;                // bytes per k-row of the B slab
  static constexpr int kPieces = kBRow / 16;                  // 16-byte pieces per k-row
  static constexpr int kRowsPerLoad = 1024 / kBRow;           // k-rows per 1 KB wave load
  static constexpr int kAVBytes = kTM * kTK / 2 * E::kElem;   // 16 KB compressed values
  static constexpr int kAMBytes = kTM * kTK / 8;              // index bytes
  static constexpr int kBBytes = kTK * kBRow;                 // 16 KB
  static constexpr int kStageBytes = kAVBytes + kAMBytes + kBBytes;
  static constexpr int kLdsBytes = T::kStages * kStageBytes;  // 72 KB int8, 68 KB bf16
  static constexpr int kMLanes = kAMBytes / T::kWaves / 16;   // lanes of a wave that load index bytes
  static_assert(kLdsBytes <= 160 * 1024, "LDS");
  static_assert(kAVBytes == T::kAL * T::kWaves * 1024 && kBBytes == T::kBL * T::kWaves * 1024,
                "loads per wave");
  static_assert(kMLanes <= 64, "one index load per wave");
  static_assert(kAMBytes == 2 * 64 * 8 * E::kIdx, "index layout");
};

// Physical 16-byte piece of logical piece c in k-row r of the B slab.  A
// transpose read is served 32 lanes at a time, 256 bytes over the 64 banks
// (16 groups of 16 bytes); those lanes touch 16 k-rows of one piece (int8:
// rows 0..7 and 16..23 of a 32-row group) or 8 k-rows of two neighbouring
// pieces (bf16: rows 0..3 and 8..11 of a 16-row group).  The XOR spreads
// them over the 16 bank groups.  bf16 rows are 256 bytes, so a piece's bank
// group is its index.  int8 rows are 128 bytes, so the bank group is the
// row's parity times 8 plus the index, and the 8 rows of each parity take
// the 8 indices.
template <class E, int kN>
__device__ __forceinline__ int swz(int r, int c) {
  static_assert(kN == 128, "slab rows of 128 int8 or bf16 columns");
  if constexpr (E::kElem == 1) return c ^ (((r >> 1) & 3) | (((r >> 4) & 1) << 2));
  else return c ^ (((r & 3) | (((r >> 3) & 1) << 2)) << 1);
}


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


// B operand of column tile j (16 columns) of wave column wn from the slab sbb.
// int8: in a 16-lane group, lane p supplies the 8 columns 8*(p%2).. of k-row
// p/2, and lane i then holds k-rows 0..7 of column i; bf16: lane p supplies
// the 4 columns 4*(p%4).. of k-row p/4, lane i then holds k-rows 0..3.
template <class E, int kN>
__device__ __forceinline__ i32x8 read_b(const char *sbb, int lane, int wn, int j) {
  using G = Geo<E, kN>;
  const int g = lane >> 4, pl = lane & 15;
  i32x2 q[4];
  if constexpr (E::kElem == 1) {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int r = 16 * g + (pl >> 1) + (h & 1) * 8 + (h >> 1) * 64;
      const int c = wn * 64 + 8 * (pl & 1) + 16 * j;  // byte column
      q[h] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (lds_i32x2 *)(sbb + r * G::kBRow + swz<E, kN>(r, c >> 4) * 16 + (c & 15)));
    }
  } else {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int r = 8 * g + (pl >> 2) + (h & 1) * 4 + (h >> 1) * 32;
      const int c = wn * 64 + 4 * (pl & 3) + 16 * j;  // element column
      q[h] = __builtin_bit_cast(i32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4 *)(sbb + r * G::kBRow + swz<E, kN>(r, c >> 3) * 16 + (c & 7) * 2)));
    }
  }
  return i32x8{q[0][0], q[0][1], q[1][0], q[1][1], q[2][0], q[2][1], q[3][0], q[3][1]};
}

template <class E>
__device__ __forceinline__ typename E::Acc mma(i32x4 a, i32x8 b, typename E::Acc c, int idx) {
  if constexpr (E::kElem == 1)
    return __builtin_amdgcn_smfmac_i32_16x16x128_i8(a, b, c, idx, 0, 0);
  else
    return __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, a),
                                                     __builtin_bit_cast(bf16x16, b), c, idx, 0, 0);
}

// kTiles: A is tile-vector-wise; row tile T holds the stored k-steps
// tile_step[tile_ptr[T] .. tile_ptr[T+1]), their values and index words in
// that order.  Otherwise every k-step of every row tile is stored.  ldb and
// ldc count elements.
// kMap: slab k-row j multiplies B row b_rows[j] (sliding-window A, whose
// lifted k-rows repeat B's rows; the table is padded with row 0 to whole
// k-steps).  Otherwise slab k-row j multiplies B row j.
// kRagged: k is not a whole number of k-steps (plain 2:4 only); the last
// step's slab rows past k are then zeroed in LDS before use.
template <class E, int kN, bool kTiles, bool kMap, bool kRagged>
__device__ __forceinline__ void sp24_body(
    const char *__restrict__ vals, const uint8_t *__restrict__ meta,
    const int32_t *__restrict__ tile_ptr, const int32_t *__restrict__ tile_step, int64_t m,
    int64_t k, int64_t n, int64_t k_pad, int32_t mtiles, int32_t ntiles, int32_t tiles,
    int32_t per_xcd, const char *__restrict__ B, int64_t ldb, void *__restrict__ C, int64_t ldc,
    const int32_t *__restrict__ b_rows, const int32_t *__restrict__ row_order) {
  using G = Geo<E, kN>;
  using T = Tile<kN>;
  constexpr int kTK = G::kTK, kAVBytes = G::kAVBytes, kAMBytes = G::kAMBytes;
  constexpr int kStageBytes = G::kStageBytes, kMLanes = G::kMLanes;
  constexpr int kStages = T::kStages, kLoads = T::kLoads, kAL = T::kAL, kBL = T::kBL;
  extern __shared__ __attribute__((aligned(1024))) char lds[];

  // logical tile t: groups of kMG row tiles x every column tile, contiguous
  // per XCD (workgroup b runs on XCD b % 8)
  const int t = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (t >= tiles) return;
  const int grp = t / (kMG * ntiles), rem = t % (kMG * ntiles);
  const int gsize = min(kMG, mtiles - grp * kMG);
  int64_t m0, n0;
  if constexpr (kTiles) {
    // row tiles of unequal work, in the plan's order (row_order), row slot
    // slowest: with 16 column tiles the two workgroups a CU holds
    // (workgroups j and j + 32 of an XCD) are slots 0 and 2, or 1 and 3, of
    // the group, in the same column tile, and the plan puts a heavy and a
    // light row tile in those slots
    m0 = static_cast<int64_t>(row_order[grp * kMG + rem / ntiles]) * kTM;
    n0 = static_cast<int64_t>(rem % ntiles) * kN;
  } else {
    m0 = static_cast<int64_t>(grp * kMG + rem % gsize) * kTM;
    n0 = static_cast<int64_t>(rem / gsize) * kN;
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / T::kWN, wn = wave % T::kWN;
  // this row tile's stored k-steps and their tiled values and index words
  int64_t first, ksteps;
  if constexpr (kTiles) {
    first = tile_ptr[m0 / kTM];
    ksteps = tile_ptr[m0 / kTM + 1] - first;
  } else {
    ksteps = k_pad / kTK;
    first = (m0 / kTM) * ksteps;
  }
  const char *vt = vals + first * kAVBytes;
  const uint8_t *mtl = meta + first * kAMBytes;
  // k-step of B for the ks-th stored step
  auto kstep = [&](int64_t ks) -> int64_t {
    if constexpr (kTiles) return tile_step[first + ks];
    else return ks;
  };

  // Loads of one k-step, per wave: A values kAL x 1 KB and kMLanes x 16
  // bytes of index words, all consecutive bytes of the tiled copies; B kBL x
  // 1 KB (whole k-rows of the slab).
  const uint32_t lds_base = lds_addr(lds);
  const int64_t ldb_bytes = ldb * E::kElem;
  uint32_t b_off[kBL];  // kMap: the column part only
#pragma unroll
  for (int i = 0; i < kBL; ++i) {
    const int r = (wave * kBL + i) * G::kRowsPerLoad + lane / G::kPieces;  // k-row of the slab
    const int c = swz<E, kN>(r, lane % G::kPieces);  // logical 16-byte piece
    constexpr int per_piece = 16 / E::kElem;    // columns per piece
    const int64_t col = (n0 + c * per_piece < n) ? n0 + c * per_piece : n0;
    b_off[i] = static_cast<uint32_t>((kMap ? 0 : r * ldb_bytes) + col * E::kElem);
  }
  // kMap: the B rows of this wave's kBL * kRowsPerLoad slab k-rows of one
  // step, one piece of the table, read with scalar loads a step before its
  // loads go out (lane group q of load i takes row kRowsPerLoad * i + q)
  constexpr int kRPL = G::kRowsPerLoad, kWRows = kBL * kRPL;
  static_assert(!kMap || kWRows <= 32, "row map: at most 32 table entries per wave and step");
  int trow[kMap ? kWRows : 1];
  auto lookup = [&](int64_t ks) {
    if constexpr (kMap) {
      const int32_t *t = b_rows + ks * kTK + wave * kWRows;
#pragma unroll
      for (int q = 0; q < kWRows; ++q) trow[q] = t[q];
    }
  };
  // load `part` of k-step ks into stage `stage`: A values 0 .. kAL-1,
  // index words kAL, B after them.  Every wave issues all kLoads parts per
  // step (the vmcnt waits count them).
  auto issue_part = [&](int64_t ks, int stage, int part) {
    const uint32_t sb = lds_base + stage * kStageBytes;
    if (part < kAL) {
      const uint32_t o = (wave * kAL + part) * 1024;
      load_lds16(sb + o, vt + ks * kAVBytes, o + lane * 16);
    } else if (part == kAL) {
      const uint32_t o = wave * kMLanes * 16;
      if (lane < kMLanes) load_lds16(sb + kAVBytes + o, mtl + ks * kAMBytes, o + lane * 16);
    } else {
      // k-rows past k (the last step when k is not a whole number of steps)
      // are read from row 0: the matching A values are zero-padded, so they
      // add nothing
      const int i = part - kAL - 1;
      uint32_t off;
      if constexpr (kMap) {
        // lane group q takes trow[kRPL i + q]; written as masks so the
        // values stay in scalar registers (a select chain becomes an
        // indexed private array)
        const int q = lane / G::kPieces;
        int row = 0;
#pragma unroll
        for (int j = 0; j < kRPL; ++j) row |= trow[kRPL * i + j] & -(q == j);
        off = static_cast<uint32_t>(row * ldb_bytes) + b_off[i];
      } else {
        // k-rows past k (the last step when k is not a whole number of
        // steps) are read from row 0 and overwritten with zeros once they
        // have landed (see the main loop)
        const int64_t krow0 = kstep(ks) * kTK;
        const int r = (wave * kBL + i) * G::kRowsPerLoad + lane / G::kPieces;
        off = krow0 + r < k ? static_cast<uint32_t>(krow0 * ldb_bytes) + b_off[i]
                            : b_off[i] - static_cast<uint32_t>(r * ldb_bytes);
      }
      load_lds16(sb + kAVBytes + kAMBytes + (wave * kBL + i) * 1024, B, off);
    }
  };
  auto issue = [&](int64_t ks, int stage) {
#pragma unroll
    for (int part = 0; part < kLoads; ++part) issue_part(ks, stage, part);
  };

  typename E::Acc acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = 0;

  for (int s = 0; s < kStages - 1; ++s)
    if (s < ksteps) {
      lookup(s);
      issue(s, s);
    }
  if (kStages - 1 < ksteps) lookup(kStages - 1);
  for (int64_t ks = 0; ks < ksteps; ++ks) {
    // this step's loads have landed (nothing else is in flight: two stages)
    static_assert(kStages == 2, "one k-step in flight");
    wait_vm<0>();
    barrier();  // ... for every wave; and the stage of step ks-1 is free
    if constexpr (kRagged) {
      if (ks == ksteps - 1) {
        // the slab rows past k hold copies of B's row 0; zero them so the
        // zero-padded A values meet zeros (0 * Inf would give NaN in bf16)
        char *tail = lds + (ks % kStages) * kStageBytes + kAVBytes + kAMBytes;
        const int r0 = static_cast<int>(k - (ksteps - 1) * kTK);
        for (int o = r0 * G::kBRow + tid * 16; o < G::kBBytes; o += T::kThreads * 16)
          *reinterpret_cast<i32x4 *>(tail + o) = i32x4{0, 0, 0, 0};
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the zeros are written
        barrier();
      }
    }
    // The loads of step ks+kStages-1 go out first: inline asm between the
    // LDS reads and the MFMAs would make the compiler wait for every read
    // before it.
    const int64_t kn = ks + kStages - 1;
    if (kn < ksteps) issue(kn, static_cast<int>(kn % kStages));
    const char *sb = lds + (ks % kStages) * kStageBytes;
    const char *sbb = sb + kAVBytes + kAMBytes;
    // The index words of a wave's 8 row tiles sit together per lane (one or
    // two 16-byte reads, consecutive lanes 16 bytes apart), then its 8 A
    // fragments.
    int idx[8];
    if constexpr (E::kIdx == 4) {
      const i32x4 *mfr = reinterpret_cast<const i32x4 *>(sb + kAVBytes) + wm * 128 + lane;
      const i32x4 lo = mfr[0], hi = mfr[64];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        idx[i] = lo[i];
        idx[4 + i] = hi[i];
      }
    } else {
      const i32x4 w = reinterpret_cast<const i32x4 *>(sb + kAVBytes)[wm * 64 + lane];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        idx[i] = static_cast<int>((static_cast<uint32_t>(w[i >> 1]) >> (16 * (i & 1))) & 0xffffu);
    }
    const i32x4 *afr = reinterpret_cast<const i32x4 *>(sb);
    i32x4 aop[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) aop[i] = afr[(wm * 8 + i) * 64 + lane];
    // B one column tile ahead: tile j+1's 4 transpose reads are in flight
    // while tile j's 8 MFMAs issue.  At most 18 reads are outstanding, few
    // enough for each wait to name a count (lgkmcnt holds at most 15).
    i32x8 bop[4];
    bop[0] = read_b<E, kN>(sbb, lane, wn, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j + 1 < 4) bop[j + 1] = read_b<E, kN>(sbb, lane, wn, j + 1);
      __builtin_amdgcn_sched_barrier(0);
      if (j + 1 < 4) __builtin_amdgcn_s_waitcnt(0xc07f | (4 << 8));  // lgkmcnt(4)
      else __builtin_amdgcn_s_waitcnt(0xc07f);                        // lgkmcnt(0)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i][j] = mma<E>(aop[i], bop[j], acc[i][j], idx[i]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // the table rows of step ks+3, after this step's last LDS wait (a scalar
    // load in flight would force the LDS waits above down to zero)
    if (kn + 1 < ksteps) lookup(kn + 1);
  }

  // D element r of lane l is row 4*(l/16) + r, column l%16 of its 16 x 16
  // tile.  A 4 x 4 transpose inside each quad of lanes gives lane q of the
  // quad row 4*(l/16) + q and the quad's 4 columns: one 16-byte (int32) or
  // 8-byte (bf16) store.
  const int g = lane >> 4;
  const int q = lane & 3;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const i32x4 bits = __builtin_bit_cast(i32x4, acc[i][j]);
      int v[4] = {bits[0], bits[1], bits[2], bits[3]};
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
      // plain stores: measured 5% faster here than non-temporal ones (the
      // C tile is written once, at the very end, with nothing left to keep
      // in L2)
      if (row < m && col < n) {
        if constexpr (E::kElem == 1) {
          *reinterpret_cast<i32x4 *>(static_cast<int32_t *>(C) + row * ldc + col) =
              i32x4{v[0], v[1], v[2], v[3]};
        } else {
          // float -> bf16 rounds to nearest even
          uint32_t h[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            h[e] = __builtin_bit_cast(unsigned short, static_cast<__bf16>(__int_as_float(v[e])));
          *reinterpret_cast<i32x2 *>(static_cast<uint16_t *>(C) + row * ldc + col) =
              i32x2{static_cast<int>(h[0] | (h[1] << 16)), static_cast<int>(h[2] | (h[3] << 16))};
        }
      }
    }
}

#define SP24_ARGS                                                                              \
  const char *__restrict__ vals, const uint8_t *__restrict__ meta,                              \
      const int32_t *__restrict__ tile_ptr, const int32_t *__restrict__ tile_step, int64_t m,   \
      int64_t k, int64_t n, int64_t k_pad, int32_t mtiles, int32_t ntiles, int32_t tiles,       \
      int32_t per_xcd, const char *__restrict__ B, int64_t ldb, void *__restrict__ C, int64_t ldc, \
      const int32_t *__restrict__ b_rows, const int32_t *__restrict__ row_order
#define SP24_PASS vals, meta, tile_ptr, tile_step, m, k, n, k_pad, mtiles, ntiles, tiles, per_xcd, B, ldb, C, ldc, b_rows, row_order

template <int kN, bool kTiles, bool kMap, bool kRagged>
__global__ __launch_bounds__(Tile<kN>::kThreads) void sp24_i8_smfmac(SP24_ARGS) {
  sp24_body<I8, kN, kTiles, kMap, kRagged>(SP24_PASS);
}

template <int kN, bool kTiles, bool kRagged>
__global__ __launch_bounds__(Tile<kN>::kThreads) void sp24_bf16_smfmac(SP24_ARGS) {
  sp24_body<Bf16, kN, kTiles, false, kRagged>(SP24_PASS);
}

#undef SP24_ARGS
#undef SP24_PASS

// One (row tile, k-step) piece of the plan layout.  v points at the piece's
// first compressed value byte (row stride vs bytes), mt at its first index
// byte (row stride ms); rows >= rows_ok and value / index byte columns >=
// vcols / mcols read as zero.  The step's 64 value bytes of a row are the
// same for both element types; a lane's index bytes are kIdx of them.
template <class E>
void sp24_piece(const char *v, int64_t vs, const uint8_t *mt, int64_t ms, int64_t rows_ok,
                int64_t vcols, int64_t mcols, char *vdst, uint8_t *mdst) {
  // values: [16-row tile][lane][16 bytes], lane l holding row l%16 and
  // bytes 16*(l/16).. of the step's 64 compressed bytes
  for (int t16 = 0; t16 < kTM / 16; ++t16)
    for (int l = 0; l < 64; ++l) {
      const int64_t row = t16 * 16 + (l & 15);
      const int64_t c0 = (l >> 4) * 16;
      for (int b = 0; b < 16; ++b)
        vdst[(t16 * 64 + l) * 16 + b] = (row < rows_ok && c0 + b < vcols) ? v[row * vs + c0 + b] : 0;
    }
  // index words: lane l of row half wm gets, for its 8 row tiles i, bytes
  // kIdx*(l/16).. of row (8*wm + i)*16 + l%16, as 16-byte pieces that
  // consecutive lanes read 16 bytes apart (no LDS bank conflict):
  // int8 [wm 2][i/4 2][lane 64][i%4 4][4 bytes], bf16 [wm 2][lane 64][i 8][2 bytes]
  constexpr int kI = E::kIdx;
  constexpr int kPer = 16 / kI;  // row tiles per 16-byte piece
  for (int wm = 0; wm < 2; ++wm)
    for (int l = 0; l < 64; ++l)
      for (int i = 0; i < 8; ++i) {
        const int64_t row = (wm * 8 + i) * 16 + (l & 15);
        const int64_t c0 = (l >> 4) * kI;
        const int64_t piece = (wm * (8 / kPer) + i / kPer) * 64 + l;
        for (int b = 0; b < kI; ++b)
          mdst[piece * 16 + (i % kPer) * kI + b] =
              (row < rows_ok && c0 + b < mcols) ? mt[row * ms + c0 + b] : uint8_t(0);
      }
}

template <class E>
void tile_layout(const char *vals, const uint8_t *meta, int64_t m, int64_t k, int64_t m_pad,
                 int64_t k_pad, char *vals_tiled, uint8_t *meta_tiled) {
  using G = Geo<E, 128>;  // the A layout does not depend on the tile width
  const int64_t ksteps = k_pad / G::kTK;
  const int64_t vrow = k / 2 * E::kElem, vstep = G::kTK / 2 * E::kElem;
  for (int64_t t = 0; t < m_pad / kTM; ++t)
    for (int64_t s = 0; s < ksteps; ++s)
      sp24_piece<E>(vals + t * kTM * vrow + s * vstep, vrow,
                    meta + t * kTM * (k / 8) + s * (G::kTK / 8), k / 8, m - t * kTM,
                    vrow - s * vstep, k / 8 - s * (G::kTK / 8),
                    vals_tiled + (t * ksteps + s) * G::kAVBytes,
                    meta_tiled + (t * ksteps + s) * G::kAMBytes);
}

template <class E>
void tvw_layout(const char *tile_vals, const uint8_t *tile_meta, int64_t ntiles, int32_t tk,
                char *vals_tiled, uint8_t *meta_tiled) {
  using G = Geo<E, 128>;
  const int64_t per = tk / G::kTK;  // k-steps per stored tile
  const int64_t vrow = tk / 2 * E::kElem, vstep = G::kTK / 2 * E::kElem;
  for (int64_t t = 0; t < ntiles; ++t)
    for (int64_t s = 0; s < per; ++s)
      sp24_piece<E>(tile_vals + t * kTM * vrow + s * vstep, vrow,
                    tile_meta + t * kTM * (tk / 8) + s * (G::kTK / 8), tk / 8, kTM, vstep,
                    G::kTK / 8, vals_tiled + (t * per + s) * G::kAVBytes,
                    meta_tiled + (t * per + s) * G::kAMBytes);
}

template <class E, int kN, bool kTiles, bool kMap, bool kRagged = false>
hipError_t launch(const Sp24Launch &a, hipStream_t s) {
  using G = Geo<E, kN>;
  const int64_t mtiles = (a.m + kTM - 1) / kTM;
  const int64_t ntiles = (a.n + kN - 1) / kN;
  const int64_t tiles = mtiles * ntiles;
  if (tiles == 0) return hipSuccess;
  if (tiles > INT32_MAX / 2 || a.k_pad * a.ldb * E::kElem > UINT32_MAX)
    return hipErrorInvalidValue;
  if (kTiles && !a.row_order) return hipErrorInvalidValue;
  auto kernel = [] {
    if constexpr (E::kElem == 1) return sp24_i8_smfmac<kN, kTiles, kMap, kRagged>;
    else return sp24_bf16_smfmac<kN, kTiles, kRagged>;
  }();
  hipError_t e = allow_dynamic_lds(reinterpret_cast<const void *>(kernel), G::kLdsBytes);
  if (e != hipSuccess) return e;
  const int64_t per_xcd = (tiles + 7) / 8;
  hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(8 * per_xcd)), dim3(Tile<kN>::kThreads),
                     G::kLdsBytes, s, static_cast<const char *>(a.vals), a.meta, a.tile_ptr,
                     a.tile_step, a.m, a.k, a.n, a.k_pad, static_cast<int32_t>(mtiles),
                     static_cast<int32_t>(ntiles), static_cast<int32_t>(tiles),
                     static_cast<int32_t>(per_xcd), static_cast<const char *>(a.B), a.ldb, a.C,
                     a.ldc, a.b_rows, a.row_order);
  return hipGetLastError();
}

}  // namespace

vec<int32_t> tvw_row_order(const int32_t *tile_ptr, int64_t mtiles) {
  vec<int32_t> by_work(static_cast<size_t>(mtiles));
  for (int64_t T = 0; T < mtiles; ++T) by_work[T] = static_cast<int32_t>(T);
  std::stable_sort(by_work.begin(), by_work.end(), [&](int32_t x, int32_t y) {
    return tile_ptr[x + 1] - tile_ptr[x] > tile_ptr[y + 1] - tile_ptr[y];
  });
  const int64_t groups = (mtiles + 3) / 4;
  vec<vec<int32_t>> members(static_cast<size_t>(groups));
  // only the last group may hold fewer than four (when mtiles % 4 != 0)
  auto room = [&](int64_t g) {
    return static_cast<int64_t>(members[static_cast<size_t>(g)].size()) < std::min<int64_t>(4, mtiles - 4 * g);
  };
  int64_t g = 0, dir = 1;
  auto next_group = [&]() {  // snake order: 0 .. G-1, G-1 .. 0, 0 ..
    if (g + dir < 0 || g + dir >= groups) dir = -dir;
    else g += dir;
  };
  for (int64_t i = 0; i < mtiles; ++i) {
    while (!room(g)) next_group();
    members[static_cast<size_t>(g)].push_back(by_work[i]);
    next_group();
  }
  vec<int32_t> order;
  order.reserve(static_cast<size_t>(mtiles));
  for (auto &mem : members) {
    if (mem.size() == 4) std::swap(mem[2], mem[3]);  // heaviest, second, lightest, third
    order.insert(order.end(), mem.begin(), mem.end());
  }
  return order;
}

void sp24_tile_layout(const void *vals, const uint8_t *meta, int64_t m, int64_t k, int64_t m_pad,
                      int64_t k_pad, bool bf16, void *vals_tiled, uint8_t *meta_tiled) {
  const char *v = static_cast<const char *>(vals);
  char *vt = static_cast<char *>(vals_tiled);
  if (bf16) tile_layout<Bf16>(v, meta, m, k, m_pad, k_pad, vt, meta_tiled);
  else tile_layout<I8>(v, meta, m, k, m_pad, k_pad, vt, meta_tiled);
}

void tvw_tile_layout(const void *tile_vals, const uint8_t *tile_meta, int64_t ntiles, int32_t tk,
                     bool bf16, void *vals_tiled, uint8_t *meta_tiled) {
  const char *v = static_cast<const char *>(tile_vals);
  char *vt = static_cast<char *>(vals_tiled);
  if (bf16) tvw_layout<Bf16>(v, tile_meta, ntiles, tk, vt, meta_tiled);
  else tvw_layout<I8>(v, tile_meta, ntiles, tk, vt, meta_tiled);
}

int sp24_tile_m() { return kTM; }
int sp24_tile_n(int64_t n, bool mapped) {
  (void)n;
  (void)mapped;
  return 128;  // two workgroups per CU
}
int sp24_tile_k(bool bf16) { return bf16 ? Bf16::kTK : I8::kTK; }

int64_t sp24_grid(int64_t m, int64_t n, int tn) {
  const int64_t tiles = ((m + kTM - 1) / kTM) * ((n + tn - 1) / tn);
  return 8 * ((tiles + 7) / 8);
}

namespace {
template <int kN>
hipError_t launch_n(const Sp24Launch &a, hipStream_t s) {
  const bool ragged = a.k_pad > a.k;  // plain 2:4 only: a tile table keeps whole steps
  if (a.bf16) {
    if (a.tile_ptr) return launch<Bf16, kN, true, false>(a, s);
    return ragged ? launch<Bf16, kN, false, false, true>(a, s) : launch<Bf16, kN, false, false>(a, s);
  }
  if (a.tile_ptr) return launch<I8, kN, true, false>(a, s);
  return ragged ? launch<I8, kN, false, false, true>(a, s) : launch<I8, kN, false, false>(a, s);
}
}  // namespace

hipError_t launch_sp24(const Sp24Launch &a, hipStream_t s) {
  if (a.b_rows) {
    // sliding-window A: int8, every k-step stored, B read through the row map
    if (a.bf16 || a.tile_ptr || a.tn != 128) return hipErrorInvalidValue;
    return launch<I8, 128, false, true>(a, s);
  }
  if (a.tn != 128) return hipErrorInvalidValue;
  return launch_n<128>(a, s);
}

}  // namespace sdm

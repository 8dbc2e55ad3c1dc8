// bcsr_bf16.hip -- C = A * B with A in BCSR (64 x 64 bf16 blocks), B and C
// dense row-major bf16, fp32 accumulation, round-to-nearest-even output.
//
// Block-structured SpMM of the AsyncSparse page (abstract; Figure 2
// caption): only the stored blocks of a block row are multiplied.  The page
// overlaps TMA copies with WGMMA through producer/consumer warps; on gfx950
// the same overlap comes from direct global->LDS loads (no registers in
// between) into a ring of kStages LDS stages, every wave both issuing loads
// and running MFMAs:
//   - a tile is a 64-row block row times kTN (256 or 512) columns of C; each
//     of the kTN/64 waves owns 64 x 64 of it as 2 x 2 MFMA 32x32x16 bf16
//     tiles;
//   - a stage holds one stored block: the B slab (64 k-rows x kTN columns,
//     row-major) and the A block, pre-arranged by the plan in MFMA fragment
//     order; or, for rows of few blocks at kTN = 256, half a block (32
//     k-rows), so that a stage is 20 KB and more workgroups share a CU;
//   - B is n-contiguous but the MFMA wants k-contiguous operands: the gfx950
//     LDS transpose read (ds_read_b64_tr_b16) gives each lane 4 k-values of
//     one column, two reads make an operand.  The slab's 16-byte pieces are
//     XOR-swizzled by k-row so those reads hit 64 distinct banks;
//   - the ring has two stages (80 KB at kTN = 256, 40 KB with half blocks,
//     so two or three workgroups share a CU and each hides the others'
//     barriers, pipeline fill and epilogue; 144 KB at kTN = 512);
//   - the finished tile is rounded to bf16, staged in the (now idle) ring and
//     written to C with 16-byte non-temporal stores, which keep the streaming
//     C writes from evicting B from L2;
//   - tiles are dealt so that each XCD walks a contiguous range, block rows
//     fastest: the workgroups resident on one XCD share the B column slab of
//     one N tile in that XCD's L2.  When A is too large to stay in L2 while
//     every N tile walks all of it, the plan splits the block rows into row
//     groups of about equal work and deals each group's tiles to its own
//     XCDs (one, or two with half the N tiles each), so that share of A
//     stays resident.  Within an N tile the block rows with
//     the most stored blocks come first (longest job first), so short tiles
//     fill the end of the launch instead of long ones.
// A 64-row block gives at most 64 flop per byte of B moved into LDS.  When
// block rows share block columns, bcsr_bf16_pair (below) computes two block
// rows per tile over the union of their block columns, so a B slab both
// rows use is moved into LDS once.
#include <algorithm>

#include "internal.h"

// load_lds16 below names m0 as clobbered on purpose (it sets m0 for the
// LDS-DMA instruction); clang warns about clobbering a reserved register.
#pragma clang diagnostic ignored "-Winline-asm"

namespace sdm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kBlk = 64;                  // block edge
constexpr int kStages = 2;                // one block in flight while one is used
constexpr int kABytes = kBlk * kBlk * 2;  // 8 KB
constexpr int kCPitch = 144;              // bytes per row of a wave's staged C tile

// Tile geometry for kTN columns of C per workgroup (one wave per 64 columns)
// and kKH k-rows (a whole block, or half of one) per stage.
template <int kTN, int kKH = kBlk>
struct Geo {
  static constexpr int kWaves = kTN / 64;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kSteps = kKH / 16;         // MFMA k-steps per stage
  static constexpr int kPer = kBlk / kKH;         // stages per block
  static constexpr int kBRow = kTN * 2;           // bytes per k-row of the B slab
  static constexpr int kBBytes = kKH * kBRow;
  static constexpr int kAStage = kABytes / kPer;  // the stage's share of the A block
  static constexpr int kStageBytes = kBBytes + kAStage;
  static constexpr int kBLoads = kBBytes / 1024 / kWaves;  // 1 KB wave loads per wave per stage
  static constexpr int kALoads = kAStage / 1024 / kWaves;
  static constexpr int kLdsBytes = kStages * kStageBytes;
  static_assert(kKH == 64 || kKH == 32, "whole or half blocks");
  static_assert(kBLoads * kWaves * 1024 == kBBytes && kALoads * kWaves * 1024 == kAStage, "split");
  static_assert(kWaves * 64 * kCPitch <= kLdsBytes, "C staging fits in the ring");
  static_assert(kLdsBytes <= 160 * 1024, "LDS");
};

// physical 16-byte piece of logical piece c in k-row r of the B slab
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r & 3) << 2); }

// s_waitcnt vmcnt(n), leaving the other counters alone
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Direct global->LDS load of 16 bytes per lane: LDS[lds + 16 * lane] =
// global[base + voff].  Issued as inline asm so the compiler neither waits
// on it (the kernel counts vmcnt itself) nor assumes every later LDS read
// depends on it.
__device__ __forceinline__ void load_lds16(uint32_t lds, const void *base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds), "v"(voff), "s"(base)
               : "memory", "m0");
}

// Workgroup barrier without the memory fence __syncthreads() adds (the fence
// would wait for every in-flight load); global loads are ordered by the
// explicit vmcnt waits before it.  Every LDS read of a block feeds that
// block's MFMAs, so its wait comes before the loop's back edge and no read of
// a stage is in flight when the next block refills it.
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char *)(p)));
}

// With B as the left MFMA operand the accumulators hold a tile transposed:
// lane l has row 32 rb + (l & 31) of the wave's 64-row tile, and registers
// 4q..4q+3 of acc[rb][cb] are its four consecutive columns
// 32 cb + 8q + 4 (l >> 5) ...  Round them to bf16 two at a time and stage
// the tile as rows of kPitch bytes, 8 bytes per write.
template <int kCb, int kPitch>
__device__ __forceinline__ void stage_c(char *ct, const f32x16 (&acc)[2][kCb], int lane) {
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < kCb; ++cb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = rb * 32 + (lane & 31);
        const int col = cb * 32 + 8 * q + 4 * (lane >> 5);
        const f32x16 &v = acc[rb][cb];
        const bf16x2 lo = __builtin_convertvector((f32x2){v[4 * q], v[4 * q + 1]}, bf16x2);
        const bf16x2 hi = __builtin_convertvector((f32x2){v[4 * q + 2], v[4 * q + 3]}, bf16x2);
        *reinterpret_cast<u32x2 *>(ct + row * kPitch + col * 2) =
            (u32x2){__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
      }
}

// Write a staged 64 x (32 kCb) tile to C rows row0 .. row0 + 63 (through
// c_rows when A was packed with its rows permuted), columns c0 ..: 16-byte
// pieces, every piece read from LDS before the first store.
template <int kCb, int kPitch>
__device__ __forceinline__ void store_c(const char *ct, int lane, int64_t row0, int64_t c0, int64_t n,
                                        const int32_t *__restrict__ c_rows, uint16_t *__restrict__ C,
                                        int64_t ldc) {
  constexpr int kPieces = kCb * 4, kRowsPer = 64 / kPieces, kQ = 64 / kRowsPer;
  const int64_t col = c0 + (lane % kPieces) * 8;
  if (col >= n) return;
  u32x4 v[kQ];
#pragma unroll
  for (int q = 0; q < kQ; ++q)
    v[q] = *reinterpret_cast<const u32x4 *>(ct + (q * kRowsPer + lane / kPieces) * kPitch +
                                            (lane % kPieces) * 16);
  const int64_t r = row0 + lane / kPieces;
  if (c_rows) {
#pragma unroll
    for (int q = 0; q < kQ; ++q)
      __builtin_nontemporal_store(
          v[q], reinterpret_cast<u32x4 *>(C + static_cast<int64_t>(c_rows[r + q * kRowsPer]) * ldc + col));
  } else {
#pragma unroll
    for (int q = 0; q < kQ; ++q)
      __builtin_nontemporal_store(v[q], reinterpret_cast<u32x4 *>(C + (r + q * kRowsPer) * ldc + col));
  }
}

struct Operands {
  bf16x8 a[2];
  bf16x8 b[2];
};

// kMap: the packed k-row j of A multiplies B row b_rows[j] (A packed with
// its columns permuted); each lane then reads its B rows through the map,
// looked up one block ahead.  Otherwise k-row j multiplies B row j.
// kKH: k-rows per stage (64: one block per stage; 32: two stages per block).
template <int kTN, bool kMap, int kKH>
__global__ __launch_bounds__(Geo<kTN>::kThreads) void bcsr_bf16_mfma(
    const int32_t *__restrict__ row_ptr, const int32_t *__restrict__ col_idx,
    const uint16_t *__restrict__ frag, const int32_t *__restrict__ row_order,
    const int32_t *__restrict__ row_seg, int32_t row_groups, int32_t ntn, int64_t n,
    const uint16_t *__restrict__ B, int64_t ldb,
    uint16_t *__restrict__ C, int64_t ldc, const int32_t *__restrict__ c_rows,
    const int32_t *__restrict__ b_rows) {
  using G = Geo<kTN, kKH>;
  constexpr int kSteps = G::kSteps, kPer = G::kPer;
  constexpr int kBRow = G::kBRow, kBBytes = G::kBBytes, kStageBytes = G::kStageBytes;
  constexpr int kBLoads = G::kBLoads, kALoads = G::kALoads;
  extern __shared__ __attribute__((aligned(1024))) char lds[];

  // XCD-aware tile order: workgroup b runs on XCD x = b % 8, which serves
  // row group x % row_groups (block rows row_order[row_seg[g] ..
  // row_seg[g+1]), most stored blocks first) and a contiguous range of that
  // group's tiles, block rows fastest.
  const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int grp = x % row_groups, part = x / row_groups, parts = 8 / row_groups;
  const int r0 = row_seg[grp], cnt = row_seg[grp + 1] - r0;
  const int tg = cnt * ntn;                      // tiles of the row group
  const int per = (tg + parts - 1) / parts;      // ... per XCD serving it
  const int t = part * per + j;
  if (j >= per || t >= tg) return;
  const int br = row_order[r0 + t % cnt];
  const int64_t n0 = static_cast<int64_t>(t / cnt) * kTN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int p0 = row_ptr[br], p1 = row_ptr[br + 1];
  const int nblk = p1 - p0;

  // Per-lane byte offsets of this wave's B loads relative to the block's
  // first k-row; columns past n are read from column n0 of the same row
  // (they only feed C columns that are never stored).
  // With kMap, boff holds only the column part and brow the lane's k-row in
  // the block; the row comes from b_rows (brow_next: the B rows of the next
  // block, loaded one block ahead).
  uint32_t boff[kBLoads];
  int brow[kBLoads];
#pragma unroll
  for (int i = 0; i < kBLoads; ++i) {
    const int o = (wave * kBLoads + i) * 1024 + lane * 16;  // byte offset in the slab
    const int r = o / kBRow;
    const int c = swz(r, (o % kBRow) / 16) * 8;
    const int64_t col = (n0 + c < n) ? n0 + c : n0;
    boff[i] = static_cast<uint32_t>(((kMap ? 0 : r * ldb) + col) * 2);
    brow[i] = r;
  }
  int brow_next[kBLoads];
  // B rows (through the map) of stage unit `unit` of the row: part
  // unit % kPer of block p0 + unit / kPer
  auto lookup_rows = [&](int unit) {
    if constexpr (kMap) {
      const int64_t k0 = static_cast<int64_t>(col_idx[p0 + unit / kPer]) * kBlk + (unit % kPer) * kKH;
#pragma unroll
      for (int i = 0; i < kBLoads; ++i) brow_next[i] = b_rows[k0 + brow[i]];
    }
  };
  const uint32_t lds_base = lds_addr(lds);
  // loads of stage unit `unit` of the row: part unit % kPer of block
  // p0 + unit / kPer
  auto issue = [&](int unit, int stage) {
    const int blk = p0 + unit / kPer, part = unit % kPer;
    const uint32_t sb = lds_base + stage * kStageBytes;
    if constexpr (kMap) {
#pragma unroll
      for (int i = 0; i < kBLoads; ++i)
        load_lds16(sb + (wave * kBLoads + i) * 1024, B,
                   static_cast<uint32_t>(brow_next[i] * ldb * 2) + boff[i]);
    } else {
      const uint16_t *bsrc = B + (static_cast<int64_t>(col_idx[blk]) * kBlk + part * kKH) * ldb;
#pragma unroll
      for (int i = 0; i < kBLoads; ++i) load_lds16(sb + (wave * kBLoads + i) * 1024, bsrc, boff[i]);
    }
    const uint16_t *asrc = frag + static_cast<int64_t>(blk) * (kABytes / 2);
#pragma unroll
    for (int i = 0; i < kALoads; ++i) {
      // 1 KB piece q of the stage: row half q / kSteps, k-step q % kSteps
      const int q = wave * kALoads + i;
      const int go = ((q / kSteps) * 4 + part * kSteps + q % kSteps) * 1024;
      load_lds16(sb + kBBytes + q * 1024, asrc, static_cast<uint32_t>(go + lane * 16));
    }
  };

  // transpose-read addressing: within a 16-lane group, lane p supplies the
  // 4 columns 4*(p%4).. of k-row p/4; lane i then holds k-rows 0..3 of
  // column i.  Lanes 32..63 take k-rows 8..15 of each 16-row step.
  const int g = lane >> 5;
  const int pl = lane & 15;
  const int tr_row = 8 * g + (pl >> 2);                                  // + 16 s + 4 h
  const int tr_col = wave * 64 + ((lane >> 4) & 1) * 16 + 4 * (pl & 3);  // + 32 cb
  auto read_ops = [&](const char *sb, int s) {
    Operands o;
    const bf16x8 *afr = reinterpret_cast<const bf16x8 *>(sb + kBBytes);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) o.a[rb] = afr[(rb * kSteps + s) * 64 + lane];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      s16x4 part[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = 16 * s + tr_row + 4 * h;
        const int c = tr_col + 32 * cb;
        part[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4 *)(sb + r * kBRow + swz(r, c >> 3) * 16 + (c & 7) * 2));
      }
      s16x8 bs;
      bs[0] = part[0][0]; bs[1] = part[0][1]; bs[2] = part[0][2]; bs[3] = part[0][3];
      bs[4] = part[1][0]; bs[5] = part[1][1]; bs[6] = part[1][2]; bs[7] = part[1][3];
      o.b[cb] = __builtin_bit_cast(bf16x8, bs);
    }
    return o;
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nunit = nblk * kPer;  // stages to run
  if (nunit > 0) {
    lookup_rows(0);
    issue(0, 0);
    if (nunit > 1) lookup_rows(1);
  }
  for (int it = 0; it < nunit; ++it) {
    wait_vm<0>();  // this stage's loads (and the next unit's row lookups) have landed
    barrier();     // ... for every wave; and the stage of unit it-1 is free
    if (it + 1 < nunit) {
      issue(it + 1, (it + 1) & 1);
      if (it + 2 < nunit) lookup_rows(it + 2);
    }
    const char *sb = lds + (it & 1) * kStageBytes;
    // every operand of the block is read before the first MFMA, so the LDS
    // latency is paid once per block instead of once per k-step
    Operands ops[kSteps];
#pragma unroll
    for (int s = 0; s < kSteps; ++s) ops[s] = read_ops(sb, s);
    __builtin_amdgcn_sched_barrier(0);  // keep the compiler from interleaving them again
#pragma unroll
    for (int s = 0; s < kSteps; ++s)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
          acc[rb][cb] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(ops[s].b[cb], ops[s].a[rb], acc[rb][cb], 0, 0, 0);
  }

  // epilogue: round to bf16, stage the wave's 64 x 64 tile in the idle ring
  // (B was the left MFMA operand, so the accumulators hold it transposed),
  // then write 16-byte pieces of C rows.
  barrier();  // every wave is done reading the ring
  char *ct = lds + wave * 64 * kCPitch;
  stage_c<2, kCPitch>(ct, acc, lane);
  __builtin_amdgcn_wave_barrier();
  store_c<2, kCPitch>(ct, lane, static_cast<int64_t>(br) * kBlk, n0 + wave * 64, n, c_rows, C, ldc);
}

// Paired block rows: a tile is two block rows times 256 columns of C.  Each
// wave owns 64 rows x kWC columns of one of the two rows (kWC = 128: 2 x 4
// MFMA tiles, so each A fragment read from LDS feeds 4 MFMAs; four waves).
// The pair walks the union of its rows' block columns in column order
// (units: column, block of the first row, block of the second, -1 for
// none), half a block per stage: a stage holds the 32 x 256 B half-slab and
// both rows' A halves, so a B slab both rows use is loaded once instead of
// twice.  Waves whose row has no block in a unit skip its MFMAs.
// The ring has three stages (two units in flight while one is used), no
// more LDS than the C staging takes anyway.  The unit descriptors sit in
// registers, one per lane, and are read with v_readlane, so the loop never
// waits on a scalar load.  Everything else (DMA loads, swizzle, transpose
// reads, epilogue, tile dealing with pairs in place of block rows) is the
// single-row kernel's.
constexpr int kPairWaveCols = 128;  // C columns per wave in the paired kernel

template <int kWC>
struct PairGeo {
  static constexpr int kTN = 256, kKH = 32;
  static constexpr int kRingStages = 3;
  static constexpr int kColWaves = kTN / kWC;   // waves per block row
  static constexpr int kWaves = 2 * kColWaves;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kCb = kWC / 32;          // MFMA column tiles per wave
  static constexpr int kPitch = kWC * 2 + 16;   // bytes per row of a wave's staged C tile
  static constexpr int kSteps = kKH / 16;
  static constexpr int kPer = kBlk / kKH;
  static constexpr int kBRow = kTN * 2;
  static constexpr int kBBytes = kKH * kBRow;  // 16 KB
  static constexpr int kAStage = kABytes / kPer;  // one row's share, 4 KB
  static constexpr int kStageBytes = kBBytes + 2 * kAStage;
  static constexpr int kBLoads = kBBytes / 1024 / kWaves;
  static constexpr int kALoads = kAStage / 1024 / kColWaves;  // per wave of a row
  static constexpr int kRing = kRingStages * kStageBytes;
  static constexpr int kCBytes = kWaves * 64 * kPitch;  // staged C of the two rows
  static constexpr int kLdsBytes = kRing > kCBytes ? kRing : kCBytes;
  static_assert(kBLoads * kWaves * 1024 == kBBytes, "split");
  static_assert(kALoads * kColWaves * 1024 == kAStage, "A split");
  static_assert(kWC == 64 || kWC == 128, "64 or 128 columns per wave");
  static_assert(2 * kLdsBytes <= 160 * 1024, "two workgroups per CU");
  static_assert(kTN == kBcsrPairTN && kKH == kBcsrPairKH, "the plan's pair tile");
};

template <int kWC>
__global__ __launch_bounds__(PairGeo<kWC>::kThreads, 2) void bcsr_bf16_pair(
    const int4 *__restrict__ units, const int32_t *__restrict__ pair_ptr,
    const int32_t *__restrict__ pair_rows, const uint16_t *__restrict__ frag,
    const int32_t *__restrict__ pair_order, const int32_t *__restrict__ pair_seg,
    int32_t row_groups, int32_t ntn, int64_t n, const uint16_t *__restrict__ B, int64_t ldb,
    uint16_t *__restrict__ C, int64_t ldc, const int32_t *__restrict__ c_rows) {
  using G = PairGeo<kWC>;
  constexpr int kSteps = G::kSteps, kPer = G::kPer, kTN = G::kTN, kCb = G::kCb;
  constexpr int kALoads = G::kALoads, kPitch = G::kPitch;
  constexpr int kBRow = G::kBRow, kBBytes = G::kBBytes, kStageBytes = G::kStageBytes;
  constexpr int kBLoads = G::kBLoads;
  extern __shared__ __attribute__((aligned(1024))) char lds[];

  const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int grp = x % row_groups, part = x / row_groups, parts = 8 / row_groups;
  const int r0 = pair_seg[grp], cnt = pair_seg[grp + 1] - r0;
  const int tg = cnt * ntn;
  const int per = (tg + parts - 1) / parts;
  const int t = part * per + j;
  if (j >= per || t >= tg) return;
  const int pr = pair_order[r0 + t % cnt];
  const int64_t n0 = static_cast<int64_t>(t / cnt) * kTN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = wave / G::kColWaves;  // which row of the pair
  const int cw = wave % G::kColWaves;    // which kWC columns
  const int u0 = pair_ptr[pr], nu = pair_ptr[pr + 1] - u0;
  const int br = pair_rows[2 * pr + half];  // block row of C this wave writes (-1: none)

  uint32_t boff[kBLoads];
#pragma unroll
  for (int i = 0; i < kBLoads; ++i) {
    const int o = (wave * kBLoads + i) * 1024 + lane * 16;
    const int r = o / kBRow;
    const int c = swz(r, (o % kBRow) / 16) * 8;
    const int64_t col = (n0 + c < n) ? n0 + c : n0;
    boff[i] = static_cast<uint32_t>((r * ldb + col) * 2);
  }
  const uint32_t lds_base = lds_addr(lds);
  // the block of this wave's row in unit u of the pair (-1: none)
  auto row_block = [&](const int4 &un) { return half ? un.z : un.y; };
  auto issue = [&](int unit, int stage, const int4 &un) {
    const int p = unit % kPer;
    const uint32_t sb = lds_base + stage * kStageBytes;
    const uint16_t *bsrc = B + (static_cast<int64_t>(un.x) * kBlk + p * G::kKH) * ldb;
#pragma unroll
    for (int i = 0; i < kBLoads; ++i) load_lds16(sb + (wave * kBLoads + i) * 1024, bsrc, boff[i]);
    const int blk = row_block(un);
    if (blk >= 0) {
#pragma unroll
      for (int i = 0; i < kALoads; ++i) {
        // 1 KB piece q of the row's stage share: row half q / kSteps, k-step q % kSteps
        const int q = cw * kALoads + i;
        const int go = ((q / kSteps) * 4 + p * kSteps + q % kSteps) * 1024;
        load_lds16(sb + kBBytes + half * G::kAStage + q * 1024,
                   frag + static_cast<int64_t>(blk) * (kABytes / 2), static_cast<uint32_t>(go + lane * 16));
      }
    }
  };

  const int g = lane >> 5;
  const int pl = lane & 15;
  const int tr_row = 8 * g + (pl >> 2);
  const int tr_col = cw * kWC + ((lane >> 4) & 1) * 16 + 4 * (pl & 3);
  struct Ops {
    bf16x8 a[2];
    bf16x8 b[kCb];
  };
  auto read_ops = [&](const char *sb, int s) {
    Ops o;
    const bf16x8 *afr = reinterpret_cast<const bf16x8 *>(sb + kBBytes + half * G::kAStage);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) o.a[rb] = afr[(rb * kSteps + s) * 64 + lane];
#pragma unroll
    for (int cb = 0; cb < kCb; ++cb) {
      s16x4 part[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = 16 * s + tr_row + 4 * h;
        const int c = tr_col + 32 * cb;
        part[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4 *)(sb + r * kBRow + swz(r, c >> 3) * 16 + (c & 7) * 2));
      }
      s16x8 bs;
      bs[0] = part[0][0]; bs[1] = part[0][1]; bs[2] = part[0][2]; bs[3] = part[0][3];
      bs[4] = part[1][0]; bs[5] = part[1][1]; bs[6] = part[1][2]; bs[7] = part[1][3];
      o.b[cb] = __builtin_bit_cast(bf16x8, bs);
    }
    return o;
  };

  f32x16 acc[2][kCb];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jj = 0; jj < kCb; ++jj)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][jj][r] = 0.0f;

  const int nunit = nu * kPer;
  // Unit descriptors sit in registers: lane l holds unit l of the pair (the
  // plan pairs rows only while every pair has at most 64 units), and a wave
  // reads one out with v_readlane, so no load waits inside the loop.
  const int4 win = lane < nu ? units[u0 + lane] : make_int4(0, -1, -1, 0);
  // descriptor of stage unit i; past the end, the last one again (unused:
  // nothing is issued or computed for it)
  const int last = nunit > 0 ? nunit - 1 : 0;
  auto desc = [&](int i) {
    const int l = min(i, last) / kPer;
    return make_int4(__builtin_amdgcn_readlane(win.x, l), __builtin_amdgcn_readlane(win.y, l),
                     __builtin_amdgcn_readlane(win.z, l), 0);
  };
  // descriptors of stage units it, it + 1, it + 2
  int4 d0 = desc(0), d1 = desc(1), d2 = desc(2);
  if (nunit > 0) issue(0, 0, d0);
  if (nunit > 1) issue(1, 1, d1);
  int cur = 0;  // stage of unit it
  for (int it = 0; it < nunit; ++it) {
    // this unit's loads have landed; the next unit's may still be in flight
    // (loads complete in issue order)
    if (it + 1 >= nunit) wait_vm<0>();
    else if (row_block(d1) >= 0) wait_vm<kBLoads + kALoads>();
    else wait_vm<kBLoads>();
    barrier();  // ... for every wave; and the stage of unit it-1 is free
    if (it + 2 < nunit) issue(it + 2, cur == 0 ? 2 : cur - 1, d2);
    const int4 d3 = desc(it + 3);  // used two stages from now
    if (row_block(d0) >= 0) {
      const char *sb = lds + cur * kStageBytes;
      Ops ops[kSteps];
#pragma unroll
      for (int s = 0; s < kSteps; ++s) ops[s] = read_ops(sb, s);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < kSteps; ++s)
#pragma unroll
        for (int cb = 0; cb < kCb; ++cb)
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
            // B is the left operand: the accumulators hold the tile transposed
            acc[rb][cb] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(ops[s].b[cb], ops[s].a[rb], acc[rb][cb], 0, 0, 0);
    }
    cur = cur == 2 ? 0 : cur + 1;
    d0 = d1;
    d1 = d2;
    d2 = d3;
  }

  barrier();  // every wave is done reading the ring
  char *ct = lds + wave * 64 * kPitch;
  stage_c<kCb, kPitch>(ct, acc, lane);
  __builtin_amdgcn_wave_barrier();
  if (br >= 0) store_c<kCb, kPitch>(ct, lane, static_cast<int64_t>(br) * kBlk, n0 + cw * kWC, n, c_rows, C, ldc);
}

}  // namespace

void bcsr_fragment_order(const uint16_t *blk, uint16_t *frag) {
  for (int rb = 0; rb < 2; ++rb)
    for (int s = 0; s < 4; ++s)
      for (int l = 0; l < 64; ++l)
        for (int i = 0; i < 8; ++i)
          frag[((rb * 4 + s) * 64 + l) * 8 + i] =
              blk[(32 * rb + (l & 31)) * kBlk + 16 * s + 8 * (l >> 5) + i];
}

BcsrSchedule bcsr_schedule(const int32_t *row_ptr, int32_t mb, int64_t n) {
  BcsrSchedule sc;
  // Wider tiles re-read each A block fewer times (once per tn columns); for
  // small n the narrower tile gives more workgroups to fill the CUs.
  sc.tn = n >= 8192 ? 512 : 256;
  sc.row_groups = 1;
  // Row groups when A would otherwise be walked from beyond L2 again for
  // every N tile of an XCD (A larger than half an XCD's 4 MB L2) while an
  // eighth of it fits in that half, and every group still has enough block
  // rows to fill an XCD's CUs.  The N tile is then 256 wide: its B slab
  // shares L2 with the group's A, and two workgroups fit in a CU.  Four
  // groups, each served by two XCDs over half of the N tiles each, measured
  // slightly faster than eight (a quarter of A per XCD, but half as many N
  // tiles in flight per group).  A larger A does not stay resident either
  // way, and the split only costs B reuse.
  const int64_t a_bytes = static_cast<int64_t>(row_ptr[mb]) * kABytes, half_l2 = 2 << 20;
  if (n >= 8192 && a_bytes > half_l2 && a_bytes <= 8 * half_l2 && mb >= 8 * 32) {
    sc.row_groups = 4;
    sc.tn = 256;
  }
  // Half-block stages at 256 columns when block rows hold few blocks (at
  // most 16 on average): a 20 KB stage lets a third workgroup onto the CU.
  // Rows of many blocks keep whole-block stages: there a barrier per 8
  // MFMAs costs more than the extra workgroup gains.
  sc.kh = (sc.tn == 256 && row_ptr[mb] <= 16 * static_cast<int64_t>(mb)) ? 32 : 64;
  return sc;
}

int64_t bcsr_grid(const int32_t *row_seg, const BcsrSchedule &sc, int64_t n) {
  const int64_t ntn = (n + sc.tn - 1) / sc.tn, parts = 8 / sc.row_groups;
  int64_t per = 0;
  for (int g = 0; g < sc.row_groups; ++g)
    per = std::max(per, ((row_seg[g + 1] - row_seg[g]) * ntn + parts - 1) / parts);
  return 8 * per;
}

double bcsr_pairing(const int32_t *row_ptr, const int32_t *col_idx, int32_t mb, int32_t kb,
                    vec<int32_t> &pair_rows, vec<int32_t> &pair_ptr, vec<int32_t> &units) {
  pair_rows.clear();
  pair_ptr.assign(1, 0);
  units.clear();
  const int64_t nnzb = row_ptr[mb];
  // block rows of each block column, ascending
  vec<int32_t> cptr(static_cast<size_t>(kb) + 1, 0), crows(static_cast<size_t>(nnzb));
  for (int64_t q = 0; q < nnzb; ++q) ++cptr[col_idx[q] + 1];
  // the search below visits, for every block, the rows of its block column:
  // the sum of the squared column counts; past kBcsrPairMaxWork the plan
  // would take too long, and the rows are not paired
  double visits = 0.0;
  for (int32_t c = 0; c < kb; ++c) visits += static_cast<double>(cptr[c + 1]) * cptr[c + 1];
  if (visits > kBcsrPairMaxWork) return 0.0;
  for (int32_t c = 0; c < kb; ++c) cptr[c + 1] += cptr[c];
  {
    vec<int32_t> fill(cptr.begin(), cptr.end() - 1);
    for (int32_t r = 0; r < mb; ++r)
      for (int32_t q = row_ptr[r]; q < row_ptr[r + 1]; ++q) crows[fill[col_idx[q]]++] = r;
  }
  auto blocks = [&](int32_t r) { return row_ptr[r + 1] - row_ptr[r]; };
  vec<int32_t> order(static_cast<size_t>(mb));
  for (int32_t i = 0; i < mb; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(),
                   [&](int32_t x, int32_t y) { return blocks(x) > blocks(y); });
  vec<char> used(static_cast<size_t>(mb), 0);
  vec<int32_t> shared(static_cast<size_t>(mb), 0), touched;
  size_t next = 0;  // first row of `order` that may still be unpaired
  for (int32_t r : order) {
    if (used[r]) continue;
    used[r] = 1;
    touched.clear();
    for (int32_t q = row_ptr[r]; q < row_ptr[r + 1]; ++q)
      for (int32_t i = cptr[col_idx[q]]; i < cptr[col_idx[q] + 1]; ++i)
        if (!used[crows[i]] && shared[crows[i]]++ == 0) touched.push_back(crows[i]);
    int32_t best = -1, best_shared = 0;
    for (int32_t s2 : touched) {
      if (shared[s2] > best_shared || (shared[s2] == best_shared && s2 < best)) {
        best = s2;
        best_shared = shared[s2];
      }
      shared[s2] = 0;
    }
    if (best < 0) {  // no unpaired row shares a column: take the longest one left
      while (next < order.size() && used[order[next]]) ++next;
      if (next < order.size()) best = order[next];
    }
    if (best >= 0) used[best] = 1;
    pair_rows.push_back(r);
    pair_rows.push_back(best);
    // the union of the two rows' block columns, ascending
    int32_t q0 = row_ptr[r], e0 = row_ptr[r + 1];
    int32_t q1 = best >= 0 ? row_ptr[best] : 0, e1 = best >= 0 ? row_ptr[best + 1] : 0;
    while (q0 < e0 || q1 < e1) {
      const int32_t c0 = q0 < e0 ? col_idx[q0] : INT32_MAX, c1 = q1 < e1 ? col_idx[q1] : INT32_MAX;
      const int32_t c = std::min(c0, c1);
      units.push_back(c);
      units.push_back(c0 == c ? q0++ : -1);
      units.push_back(c1 == c ? q1++ : -1);
      units.push_back(0);
    }
    pair_ptr.push_back(static_cast<int32_t>(units.size() / 4));
    if (pair_ptr.back() - pair_ptr[pair_ptr.size() - 2] > kBcsrPairMaxUnits) return 0.0;
  }
  const double stored = static_cast<double>(units.size() / 4);
  return nnzb > 0 ? 1.0 - stored / static_cast<double>(nnzb) : 0.0;
}

namespace {
template <int kTN, bool kMap, int kKH>
hipError_t launch_tn(const BcsrLaunch &a, hipStream_t s) {
  using G = Geo<kTN, kKH>;
  const int64_t ntn = (a.n + kTN - 1) / kTN;
  const int64_t tiles = static_cast<int64_t>(a.mb) * ntn;
  if (tiles == 0) return hipSuccess;
  if (tiles > INT32_MAX / 2 || a.ldb > (1 << 24)) return hipErrorInvalidValue;
  if (a.row_groups < 1 || a.row_groups > 8 || 8 % a.row_groups != 0) return hipErrorInvalidValue;
  // through the row map every B byte offset is a 32-bit offset from B
  if (kMap && a.k_rows * a.ldb * 2 > UINT32_MAX) return hipErrorInvalidValue;
  auto kernel = bcsr_bf16_mfma<kTN, kMap, kKH>;
  hipError_t e = allow_dynamic_lds(reinterpret_cast<const void *>(kernel), G::kLdsBytes);
  if (e != hipSuccess) return e;
  if (a.grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(a.grid)), dim3(G::kThreads),
                     G::kLdsBytes, s, a.row_ptr, a.col_idx, a.frag, a.row_order, a.row_seg,
                     a.row_groups, static_cast<int32_t>(ntn), a.n, a.B, a.ldb, a.C, a.ldc, a.c_rows,
                     a.col_perm);
  return hipGetLastError();
}

template <int kWC>
hipError_t launch_pair(const BcsrLaunch &a, hipStream_t s) {
  using G = PairGeo<kWC>;
  if (a.tn != G::kTN || a.kh != G::kKH || a.col_perm) return hipErrorInvalidValue;
  const int64_t ntn = (a.n + G::kTN - 1) / G::kTN;
  const int64_t tiles = static_cast<int64_t>(a.npairs) * ntn;
  if (tiles == 0) return hipSuccess;
  if (tiles > INT32_MAX / 2 || a.ldb > (1 << 24)) return hipErrorInvalidValue;
  if (a.row_groups < 1 || a.row_groups > 8 || 8 % a.row_groups != 0) return hipErrorInvalidValue;
  auto kernel = bcsr_bf16_pair<kWC>;
  hipError_t e = allow_dynamic_lds(reinterpret_cast<const void *>(kernel), G::kLdsBytes);
  if (e != hipSuccess) return e;
  if (a.grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(a.grid)), dim3(G::kThreads),
                     G::kLdsBytes, s, a.units, a.pair_ptr, a.pair_rows, a.frag, a.row_order,
                     a.row_seg, a.row_groups, static_cast<int32_t>(ntn), a.n, a.B, a.ldb, a.C,
                     a.ldc, a.c_rows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bcsr_bf16(const BcsrLaunch &a, hipStream_t s) {
  if (a.paired) return launch_pair<kPairWaveCols>(a, s);
  if (a.tn != 256 && a.tn != 512) return hipErrorInvalidValue;
  if (a.kh != 64 && (a.kh != 32 || a.tn != 256)) return hipErrorInvalidValue;
  const bool wide = a.tn == 512;
  if (a.col_perm) {
    if (wide) return launch_tn<512, true, 64>(a, s);
    return a.kh == 32 ? launch_tn<256, true, 32>(a, s) : launch_tn<256, true, 64>(a, s);
  }
  if (wide) return launch_tn<512, false, 64>(a, s);
  return a.kh == 32 ? launch_tn<256, false, 32>(a, s) : launch_tn<256, false, 64>(a, s);
}

}  // namespace sdm

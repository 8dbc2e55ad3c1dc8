// bcsr_bf16.hip -- C = A * B with A in BCSR (64 x 64 bf16 blocks), B and C
// dense row-major bf16, fp32 accumulation, round-to-nearest-even output.
//
// Block-structured SpMM of the AsyncSparse page (abstract; Figure 2 caption):
// only the stored blocks of a block row are multiplied.  Design for gfx950:
//   - one workgroup (4 waves) owns a 64-row block row and a 256-column tile
//     of C; each wave owns 64 x 64 of it as 2 x 2 MFMA 32x32x16 bf16 tiles;
//   - per stored block the B slab (64 k-rows x 256 columns) and the A block
//     (8 KB, pre-arranged in MFMA fragment order by the plan) are staged in
//     LDS; the next block's loads are issued to registers before the current
//     block's MFMAs (software pipelining instead of the pages' TMA producer
//     warps);
//   - B is row-major (n contiguous) but the MFMA wants k contiguous per lane:
//     the gfx950 LDS transpose read (ds_read_b64_tr_b16) delivers 4 k-values
//     of one column per lane, two reads per operand;
//   - workgroups are mapped so that each XCD walks contiguous tiles, block
//     rows fastest: the workgroups resident on one XCD share the B column
//     slab of one N tile in that XCD's L2.
#include "internal.h"

namespace sdm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kBlk = 64;                        // block edge
constexpr int kTN = 256;                        // C columns per workgroup
constexpr int kThreads = 256;                   // 4 waves
constexpr int kBPitch = kTN * 2 + 64;           // bytes per k-row of the LDS B slab
constexpr int kBBytes = kBlk * kBPitch;         // 36,864
constexpr int kABytes = kBlk * kBlk * 2;        // 8,192
constexpr int kBPieces = kBlk * kTN * 2 / 16 / kThreads;  // 16-byte pieces per thread: 8
constexpr int kAPieces = kABytes / 16 / kThreads;        // 2

__device__ __forceinline__ unsigned short to_bf16_rne(float f) {
  // float -> bf16 conversion rounds to nearest even (v_cvt_pk_bf16_f32)
  return __builtin_bit_cast(unsigned short, static_cast<__bf16>(f));
}

__global__ __launch_bounds__(kThreads) void bcsr_bf16_mfma(
    const int32_t *__restrict__ row_ptr, const int32_t *__restrict__ col_idx,
    const uint4 *__restrict__ frag, int32_t mb, int32_t tiles, int32_t per_xcd, int64_t n,
    const uint16_t *__restrict__ B, int64_t ldb, uint16_t *__restrict__ C, int64_t ldc) {
  __shared__ __attribute__((aligned(16))) char lds[kBBytes + kABytes];

  // XCD-aware tile order: workgroup b runs on XCD b % 8; give each XCD a
  // contiguous range of logical tiles, block rows fastest.
  const int bid = blockIdx.x;
  const int t = (bid & 7) * per_xcd + (bid >> 3);
  if (t >= tiles) return;
  const int br = t % mb;
  const int64_t n0 = static_cast<int64_t>(t / mb) * kTN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int p0 = row_ptr[br], p1 = row_ptr[br + 1];

  // global -> register staging: piece q = tid + 256 j of the B slab is row
  // q / 32, 16-byte column piece q % 32 (32 threads cover a 512-byte row)
  uint4 breg[kBPieces];
  uint4 areg[kAPieces];
  auto load_block = [&](int p) {
    const int64_t kb = static_cast<int64_t>(col_idx[p]) * kBlk;
    const uint16_t *src = B + kb * ldb + n0;
#pragma unroll
    for (int j = 0; j < kBPieces; ++j) {
      const int q = tid + kThreads * j;
      const int row = q >> 5, cp = q & 31;
      if (n0 + cp * 8 < n)
        breg[j] = *reinterpret_cast<const uint4 *>(src + row * ldb + cp * 8);
      else
        breg[j] = make_uint4(0, 0, 0, 0);
    }
    const uint4 *asrc = frag + static_cast<int64_t>(p) * (kABytes / 16);
#pragma unroll
    for (int j = 0; j < kAPieces; ++j) areg[j] = asrc[tid + kThreads * j];
  };
  auto store_block = [&]() {
#pragma unroll
    for (int j = 0; j < kBPieces; ++j) {
      const int q = tid + kThreads * j;
      *reinterpret_cast<uint4 *>(lds + (q >> 5) * kBPitch + (q & 31) * 16) = breg[j];
    }
    uint4 *al = reinterpret_cast<uint4 *>(lds + kBBytes);
#pragma unroll
    for (int j = 0; j < kAPieces; ++j) al[tid + kThreads * j] = areg[j];
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // transpose-read addressing: within a 16-lane group, lane p supplies the
  // 4 columns 4*(p%4).. of k-row p/4; lane i then holds k-rows 0..3 of
  // column i.  Lanes 32..63 take k-rows 8..15 of the 16-row step.
  const int g = lane >> 5;
  const int pl = lane & 15;
  const int tr_row = 8 * g + (pl >> 2);
  const int tr_col = wave * 64 + ((lane >> 4) & 1) * 16 + 4 * (pl & 3);

  if (p0 < p1) {
    load_block(p0);
    store_block();
  }
  __syncthreads();
  for (int p = p0; p < p1; ++p) {
    if (p + 1 < p1) load_block(p + 1);
    const bf16x8 *afr = reinterpret_cast<const bf16x8 *>(lds + kBBytes);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 af[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) af[rb] = afr[(rb * 4 + s) * 64 + lane];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const char *base = lds + (16 * s + tr_row) * kBPitch + (tr_col + 32 * cb) * 2;
        s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(base));
        s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(base + 4 * kBPitch));
        s16x8 bs;
        bs[0] = lo[0]; bs[1] = lo[1]; bs[2] = lo[2]; bs[3] = lo[3];
        bs[4] = hi[0]; bs[5] = hi[1]; bs[6] = hi[2]; bs[7] = hi[3];
        const bf16x8 bfr = __builtin_bit_cast(bf16x8, bs);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[rb], bfr, acc[rb][cb], 0, 0, 0);
      }
    }
    __syncthreads();
    if (p + 1 < p1) store_block();
    __syncthreads();
  }

  // epilogue: accumulator element r of lane l is row 8*(r/4) + 4*(l/32) + r%4,
  // column l%32 of its 32 x 32 tile
  const int64_t row0 = static_cast<int64_t>(br) * kBlk;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int64_t col = n0 + wave * 64 + cb * 32 + (lane & 31);
      if (col < n) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = row0 + rb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          C[row * ldc + col] = to_bf16_rne(acc[rb][cb][r]);
        }
      }
    }
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

int bcsr_tile_n() { return kTN; }

int64_t bcsr_grid(int32_t mb, int64_t n) {
  const int64_t tiles = static_cast<int64_t>(mb) * ((n + kTN - 1) / kTN);
  return 8 * ((tiles + 7) / 8);
}

hipError_t launch_bcsr_bf16(const BcsrLaunch &a, hipStream_t s) {
  const int64_t ntn = (a.n + kTN - 1) / kTN;
  const int64_t tiles = static_cast<int64_t>(a.mb) * ntn;
  if (tiles == 0) return hipSuccess;
  if (tiles > INT32_MAX / 2) return hipErrorInvalidValue;
  const int64_t per_xcd = (tiles + 7) / 8;
  hipLaunchKernelGGL(bcsr_bf16_mfma, dim3(static_cast<unsigned>(8 * per_xcd)), dim3(kThreads), 0, s,
                     a.row_ptr, a.col_idx, reinterpret_cast<const uint4 *>(a.frag), a.mb,
                     static_cast<int32_t>(tiles), static_cast<int32_t>(per_xcd), a.n, a.B, a.ldb,
                     a.C, a.ldc);
  return hipGetLastError();
}

}  // namespace sdm

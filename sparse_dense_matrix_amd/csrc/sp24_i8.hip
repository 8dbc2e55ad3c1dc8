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
// One workgroup (4 waves, 2 x 2) computes a 128 x 128 tile of C; k advances
// 128 dense columns per step with register prefetch of the next step.
#include "internal.h"

namespace sdm {
namespace {

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr int kTM = 128, kTN = 128, kTK = 128;  // dense k per step
constexpr int kThreads = 256;
constexpr int kBPitch = kTN + 16;               // bytes per k-row of the LDS B slab
constexpr int kBBytes = kTK * kBPitch;          // 18,432
constexpr int kABytes = kTM * kTK / 2;          // 8,192 compressed values
constexpr int kMBytes = kTM * kTK / 8;          // 2,048 metadata
constexpr int kAPieces = kABytes / 16 / kThreads;   // 2
constexpr int kBPieces = kTK * kTN / 16 / kThreads; // 4

__global__ __launch_bounds__(kThreads) void sp24_i8_smfmac(
    const int8_t *__restrict__ vals, const uint8_t *__restrict__ meta, int64_t m, int64_t k,
    int64_t n, int64_t k_pad, int32_t mtiles, int32_t tiles, int32_t per_xcd,
    const int8_t *__restrict__ B, int64_t ldb, int32_t *__restrict__ C, int64_t ldc) {
  __shared__ __attribute__((aligned(16))) char lds[kBBytes + kABytes + kMBytes];
  char *const lds_b = lds;
  char *const lds_a = lds + kBBytes;
  char *const lds_m = lds + kBBytes + kABytes;

  const int bid = blockIdx.x;
  const int t = (bid & 7) * per_xcd + (bid >> 3);
  if (t >= tiles) return;
  const int64_t m0 = static_cast<int64_t>(t % mtiles) * kTM;
  const int64_t n0 = static_cast<int64_t>(t / mtiles) * kTN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t arow_bytes = k_pad / 2, mrow_bytes = k_pad / 8;

  uint4 areg[kAPieces], breg[kBPieces], mreg;
  auto load_step = [&](int64_t ks) {
    // A: piece q -> row q/4, 16-byte piece q%4 (= lane group) of the row's 64
#pragma unroll
    for (int j = 0; j < kAPieces; ++j) {
      const int q = tid + kThreads * j;
      areg[j] = *reinterpret_cast<const uint4 *>(vals + (m0 + (q >> 2)) * arow_bytes +
                                                 ks * (kTK / 2) + (q & 3) * 16);
    }
    if (tid < kTM)
      mreg = *reinterpret_cast<const uint4 *>(meta + (m0 + tid) * mrow_bytes + ks * (kTK / 8));
    // B: piece q -> k-row q/8, 16-byte column piece q%8
#pragma unroll
    for (int j = 0; j < kBPieces; ++j) {
      const int q = tid + kThreads * j;
      const int64_t kr = ks * kTK + (q >> 3);
      const int64_t cc = n0 + (q & 7) * 16;
      if (kr < k && cc < n)
        breg[j] = *reinterpret_cast<const uint4 *>(B + kr * ldb + cc);
      else
        breg[j] = make_uint4(0, 0, 0, 0);
    }
  };
  auto store_step = [&]() {
#pragma unroll
    for (int j = 0; j < kAPieces; ++j) {
      const int q = tid + kThreads * j;
      const int r = q >> 2, g = q & 3;
      *reinterpret_cast<uint4 *>(lds_a + ((r >> 4) * 64 + g * 16 + (r & 15)) * 16) = areg[j];
    }
    if (tid < kTM) {
      const int r = tid;
      uint32_t *ml = reinterpret_cast<uint32_t *>(lds_m);
      const int base = (r >> 4) * 64 + (r & 15);
      ml[base + 0] = mreg.x;
      ml[base + 16] = mreg.y;
      ml[base + 32] = mreg.z;
      ml[base + 48] = mreg.w;
    }
#pragma unroll
    for (int j = 0; j < kBPieces; ++j) {
      const int q = tid + kThreads * j;
      *reinterpret_cast<uint4 *>(lds_b + (q >> 3) * kBPitch + (q & 7) * 16) = breg[j];
    }
  };

  i32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = i32x4{0, 0, 0, 0};

  // transpose-read addressing: in a 16-lane group, lane p supplies 8 columns
  // 8*(p%2).. of k-row p/2; lane i then holds k-rows 0..7 of column i.
  const int g = lane >> 4;
  const int pl = lane & 15;
  const int tr_row = 16 * g + (pl >> 1);
  const int tr_col = wn * 64 + 8 * (pl & 1);

  const int64_t ksteps = k_pad / kTK;
  load_step(0);
  store_step();
  __syncthreads();
  for (int64_t ks = 0; ks < ksteps; ++ks) {
    if (ks + 1 < ksteps) load_step(ks + 1);
    i32x8 bop[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const char *base = lds_b + tr_row * kBPitch + tr_col + 16 * j;
      const i32x2 q0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2 *)(base));
      const i32x2 q1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2 *)(base + 8 * kBPitch));
      const i32x2 q2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2 *)(base + 64 * kBPitch));
      const i32x2 q3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2 *)(base + 72 * kBPitch));
      bop[j] = i32x8{q0[0], q0[1], q1[0], q1[1], q2[0], q2[1], q3[0], q3[1]};
    }
    const i32x4 *afr = reinterpret_cast<const i32x4 *>(lds_a);
    const int *mfr = reinterpret_cast<const int *>(lds_m);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int mt = wm * 4 + i;
      const i32x4 aop = afr[mt * 64 + lane];
      const int idx = mfr[mt * 64 + lane];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_smfmac_i32_16x16x128_i8(aop, bop[j], acc[i][j], idx, 0, 0);
    }
    __syncthreads();
    if (ks + 1 < ksteps) store_step();
    __syncthreads();
  }

  // D element r of lane l: row 4*(l/16) + r, column l%16 of the 16 x 16 tile
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = n0 + wn * 64 + 16 * j + (lane & 15);
      if (col >= n) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = m0 + wm * 64 + 16 * i + 4 * g + r;
        if (row < m) C[row * ldc + col] = acc[i][j][r];
      }
    }
}

}  // namespace

int sp24_tile_m() { return kTM; }
int sp24_tile_n() { return kTN; }
int sp24_tile_k() { return kTK; }

int64_t sp24_grid(int64_t m, int64_t n) {
  const int64_t tiles = ((m + kTM - 1) / kTM) * ((n + kTN - 1) / kTN);
  return 8 * ((tiles + 7) / 8);
}

hipError_t launch_sp24_i8(const Sp24Launch &a, hipStream_t s) {
  const int64_t mtiles = (a.m + kTM - 1) / kTM;
  const int64_t tiles = mtiles * ((a.n + kTN - 1) / kTN);
  if (tiles == 0) return hipSuccess;
  if (tiles > INT32_MAX / 2) return hipErrorInvalidValue;
  const int64_t per_xcd = (tiles + 7) / 8;
  hipLaunchKernelGGL(sp24_i8_smfmac, dim3(static_cast<unsigned>(8 * per_xcd)), dim3(kThreads), 0, s,
                     a.vals, a.meta, a.m, a.k, a.n, a.k_pad, static_cast<int32_t>(mtiles),
                     static_cast<int32_t>(tiles), static_cast<int32_t>(per_xcd), a.B, a.ldb, a.C,
                     a.ldc);
  return hipGetLastError();
}

}  // namespace sdm

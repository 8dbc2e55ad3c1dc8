// gather.hip -- dst row j = src row map[j], 16-byte pieces.
//
// Used where a packed operand's inner dimension is not B's row order: the
// row/column-permuted BCSR (B's rows in the packed column order) and the
// sliding-window 2:4 decomposition of (2N-2):2N weights (B's rows repeated
// as the overlapping windows need them).
#include "internal.h"

namespace sdm {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// one workgroup per destination row
__global__ __launch_bounds__(256) void gather_rows(const char *__restrict__ src, int64_t ld_bytes,
                                                   const int32_t *__restrict__ map,
                                                   int64_t row_bytes, char *__restrict__ dst,
                                                   int64_t dst_ld_bytes) {
  const int64_t j = blockIdx.x;
  const u32x4 *s = reinterpret_cast<const u32x4 *>(src + static_cast<int64_t>(map[j]) * ld_bytes);
  u32x4 *d = reinterpret_cast<u32x4 *>(dst + j * dst_ld_bytes);
  for (int64_t c = threadIdx.x; c < row_bytes / 16; c += 256) d[c] = s[c];
}

}  // namespace

hipError_t launch_gather_rows(const void *src, int64_t ld_bytes, const int32_t *map, int64_t rows,
                              int64_t row_bytes, void *dst, int64_t dst_ld_bytes, hipStream_t s) {
  if (rows <= 0 || row_bytes <= 0) return hipSuccess;
  if (rows > 0x7fffffff || row_bytes % 16 != 0 || ld_bytes % 16 != 0 || dst_ld_bytes % 16 != 0)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(gather_rows, dim3(static_cast<unsigned>(rows)), dim3(256), 0, s,
                     static_cast<const char *>(src), ld_bytes, map, row_bytes,
                     static_cast<char *>(dst), dst_ld_bytes);
  return hipGetLastError();
}

}  // namespace sdm

// Five trits per byte (gfx950).
//
// "ultragraph-1bit 0.12.0" README, sections "A whole ternary GPT" (the
// deployed checkpoint stores 5 ternary values per byte, ~1.6 bits/weight)
// and "Layout" (pack.py).  3^5 = 243 <= 256, so a byte holds five trits as
// the base-3 number with digits t_j + 1:  code = 121 + sum_j t_j 3^j, t_0 at
// the lowest K position of the group.
//
// Integer-only and HBM-bound (6 B moved per 5 trits).  Bad-input counts are
// reduced per wave and added with one integer atomic per wave.
#include "ug_internal.h"

namespace ug {
namespace {

__device__ inline void count_bad(int bad, int32_t *counter) {
  if (!counter) return;
  const int tot = wave_sum_i32(bad);
  if ((threadIdx.x & 63) == 0 && tot) atomicAdd(counter, tot);
}

// One thread per output byte (row r, byte g), g in [0, ldp).
__global__ __launch_bounds__(256) void pack_kernel(const int8_t *__restrict__ wq, int64_t ldq,
                                                   int64_t N, int64_t K,
                                                   uint8_t *__restrict__ packed, int64_t ldp,
                                                   int32_t *bad_count) {
  const int64_t groups = (K + 4) / 5;
  const int64_t total = N * ldp;
  int bad = 0;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * 256) {
    const int64_t r = idx / ldp;
    const int64_t g = idx - r * ldp;
    int code = 121;
    if (g < groups) {
      const int8_t *src = wq + r * ldq + 5 * g;
      int p3 = 1;
#pragma unroll
      for (int j = 0; j < 5; ++j) {
        int t = 0;
        if (5 * g + j < K) {
          t = src[j];
          if (t < -1 || t > 1) {
            ++bad;
            t = t < -1 ? -1 : 1;
          }
        }
        code += t * p3;
        p3 *= 3;
      }
    }
    packed[idx] = (uint8_t)code;  // idx = r * ldp + g
  }
  count_bad(bad, bad_count);
}

// One thread per group (row r, byte g < ceil(K/5)): writes up to 5 trits.
__global__ __launch_bounds__(256) void unpack_kernel(const uint8_t *__restrict__ packed,
                                                     int64_t ldp, int64_t N, int64_t K,
                                                     int8_t *__restrict__ wq, int64_t ldq,
                                                     int32_t *bad_count) {
  const int64_t groups = (K + 4) / 5;
  const int64_t total = N * groups;
  int bad = 0;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * 256) {
    const int64_t r = idx / groups;
    const int64_t g = idx - r * groups;
    int code = packed[r * ldp + g];
    if (code > 242) {
      ++bad;
      code = 121;
    }
    int8_t *dst = wq + r * ldq + 5 * g;
#pragma unroll
    for (int j = 0; j < 5; ++j) {
      const int d = code % 3;
      code /= 3;
      if (5 * g + j < K) dst[j] = (int8_t)(d - 1);
    }
  }
  count_bad(bad, bad_count);
}

int64_t grid_for(int64_t total) {
  int64_t b = ceil_div(total, 256);
  if (b > 256 * 64) b = 256 * 64;
  if (b < 1) b = 1;
  return b;
}

}  // namespace

hipError_t launch_pack(const int8_t *wq, int64_t ldq, int64_t N, int64_t K, uint8_t *packed,
                       int64_t ldp, int32_t *bad, hipStream_t st) {
  hipLaunchKernelGGL(pack_kernel, dim3(grid_for(N * ldp)), dim3(256), 0, st, wq, ldq, N, K,
                     packed, ldp, bad);
  return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t *packed, int64_t ldp, int64_t N, int64_t K, int8_t *wq,
                         int64_t ldq, int32_t *bad, hipStream_t st) {
  hipLaunchKernelGGL(unpack_kernel, dim3(grid_for(N * ceil_div(K, 5))), dim3(256), 0, st, packed,
                     ldp, N, K, wq, ldq, bad);
  return hipGetLastError();
}

}  // namespace ug

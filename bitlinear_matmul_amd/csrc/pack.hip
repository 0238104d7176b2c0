// Five trits per byte (gfx950).
//
// "ultragraph-1bit 0.12.0" README, sections "A whole ternary GPT" (the
// deployed checkpoint stores 5 ternary values per byte, ~1.6 bits/weight)
// and "Layout" (pack.py).  3^5 = 243 <= 256, so a byte holds five trits as
// the base-3 number with digits t_j + 1:  code = 121 + sum_j t_j 3^j, t_0 at
// the lowest K position of the group.
//
// Integer-only and HBM-bound (6 B moved per 5 trits): each thread moves 20
// trits with 4-byte loads and stores.  Bad-input counts are reduced per
// wave and added with one integer atomic per wave.
#include "ug_internal.h"

namespace ug {
namespace {

__device__ inline void count_bad(int bad, int32_t *counter) {
  if (!counter) return;
  const int tot = wave_sum_i32(bad);
  if ((threadIdx.x & 63) == 0 && tot) atomicAdd(counter, tot);
}

// Code of five trits t0..t4 (each clamped to [-1, 1]; an entry outside
// counts as bad).
__device__ inline uint32_t encode5(const int8_t *t, int n, int &bad) {
  uint32_t code = 121;
  int p3 = 1;
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    int v = j < n ? t[j] : 0;
    if (v < -1 || v > 1) {
      ++bad;
      v = v < -1 ? -1 : 1;
    }
    code += v * p3;
    p3 *= 3;
  }
  return code;
}

// One thread per 4 output bytes (row r, bytes 4 j .. 4 j + 3 of [0, ldp)),
// i.e. the 20 entries 20 j .. 20 j + 19 of the row: five 4-byte loads and
// one 4-byte store where all 20 lie inside the row; entry by entry at the
// row's end (entries past K are 0 trits, bytes past ceil(K/5) are 121).
// Small pieces keep many loads in flight across the CU's waves.
__global__ __launch_bounds__(256) void pack_kernel(const int8_t *__restrict__ wq, int64_t ldq,
                                                   int64_t N, int64_t K,
                                                   uint8_t *__restrict__ packed, int64_t ldp,
                                                   int32_t *bad_count) {
  const int64_t groups = (K + 4) / 5;
  const int64_t vpr = ldp / 4;  // 4-byte pieces per packed row
  const int64_t total = N * vpr;
  int bad = 0;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * 256) {
    const int64_t r = idx / vpr;
    const int64_t j = idx - r * vpr;
    const int8_t *src = wq + r * ldq + 20 * j;
    uint32_t w = 0;
    if (20 * j + 20 <= K) {
      uint32_t in[5];  // the 20 entries, four per dword (4-byte aligned)
#pragma unroll
      for (int i = 0; i < 5; ++i) in[i] = *reinterpret_cast<const uint32_t *>(src + 4 * i);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        int8_t t[5];
#pragma unroll
        for (int i = 0; i < 5; ++i) {
          const int e = 5 * b + i;  // entry e: byte e % 4 of dword e / 4
          t[i] = (int8_t)(in[e >> 2] >> (8 * (e & 3)));
        }
        w |= encode5(t, 5, bad) << (8 * b);
      }
    } else {
      for (int b = 0; b < 4; ++b) {
        const int64_t g = 4 * j + b;
        uint32_t code = 121;
        if (g < groups) {
          int8_t t[5];
          const int n = (int)min((int64_t)5, K - 5 * g);
          for (int i = 0; i < n; ++i) t[i] = src[5 * b + i];
          code = encode5(t, n, bad);
        }
        w |= code << (8 * b);
      }
    }
    *reinterpret_cast<uint32_t *>(packed + r * ldp + 4 * j) = w;
  }
  count_bad(bad, bad_count);
}

// One thread per 4 packed bytes of a row (groups 4 j .. 4 j + 3 below
// ceil(K/5)): one 4-byte load and five 4-byte stores where all 20 trits lie
// inside the row; byte by byte at the row's end (pad bytes not read).
__global__ __launch_bounds__(256) void unpack_kernel(const uint8_t *__restrict__ packed,
                                                     int64_t ldp, int64_t N, int64_t K,
                                                     int8_t *__restrict__ wq, int64_t ldq,
                                                     int32_t *bad_count) {
  const int64_t groups = (K + 4) / 5;
  const int64_t vpr = (groups + 3) / 4;
  const int64_t total = N * vpr;
  int bad = 0;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * 256) {
    const int64_t r = idx / vpr;
    const int64_t j = idx - r * vpr;
    const uint8_t *src = packed + r * ldp + 4 * j;
    int8_t *dst = wq + r * ldq + 20 * j;
    auto decode = [&](uint32_t code, int8_t *t) __attribute__((always_inline)) {
      if (code > 242) {
        ++bad;
        code = 121;
      }
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        t[i] = (int8_t)((int)(code % 3) - 1);
        code /= 3;
      }
    };
    if (20 * j + 20 <= K) {
      const uint32_t c = *reinterpret_cast<const uint32_t *>(src);
      int8_t out[20];
#pragma unroll
      for (int b = 0; b < 4; ++b) decode((c >> (8 * b)) & 0xff, out + 5 * b);
#pragma unroll
      for (int i = 0; i < 5; ++i)
        *reinterpret_cast<uint32_t *>(dst + 4 * i) = *reinterpret_cast<const uint32_t *>(out + 4 * i);
    } else {
      for (int b = 0; b < 4; ++b) {
        const int64_t g = 4 * j + b;
        if (g >= groups) break;
        int8_t t[5];
        decode(src[b], t);
        for (int i = 0; i < 5; ++i)
          if (5 * g + i < K) dst[5 * b + i] = t[i];
      }
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
  hipLaunchKernelGGL(pack_kernel, dim3(grid_for(N * (ldp / 4))), dim3(256), 0, st, wq, ldq, N,
                     K, packed, ldp, bad);
  return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t *packed, int64_t ldp, int64_t N, int64_t K, int8_t *wq,
                         int64_t ldq, int32_t *bad, hipStream_t st) {
  hipLaunchKernelGGL(unpack_kernel, dim3(grid_for(N * ceil_div(ceil_div(K, 5), 4))), dim3(256), 0,
                     st, packed, ldp, N, K, wq, ldq, bad);
  return hipGetLastError();
}

}  // namespace ug

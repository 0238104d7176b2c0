// Five trits per byte (gfx950).
//
// "ultragraph-1bit 0.12.0" README, sections "A whole ternary GPT" (the
// deployed checkpoint stores 5 ternary values per byte, ~1.6 bits/weight)
// and "Layout" (pack.py).  3^5 = 243 <= 256, so a byte holds five trits as
// the base-3 number with digits t_j + 1:  code = 121 + sum_j t_j 3^j, t_0 at
// the lowest K position of the group.
//
// Integer-only and HBM-bound (6 B moved per 5 trits): each thread moves 80
// trits with 16-byte loads and stores.  Bad-input counts are reduced per
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

// One thread per 16 output bytes (row r, bytes 16 j .. 16 j + 15 of
// [0, ldp)), i.e. the 80 entries 80 j .. 80 j + 79 of the row: five 16-byte
// loads and one 16-byte store where all 80 lie inside the row; entry by
// entry at the row's end (entries past K are 0 trits, bytes past ceil(K/5)
// are 121).
__global__ __launch_bounds__(256) void pack_kernel(const int8_t *__restrict__ wq, int64_t ldq,
                                                   int64_t N, int64_t K,
                                                   uint8_t *__restrict__ packed, int64_t ldp,
                                                   int32_t *bad_count) {
  const int64_t groups = (K + 4) / 5;
  const int64_t vpr = ldp / 16;  // 16-byte pieces per packed row
  const int64_t total = N * vpr;
  int bad = 0;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * 256) {
    const int64_t r = idx / vpr;
    const int64_t j = idx - r * vpr;
    const int8_t *src = wq + r * ldq + 80 * j;
    uint32_t w[4];
    if (80 * j + 80 <= K) {
      uint32_t in[20];  // the 80 entries, four per dword
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        const uint4 v = *reinterpret_cast<const uint4 *>(src + 16 * i);
        in[4 * i] = v.x;
        in[4 * i + 1] = v.y;
        in[4 * i + 2] = v.z;
        in[4 * i + 3] = v.w;
      }
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        w[d] = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          int8_t t[5];
#pragma unroll
          for (int i = 0; i < 5; ++i) {
            const int e = 5 * (4 * d + b) + i;  // entry e: byte e % 4 of dword e / 4
            t[i] = (int8_t)(in[e >> 2] >> (8 * (e & 3)));
          }
          w[d] |= encode5(t, 5, bad) << (8 * b);
        }
      }
    } else {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        w[d] = 0;
        for (int b = 0; b < 4; ++b) {
          const int64_t g = 16 * j + 4 * d + b;
          uint32_t code = 121;
          if (g < groups) {
            int8_t t[5];
            const int n = (int)min((int64_t)5, K - 5 * g);
            for (int i = 0; i < n; ++i) t[i] = wq[r * ldq + 5 * g + i];
            code = encode5(t, n, bad);
          }
          w[d] |= code << (8 * b);
        }
      }
    }
    *reinterpret_cast<uint4 *>(packed + r * ldp + 16 * j) = make_uint4(w[0], w[1], w[2], w[3]);
  }
  count_bad(bad, bad_count);
}

// One thread per 16 packed bytes of a row (groups 16 j .. 16 j + 15 below
// ceil(K/5)): one 16-byte load and five 16-byte stores where all 80 trits
// lie inside the row; byte by byte at the row's end (pad bytes not read).
__global__ __launch_bounds__(256) void unpack_kernel(const uint8_t *__restrict__ packed,
                                                     int64_t ldp, int64_t N, int64_t K,
                                                     int8_t *__restrict__ wq, int64_t ldq,
                                                     int32_t *bad_count) {
  const int64_t groups = (K + 4) / 5;
  const int64_t vpr = (groups + 15) / 16;
  const int64_t total = N * vpr;
  int bad = 0;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * 256) {
    const int64_t r = idx / vpr;
    const int64_t j = idx - r * vpr;
    const uint8_t *src = packed + r * ldp + 16 * j;
    int8_t *dst = wq + r * ldq + 80 * j;
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
    if (80 * j + 80 <= K) {
      const uint4 v = *reinterpret_cast<const uint4 *>(src);
      const uint32_t c[4] = {v.x, v.y, v.z, v.w};
      int8_t out[80];
#pragma unroll
      for (int b = 0; b < 16; ++b) decode((c[b >> 2] >> (8 * (b & 3))) & 0xff, out + 5 * b);
#pragma unroll
      for (int i = 0; i < 5; ++i)
        *reinterpret_cast<uint4 *>(dst + 16 * i) = *reinterpret_cast<const uint4 *>(out + 16 * i);
    } else {
      for (int b = 0; b < 16; ++b) {
        const int64_t g = 16 * j + b;
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
  hipLaunchKernelGGL(pack_kernel, dim3(grid_for(N * (ldp / 16))), dim3(256), 0, st, wq, ldq, N,
                     K, packed, ldp, bad);
  return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t *packed, int64_t ldp, int64_t N, int64_t K, int8_t *wq,
                         int64_t ldq, int32_t *bad, hipStream_t st) {
  hipLaunchKernelGGL(unpack_kernel, dim3(grid_for(N * ceil_div(ceil_div(K, 5), 16))), dim3(256), 0,
                     st, packed, ldp, N, K, wq, ldq, bad);
  return hipGetLastError();
}

}  // namespace ug

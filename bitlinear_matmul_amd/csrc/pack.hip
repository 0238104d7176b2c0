// Five trits per byte (gfx950).
//
// "ultragraph-1bit 0.12.0" README, sections "A whole ternary GPT" (the
// deployed checkpoint stores 5 ternary values per byte, ~1.6 bits/weight)
// and "Layout" (pack.py).  3^5 = 243 <= 256, so a byte holds five trits as
// the base-3 number with digits t_j + 1:  code = 121 + sum_j t_j 3^j, t_0 at
// the lowest K position of the group.
//
// Integer-only and HBM-bound (6 B moved per 5 trits): each wave moves
// spans of 2560 trits in contiguous 512-byte pieces.  Bad-input counts are
// reduced per wave and added with one integer atomic per wave.
#include "ug_internal.h"

namespace ug {
namespace {

__device__ inline void count_bad(int bad, int32_t *counter) {
  if (!counter) return;
  const int tot = wave_sum_i32(bad);
  if ((threadIdx.x & 63) == 0 && tot) atomicAdd(counter, tot);
}

// A wave moves one span of a row: kSpanIn = 2560 trit bytes, which are
// kSpanOut = 512 packed bytes.  HBM sees only contiguous 512-byte pieces
// (8 bytes per lane); the regrouping into 5-trit groups goes through the
// wave's own 2560 bytes of LDS, where lane l's 40 trits (8 groups) sit at
// bytes [40 l, 40 l + 40): 8-byte accesses 10 dwords apart, which cover all
// 64 banks in each half-wave pass.  A wave's LDS accesses complete in issue
// order, so no wait separates the writes from the reads; the empty asm
// keeps the compiler from moving them past each other.
constexpr int kSpanIn = 2560, kSpanOut = 512, kSpanWaves = 4;

__device__ inline void lds_fence() { asm volatile("" ::: "memory"); }

// Items are (row r, span c) pairs: a block's four waves take four rows of
// span blockIdx.y (strided by the grid in both directions), spans cut on
// the packed side: c covers packed bytes [512 c, 512 c + 512) of [0, ldp) and trit
// bytes [2560 c, 2560 c + 2560) of [0, K).  Trit bytes past K load as 0
// (trit 0), so every packed byte at or past ceil(K/5) comes out as 121.
__global__ __launch_bounds__(256) void pack_kernel(const int8_t *__restrict__ wq, int64_t ldq,
                                                   int64_t N, int64_t K,
                                                   uint8_t *__restrict__ packed, int64_t ldp,
                                                   int32_t *bad_count) {
  __shared__ __attribute__((aligned(16))) uint8_t stage[kSpanWaves][kSpanIn];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint8_t *buf = stage[wv];
  const int64_t spans = (ldp + kSpanOut - 1) / kSpanOut;
  int bad = 0;
  for (int64_t c = blockIdx.y; c < spans; c += gridDim.y)
  for (int64_t r = (int64_t)blockIdx.x * kSpanWaves + wv; r < N;
       r += (int64_t)gridDim.x * kSpanWaves) {
    const int8_t *src = wq + r * ldq + (int64_t)kSpanIn * c;
    const int64_t left = K - (int64_t)kSpanIn * c;  // trit bytes of the row from here
    if (left >= kSpanIn) {  // (wave-uniform) the whole span lies inside the row
      uint2 v[5];
#pragma unroll
      for (int i = 0; i < 5; ++i) v[i] = *reinterpret_cast<const uint2 *>(src + 512 * i + 8 * lane);
#pragma unroll
      for (int i = 0; i < 5; ++i) *reinterpret_cast<uint2 *>(buf + 512 * i + 8 * lane) = v[i];
    } else {
#pragma unroll 1
      for (int i = 0; i < 5; ++i) {
        const int o = 512 * i + 8 * lane;
        uint64_t w = 0;
        if (o + 8 <= left) {
          const uint2 u = *reinterpret_cast<const uint2 *>(src + o);
          w = (uint64_t)u.x | (uint64_t)u.y << 32;
        } else {
#pragma unroll 1
          for (int e = 0; e < 8 && o + e < left; ++e) w |= (uint64_t)(uint8_t)src[o + e] << (8 * e);
        }
        *reinterpret_cast<uint2 *>(buf + o) = make_uint2((uint32_t)w, (uint32_t)(w >> 32));
      }
    }
    lds_fence();
    uint32_t d[10];
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const uint2 v = *reinterpret_cast<const uint2 *>(buf + 40 * lane + 8 * i);
      d[2 * i] = v.x;
      d[2 * i + 1] = v.y;
    }
    lds_fence();
    // Digits: u = (byte + 1) mod 256 per byte (2, 1, 0 for trits 1, 0, -1).
    // A byte is a trit iff its u is 0, 1 or 2: no bit above the lowest two
    // set and not both of those; clamping and counting are needed only
    // where some byte of the lane's 40 is not.
    uint32_t u[10], odd = 0;
#pragma unroll
    for (int i = 0; i < 10; ++i) {
      u[i] = ((d[i] & 0x7f7f7f7fu) + 0x01010101u) ^ (d[i] & 0x80808080u);
      odd |= (u[i] & 0xfcfcfcfcu) | (u[i] & (u[i] >> 1) & 0x01010101u);
    }
    if (odd) {
#pragma unroll 1
      for (int i = 0; i < 10; ++i) {
        uint32_t v = 0;
        for (int b = 0; b < 4; ++b) {
          const int x = (int8_t)(d[i] >> (8 * b)), cx = min(max(x, -1), 1);
          bad += x != cx;
          v |= (uint32_t)(cx + 1) << (8 * b);
        }
        u[i] = v;
      }
    }
    // code of group g = digits at bytes 5g .. 5g + 4: a 4-byte window
    // weighted 1, 3, 9, 27 and the fifth byte weighted 81 (two 4-way byte
    // dot products)
    uint32_t out[2] = {0u, 0u};
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const int p = 5 * g, w = p >> 2, o = p & 3, p4 = p + 4;
      const uint32_t win = o ? __builtin_amdgcn_alignbyte(u[w + 1], u[w], o) : u[w];
      uint32_t code = __builtin_amdgcn_udot4(win, 0x1b090301u, 0u, false);
      code = __builtin_amdgcn_udot4(u[p4 >> 2], 81u << (8 * (p4 & 3)), code, false);
      out[g >> 2] |= code << (8 * (g & 3));
    }
    const int64_t ob = (int64_t)kSpanOut * c + 8 * lane;
    if (ob < ldp)  // ldp is a multiple of 16: the 8 bytes fit
      *reinterpret_cast<uint2 *>(packed + r * ldp + ob) = make_uint2(out[0], out[1]);
  }
  count_bad(bad, bad_count);
}

// The same spans, cut on the packed side over the ceil(K/5) code bytes
// (pad bytes are not read; code bytes past them decode as 121, whose
// trits lie past K and are not written).  Codes decode through a 256-entry
// LDS table that the block fills once: entry c holds the five trit bytes of
// c in bytes 0..4 (five zeros and a flag at bit 48 for c > 242, which the
// lane sums to count bad codes).  Four codes are 20 trit bytes, five
// dwords, assembled from the entries by byte permutes.  Trit bytes go out
// as contiguous 8-byte pieces, byte by byte where a piece crosses K.
__global__ __launch_bounds__(256) void unpack_kernel(const uint8_t *__restrict__ packed,
                                                     int64_t ldp, int64_t N, int64_t K,
                                                     int8_t *__restrict__ wq, int64_t ldq,
                                                     int32_t *bad_count) {
  __shared__ __attribute__((aligned(16))) uint8_t stage[kSpanWaves][kSpanIn];
  __shared__ uint64_t dec[256];
  {
    uint32_t c = threadIdx.x;  // 256 threads: one entry each
    uint64_t e = 1ull << 48;
    if (c <= 242) {
      e = 0;
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        e |= (uint64_t)(uint8_t)((int)(c % 3) - 1) << (8 * i);
        c /= 3;
      }
    }
    dec[threadIdx.x] = e;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint8_t *buf = stage[wv];
  const int64_t groups = (K + 4) / 5;
  const int64_t spans = (groups + kSpanOut - 1) / kSpanOut;
  int bad = 0;
  for (int64_t c = blockIdx.y; c < spans; c += gridDim.y)
  for (int64_t r = (int64_t)blockIdx.x * kSpanWaves + wv; r < N;
       r += (int64_t)gridDim.x * kSpanWaves) {
    const int64_t pb = (int64_t)kSpanOut * c + 8 * lane;
    const uint8_t *src = packed + r * ldp + pb;
    uint64_t codes = 0x7979797979797979ull;  // 121: five 0 trits
    if (pb + 8 <= groups) {
      const uint2 v = *reinterpret_cast<const uint2 *>(src);
      codes = (uint64_t)v.x | (uint64_t)v.y << 32;
    } else if (pb < groups) {
#pragma unroll 1
      for (int e = 0; e < 8 && pb + e < groups; ++e)
        codes = (codes & ~(0xffull << (8 * e))) | (uint64_t)src[e] << (8 * e);
    }
    uint32_t d[10];
    uint32_t flags = 0;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      uint32_t lo[4], hi[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint64_t e = dec[(codes >> (8 * (4 * q + k))) & 0xffu];
        lo[k] = (uint32_t)e;
        hi[k] = (uint32_t)(e >> 32);
        flags += hi[k] >> 16;
      }
      // trit bytes 0..19 of codes 4q .. 4q + 3: five from each entry
      d[5 * q] = lo[0];
      d[5 * q + 1] = (hi[0] & 0xffu) | lo[1] << 8;
      d[5 * q + 2] = lo[1] >> 24 | (hi[1] & 0xffu) << 8 | lo[2] << 16;
      d[5 * q + 3] = lo[2] >> 16 | (hi[2] & 0xffu) << 16 | lo[3] << 24;
      d[5 * q + 4] = lo[3] >> 8 | hi[3] << 24;
    }
    bad += (int)flags;
#pragma unroll
    for (int i = 0; i < 5; ++i)
      *reinterpret_cast<uint2 *>(buf + 40 * lane + 8 * i) = make_uint2(d[2 * i], d[2 * i + 1]);
    lds_fence();
    int8_t *dst = wq + r * ldq + (int64_t)kSpanIn * c;
    const int64_t left = K - (int64_t)kSpanIn * c;
    if (left >= kSpanIn) {  // (wave-uniform) the whole span lies inside the row
      uint2 v[5];
#pragma unroll
      for (int i = 0; i < 5; ++i) v[i] = *reinterpret_cast<const uint2 *>(buf + 512 * i + 8 * lane);
#pragma unroll
      for (int i = 0; i < 5; ++i) *reinterpret_cast<uint2 *>(dst + 512 * i + 8 * lane) = v[i];
    } else {
#pragma unroll 1
      for (int i = 0; i < 5; ++i) {
        const int o = 512 * i + 8 * lane;
        const uint2 v = *reinterpret_cast<const uint2 *>(buf + o);
        if (o + 8 <= left) {
          *reinterpret_cast<uint2 *>(dst + o) = v;
        } else if (o < left) {
          const uint64_t w = (uint64_t)v.x | (uint64_t)v.y << 32;
#pragma unroll 1
          for (int e = 0; e < 8 && o + e < left; ++e) dst[o + e] = (int8_t)(w >> (8 * e));
        }
      }
    }
    lds_fence();
  }
  count_bad(bad, bad_count);
}

// (row groups of four, spans), each capped; the kernels stride over the rest
dim3 span_grid(int64_t N, int64_t spans) {
  const int64_t gx = std::min<int64_t>(ceil_div(N, kSpanWaves), INT64_C(1) << 20);
  const int64_t gy = std::min<int64_t>(spans, 65535);
  return dim3((unsigned)std::max<int64_t>(gx, 1), (unsigned)std::max<int64_t>(gy, 1));
}

}  // namespace

hipError_t launch_pack(const int8_t *wq, int64_t ldq, int64_t N, int64_t K, uint8_t *packed,
                       int64_t ldp, int32_t *bad, hipStream_t st) {
  hipLaunchKernelGGL(pack_kernel, span_grid(N, ceil_div(ldp, kSpanOut)), dim3(256), 0, st, wq,
                     ldq, N, K, packed, ldp, bad);
  return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t *packed, int64_t ldp, int64_t N, int64_t K, int8_t *wq,
                         int64_t ldq, int32_t *bad, hipStream_t st) {
  hipLaunchKernelGGL(unpack_kernel, span_grid(N, ceil_div(ceil_div(K, 5), kSpanOut)), dim3(256),
                     0, st, packed, ldp, N, K, wq, ldq, bad);
  return hipGetLastError();
}

}  // namespace ug

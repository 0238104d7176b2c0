// Decode GEMV (gfx950): y = (x_q W_q^T)(s beta) for 1..64 activation rows.
//
// "ultragraph - when the graph is the 1-bit LLM, part 2", section
// "autograd on a byte-graph": integer multiply-accumulate of int8
// activations against ternary weights, one rescale by s*beta at the end.
// "a 1-bit llm, from scratch" (the 20 -> 1,045 tok/s table) is the prior art
// for the inner loop: never branch on the zeros, keep independent
// accumulators.
//
// Weights stream from HBM once per group of MT activation rows with 128-bit
// loads; each wave owns whole weight rows and its 64 lanes split the row.
// A packed byte is decoded through a 256-entry table in LDS (code -> five
// int8 trits in a uint2); four decoded bytes are stitched into five dwords
// of int8 trits that line up with 20 consecutive int8 activations, and
// v_dot4_i32_i8 multiplies-and-adds four at a time into int32.  Lanes are
// then summed with cross-lane shuffles; integer addition is exact, so the
// order does not matter.
#include "ug_internal.h"

namespace ug {
namespace {

constexpr int kMT = 4;  // activation rows per pass over the weights

__device__ inline int dot4(uint32_t a, uint32_t b, int c) {
  return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// Trits of code e (0..242) as int8 in bytes 0..4 of a uint2; codes
// 243..255 decode to zeros.
__device__ inline uint2 lut_entry(int e) {
  uint32_t lo = 0, hi = 0;
  if (e <= 242) {
    int c = e;
#pragma unroll
    for (int j = 0; j < 5; ++j) {
      const uint32_t t = (uint32_t)((c % 3) - 1) & 0xffu;
      c /= 3;
      if (j < 4)
        lo |= t << (8 * j);
      else
        hi = t;
    }
  }
  return make_uint2(lo, hi);
}

// Four packed bytes -> twenty int8 trits in five dwords (trit stream order).
__device__ inline void decode4(uint32_t w, const uint2 *lut, uint32_t d[5]) {
  const uint2 L0 = lut[w & 0xff];
  const uint2 L1 = lut[(w >> 8) & 0xff];
  const uint2 L2 = lut[(w >> 16) & 0xff];
  const uint2 L3 = lut[w >> 24];
  d[0] = L0.x;
  d[1] = L0.y | (L1.x << 8);
  d[2] = (L1.x >> 24) | (L1.y << 8) | (L2.x << 16);
  d[3] = (L2.x >> 16) | (L2.y << 16) | (L3.x << 24);
  d[4] = (L3.x >> 8) | (L3.y << 24);
}

// 16 bytes of x_q row at K offset p, zero past K.  In-bounds because every
// row owns ldx >= round_up(K, 16) bytes and p < K when anything is read.
__device__ inline uint4 load_x16(const int8_t *xr, int64_t p, int64_t K) {
  if (p >= K) return make_uint4(0, 0, 0, 0);
  uint4 v = *reinterpret_cast<const uint4 *>(xr + p);
  if (p + 16 > K) {
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (p + i >= K) w[i >> 2] &= ~(0xffu << (8 * (i & 3)));
    v = make_uint4(w[0], w[1], w[2], w[3]);
  }
  return v;
}

template <int FMT>
__global__ __launch_bounds__(256) void gemv_kernel(const int8_t *__restrict__ xq, int64_t ldx,
                                                   const float *__restrict__ s,
                                                   const uint8_t *__restrict__ w, int64_t ldw,
                                                   const float *__restrict__ beta, int64_t M,
                                                   int64_t N, int64_t K, int32_t *__restrict__ acc,
                                                   int64_t ldacc, float *__restrict__ y,
                                                   int64_t ldy) {
  __shared__ uint2 lut[256];
  if (FMT == UG_W_PACK5) {
    lut[threadIdx.x] = lut_entry(threadIdx.x);
    __syncthreads();
  }
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  // Bytes of weight per row that carry data, in 16-byte chunks.
  const int64_t row_bytes = FMT == UG_W_PACK5 ? (K + 4) / 5 : K;
  const int64_t nchunks = (row_bytes + 15) / 16;
  const int64_t kchunk = FMT == UG_W_PACK5 ? 80 : 16;  // K positions per chunk
  const float b = beta[0];

  for (int64_t n = wave; n < N; n += nwaves) {
    const uint8_t *wr = w + n * ldw;
    for (int64_t m0 = 0; m0 < M; m0 += kMT) {
      int a[kMT];
#pragma unroll
      for (int i = 0; i < kMT; ++i) a[i] = 0;
      for (int64_t c = lane; c < nchunks; c += 64) {
        const uint4 wv = *reinterpret_cast<const uint4 *>(wr + 16 * c);
        const int64_t kb = c * kchunk;
        if (FMT == UG_W_PACK5) {
          uint32_t d[20];
          decode4(wv.x, lut, d);
          decode4(wv.y, lut, d + 5);
          decode4(wv.z, lut, d + 10);
          decode4(wv.w, lut, d + 15);
#pragma unroll
          for (int i = 0; i < kMT; ++i) {
            if (m0 + i < M) {
              const int8_t *xr = xq + (m0 + i) * ldx;
#pragma unroll
              for (int p = 0; p < 5; ++p) {
                const uint4 xv = load_x16(xr, kb + 16 * p, K);
                a[i] = dot4(d[4 * p + 0], xv.x, a[i]);
                a[i] = dot4(d[4 * p + 1], xv.y, a[i]);
                a[i] = dot4(d[4 * p + 2], xv.z, a[i]);
                a[i] = dot4(d[4 * p + 3], xv.w, a[i]);
              }
            }
          }
        } else {
#pragma unroll
          for (int i = 0; i < kMT; ++i) {
            if (m0 + i < M) {
              const uint4 xv = load_x16(xq + (m0 + i) * ldx, kb, K);
              a[i] = dot4(wv.x, xv.x, a[i]);
              a[i] = dot4(wv.y, xv.y, a[i]);
              a[i] = dot4(wv.z, xv.z, a[i]);
              a[i] = dot4(wv.w, xv.w, a[i]);
            }
          }
        }
      }
#pragma unroll
      for (int i = 0; i < kMT; ++i) {
        const int tot = wave_sum_i32(a[i]);
        const int64_t m = m0 + i;
        if (lane == 0 && m < M) {
          if (acc) acc[m * ldacc + n] = tot;
          if (y) {
            const float scale = s[m] * b;
            y[m * ldy + n] = (float)tot * scale;
          }
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemv(const int8_t *xq, int64_t ldx, const float *s, const void *w, int wfmt,
                       int64_t ldw, const float *beta, int64_t M, int64_t N, int64_t K,
                       int32_t *acc, int64_t ldacc, float *y, int64_t ldy, hipStream_t st) {
  int64_t blocks = ceil_div(N, 4);
  if (blocks > 256 * 8) blocks = 256 * 8;
  if (wfmt == UG_W_PACK5)
    hipLaunchKernelGGL(gemv_kernel<UG_W_PACK5>, dim3(blocks), dim3(256), 0, st, xq, ldx, s,
                       (const uint8_t *)w, ldw, beta, M, N, K, acc, ldacc, y, ldy);
  else
    hipLaunchKernelGGL(gemv_kernel<UG_W_I8>, dim3(blocks), dim3(256), 0, st, xq, ldx, s,
                       (const uint8_t *)w, ldw, beta, M, N, K, acc, ldacc, y, ldy);
  return hipGetLastError();
}

}  // namespace ug

// Absmean ternary weight quantization (gfx950).
//
// "ultragraph - when the graph is the 1-bit LLM, part 2", section "the
// bytes": beta = (1/n) sum_i |W_i| + eps, W_q = clip(round(W/beta), -1, 1);
// one beta per weight tensor.
//
// Three launches, no host synchronization, no atomics on values:
//   stage 1  one 256-thread block per 8192-element chunk; thread t keeps four
//            sums and adds element 8192c + 1024i + 4t + j (i = 0..7) to sum j
//            -- eight coalesced float4 loads per thread -- then the block
//            folds its 256 lane values pairwise;
//   stage 2  one block sums the chunk sums (lane t: chunks t, t+256, ...),
//            folds, and writes beta = fl(fl(T/n) + eps) to device memory;
//   quant    elementwise W_q = clamp(rint(W/beta), -1, 1), beta read from
//            device memory.
// Traffic: 4 B/element read twice (the second read mostly hits the MALL for
// tensors that fit) plus 1 B/element written.
#include "ug_internal.h"

namespace ug {
namespace {

__device__ inline float4 ld4(const float *p) { return *reinterpret_cast<const float4 *>(p); }

// |W| of flat element e of a pitched [N][K] matrix, +0 past the end.
__device__ inline float abs_at(const float *W, int64_t ldw, int64_t K, int64_t n, int64_t e) {
  if (e >= n) return 0.0f;
  const int64_t r = e / K, c = e - r * K;
  return fabsf(W[r * ldw + c]);
}

__global__ __launch_bounds__(256) void absmean_stage1(const float *__restrict__ W, int64_t ldw,
                                                      int64_t N, int64_t K,
                                                      float *__restrict__ partials) {
  __shared__ float lds[256];
  const int t = threadIdx.x;
  const int64_t c = blockIdx.x;
  const int64_t n = N * K;
  const int64_t base = c * kAbsmeanChunk;
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  if (ldw == K && base + kAbsmeanChunk <= n) {
    // Whole chunk inside a contiguous tensor: eight float4 loads, issued
    // together before any add.
    float4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = ld4(W + base + 1024 * i + 4 * t);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a0 = a0 + fabsf(v[i].x);
      a1 = a1 + fabsf(v[i].y);
      a2 = a2 + fabsf(v[i].z);
      a3 = a3 + fabsf(v[i].w);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t e = base + 1024 * i + 4 * t;
      a0 = a0 + abs_at(W, ldw, K, n, e);
      a1 = a1 + abs_at(W, ldw, K, n, e + 1);
      a2 = a2 + abs_at(W, ldw, K, n, e + 2);
      a3 = a3 + abs_at(W, ldw, K, n, e + 3);
    }
  }
  const float lo = a0 + a1;
  const float hi = a2 + a3;
  const float p = fold256(lo + hi, lds);
  if (t == 0) partials[c] = p;
}

__global__ __launch_bounds__(256) void absmean_stage2(const float *__restrict__ partials,
                                                      int64_t nchunks, float n_f, float eps,
                                                      float *__restrict__ beta) {
  __shared__ float lds[256];
  const int t = threadIdx.x;
  float acc = 0.0f;
  for (int64_t c = t; c < nchunks; c += 256) acc = acc + partials[c];
  const float T = fold256(acc, lds);
  if (t == 0) {
    const float mean = T / n_f;
    beta[0] = mean + eps;
  }
}

__device__ inline int tern(float w, float b) { return rint_clamp(w / b, -1.0f, 1.0f); }

// One thread per 4 consecutive elements of a row; rows are split into
// ceil(K/4) vector slots.
__global__ __launch_bounds__(256) void ternary_quant(const float *__restrict__ W, int64_t ldw,
                                                     int64_t N, int64_t K,
                                                     const float *__restrict__ beta_p,
                                                     int8_t *__restrict__ wq, int64_t ldq) {
  const float b = beta_p[0];
  const int64_t kv = (K + 3) / 4;
  const int64_t total = N * kv;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * 256) {
    const int64_t r = idx / kv;
    const int64_t k = (idx - r * kv) * 4;
    const float4 v = ld4(W + r * ldw + k);  // in-bounds: ldw >= round_up(K, 4)
    const int q0 = tern(v.x, b), q1 = tern(v.y, b), q2 = tern(v.z, b), q3 = tern(v.w, b);
    int8_t *dst = wq + r * ldq + k;
    if (k + 3 < K) {
      const uint32_t p = (uint32_t)(q0 & 0xff) | ((uint32_t)(q1 & 0xff) << 8) |
                         ((uint32_t)(q2 & 0xff) << 16) | ((uint32_t)(q3 & 0xff) << 24);
      *reinterpret_cast<uint32_t *>(dst) = p;
    } else {
      dst[0] = (int8_t)q0;
      if (k + 1 < K) dst[1] = (int8_t)q1;
      if (k + 2 < K) dst[2] = (int8_t)q2;
    }
  }
}

}  // namespace

hipError_t launch_absmean(const float *W, int64_t ldw, int64_t N, int64_t K, float eps,
                          int8_t *wq, int64_t ldq, float *beta, float *partials,
                          hipStream_t st) {
  const int64_t n = N * K;
  const int64_t nchunks = ceil_div(n, kAbsmeanChunk);
  hipLaunchKernelGGL(absmean_stage1, dim3(nchunks), dim3(256), 0, st, W, ldw, N, K, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(absmean_stage2, dim3(1), dim3(256), 0, st, partials, nchunks, (float)n,
                     eps, beta);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t total = N * ceil_div(K, 4);
  int64_t blocks = ceil_div(total, 256);
  if (blocks > 256 * 64) blocks = 256 * 64;
  hipLaunchKernelGGL(ternary_quant, dim3(blocks), dim3(256), 0, st, W, ldw, N, K, beta, wq, ldq);
  return hipGetLastError();
}

}  // namespace ug

// Absmean ternary weight quantization (gfx950).
//
// "ultragraph - when the graph is the 1-bit LLM, part 2", section "the
// bytes": beta = (1/n) sum_i |W_i| + eps, W_q = clip(round(W/beta), -1, 1);
// one beta per weight tensor.
//
// Two launches, no host synchronization, no atomics on values:
//   stage 1  one 256-thread block per 8192-element chunk; thread t keeps four
//            sums and adds element 8192c + 1024i + 4t + j (i = 0..7) to sum j
//            -- eight coalesced float4 loads per thread -- then the block
//            folds its 256 lane values pairwise;
//   quant    every block first forms beta the same way (lane t sums the
//            chunk sums t, t+256, ..., the block folds them, beta =
//            fl(fl(T/n) + eps); block 0 stores it), then quantizes its share
//            of the elements: W_q = clamp(rint(W/beta), -1, 1).
// Traffic: 4 B/element read twice (the second read mostly hits the MALL for
// tensors that fit) plus 1 B/element written.
#include <mutex>

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

// beta from the chunk sums, in the fixed order (every block gets the same bits).
__device__ inline float beta_from(const float *__restrict__ partials, int64_t nchunks, float n_f,
                                  float eps, float *lds) {
  const int t = threadIdx.x;
  float acc = 0.0f;
  for (int64_t c = t; c < nchunks; c += 256) acc = acc + partials[c];
  const float T = fold256(acc, lds);
  const float mean = T / n_f;
  return mean + eps;
}

__device__ inline int tern(float w, float b) { return rint_clamp(w / b, -1.0f, 1.0f); }

// The same code without the division in almost every case: with
// q' = w * rb (rb = v_rcp_f32(b), at most 1 ulp from 1/b), |q' - fl(w/b)|
// stays below 2.5 ulp of |q'|, so only |q'| within kBand of 1/2 (the one
// rounding boundary that survives the clamp to [-1, 1]) needs the exact
// quotient; elsewhere the code is sign(q') if |q'| > 1/2, else 0.  Used
// only for a normal beta of moderate size (the caller checks), so that rb
// is finite and accurate; NaN elements take the exact path.
constexpr float kBand = 6.103515625e-05f;  // 2^-14
__device__ inline int tern_fast(float w, float b, float rb) {
  const float q = w * rb;
  const float aq = fabsf(q);
  if (__builtin_expect(!(fabsf(aq - 0.5f) > kBand), 0)) return tern(w, b);
  return aq > 0.5f ? (q > 0.0f ? 1 : -1) : 0;
}

__device__ inline uint32_t tern4(float4 v, float b, float rb, bool fast) {
  int q0, q1, q2, q3;
  if (fast) {
    q0 = tern_fast(v.x, b, rb);
    q1 = tern_fast(v.y, b, rb);
    q2 = tern_fast(v.z, b, rb);
    q3 = tern_fast(v.w, b, rb);
  } else {
    q0 = tern(v.x, b);
    q1 = tern(v.y, b);
    q2 = tern(v.z, b);
    q3 = tern(v.w, b);
  }
  return (uint32_t)(q0 & 0xff) | ((uint32_t)(q1 & 0xff) << 8) | ((uint32_t)(q2 & 0xff) << 16) |
         ((uint32_t)(q3 & 0xff) << 24);
}

// Grid-stride over float4 slots.  Contiguous tensors (ldw == ldq == K) are
// walked as one flat array; pitched ones as ceil(K/4) slots per row.
__global__ __launch_bounds__(256) void ternary_quant(const float *__restrict__ W, int64_t ldw,
                                                     int64_t N, int64_t K,
                                                     const float *__restrict__ partials,
                                                     int64_t nchunks, float n_f, float eps,
                                                     float *__restrict__ beta_out,
                                                     int8_t *__restrict__ wq, int64_t ldq) {
  __shared__ float lds[256];
  const float b = beta_from(partials, nchunks, n_f, eps, lds);
  if (blockIdx.x == 0 && threadIdx.x == 0) beta_out[0] = b;
  const bool fast = b >= 0x1p-100f && b <= 0x1p100f;
  const float rb = fast ? __builtin_amdgcn_rcpf(b) : 0.0f;
  const int64_t stride = (int64_t)gridDim.x * 256;
  if (ldw == K && ldq == K) {
    const int64_t n = N * K, n4 = n / 4;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride)
      *reinterpret_cast<uint32_t *>(wq + 4 * i) = tern4(ld4(W + 4 * i), b, rb, fast);
    // the last n % 4 elements
    const int64_t e = 4 * n4 + (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e < n) wq[e] = (int8_t)tern(W[e], b);
    return;
  }
  const int64_t kv = (K + 3) / 4;
  const int64_t total = N * kv;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += stride) {
    const int64_t r = idx / kv;
    const int64_t k = (idx - r * kv) * 4;
    const float4 v = ld4(W + r * ldw + k);  // in-bounds: ldw >= round_up(K, 4)
    const uint32_t p = tern4(v, b, rb, fast);
    int8_t *dst = wq + r * ldq + k;
    if (k + 3 < K) {
      *reinterpret_cast<uint32_t *>(dst) = p;
    } else {
      dst[0] = (int8_t)(p & 0xff);
      if (k + 1 < K) dst[1] = (int8_t)((p >> 8) & 0xff);
      if (k + 2 < K) dst[2] = (int8_t)((p >> 16) & 0xff);
    }
  }
}

// One PACK5 byte from the five fp32 weights of its group:
// 121 + sum_j W_q(w_j) 3^j (README "A whole ternary GPT": five ternary values
// per byte), each W_q as in ternary_quant.
__device__ inline uint32_t pack5_code(float w0, float w1, float w2, float w3, float w4, float b,
                                      float rb, bool fast) {
  int t0, t1, t2, t3, t4;
  if (fast) {
    t0 = tern_fast(w0, b, rb);
    t1 = tern_fast(w1, b, rb);
    t2 = tern_fast(w2, b, rb);
    t3 = tern_fast(w3, b, rb);
    t4 = tern_fast(w4, b, rb);
  } else {
    t0 = tern(w0, b);
    t1 = tern(w1, b);
    t2 = tern(w2, b);
    t3 = tern(w3, b);
    t4 = tern(w4, b);
  }
  return (uint32_t)(121 + t0 + 3 * t1 + 9 * t2 + 27 * t3 + 81 * t4);
}

// Requantization straight to five trits per byte: beta as in ternary_quant,
// then every output dword (4 bytes = 20 consecutive weights of a row) from
// five float4 loads.  Row bytes from ceil(K/5) to ldp are 121 (five zero
// trits); weights past K count as zero trits.  The same bytes as
// ternary_quant followed by pack_kernel, without the int8 tensor between.
__global__ __launch_bounds__(256) void ternary_pack5(const float *__restrict__ W, int64_t ldw,
                                                     int64_t N, int64_t K,
                                                     const float *__restrict__ partials,
                                                     int64_t nchunks, float n_f, float eps,
                                                     float *__restrict__ beta_out,
                                                     uint8_t *__restrict__ packed, int64_t ldp) {
  __shared__ float lds[256];
  const float b = beta_from(partials, nchunks, n_f, eps, lds);
  if (blockIdx.x == 0 && threadIdx.x == 0) beta_out[0] = b;
  const bool fast = b >= 0x1p-100f && b <= 0x1p100f;
  const float rb = fast ? __builtin_amdgcn_rcpf(b) : 0.0f;
  const int64_t groups = (K + 4) / 5;
  const int64_t dpr = ldp / 4;  // output dwords per row
  const int64_t total = N * dpr;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += stride) {
    const int64_t r = idx / dpr;
    const int64_t j = idx - r * dpr;
    const int64_t e0 = 20 * j;  // first weight of the dword's four groups
    const float *src = W + r * ldw + e0;
    uint32_t word;
    if (e0 + 20 <= K) {
      // 80 contiguous bytes, 16-byte aligned (ldw is a multiple of 4)
      const float4 a = ld4(src), c = ld4(src + 4), d = ld4(src + 8), e = ld4(src + 12),
                   f = ld4(src + 16);
      word = pack5_code(a.x, a.y, a.z, a.w, c.x, b, rb, fast) |
             pack5_code(c.y, c.z, c.w, d.x, d.y, b, rb, fast) << 8 |
             pack5_code(d.z, d.w, e.x, e.y, e.z, b, rb, fast) << 16 |
             pack5_code(e.w, f.x, f.y, f.z, f.w, b, rb, fast) << 24;
    } else {
      word = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t g = 4 * j + q;
        uint32_t code = 121;
        if (g < groups) {
          float v[5];
#pragma unroll
          for (int i = 0; i < 5; ++i) v[i] = 5 * g + i < K ? src[5 * q + i] : 0.0f;
          code = pack5_code(v[0], v[1], v[2], v[3], v[4], b, rb, fast);
        }
        word |= code << (8 * q);
      }
    }
    *reinterpret_cast<uint32_t *>(packed + r * ldp + 4 * j) = word;
  }
}

// Stage-1 partials of the allocation-free entry point: one float per
// 8192-element chunk, so tensors of up to kStaticChunks * 8192 elements.
// Each device holds its own copy for the life of the process.
static __device__ __align__(256) float scratch[kStaticChunks];

}  // namespace

// The device address of this device's `scratch` array, looked up once per
// device (with that device current) and cached; host code uses only this
// pointer, never the array's name.
hipError_t static_scratch(float **out) {
  static std::mutex mu;
  static float *ptrs[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptrs[dev] = static_cast<float *>(p);
  }
  *out = ptrs[dev];
  return hipSuccess;
}

hipError_t launch_absmean(const float *W, int64_t ldw, int64_t N, int64_t K, float eps,
                          int8_t *wq, int64_t ldq, float *beta, float *partials,
                          hipStream_t st) {
  const int64_t n = N * K;
  const int64_t nchunks = ceil_div(n, kAbsmeanChunk);
  hipLaunchKernelGGL(absmean_stage1, dim3(nchunks), dim3(256), 0, st, W, ldw, N, K, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // every quantization block re-forms beta from the chunk sums: keep them
  // few (4 per CU), each streaming a long range
  const int64_t total = ldw == K && ldq == K ? ceil_div(n, 4) : N * ceil_div(K, 4);
  int64_t blocks = ceil_div(total, 256);
  if (blocks > 256 * 4) blocks = 256 * 4;
  hipLaunchKernelGGL(ternary_quant, dim3(blocks), dim3(256), 0, st, W, ldw, N, K, partials,
                     nchunks, (float)n, eps, beta, wq, ldq);
  return hipGetLastError();
}

hipError_t launch_absmean_pack5(const float *W, int64_t ldw, int64_t N, int64_t K, float eps,
                                uint8_t *packed, int64_t ldp, float *beta, float *partials,
                                hipStream_t st) {
  const int64_t n = N * K;
  const int64_t nchunks = ceil_div(n, kAbsmeanChunk);
  hipLaunchKernelGGL(absmean_stage1, dim3(nchunks), dim3(256), 0, st, W, ldw, N, K, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int64_t blocks = ceil_div(N * (ldp / 4), 256);
  if (blocks > 256 * 4) blocks = 256 * 4;
  hipLaunchKernelGGL(ternary_pack5, dim3(blocks), dim3(256), 0, st, W, ldw, N, K, partials,
                     nchunks, (float)n, eps, beta, packed, ldp);
  return hipGetLastError();
}

}  // namespace ug

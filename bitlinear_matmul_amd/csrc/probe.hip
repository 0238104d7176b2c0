// Rate probes (gfx950): measurement helpers beside the forward path, not
// steps of it.
//
// Matrix-core rate.
// The published dense peaks (5.0 POP/s int8, 157.3 TFLOP/s fp32) assume
// the 2.4 GHz peak engine clock on all 256 CUs.  Under a full matrix-core
// load the board's power limit lowers that clock, so the rate a GEMM can
// reach is set by what the matrix cores sustain.  This kernel measures it:
// one block of four waves per CU (one per SIMD), each wave issuing
// back-to-back matrix instructions on 16 independent accumulators, with
// operands from four register sets per side that change from one
// instruction to the next (as a GEMM's fragments do), no memory traffic in
// the loop.  Each wave finally writes one word derived from its
// accumulators, so the compiler keeps every instruction.
#include "ug_internal.h"

namespace ug {
namespace {

typedef int v4i_p __attribute__((ext_vector_type(4)));
typedef int v16i_p __attribute__((ext_vector_type(16)));
typedef float v4f_p __attribute__((ext_vector_type(4)));

// 32-bit mix of (block, lane, i): operand bits that differ between lanes
__device__ inline uint32_t mix(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

template <int KIND>
__global__ __launch_bounds__(256) void mfma_rate_kernel(int iters, int32_t *__restrict__ sink) {
  const uint32_t lane = threadIdx.x & 63, seed = blockIdx.x * 256 + threadIdx.x;
  uint32_t word = 0;
  if (KIND == 0) {
    v4i_p a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a[i][e] = (int)mix(seed * 32 + 8 * i + e);
        b[i][e] = (int)mix(seed * 32 + 8 * i + 4 + e + 0x9e3779b9u);
      }
    v16i_p c[16];
#pragma unroll
    for (int g = 0; g < 16; ++g) c[g] = (v16i_p){};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int g = 0; g < 16; ++g)
        c[g] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[g & 3], b[(g >> 2) & 3], c[g], 0, 0, 0);
    }
#pragma unroll
    for (int g = 0; g < 16; ++g)
#pragma unroll
      for (int e = 0; e < 16; ++e) word ^= (uint32_t)c[g][e];
  } else {
    float a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // values in [-1, 1): the sums stay far from overflow
      a[i] = (float)(int)(mix(seed * 8 + i) >> 8) * 0x1p-23f - 1.0f;
      b[i] = (float)(int)(mix(seed * 8 + 4 + i) >> 8) * 0x1p-23f - 1.0f;
    }
    v4f_p c[16];
#pragma unroll
    for (int g = 0; g < 16; ++g) c[g] = (v4f_p){};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int g = 0; g < 16; ++g)
        c[g] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[g & 3], b[(g >> 2) & 3], c[g], 0, 0, 0);
    }
#pragma unroll
    for (int g = 0; g < 16; ++g)
#pragma unroll
      for (int e = 0; e < 4; ++e) word ^= __float_as_uint(c[g][e]);
  }
  // one word per wave: the XOR over its lanes
#pragma unroll
  for (int h = 32; h >= 1; h >>= 1) word ^= (uint32_t)__shfl_xor((int)word, h, 64);
  if (lane == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = (int32_t)word;
}

// HBM read rate: the rate a plain streaming read reaches on this GPU, the
// measured ceiling for the bandwidth-bound kernels (which read far more
// than they write).  Threads walk the buffer's 16-byte words (a wave's load
// instruction reads 1 KB contiguous), eight loads in flight, and fold each
// word into an XOR; each wave writes the XOR over its lanes, so the XOR of
// all sink words is the XOR of every 32-bit word of the buffer.  Walk 0:
// one grid stride over the whole buffer; walk 1: block b takes the b-th of
// gridDim.x contiguous ranges (whole 16-byte words) and its threads walk
// that range with a block stride, as the streaming GEMV's blocks each walk
// their own range of weight rows.
template <int WALK>
__global__ __launch_bounds__(256) void hbm_read_kernel(const uint4 *__restrict__ buf, uint64_t n16,
                                                       uint32_t *__restrict__ sink) {
  uint64_t stride, i, end;
  if (WALK == 0) {
    stride = (uint64_t)gridDim.x * 256;
    i = (uint64_t)blockIdx.x * 256 + threadIdx.x;
    end = n16;
  } else {
    stride = 256;
    i = n16 * blockIdx.x / gridDim.x + threadIdx.x;
    end = n16 * (blockIdx.x + 1) / gridDim.x;
  }
  const uint64_t n16_ = end;  // (walk 0: the whole buffer)
  uint32_t x = 0;
  for (; i + 7 * stride < n16_; i += 8 * stride) {
    uint4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = buf[i + j * stride];
#pragma unroll
    for (int j = 0; j < 8; ++j) x ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  for (; i < n16_; i += stride) {
    const uint4 v = buf[i];
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int h = 32; h >= 1; h >>= 1) x ^= (uint32_t)__shfl_xor((int)x, h, 64);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = x;
}

}  // namespace

hipError_t launch_hbm_read(const void *buf, uint64_t bytes, int blocks, int walk, uint32_t *sink,
                           hipStream_t st) {
  if (walk == 0)
    hipLaunchKernelGGL(hbm_read_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, st,
                       static_cast<const uint4 *>(buf), bytes / 16, sink);
  else
    hipLaunchKernelGGL(hbm_read_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, st,
                       static_cast<const uint4 *>(buf), bytes / 16, sink);
  return hipGetLastError();
}

hipError_t launch_mfma_rate(int kind, int blocks, int iters, int32_t *sink, hipStream_t st) {
  if (kind == 0)
    hipLaunchKernelGGL(mfma_rate_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, st, iters, sink);
  else
    hipLaunchKernelGGL(mfma_rate_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, st, iters, sink);
  return hipGetLastError();
}

}  // namespace ug

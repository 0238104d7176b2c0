// Per-token activation quantizers (gfx950).
//
// "ultragraph - when the graph is the 1-bit LLM, part 2", section "the
// bytes": s = max|x|/127 + eps, x_q = clip(round(x/s), -127, 127), one scale
// per row ("attention, as graph ops": per-token scales keep rows
// independent).  The RMSNorm variant applies x / sqrt(mean x^2 + eps) * g
// first (same page, "attention, as graph ops").
//
// HBM-bound: 4 bytes read + 1 byte written per element.  A row is read from
// HBM once: each thread keeps its float4 slices in registers between the
// max-reduction and the quantization.  Rows longer than the register budget
// are read twice (the second read mostly hits L2).
#include "ug_internal.h"

namespace ug {
namespace {

__device__ inline float4 ld4(const float *p) {
  return *reinterpret_cast<const float4 *>(p);
}

// q8 and q8x4 (the row codes with and without the division) come from
// ug_internal.h, shared with the fused GEMV.

__device__ inline void store_q4(int8_t *dst, int64_t k, int64_t K, float4 v, float s) {
  int a, b, c, d;
  q8x4(v, s, a, b, c, d);
  if (k + 3 < K) {
    uint32_t packed = (uint32_t)(a & 0xff) | ((uint32_t)(b & 0xff) << 8) |
                      ((uint32_t)(c & 0xff) << 16) | ((uint32_t)(d & 0xff) << 24);
    *reinterpret_cast<uint32_t *>(dst + k) = packed;
  } else {
    dst[k] = (int8_t)a;
    if (k + 1 < K) dst[k + 1] = (int8_t)b;
    if (k + 2 < K) dst[k + 2] = (int8_t)c;
  }
}

// Zero the lanes of v at positions >= K (row pad or past the row).
__device__ inline float4 mask4(float4 v, int64_t k, int64_t K) {
  if (k + 3 >= K) {
    if (k + 1 >= K) v.y = 0.0f;
    if (k + 2 >= K) v.z = 0.0f;
    if (k + 3 >= K) v.w = 0.0f;
  }
  return v;
}

__device__ inline float amax4(float4 v) {
  return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}

// TPR threads per row (64: one wave per row, 4 rows per block; 256: one
// block per row).  VPT = float4 slices held per thread.  If K > TPR*4*VPT the
// row is streamed twice.
template <int TPR, int VPT>
__global__ __launch_bounds__(256) void quant_act_kernel(const float *__restrict__ x, int64_t ldx,
                                                        int64_t M, int64_t K, float eps,
                                                        int8_t *__restrict__ xq, int64_t ldq,
                                                        float *__restrict__ s) {
  constexpr int RPB = 256 / TPR;
  __shared__ float red[4];
  const int tid = threadIdx.x;
  const int lane_in_row = tid % TPR;
  const int64_t m = (int64_t)blockIdx.x * RPB + tid / TPR;
  const bool row_ok = m < M;
  const float *xr = x + (row_ok ? m : 0) * ldx;
  const int64_t nvec = (K + 3) / 4;
  const bool fits = nvec <= (int64_t)TPR * VPT;

  float4 v[VPT];
  float a = 0.0f;
  if (fits) {
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int64_t f = lane_in_row + (int64_t)i * TPR;
      if (row_ok && f < nvec) {
        v[i] = mask4(ld4(xr + 4 * f), 4 * f, K);
        a = fmaxf(a, amax4(v[i]));
      } else {
        v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  } else {
    for (int64_t f = lane_in_row; f < nvec; f += TPR)
      if (row_ok) a = fmaxf(a, amax4(mask4(ld4(xr + 4 * f), 4 * f, K)));
  }
  a = wave_max(a);
  if (TPR == 256) {
    if ((tid & 63) == 0) red[tid >> 6] = a;
    __syncthreads();
    a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  }
  // s = fl(fl(a / 127) + eps): correctly rounded division, then the add.
  const float a127 = a / 127.0f;
  const float sc = a127 + eps;
  if (!row_ok) return;
  if (lane_in_row == 0) s[m] = sc;
  int8_t *qr = xq + m * ldq;
  if (fits) {
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int64_t f = lane_in_row + (int64_t)i * TPR;
      if (f < nvec) store_q4(qr, 4 * f, K, v[i], sc);
    }
  } else {
    for (int64_t f = lane_in_row; f < nvec; f += TPR)
      store_q4(qr, 4 * f, K, mask4(ld4(xr + 4 * f), 4 * f, K), sc);
  }
}

// fl(v / r) given y = fl(1 / r), without the division sequence: q0 = v y is
// within an ulp of v / r, the residual v - q0 r is exact with a fused
// multiply-add, and q0 + residual * y rounded once is the correctly rounded
// quotient (Markstein's theorem on division by a correctly rounded
// reciprocal).  Its conditions need v and the quotient in the normal range
// away from overflow: outside [2^-80, 2^100] the division is done as
// written.
__device__ __forceinline__ float div_by(float v, float r, float y) {
  const float q0 = v * y;
  const float aq = fabsf(q0);
  if (__builtin_expect(fabsf(v) >= 0x1p-80f && aq >= 0x1p-80f && aq <= 0x1p100f, 1))
    return __builtin_fmaf(__builtin_fmaf(-q0, r, v), y, q0);
  return v == 0.0f ? q0 : v / r;
}

// RMSNorm + quantization; one 256-thread block per row.  Thread t owns the
// float4 slices f = t + 256 i, i.e. the elements k with floor(k/4) mod 256
// = t, which it squares and adds from +0 in increasing k.  The 256 slot
// sums are folded in the documented order (fold256's: v_t + v_t+128, then
// + (v_t+64 + v_t+192), then lanes t + h for h = 32 .. 1) by every wave
// itself, which takes lane 0's bits: one barrier instead of four.
template <int VPT>
__global__ __launch_bounds__(256) void rmsnorm_quant_kernel(const float *__restrict__ x, int64_t ldx,
                                                            const float *__restrict__ g, int64_t M,
                                                            int64_t K, float eps_n, float eps,
                                                            int8_t *__restrict__ xq, int64_t ldq,
                                                            float *__restrict__ s) {
  __shared__ float lds[256];
  __shared__ float red[4];
  const int t = threadIdx.x;
  const int64_t m = blockIdx.x;
  const float *xr = x + m * ldx;
  const int64_t nvec = (K + 3) / 4;
  const bool fits = nvec <= 256LL * VPT;

  float4 v[VPT];
  float acc = 0.0f;
  if (fits) {
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int64_t f = t + 256LL * i;
      if (f < nvec) {
        v[i] = mask4(ld4(xr + 4 * f), 4 * f, K);
        float q0 = v[i].x * v[i].x;
        acc = acc + q0;
        float q1 = v[i].y * v[i].y;
        acc = acc + q1;
        float q2 = v[i].z * v[i].z;
        acc = acc + q2;
        float q3 = v[i].w * v[i].w;
        acc = acc + q3;
      } else {
        v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  } else {
    for (int64_t f = t; f < nvec; f += 256) {
      float4 u = mask4(ld4(xr + 4 * f), 4 * f, K);
      float q0 = u.x * u.x;
      acc = acc + q0;
      float q1 = u.y * u.y;
      acc = acc + q1;
      float q2 = u.z * u.z;
      acc = acc + q2;
      float q3 = u.w * u.w;
      acc = acc + q3;
    }
  }
  // Masked lanes contribute +0 (0*0), which leaves a sum >= +0 unchanged.
  lds[t] = acc;
  __syncthreads();
  const int lane = t & 63;
  float u = (lds[lane] + lds[lane + 128]) + (lds[lane + 64] + lds[lane + 192]);
#pragma unroll
  for (int h = 32; h >= 1; h >>= 1) {
    const float o = __shfl_down(u, h, 64);
    u = u + o;
  }
  const float T = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, u), 0));
  const float ms = T / (float)K;
  const float r = sqrtf(ms + eps_n);
  const float y = 1.0f / r;

  auto norm4 = [&](float4 u, int64_t k) {
    float4 o;
    o.x = div_by(u.x, r, y);
    o.y = div_by(u.y, r, y);
    o.z = div_by(u.z, r, y);
    o.w = div_by(u.w, r, y);
    if (g) {
      // g holds exactly K floats: no vector read past its end.
      float4 gg;
      if (k + 3 < K) {
        gg = ld4(g + k);
      } else {
        gg.x = g[k];
        gg.y = k + 1 < K ? g[k + 1] : 0.0f;
        gg.z = k + 2 < K ? g[k + 2] : 0.0f;
        gg.w = 0.0f;
      }
      o.x = o.x * gg.x;
      o.y = o.y * gg.y;
      o.z = o.z * gg.z;
      o.w = o.w * gg.w;
    }
    return o;
  };

  float a = 0.0f;
  if (fits) {
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int64_t f = t + 256LL * i;
      if (f < nvec) {
        v[i] = norm4(v[i], 4 * f);
        a = fmaxf(a, amax4(v[i]));
      }
    }
  } else {
    for (int64_t f = t; f < nvec; f += 256)
      a = fmaxf(a, amax4(norm4(mask4(ld4(xr + 4 * f), 4 * f, K), 4 * f)));
  }
  a = wave_max(a);
  if ((t & 63) == 0) red[t >> 6] = a;
  __syncthreads();
  a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float a127 = a / 127.0f;
  const float sc = a127 + eps;
  if (t == 0) s[m] = sc;
  int8_t *qr = xq + m * ldq;
  if (fits) {
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int64_t f = t + 256LL * i;
      if (f < nvec) store_q4(qr, 4 * f, K, v[i], sc);
    }
  } else {
    for (int64_t f = t; f < nvec; f += 256)
      store_q4(qr, 4 * f, K, norm4(mask4(ld4(xr + 4 * f), 4 * f, K), 4 * f), sc);
  }
}

}  // namespace

hipError_t launch_quant_act(const float *x, int64_t ldx, int64_t M, int64_t K, float eps,
                            int8_t *xq, int64_t ldq, float *s, hipStream_t st) {
  const int64_t nvec = ceil_div(K, 4);
  if (nvec <= 64) {
    hipLaunchKernelGGL((quant_act_kernel<64, 1>), dim3(ceil_div(M, 4)), dim3(256), 0, st, x, ldx,
                       M, K, eps, xq, ldq, s);
  } else if (nvec <= 128) {
    hipLaunchKernelGGL((quant_act_kernel<64, 2>), dim3(ceil_div(M, 4)), dim3(256), 0, st, x, ldx,
                       M, K, eps, xq, ldq, s);
  } else if (nvec <= 256) {
    hipLaunchKernelGGL((quant_act_kernel<64, 4>), dim3(ceil_div(M, 4)), dim3(256), 0, st, x, ldx,
                       M, K, eps, xq, ldq, s);
  } else if (nvec <= 512) {
    hipLaunchKernelGGL((quant_act_kernel<256, 2>), dim3(M), dim3(256), 0, st, x, ldx, M, K, eps,
                       xq, ldq, s);
  } else if (nvec <= 1024) {
    hipLaunchKernelGGL((quant_act_kernel<256, 4>), dim3(M), dim3(256), 0, st, x, ldx, M, K, eps,
                       xq, ldq, s);
  } else {
    hipLaunchKernelGGL((quant_act_kernel<256, 8>), dim3(M), dim3(256), 0, st, x, ldx, M, K, eps,
                       xq, ldq, s);
  }
  return hipGetLastError();
}

hipError_t launch_rmsnorm_quant_act(const float *x, int64_t ldx, const float *g, int64_t M,
                                    int64_t K, float eps_n, float eps, int8_t *xq, int64_t ldq,
                                    float *s, hipStream_t st) {
  const int64_t nvec = ceil_div(K, 4);
  if (nvec <= 256) {
    hipLaunchKernelGGL((rmsnorm_quant_kernel<1>), dim3(M), dim3(256), 0, st, x, ldx, g, M, K,
                       eps_n, eps, xq, ldq, s);
  } else if (nvec <= 512) {
    hipLaunchKernelGGL((rmsnorm_quant_kernel<2>), dim3(M), dim3(256), 0, st, x, ldx, g, M, K,
                       eps_n, eps, xq, ldq, s);
  } else if (nvec <= 1024) {
    hipLaunchKernelGGL((rmsnorm_quant_kernel<4>), dim3(M), dim3(256), 0, st, x, ldx, g, M, K,
                       eps_n, eps, xq, ldq, s);
  } else {
    hipLaunchKernelGGL((rmsnorm_quant_kernel<8>), dim3(M), dim3(256), 0, st, x, ldx, g, M, K,
                       eps_n, eps, xq, ldq, s);
  }
  return hipGetLastError();
}

}  // namespace ug

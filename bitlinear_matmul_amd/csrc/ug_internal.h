// Internal declarations shared by the libug translation units: kernel
// launchers (called by the entry points in api.hip after validation) and
// small device helpers.  Nothing here is part of the ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <vector>
#include <stdint.h>

#include "../../include/ug.h"

namespace ug {

constexpr int kAbsmeanChunk = 8192;   // elements per stage-1 chunk
constexpr int kAbsmeanLanes = 256;    // lanes per chunk / per fold

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

// Launchers: return the hipError_t of the launch (hipSuccess on success).
hipError_t launch_quant_act(const float *x, int64_t ldx, int64_t M, int64_t K,
                            float eps, int8_t *xq, int64_t ldq, float *s,
                            hipStream_t st);
hipError_t launch_rmsnorm_quant_act(const float *x, int64_t ldx, const float *g,
                                    int64_t M, int64_t K, float eps_n, float eps,
                                    int8_t *xq, int64_t ldq, float *s,
                                    hipStream_t st);
hipError_t launch_absmean(const float *W, int64_t ldw, int64_t N, int64_t K,
                          float eps, int8_t *wq, int64_t ldq, float *beta,
                          float *partials, hipStream_t st);
hipError_t launch_pack(const int8_t *wq, int64_t ldq, int64_t N, int64_t K,
                       uint8_t *packed, int64_t ldp, int32_t *bad,
                       hipStream_t st);
hipError_t launch_unpack(const uint8_t *packed, int64_t ldp, int64_t N,
                         int64_t K, int8_t *wq, int64_t ldq, int32_t *bad,
                         hipStream_t st);
// One GEMV problem as the matrix-core GEMV kernel sees it (device-side
// descriptor; also the element of a grouped plan).
struct GemvDesc {
  const float *x;      // fp32 activations quantized inside the launch, or null
  int64_t ldx;
  const int8_t *xq;    // int8 activations (x == null), else optional output
  int64_t ldxq;
  float *s;            // row scales: input (x == null) or optional output
  const uint8_t *w;    // weights, UG_W_I8 or UG_W_PACK5 rows of ldw bytes
  int64_t ldw;
  const float *beta;
  int32_t *acc;
  int64_t ldacc;
  float *y;
  int64_t ldy;
  float eps;           // activation-quantization eps (x != null)
  int32_t wfmt;
  int32_t M, N, K;
  int32_t mb;          // 16-row activation blocks: 1, 2 or 4
  int32_t items;       // work items (sets of 16-row groups) of this problem
  int32_t item_begin;  // first item of this problem in a grouped plan
};

constexpr int kGemvBlocks = 256;  // at most one GEMV block per CU

// One block of a GEMV launch: problem p and its item range [i0, i1) (fine
// split), or the first problem p and the plan-wide item range (stream split),
// with a copy of problem p's descriptor (one load at block start).
struct GemvBlock {
  GemvDesc d;
  int32_t p, i0, i1, pad;
};

// Plans a group of problems for the matrix-core GEMV: picks the split (fine
// or stream), fills mb, items and item_begin of every descriptor and one
// GemvBlock per block to launch.  Returns the variant
// (512 * fused + 256 * fine + 16 * wfmt + mb; fused: the fine split with fp32
// activations), or -1 if the problems cannot share a launch.
int gemv_plan(GemvDesc *descs, int count, std::vector<GemvBlock> &blocks);
// Blocks to launch for `total_items` items of the stream split.
int gemv_grid(int64_t total_items);
// Whether the activations of a problem fit the kernel's LDS staging area
// (required when the launch quantizes fp32 activations).
bool gemv_stages_x(int wfmt, int64_t M, int64_t K);
hipError_t launch_gemv_grouped(const GemvDesc *plan_dev, const GemvBlock *blocks_dev, int32_t count,
                               int32_t grid, int32_t variant, hipStream_t st);
hipError_t launch_gemv(const int8_t *xq, int64_t ldx, const float *s,
                       const void *w, int wfmt, int64_t ldw, const float *beta,
                       int64_t M, int64_t N, int64_t K, int32_t *acc,
                       int64_t ldacc, float *y, int64_t ldy, hipStream_t st);
// Bytes of the GEMM's K-split area (tile counters at offset 0, then one
// partial tile per block); the same size and layout for every shape.
size_t gemm_split_area_bytes();
// split: NULL, or gemm_split_area_bytes() bytes of device memory (any
// contents: counters are tagged per launch).
hipError_t launch_gemm_i8(const int8_t *xq, int64_t ldx, const float *s,
                          const int8_t *w, int64_t ldw, const float *beta,
                          int64_t M, int64_t N, int64_t K, int32_t *acc,
                          int64_t ldacc, float *y, int64_t ldy, void *split,
                          hipStream_t st);

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------

// Fold 256 per-thread values pairwise in the fixed order
//   v_t += v_{t+h} for h = 128, 64, ..., 1
// (256-thread block; lds must hold 256 floats).  The result is valid in
// thread 0 and is also returned to every thread.  Ends with a barrier, so
// lds may be reused afterwards.
__device__ inline float fold256(float v, float *lds) {
  const int t = threadIdx.x;
  lds[t] = v;
  __syncthreads();
  if (t < 128) lds[t] = lds[t] + lds[t + 128];
  __syncthreads();
  if (t < 64) {
    float u = lds[t] + lds[t + 64];
    // h = 32 .. 1 inside wave 0: lane t takes lane t+h's value.
#pragma unroll
    for (int h = 32; h >= 1; h >>= 1) {
      float o = __shfl_down(u, h, 64);
      u = u + o;
    }
    if (t == 0) lds[0] = u;
  }
  __syncthreads();
  float r = lds[0];
  __syncthreads();
  return r;
}

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int h = 32; h >= 1; h >>= 1) v = fmaxf(v, __shfl_xor(v, h, 64));
  return v;
}

__device__ inline int wave_sum_i32(int v) {
#pragma unroll
  for (int h = 32; h >= 1; h >>= 1) v += __shfl_xor(v, h, 64);
  return v;
}

// clamp(rint(q), lo, hi) as an int; rintf rounds half to even.
__device__ inline int rint_clamp(float q, float lo, float hi) {
  float r = rintf(q);
  r = fminf(fmaxf(r, lo), hi);
  return (int)r;
}

}  // namespace ug

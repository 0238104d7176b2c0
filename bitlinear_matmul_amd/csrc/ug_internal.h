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
// The same beta, then the ternary weights written straight as UG_W_PACK5
// rows of ldp bytes (ldp a multiple of 16, >= ceil(K/5)).
hipError_t launch_absmean_pack5(const float *W, int64_t ldw, int64_t N, int64_t K,
                                float eps, uint8_t *packed, int64_t ldp, float *beta,
                                float *partials, hipStream_t st);
// Chunks the allocation-free absmean's static scratch array holds (64 KB).
constexpr int64_t kStaticChunks = 16384;
// Device address of the current device's static absmean scratch array.
hipError_t static_scratch(float **out);
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
  const float *bias;   // fp32 [N] added to y, or null
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

constexpr int kGemvBlocks = 256;    // at most one GEMV block per CU
constexpr int kGemvFineWaves = 8;   // waves of a fine-split GEMV block

// One block of the fine GEMV split: every value its waves need, precomputed,
// in 144 bytes that the planner places in a table starting at a 128-byte
// boundary; the block reads all of it with scalar loads issued together
// (one round trip).
struct FineBlock {
  const void *x;       // fp32 activations (quantized in the launch) or x_q
  const uint8_t *w;    // weight rows of ldw bytes
  const float *beta;
  const float *bias;   // fp32 [N] added to y, or null
  float *y;            // [M][ldy], or null
  int32_t *acc;        // [M][ldacc], or null
  float *s;            // x_q given: its row scales; fp32 given: output or null
  int8_t *xq_out;      // fp32 given: x_q output [M][ldxq_out], or null
  int32_t ldx;         // bytes between activation rows
  int32_t ldw, ldy, ldacc, ldxq_out;
  float eps;
  int32_t N, K;
  int32_t i0;          // the block's first item (16 weight rows)
  // M | items << 8 | S << 16: activation rows (1..16), items of the block
  // (1..16), K steps (64 weight bytes of a row) per item (one dword: scalar
  // loads fetch whole dwords)
  uint32_t shape;
  // wave w: byte 0 = item (from i0) and byte 1 = step of its first piece
  // (a block orders its pieces step-major);
  // byte 2 = row and byte 3 = chunk of its first activation tile
  uint32_t wave_start[kGemvFineWaves];
  int32_t pad[2];
};
static_assert(sizeof(FineBlock) == 144, "fine block layout");

// One block of a GEMV launch: problem p and its item range [i0, i1) (fine
// split), or the first problem p and the plan-wide item range (stream split),
// with a copy of problem p's descriptor (one load at block start).
struct GemvBlock {
  GemvDesc d;
  int32_t p, i0, i1, pad;
};

// Plans a group of problems for the matrix-core GEMV: picks the split (fine
// or stream), fills mb, items and item_begin of every descriptor and one
// table entry per block to launch.  Returns the variant
// (8192 * spread + 4096 * tiny + 2048 * chunked + 1024 * short + 512 * fused +
// 256 * fine + 16 * wfmt + mb; spread: the stream split of five-trit weights
// at mb 1 with the spread activation staging (every problem's rows fit it);
// fused: the fine split with fp32 activations; short: the
// fine split's variant for at most 4 pieces and 2 activation tiles per wave;
// tiny (with short): at most 3 pieces and 1 tile per wave; chunked: the
// stream split staging activations chunk by chunk, when some problem's rows
// do not fit the staging area), -1 if the problems cannot share a launch, or
// -2 if the group needs the chunked split and also has fp32 activations to
// quantize (the chunked kernel takes x_q only).
// The fine split fills `fine` (and leaves `blocks` empty), the stream split
// fills `blocks`.
int gemv_plan(GemvDesc *descs, int count, std::vector<GemvBlock> &blocks,
              std::vector<FineBlock> &fine);
// Blocks to launch for `total_items` items of the stream split.
int gemv_grid(int64_t total_items);
// Reorders a grouped launch's fine-split block table so that the blocks of
// one problem run on as few XCDs as possible: each XCD's L2 then fetches the
// problem's activation row once instead of every XCD fetching it.
void fine_xcd_order(std::vector<FineBlock> &fine);
// Whether the activations of a problem fit the kernel's LDS staging area
// (required when the launch quantizes fp32 activations).
bool gemv_stages_x(int wfmt, int64_t M, int64_t K);
// table: the plan's GemvBlock table (stream split) or FineBlock table (fine
// split, 128-byte aligned).
hipError_t launch_gemv_grouped(const GemvDesc *plan_dev, const void *table, int32_t count,
                               int32_t grid, int32_t variant, hipStream_t st);
hipError_t launch_gemv(const int8_t *xq, int64_t ldx, const float *s,
                       const void *w, int wfmt, int64_t ldw, const float *beta,
                       const float *bias,
                       int64_t M, int64_t N, int64_t K, int32_t *acc,
                       int64_t ldacc, float *y, int64_t ldy, hipStream_t st);
// Compute units of the current device (0 if it cannot be queried).
int device_cus();
// Straight-through backward: dx = g W and dW = g^T x on the fp32 matrix
// cores, db = column sums of g; `part` (backward_workspace_bytes) holds the
// column chunk sums and the products' partial tiles.  Null outputs are
// skipped.
size_t backward_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_backward(const float *g, int64_t ldg, const float *x, int64_t ldx,
                           const float *W, int64_t ldw, int64_t M, int64_t N, int64_t K,
                           float *dx, int64_t lddx, float *dW, int64_t lddw, float *db,
                           float *part, hipStream_t st);
// Matrix-core issue-rate probe: `blocks` blocks of back-to-back MFMAs.
hipError_t launch_mfma_rate(int kind, int blocks, int iters, int32_t *sink, hipStream_t st);
hipError_t launch_hbm_read(const void *buf, uint64_t bytes, int blocks, int walk, uint32_t *sink,
                           hipStream_t st);
// Top-k sampling: one block per row of logits.
hipError_t launch_sample_topk(const float *logits, int64_t ld, int64_t B, int64_t V, int64_t k,
                              float temp, const float *u, int32_t *tok, int32_t *idx_out,
                              int64_t ldi, float *val_out, int64_t ldv, float *prob_out,
                              int64_t ldp, hipStream_t st);
// Causal attention over a key/value cache: partials per 256-key chunk in
// `part` (attention_workspace_bytes), then one combine per (row, head).
size_t attention_workspace_bytes(int64_t M, int64_t pos0, int64_t H, int64_t dh);
hipError_t launch_attention(const float *q, int64_t ldq, const float *kc, int64_t ldk,
                            const float *vc, int64_t ldv, int64_t M, int64_t pos0, int64_t H,
                            int64_t dh, float *out, int64_t ldo, float *part, hipStream_t st);
// Bytes of the GEMM's K-split area (tile counters at offset 0, then one
// partial tile per block); the same size and layout for every shape.
size_t gemm_split_area_bytes();
// Bytes at the start of a GEMM workspace that hold the K-split tile
// counters; nothing else is ever written there.
constexpr size_t kGemmCounterBytes = 2048;
// split: NULL, or gemm_split_area_bytes() bytes of device memory (any
// contents: counters are tagged per launch).  tile: -1 (the time model's
// choice), 0 (256 x 256 tiles) or 1 (256 x 160); splits: -1 (the model's
// choice) or a K-split count, used where it fits (else 1).
hipError_t launch_gemm_i8(const int8_t *xq, int64_t ldx, const float *s,
                          const int8_t *w, int64_t ldw, const float *beta,
                          const float *bias,
                          int64_t M, int64_t N, int64_t K, int32_t *acc,
                          int64_t ldacc, float *y, int64_t ldy, void *split,
                          int tile, int splits, hipStream_t st);

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

// Max over the 64 lanes of a wave, returned to every lane.  Registers only
// (cross-lane shuffles through ds_bpermute would be LDS round trips, queued
// behind whatever else the block has sent to LDS): DPP butterflies give
// every lane its 16-lane row's max, then the four row maxima are read out.
template <int CTRL>
__device__ inline float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xf, 0xf, false));
}
__device__ inline float wave_max(float v) {
  v = fmaxf(v, dpp_f32<0xb1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f32<0x4e>(v));   // quad_perm [2,3,0,1]: quad max
  v = fmaxf(v, dpp_f32<0x141>(v));  // row_half_mirror: max of 8
  v = fmaxf(v, dpp_f32<0x140>(v));  // row_mirror: max of the 16-lane row
  const int b = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
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

// Activation code of v with the row scale s: clamp(rint(v / s), -127, 127).
__device__ inline int q8(float v, float s) { return rint_clamp(v / s, -127.0f, 127.0f); }

// The same code without the division in almost every case.  q' = v * rs,
// with rs = v_rcp_f32(s) (at most 1 ulp from 1/s), is within
// 1.5 ulp + 0.5 ulp of the correctly rounded quotient fl(v/s): below 3.1e-5
// wherever |v/s| < 128.  rint(fl(v/s)) can differ from rint(q') only if a
// half-integer lies between them, so when q' is more than kTieBand from
// every half-integer the codes agree; otherwise (about 1e-4 of the values)
// the exact quotient is formed.  Above 127.5 both sides clamp to 127 (and
// likewise below -127.5), NaN and infinities take the same clamp in both.
// Only for scales with scale_fast_ok(s), so that rs is finite and accurate.
constexpr float kTieBand = 6.103515625e-05f;  // 2^-14, twice the bound above
__device__ inline int q8_fast(float v, float s, float rs) {
  const float q = v * rs;
  const float r = rintf(q);
  if (__builtin_expect(fabsf(q - r) > 0.5f - kTieBand, 0)) return q8(v, s);
  return (int)fminf(fmaxf(r, -127.0f), 127.0f);
}
__device__ inline bool scale_fast_ok(float s) { return s >= 0x1p-100f && s <= 0x1p100f; }

// The codes of four values with one scale: q8 of each, bit for bit.  The
// fast products decide all four unless the scale is out of the fast range
// or a product lies near a tie (q8_fast's test); then all four take the
// exact quotient.  One branch per four codes instead of one per code.
__device__ inline void q8x4(float4 v, float s, int &a, int &b, int &c, int &d) {
  const float rs = __builtin_amdgcn_rcpf(s);
  const float qa = v.x * rs, qb = v.y * rs, qc = v.z * rs, qd = v.w * rs;
  const float ra = rintf(qa), rb = rintf(qb), rc = rintf(qc), rd = rintf(qd);
  const float lim = 0.5f - kTieBand;
  const bool exact = !scale_fast_ok(s) | (fabsf(qa - ra) > lim) | (fabsf(qb - rb) > lim) |
                     (fabsf(qc - rc) > lim) | (fabsf(qd - rd) > lim);
  if (__builtin_expect(exact, 0)) {
    a = q8(v.x, s);
    b = q8(v.y, s);
    c = q8(v.z, s);
    d = q8(v.w, s);
  } else {
    a = (int)fminf(fmaxf(ra, -127.0f), 127.0f);
    b = (int)fminf(fmaxf(rb, -127.0f), 127.0f);
    c = (int)fminf(fmaxf(rc, -127.0f), 127.0f);
    d = (int)fminf(fmaxf(rd, -127.0f), 127.0f);
  }
}

}  // namespace ug

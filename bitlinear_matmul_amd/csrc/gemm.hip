// Prefill GEMM (gfx950): y = (x_q W_q^T)(s beta) for any number of rows,
// as a dense int8 contraction on the matrix cores.
//
// "ultragraph - when the graph is the 1-bit LLM, part 2", section
// "autograd on a byte-graph": integer matmul x_q W_q^T, then one rescale by
// s*beta.  Ternary weights are exact in int8, so the contraction runs on
// v_mfma_i32_16x16x64_i8 with int32 accumulators; nothing is approximated.
//
// Both operands are K-contiguous (x_q [M][K], W_q [N][K]), which is the
// layout the MFMA operands want: a lane holds 16 consecutive K bytes of one
// row of A and the same 16 K positions of one row of W.  Any K order that
// is the same for A and B gives the same exact integer sum.
//
// Tiling: 128 x 128 output tile per 256-thread block, 2 x 2 waves of 64 x 64
// (4 x 4 MFMA tiles each), K step 64, operands staged through LDS with a
// 16-byte row pad, next K step prefetched into registers while the MFMAs of
// the current one run.
#include "ug_internal.h"

namespace ug {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDS_STRIDE = BK + 16;  // bytes per staged row

// Load the 16-byte piece (row, k0..k0+15) of a K-contiguous int8 matrix,
// zero outside rows < R or K positions >= K.
__device__ inline uint4 load_piece(const int8_t *base, int64_t ld, int64_t row, int64_t R,
                                   int64_t k0, int64_t K, bool mask_k) {
  if (row >= R || k0 >= K) return make_uint4(0, 0, 0, 0);
  uint4 v = *reinterpret_cast<const uint4 *>(base + row * ld + k0);
  if (mask_k && k0 + 16 > K) {
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (k0 + i >= K) w[i >> 2] &= ~(0xffu << (8 * (i & 3)));
    v = make_uint4(w[0], w[1], w[2], w[3]);
  }
  return v;
}

__global__ __launch_bounds__(256) void gemm_i8_kernel(const int8_t *__restrict__ xq, int64_t ldx,
                                                      const float *__restrict__ s,
                                                      const int8_t *__restrict__ w, int64_t ldw,
                                                      const float *__restrict__ beta, int64_t M,
                                                      int64_t N, int64_t K,
                                                      int32_t *__restrict__ acc, int64_t ldacc,
                                                      float *__restrict__ y, int64_t ldy) {
  __shared__ __attribute__((aligned(16))) int8_t As[BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) int8_t Bs[BN * LDS_STRIDE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int64_t tm = (int64_t)blockIdx.y * BM;
  const int64_t tn = (int64_t)blockIdx.x * BN;

  // Global -> LDS mapping: 512 pieces of 16 B per operand tile, 2 per thread.
  int prow[2], pcol[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = tid + 256 * i;
    prow[i] = p >> 2;
    pcol[i] = (p & 3) * 16;
  }

  v4i c[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) c[i][j] = v4i{0, 0, 0, 0};

  uint4 ra[2], rb[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    ra[i] = load_piece(xq, ldx, tm + prow[i], M, pcol[i], K, true);
    rb[i] = load_piece(w, ldw, tn + prow[i], N, pcol[i], K, false);
  }

  const int arow = lane & 15;        // row of the 16x16 operand tile
  const int akof = (lane >> 4) * 16;  // K bytes [akof, akof + 16) of the step

  for (int64_t k0 = 0; k0 < K; k0 += BK) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      *reinterpret_cast<uint4 *>(As + prow[i] * LDS_STRIDE + pcol[i]) = ra[i];
      *reinterpret_cast<uint4 *>(Bs + prow[i] * LDS_STRIDE + pcol[i]) = rb[i];
    }
    __syncthreads();
    if (k0 + BK < K) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        ra[i] = load_piece(xq, ldx, tm + prow[i], M, k0 + BK + pcol[i], K, true);
        rb[i] = load_piece(w, ldw, tn + prow[i], N, k0 + BK + pcol[i], K, false);
      }
    }
    v4i a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a[i] = *reinterpret_cast<const v4i *>(As + (wm * 64 + 16 * i + arow) * LDS_STRIDE + akof);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      b[j] = *reinterpret_cast<const v4i *>(Bs + (wn * 64 + 16 * j + arow) * LDS_STRIDE + akof);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        c[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i], b[j], c[i][j], 0, 0, 0);
  }

  // Epilogue: lane holds C[4*(lane/16) + r][lane % 16] of each 16x16 tile.
  const float bt = beta[0];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t m = tm + wm * 64 + 16 * i + 4 * (lane >> 4) + r;
      if (m >= M) continue;
      const float scale = s[m] * bt;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t n = tn + wn * 64 + 16 * j + (lane & 15);
        if (n >= N) continue;
        const int v = c[i][j][r];
        if (acc) acc[m * ldacc + n] = v;
        if (y) y[m * ldy + n] = (float)v * scale;
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_i8(const int8_t *xq, int64_t ldx, const float *s, const int8_t *w,
                          int64_t ldw, const float *beta, int64_t M, int64_t N, int64_t K,
                          int32_t *acc, int64_t ldacc, float *y, int64_t ldy, hipStream_t st) {
  dim3 grid((unsigned)ceil_div(N, BN), (unsigned)ceil_div(M, BM));
  hipLaunchKernelGGL(gemm_i8_kernel, grid, dim3(256), 0, st, xq, ldx, s, w, ldw, beta, M, N, K,
                     acc, ldacc, y, ldy);
  return hipGetLastError();
}

}  // namespace ug

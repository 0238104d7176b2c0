// Straight-through backward of the BitLinear layer (gfx950).
//
// "ultragraph - when the graph is the 1-bit LLM, part 2", section "autograd
// on a byte-graph": backward, the straight-through estimator pretends the
// quantizers and the per-row scale were the identity and routes the
// gradient into the fp32 master weights:
//     dL/dx = g W,   dL/dW = g^T x,   dL/db = sum over rows of g
// with g = dL/dy [M][N], W [N][K] (the masters) and x [M][K] (the layer's
// fp32 input).  The two products are dense fp32 contractions and run on the
// fp32 matrix cores (v_mfma_f32_16x16x4f32); the bias gradient is a column
// sum in a fixed order.
//
// gemm_f32 computes C[i][j] = sum_p A(i, p) B(p, j) with B(p, j) = b[p][j]
// (j contiguous) and A either p-contiguous (A(i, p) = a[i][p]: dx, A = g) or
// i-contiguous (A(i, p) = a[p][i]: dW, A = g read as g^T).  Blocks of 256
// threads own 128 x 128 tiles of C, each wave a 64 x 64 quarter (4 x 4 MFMA
// tiles).  A product with too few tiles to fill the chip for several rounds
// (dx at 2048 x 2560: 320 tiles on 256 compute units) is cut along the
// contraction into S pieces whose partial tiles a second kernel adds in
// piece order (no atomics: the same bits on every run); the reduction moves 16 p at a time through double-buffered LDS
// (p-major rows padded to 144 floats, so the four p-rows one fragment read
// touches fall in different banks), the next step's loads in registers
// while the current one multiplies, one barrier per step.
#include "ug_internal.h"

namespace ug {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kTile = 128;     // C tile edge
constexpr int kStep = 16;      // p per step
constexpr int kPitch = 144;    // LDS row (one p) in floats
constexpr int kXcd = 8;
constexpr int kMaxPieces = 8;  // contraction pieces of a few-tile product

__device__ inline float4 load4_guarded(const float *base, int64_t row, int64_t ld, int col,
                                       int64_t rows, int cols) {
  if (row >= rows) return make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  const float *p = base + row * ld + col;
  if (col + 3 < cols) return *reinterpret_cast<const float4 *>(p);
  float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if (col < cols) v.x = p[0];
  if (col + 1 < cols) v.y = p[1];
  if (col + 2 < cols) v.z = p[2];
  return v;
}

template <bool A_PCONTIG>
__global__ __launch_bounds__(256) void gemm_f32(const float *__restrict__ a, int64_t lda,
                                                const float *__restrict__ b, int64_t ldb, int I,
                                                int J, int P, int S, float *__restrict__ c,
                                                int64_t ldc, int64_t slab) {
  __shared__ __attribute__((aligned(16))) float As[2][kStep * kPitch];  // [p][i]
  __shared__ __attribute__((aligned(16))) float Bs[2][kStep * kPitch];  // [p][j]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wi = wave >> 1, wj = wave & 1;
  // XCD x runs blocks x, x + 8, ...: give it a contiguous run of tiles
  // (neighbours along j share the A panel in that XCD's L2)
  const int nj = (J + kTile - 1) / kTile;
  const int tiles = nj * ((I + kTile - 1) / kTile);
  const int per = (int)(gridDim.x / kXcd);
  const int vb0 = (int)(blockIdx.x % kXcd) * per + (int)(blockIdx.x / kXcd);
  if (vb0 >= tiles * S) return;
  // work item vb0: tile vb0 % tiles, contraction piece vb0 / tiles (of S
  // pieces of whole steps); piece s writes its partial tile to slab s of c
  const int vb = vb0 % tiles, sp = vb0 / tiles;
  const int nsteps = (P + kStep - 1) / kStep;
  const int pb = (int)((int64_t)sp * nsteps / S) * kStep;
  const int pe = min(P, (int)((int64_t)(sp + 1) * nsteps / S) * kStep);
  c += (int64_t)sp * slab;
  const int i0 = (vb / nj) * kTile, j0 = (vb % nj) * kTile;

  float4 ra[2], rb[2];
  auto gload = [&](int p0) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // B: rows p (16), 128 j; thread: row (tid >> 5) + 8h, four j at (tid & 31) * 4
      const int r = (tid >> 5) + 8 * h, c4 = (tid & 31) * 4;
      rb[h] = load4_guarded(b, p0 + r, ldb, j0 + c4, pe, J);
      if (A_PCONTIG) {
        // A rows i (128) x 16 p (64 bytes): thread t takes row t / 2, p
        // 8 (t % 2) + 4 h .. + 3 (two threads read a row's 64 bytes)
        ra[h] = load4_guarded(a, i0 + (tid >> 1), lda, p0 + 8 * (tid & 1) + 4 * h, I, pe);
      } else {
        ra[h] = load4_guarded(a, p0 + r, lda, i0 + c4, pe, I);
      }
    }
  };
  auto sstore = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = (tid >> 5) + 8 * h, c4 = (tid & 31) * 4;
      *reinterpret_cast<float4 *>(&Bs[buf][r * kPitch + c4]) = rb[h];
      if (A_PCONTIG) {
        const int i = tid >> 1, p = 8 * (tid & 1) + 4 * h;
        As[buf][(p + 0) * kPitch + i] = ra[h].x;
        As[buf][(p + 1) * kPitch + i] = ra[h].y;
        As[buf][(p + 2) * kPitch + i] = ra[h].z;
        As[buf][(p + 3) * kPitch + i] = ra[h].w;
      } else {
        *reinterpret_cast<float4 *>(&As[buf][r * kPitch + c4]) = ra[h];
      }
    }
  };

  v4f acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  gload(pb);
  sstore(0);
  __syncthreads();
  const int ai = wi * 64 + (lane & 15), bj = wj * 64 + (lane & 15), pq = lane >> 4;
  int cur = 0;
  for (int p0 = pb; p0 < pe; p0 += kStep) {
    const bool more = p0 + kStep < pe;
    if (more) gload(p0 + kStep);
#pragma unroll
    for (int kk = 0; kk < kStep / 4; ++kk) {
      const float *arow = &As[cur][(4 * kk + pq) * kPitch + ai];
      const float *brow = &Bs[cur][(4 * kk + pq) * kPitch + bj];
      float av[4], bv[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        av[t] = arow[16 * t];
        bv[t] = brow[16 * t];
      }
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y)
          acc[x][y] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[x], bv[y], acc[x][y], 0, 0, 0);
    }
    if (more) sstore(cur ^ 1);
    __syncthreads();
    cur ^= 1;
  }

  // lane (j = l % 16, q = l / 16) holds C[4 q + r][j] of each 16 x 16 tile
#pragma unroll
  for (int x = 0; x < 4; ++x) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = i0 + wi * 64 + 16 * x + 4 * pq + r;
      if (i >= I) continue;
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        const int j = j0 + wj * 64 + 16 * y + (lane & 15);
        if (j < J) c[(int64_t)i * ldc + j] = acc[x][y][r];
      }
    }
  }
}

// db, stage 1: thread n of block (x, y) adds g[m][n] for the 32 rows
// m in [32 y, 32 y + 32) in increasing m; stage 2: thread n adds the
// chunk sums in increasing chunk order.
constexpr int kColChunk = 32;

__global__ __launch_bounds__(256) void colsum_chunks(const float *__restrict__ g, int64_t ldg,
                                                     int M, int N, float *__restrict__ part) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  const int m0 = blockIdx.y * kColChunk, m1 = min(M, m0 + kColChunk);
  float s = 0.0f;
  for (int m = m0; m < m1; ++m) s = s + g[(int64_t)m * ldg + n];
  part[(int64_t)blockIdx.y * N + n] = s;
}

__global__ __launch_bounds__(64) void colsum_finish(const float *__restrict__ part, int chunks,
                                                    int N, float *__restrict__ db) {
  const int n = blockIdx.x * 64 + threadIdx.x;
  if (n >= N) return;
  float s = 0.0f;
  // the chunk sums in order, 16 loads in flight at a time
  int c = 0;
  for (; c + 16 <= chunks; c += 16) {
    float v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = part[(int64_t)(c + u) * N + n];
#pragma unroll
    for (int u = 0; u < 16; ++u) s = s + v[u];
  }
  for (; c < chunks; ++c) s = s + part[(int64_t)c * N + n];
  db[n] = s;
}

// C = the S partial tiles (slabs of I x J, pitch J) added in slab order.
__global__ __launch_bounds__(256) void sum_slabs(const float *__restrict__ part, int S,
                                                 int64_t slab, int I, int J,
                                                 float *__restrict__ c, int64_t ldc) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int j4 = (J + 3) / 4;
  if (idx >= (int64_t)I * j4) return;
  const int i = (int)(idx / j4), j = (int)(idx - (int64_t)i * j4) * 4;
  const float *p = part + (int64_t)i * J + j;
  if ((J & 3) == 0 && j + 3 < J) {  // 16-byte aligned: slabs have pitch J
    float4 acc = *reinterpret_cast<const float4 *>(p);
    for (int s = 1; s < S; ++s) {
      const float4 v = *reinterpret_cast<const float4 *>(p + s * slab);
      acc.x = acc.x + v.x;
      acc.y = acc.y + v.y;
      acc.z = acc.z + v.z;
      acc.w = acc.w + v.w;
    }
    *reinterpret_cast<float4 *>(c + (int64_t)i * ldc + j) = acc;
  } else {
    for (int e = j; e < J; ++e) {
      float acc = p[e - j];
      for (int s = 1; s < S; ++s) acc = acc + p[e - j + s * slab];
      c[(int64_t)i * ldc + e] = acc;
    }
  }
}

// Pieces of the contraction: enough work items to fill four rounds of the
// chip when the tiles alone are fewer, each piece at least 256 deep.
int contraction_pieces(int64_t I, int64_t J, int64_t P) {
  const int64_t tiles = ceil_div(I, kTile) * ceil_div(J, kTile);
  int64_t S = 1;
  while (S < kMaxPieces && tiles * S < 1024 && P / (2 * S) >= 256) S *= 2;
  return (int)S;
}

template <bool A_PCONTIG>
hipError_t launch_gemm_f32(const float *a, int64_t lda, const float *b, int64_t ldb, int64_t I,
                           int64_t J, int64_t P, float *c, int64_t ldc, float *pieces,
                           hipStream_t st) {
  const int64_t tiles = ceil_div(I, kTile) * ceil_div(J, kTile);
  const int S = pieces ? contraction_pieces(I, J, P) : 1;
  const int64_t blocks = ceil_div(tiles * S, kXcd) * kXcd;
  const int64_t slab = I * J;  // a partial tile set, pitch J
  hipLaunchKernelGGL(gemm_f32<A_PCONTIG>, dim3((unsigned)blocks), dim3(256), 0, st, a, lda, b,
                     ldb, (int)I, (int)J, (int)P, S, S > 1 ? pieces : c, S > 1 ? J : ldc, slab);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1) return e;
  hipLaunchKernelGGL(sum_slabs, dim3((unsigned)ceil_div(I * ceil_div(J, 4), 256)), dim3(256), 0,
                     st, pieces, S, slab, (int)I, (int)J, c, ldc);
  return hipGetLastError();
}

}  // namespace

size_t backward_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  const size_t db = (size_t)(4 * ceil_div(M, kColChunk) * N);
  const int S = contraction_pieces(M, K, N);  // dx = g W: M x K tiles, N deep
  const size_t dx = S > 1 ? (size_t)(4 * S * M * K) : 0;
  return std::max(db, dx);
}

hipError_t launch_backward(const float *g, int64_t ldg, const float *x, int64_t ldx,
                           const float *W, int64_t ldw, int64_t M, int64_t N, int64_t K,
                           float *dx, int64_t lddx, float *dW, int64_t lddw, float *db,
                           float *part, hipStream_t st) {
  hipError_t e = hipSuccess;
  if (dx) {  // dx[m][k] = sum_n g[m][n] W[n][k]
    e = launch_gemm_f32<true>(g, ldg, W, ldw, M, K, N, dx, lddx, part, st);
    if (e != hipSuccess) return e;
  }
  if (dW) {  // dW[n][k] = sum_m g[m][n] x[m][k]
    e = launch_gemm_f32<false>(g, ldg, x, ldx, N, K, M, dW, lddw, nullptr, st);
    if (e != hipSuccess) return e;
  }
  if (db) {
    const int chunks = (int)ceil_div(M, kColChunk);
    hipLaunchKernelGGL(colsum_chunks, dim3((unsigned)ceil_div(N, 256), (unsigned)chunks),
                       dim3(256), 0, st, g, ldg, (int)M, (int)N, part);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(colsum_finish, dim3((unsigned)ceil_div(N, 64)), dim3(64), 0, st, part,
                       chunks, (int)N, db);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace ug

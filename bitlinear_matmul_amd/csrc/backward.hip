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
// tiles); the reduction moves 16 p at a time through double-buffered LDS
// (p-major rows padded to 144 floats, so the four p-rows one fragment read
// touches fall in different banks), the next step's loads in registers
// while the current one multiplies, one barrier per step.
//
// Four blocks fit a compute unit, so a launch runs in rounds of 4 x CUs
// blocks; a tile count just past a whole number of rounds (dW at
// 6912 x 2560: 1080 tiles on 1024 slots) or short of one round (dx at
// 2048 x 2560: 320 tiles) would leave most of the chip idle for part of
// the run.  So the tiles beyond the last whole round are cut along the
// contraction into S equal pieces, enough for a round of their own (dW: 56
// tiles x 16 pieces of 8 steps; dx: 320 tiles x 4 pieces of 108 steps),
// which run after the whole tiles, one block each.  Blocks that run at the
// same time take the same piece of neighbouring tiles, so they read the
// same contraction rows of the shared operand at the same time (one XCD's
// L2 serves them all), as the whole tiles do.  The pieces land as partial
// tiles in the workspace and a second kernel adds each tile's pieces in
// piece order (no atomics: the same bits on every run on a given device,
// since the cut depends only on the shape and the CU count).
#include "ug_internal.h"

namespace ug {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kTile = 128;     // C tile edge
constexpr int kStep = 16;      // p per step
constexpr int kPitch = 144;    // LDS row (one p) in floats
constexpr int kXcd = 8;

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

// How one product's tiles are dealt to the blocks (one tile or piece
// each): blocks 0 .. dp-1 compute tiles 0 .. dp-1 whole; the rem tiles
// dp .. T-1 are cut into S pieces of the contraction, and the blocks after
// them compute piece v = piece v / rem of tile dp + v mod rem (v < rem S).
struct Share {
  int64_t T;   // tiles of C
  int64_t dp;  // tiles computed whole (a multiple of kXcd)
  int nj;      // tiles along j
  int ns;      // contraction steps (kStep deep) per tile
  int rem;     // tiles cut into pieces
  int S;       // pieces per cut tile
  int npb;     // blocks for the pieces: rem S rounded up to a multiple of kXcd
};

// floats of one partial tile (row-major, pitch kTile)
constexpr int kSlotFloats = kTile * kTile;

template <bool A_PCONTIG>
__global__ __launch_bounds__(256) void gemm_f32(const float *__restrict__ a, int64_t lda,
                                                const float *__restrict__ b, int64_t ldb, int I,
                                                int J, int P, float *__restrict__ c,
                                                int64_t ldc, Share sh, float *__restrict__ part) {
  __shared__ __attribute__((aligned(16))) float As[2][kStep * kPitch];  // [p][i]
  __shared__ __attribute__((aligned(16))) float Bs[2][kStep * kPitch];  // [p][j]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wi = wave >> 1, wj = wave & 1;

  int i0 = 0, j0 = 0, pe = 0;  // the current tile's corner and contraction end
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
  const int ai = wi * 64 + (lane & 15), bj = wj * 64 + (lane & 15), pq = lane >> 4;
  // acc = steps s0 .. s1-1 of tile t's contraction
  auto run = [&](int64_t t, int s0, int s1) __attribute__((always_inline)) {
    i0 = (int)(t / sh.nj) * kTile;
    j0 = (int)(t % sh.nj) * kTile;
    pe = min(P, s1 * kStep);
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y) acc[x][y] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    // (the previous run ended with a barrier: no wave still reads buffer 0)
    gload(s0 * kStep);
    sstore(0);
    __syncthreads();
    int cur = 0;
    for (int p0 = s0 * kStep; p0 < pe; p0 += kStep) {
      const bool more = p0 + kStep < pe;
      if (more) gload(p0 + kStep);
#pragma unroll
      for (int kk = 0; kk < kStep / 4; ++kk) {
        const float *arow = &As[cur][(4 * kk + pq) * kPitch + ai];
        const float *brow = &Bs[cur][(4 * kk + pq) * kPitch + bj];
        float av[4], bv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          av[q] = arow[16 * q];
          bv[q] = brow[16 * q];
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
  };
  // lane (j = l % 16, q = l / 16) holds C[4 q + r][j] of each 16 x 16 tile
  auto store_tile = [&](float *dst, int64_t ld, int rows, int cols) __attribute__((always_inline)) {
#pragma unroll
    for (int x = 0; x < 4; ++x) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = wi * 64 + 16 * x + 4 * pq + r;
        if (i >= rows) continue;
#pragma unroll
        for (int y = 0; y < 4; ++y) {
          const int j = wj * 64 + 16 * y + (lane & 15);
          if (j < cols) dst[(int64_t)i * ld + j] = acc[x][y][r];
        }
      }
    }
  };

  // XCD x runs blocks x, x + 8, ...: give it a contiguous range of the
  // whole tiles and then of the pieces (neighbouring tiles share operand
  // panels in that XCD's L2)
  const int64_t bid = blockIdx.x;
  const int xcd = (int)(bid % kXcd);
  int64_t t;
  int s0 = 0, s1 = sh.ns;
  float *dst;
  int64_t ld = ldc;
  int rows, cols;
  if (bid < sh.dp) {
    t = xcd * (sh.dp / kXcd) + bid / kXcd;
    run(t, s0, s1);
    dst = c + (int64_t)i0 * ldc + j0;
    rows = I - i0;
    cols = J - j0;
  } else {
    const int v = xcd * (sh.npb / kXcd) + (int)((bid - sh.dp) / kXcd);
    if (v >= sh.rem * sh.S) return;
    t = sh.dp + v % sh.rem;
    const int k = v / sh.rem;
    s0 = (int)((int64_t)k * sh.ns / sh.S);
    s1 = (int)((int64_t)(k + 1) * sh.ns / sh.S);
    run(t, s0, s1);
    if (sh.S > 1) {
      dst = part + (int64_t)v * kSlotFloats;
      ld = kTile;
      rows = cols = kTile;
    } else {
      dst = c + (int64_t)i0 * ldc + j0;
      rows = I - i0;
      cols = J - j0;
    }
  }
  store_tile(dst, ld, rows, cols);
}

// C tiles dp .. dp + rem - 1 = their S partial tiles added in piece order;
// thread: four consecutive floats of one tile row.
__global__ __launch_bounds__(256) void sum_pieces(const float *__restrict__ part, int rem, int S,
                                                  int64_t dp, int nj, int I, int J,
                                                  float *__restrict__ c, int64_t ldc) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)rem * (kSlotFloats / 4)) return;
  const int r = (int)(idx / (kSlotFloats / 4)), e = (int)(idx % (kSlotFloats / 4)) * 4;
  const int64_t t = dp + r;
  const int i = (int)(t / nj) * kTile + e / kTile, j = (int)(t % nj) * kTile + e % kTile;
  if (i >= I || j >= J) return;
  const float4 *p = reinterpret_cast<const float4 *>(part + (int64_t)r * kSlotFloats + e);
  const int64_t step = (int64_t)rem * (kSlotFloats / 4);  // piece to piece
  float4 acc = p[0];
  int s = 1;
  for (; s + 4 <= S; s += 4) {  // four pieces' loads in flight
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = p[(s + u) * step];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      acc.x = acc.x + v[u].x;
      acc.y = acc.y + v[u].y;
      acc.z = acc.z + v[u].z;
      acc.w = acc.w + v[u].w;
    }
  }
  for (; s < S; ++s) {
    const float4 v = p[s * step];
    acc.x = acc.x + v.x;
    acc.y = acc.y + v.y;
    acc.z = acc.z + v.z;
    acc.w = acc.w + v.w;
  }
  float *dst = c + (int64_t)i * ldc + j;
  if (j + 3 < J) {
    *reinterpret_cast<float4 *>(dst) = acc;  // ldc % 4 == 0, 16-byte aligned c
  } else {
    dst[0] = acc.x;
    if (j + 1 < J) dst[1] = acc.y;
    if (j + 2 < J) dst[2] = acc.z;
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

// Blocks resident at once: four per compute unit (about 104 VGPRs and
// 36 KB of LDS each).
int resident_blocks() {
  const int cus = device_cus();
  return 4 * (cus > 0 ? cus : 256);
}

// A piece is at least kMinRun steps deep (each costs a 64 KB partial tile
// written and read back) and no tile is cut into more than kMaxPieces.
constexpr int kMinRun = 8;
constexpr int kMaxPieces = 16;

// The tiles beyond the last whole round of B resident blocks (all tiles
// when there are fewer than B) are cut into enough pieces for a round:
// S = ceil(B / rem), at most kMaxPieces and each piece at least kMinRun
// steps deep.
Share plan_share(int64_t I, int64_t J, int64_t P) {
  Share sh{};
  const int B = resident_blocks();
  sh.nj = (int)ceil_div(J, kTile);
  sh.T = ceil_div(I, kTile) * sh.nj;
  sh.ns = (int)ceil_div(P, kStep);
  sh.rem = (int)(sh.T % B);
  sh.dp = sh.T - sh.rem;
  sh.S = 1;
  if (sh.rem > 0)
    sh.S = (int)std::max<int64_t>(
        1, std::min<int64_t>({ceil_div(B, sh.rem), sh.ns / kMinRun, (int64_t)kMaxPieces}));
  sh.npb = (int)round_up((int64_t)sh.rem * sh.S, kXcd);
  return sh;
}

// Workspace of the pieces: one partial tile each (fewer than 2B).
int64_t share_bytes(const Share &sh) {
  return sh.S > 1 ? (int64_t)sh.rem * sh.S * kSlotFloats * 4 : 0;
}

template <bool A_PCONTIG>
hipError_t launch_gemm_f32(const float *a, int64_t lda, const float *b, int64_t ldb, int64_t I,
                           int64_t J, int64_t P, float *c, int64_t ldc, float *part,
                           hipStream_t st) {
  const Share sh = plan_share(I, J, P);
  hipLaunchKernelGGL(gemm_f32<A_PCONTIG>, dim3((unsigned)(sh.dp + sh.npb)), dim3(256), 0, st, a, lda, b,
                     ldb, (int)I, (int)J, (int)P, c, ldc, sh, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || sh.S == 1) return e;
  hipLaunchKernelGGL(sum_pieces,
                     dim3((unsigned)ceil_div((int64_t)sh.rem * (kSlotFloats / 4), 256)),
                     dim3(256), 0, st, part, sh.rem, sh.S, sh.dp, sh.nj, (int)I, (int)J, c, ldc);
  return hipGetLastError();
}

}  // namespace

size_t backward_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  const int64_t db = 4 * ceil_div(M, kColChunk) * N;
  const int64_t dx = share_bytes(plan_share(M, K, N));  // dx = g W: M x K tiles, N deep
  const int64_t dw = share_bytes(plan_share(N, K, M));  // dW = g^T x: N x K tiles, M deep
  return (size_t)std::max({db, dx, dw});
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
    e = launch_gemm_f32<false>(g, ldg, x, ldx, N, K, M, dW, lddw, part, st);
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

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

#include <atomic>
#include <chrono>
#include <random>
#include <type_traits>

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
                                                      const float *__restrict__ beta,
                                                      const float *__restrict__ bias, int64_t M,
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
        if (y) {
          const float o = (float)v * scale;
          y[m * ldy + n] = bias ? o + bias[n] : o;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Large GEMM on v_mfma_i32_32x32x32_i8 (the same int8 rate as the 16x16x64
// form, twice its products per fragment byte read from LDS).  Lane l of that
// MFMA holds A row l%32 and B column l%32 at K bytes [16 (l/32), +16), and
// accumulator element i of lane l is D[8 (i/4) + 4 (l/32) + i%4][l%32].
//
// Output tiles of 256 rows x BN = 32 NT columns per 256-thread block, four
// waves in a WM x WN grid, each with IT x JT MFMA tiles (int32 accumulators
// in AGPRs; one wave per SIMD): 256 x 256 as 2 x 2 waves of 4 x 4 tiles, and
// 256 x 160 as 4 x 1 waves of 2 x 5, which lets N = 2560 fill the GPU with
// whole rounds of tiles.  K step 64, four LDS stages per operand.
//
// Operands go from global memory straight into LDS (buffer loads with the
// LDS destination bit), so no register staging and no LDS store
// instructions.  One such load moves 1 KB: lane l's 16 bytes land at 16 l.
// A stage holds 256 rows x 64 bytes; within row r the 16-byte chunk x sits at
// slot x ^ ((r >> 2) & 3), which makes every MFMA fragment read a
// conflict-free ds_read_b128 (16 consecutive lanes cover all 64 banks) while
// each load still fetches whole 64-byte row pieces.
//
// Step k: MFMAs of its first K half run while the second half's fragments
// are read; then each wave waits for its own loads of step k+1, one barrier
// makes them visible block-wide (and frees the stage read in step k-1), the
// loads of step k+3 are issued into that stage, and the second-half MFMAs run
// while the first-half fragments of step k+1 are read.  Loads therefore have
// two steps to arrive.  Past the last step the loads repeat the last step's
// data into stages nobody reads again, so every step issues the same number
// of loads and the wait counts stay exact.
//
// Edges: buffer loads of rows past M or N return zeros (or leave old data:
// either way only rows and columns that are never stored see it).  In the
// last step the activation bytes past K are zeroed in LDS before use, so
// whatever the weight rows hold there multiplies zeros.  Blocks are mapped to
// tiles so that the blocks one XCD runs together cover a compact rectangle
// of tiles.
constexpr int LBM = 256, LBK = 64;
constexpr int LTHREADS = 256;
constexpr int LTILE = LBM * LBK;  // bytes of one operand tile per stage (B uses BN rows)
constexpr int kXcds = 8;          // blocks are dealt to the XCDs round-robin
constexpr int kGroupM = 4;        // tile rows per group of the tile order

typedef int v4i_ __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// s_waitcnt with only the vector-memory count limited (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}
// Workgroup barrier that orders the compiler's memory operations but adds no
// waits of its own: the waits that make LDS data visible are explicit.
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Zero the bytes of a 16-byte piece at K positions >= K (k0 = its first).
__device__ __forceinline__ uint4 mask_k(uint4 v, int k0, int K) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int kb = K - k0 - 4 * e;  // bytes of this dword inside the row
    w[e] &= kb >= 4 ? 0xffffffffu : (kb <= 0 ? 0u : (0xffffffffu >> (8 * (4 - kb))));
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Work split.  The T output tiles are ordered (kGroupM tile rows, then along
// N) and each one's nk K steps are cut into S equal-as-possible ranges:
// block v (after the XCD remap below) computes split s = v / T of tile
// t = v % T.  Splitting by whole K ranges keeps the blocks that run at the
// same time on the same K steps of neighbouring tiles, so they keep sharing
// operand rows in L2.  With S = 1 each block computes a whole tile; with
// S > 1 a tile's blocks leave int32 partial tiles in the workspace, bump the
// tile's counter, and move on, so no block ever waits for another.  The last
// one in adds the partials (integer sums: exact in any order) and writes the
// tile.  Counters are tagged with the launch, so the workspace needs no
// clearing between calls.
template <int WM, int NT>
struct TileShape {
  static constexpr int WN = 4 / WM;       // waves along N
  static constexpr int IT = 8 / WM;       // MFMA row tiles per wave
  static constexpr int JT = NT / WN;      // MFMA column tiles per wave
  static constexpr int BN = 32 * NT;      // tile columns
  static constexpr int NMF = IT * JT;     // MFMAs per K half
  static constexpr int NFR = IT + JT;     // fragment reads per K half
  static constexpr int kTileInts = LBM * BN;
  static_assert(WM * WN == 4 && NT % WN == 0 && NT <= 8, "tile shape");
  static_assert(NMF >= NFR && NMF >= 8 && NMF <= 16, "issue slots per K half");
};

template <int WM, int NT>
__global__ __launch_bounds__(LTHREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_i8_large(const int8_t *__restrict__ xq, int64_t ldx, const float *__restrict__ s,
                   const int8_t *__restrict__ w, int64_t ldw, const float *__restrict__ beta,
                   const float *__restrict__ bias, int M,
                   int N, int K, int32_t *__restrict__ acc, int64_t ldacc, float *__restrict__ y,
                   int64_t ldy, int S, int32_t *__restrict__ part,
                   unsigned long long *__restrict__ cnt, unsigned long long epoch) {
  using TS = TileShape<WM, NT>;
  constexpr int WN = TS::WN, IT = TS::IT, JT = TS::JT, BN = TS::BN, NMF = TS::NMF,
                NFR = TS::NFR;
  // four stages per operand, as separate arrays so that the compiler can
  // tell a load into one stage from reads of another
  __shared__ __attribute__((aligned(1024))) int8_t A0[LTILE], A1[LTILE], A2[LTILE], A3[LTILE];
  __shared__ __attribute__((aligned(1024))) int8_t B0[LTILE], B1[LTILE], B2[LTILE], B3[LTILE];
  __shared__ float scale[LBM];
  __shared__ int last_flag;

  const int nbm = (M + LBM - 1) / LBM, nbn = (N + BN - 1) / BN, T = nbm * nbn;
  const int nk = (K + LBK - 1) / LBK;
  const int kv = K - (nk - 1) * LBK;  // valid K bytes of the last step, 1..64
  // XCD x runs blocks x, x + 8, ...: give it the contiguous share
  // [x per, (x + 1) per) of the work, so that its L2 sees neighbouring tiles
  const int per = (int)(gridDim.x / kXcds);
  const int vb = (int)(blockIdx.x % kXcds) * per + (int)(blockIdx.x / kXcds);
  if (vb >= T * S) return;

  // Thread coordinates, read through an empty asm, so that the compiler
  // recomputes the addresses derived from them where they are used instead
  // of keeping them all live from the kernel's start.
  int tid, lane, wid, wm, wn;  // wid, wm, wn wave-uniform
  auto refresh = [&]() __attribute__((always_inline)) {
    int t_ = (int)threadIdx.x;
    asm volatile("" : "+v"(t_));
    tid = t_;
    lane = t_ & 63;
    const int w_ = __builtin_amdgcn_readfirstlane(t_ >> 6);
    wid = w_;
    wm = w_ / WN;
    wn = w_ % WN;
  };
  const __amdgpu_buffer_rsrc_t ar = rsrc(xq, (int64_t)M * ldx);
  const __amdgpu_buffer_rsrc_t br = rsrc(w, (int64_t)N * ldw);
  const float bs = beta[0];

  // Loads: 16 per operand and step, 4 per wave; load j fills rows
  // 16 j + [0, 16) of the stage.  Lane l lands at row 16 j + l/4, slot l%4,
  // so it fetches chunk (l%4) ^ ((l/16)%4) of that row.  Weight rows past
  // the tile's BN (or past N) get an offset past the buffer: no memory
  // traffic, and nobody reads those LDS rows.
  uint32_t aoff[4], boff[4];
  int kend = 0;  // loads clamp to the last step of the block's K range
  // This wave's 4 KB part of a stage, from an opaque copy of the thread
  // index: a uniform value the compiler recomputes where it is used (one
  // scalar add per load) instead of keeping 32 hoisted sums in registers.
  auto wave_base = [&]() __attribute__((always_inline)) {
    int t_ = (int)threadIdx.x;
    asm volatile("" : "+v"(t_));
    return __builtin_amdgcn_readfirstlane((t_ >> 6) * 4096);
  };
  auto load = [&](int k, int8_t *As, int8_t *Bs) __attribute__((always_inline)) {
    const uint32_t k0 = (uint32_t)min(k, kend - 1) * LBK;
    const int wb = wave_base();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, (lds_void *)(As + wb + i * 1024), 16,
                                               aoff[i] + k0, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(br, (lds_void *)(Bs + wb + i * 1024), 16,
                                               boff[i] + k0, 0, 0, 0);
    }
  };
  // zero the activation bytes at step positions >= kv (one row per thread)
  auto fix_tail = [&](int8_t *As) __attribute__((always_inline)) {
    const int sw = (tid >> 2) & 3;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      if (16 * x + 16 <= kv) continue;
      uint4 *p = reinterpret_cast<uint4 *>(As + tid * 64 + 16 * (x ^ sw));
      *p = mask_k(*p, 16 * x, kv);
    }
  };

  v16i c[IT][JT];

  // Fragment addresses (set per block): MFMA row tile i of K half h of a
  // stage is at row (this wave's first row) + 32 i + (l & 31), chunk
  // 2 h + (l >> 5), in its swizzled slot; column tile j likewise.
  int fa[2], fb[2];
  auto frags = [&](const int8_t *As, const int8_t *Bs, int h, v4i_(&a)[IT], v4i_(&b)[JT])
                   __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < IT; ++i) a[i] = *reinterpret_cast<const v4i_ *>(As + fa[h] + 2048 * i);
#pragma unroll
    for (int j = 0; j < JT; ++j) b[j] = *reinterpret_cast<const v4i_ *>(Bs + fb[h] + 2048 * j);
  };

  // The issue order inside a K half is written out and pinned: MFMA g,
  // then (g < NFR) fragment read g and/or (g >= NMF - 8) load g - (NMF - 8).
  // The pins (scheduling barriers that only let non-matrix vector ALU and
  // scalar ALU work move) keep the compiler from regrouping the reads
  // behind the MFMAs that need them.
  auto pin = []() __attribute__((always_inline)) { __builtin_amdgcn_sched_barrier(0x0006); };
  auto mfma_g = [&](const v4i_(&a)[IT], const v4i_(&b)[JT], int g)
                    __attribute__((always_inline)) {
    c[g / JT][g % JT] =
        __builtin_amdgcn_mfma_i32_32x32x32_i8(a[g / JT], b[g % JT], c[g / JT][g % JT], 0, 0, 0);
  };
  auto frag_g = [&](const int8_t *As, const int8_t *Bs, int h, v4i_(&a)[IT], v4i_(&b)[JT], int g)
                    __attribute__((always_inline)) {
    if (g < IT)
      a[g] = *reinterpret_cast<const v4i_ *>(As + fa[h] + 2048 * g);
    else
      b[g - IT] = *reinterpret_cast<const v4i_ *>(Bs + fb[h] + 2048 * (g - IT));
  };
  auto load_g = [&](int k, int8_t *As, int8_t *Bs, int wb, int g) __attribute__((always_inline)) {
    const uint32_t k0 = (uint32_t)min(k, kend - 1) * LBK;
    const int i = g >> 1;
    if (g & 1)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(br, (lds_void *)(Bs + wb + i * 1024), 16,
                                               boff[i] + k0, 0, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, (lds_void *)(As + wb + i * 1024), 16,
                                               aoff[i] + k0, 0, 0, 0);
  };

  v4i_ a0[IT], b0[JT], a1[IT], b1[JT];
  // step k reads stage (Ac, Bc); step k+1 is in (An, Bn); step k+3 goes to (Ad, Bd)
  auto step = [&](int k, const int8_t *Ac, const int8_t *Bc, int8_t *An, int8_t *Bn, int8_t *Ad,
                  int8_t *Bd) __attribute__((always_inline)) {
    pin();
#pragma unroll
    for (int g = 0; g < NMF; ++g) {
      mfma_g(a0, b0, g);
      if (g < NFR) frag_g(Ac, Bc, 1, a1, b1, g);
      pin();
    }
    wait_vmcnt<8>();  // this wave's loads of step k+1 (those of k+2 may be in flight)
    block_barrier();
    if (k + 1 == nk - 1 && kv < LBK) {
      fix_tail(An);
      wait_lgkmcnt0();
      block_barrier();
    }
    const int wb = wave_base();
    pin();
#pragma unroll
    for (int g = 0; g < NMF; ++g) {
      mfma_g(a1, b1, g);
      if (g < NFR) frag_g(An, Bn, 0, a0, b0, g);
      if (g >= NMF - 8) load_g(k + 3, Ad, Bd, wb, g - (NMF - 8));
      pin();
    }
  };

  // Accumulate steps [ks, ke) of the tile at (tm, tn) into c.
  auto mainloop = [&](int tm, int tn, int ks, int ke) __attribute__((always_inline)) {
    // Load i of this wave: rows 16 (4 wid + i) + l/4, chunk (l%4) ^ ((l/16)%4).
    const int lrow = 16 * 4 * wid + (lane >> 2), lchunk = (lane & 3) ^ ((lane >> 4) & 3);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = lrow + 16 * i;
      aoff[i] = tm + row < M ? (uint32_t)((tm + row) * ldx + 16 * lchunk) : 0x80000000u;
      boff[i] = row < BN && tn + row < N ? (uint32_t)((tn + row) * ldw + 16 * lchunk)
                                         : 0x80000000u;
    }
    kend = ke;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int slot = 16 * ((2 * h + (lane >> 5)) ^ ((lane >> 2) & 3));
      fa[h] = (wm * 32 * IT + (lane & 31)) * 64 + slot;
      fb[h] = (wn * 32 * JT + (lane & 31)) * 64 + slot;
    }
#pragma unroll
    for (int i = 0; i < IT; ++i)
#pragma unroll
      for (int j = 0; j < JT; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) c[i][j][e] = 0;
    load(ks, A0, B0);
    load(ks + 1, A1, B1);
    load(ks + 2, A2, B2);
    wait_vmcnt<16>();
    block_barrier();
    if (ks == nk - 1 && kv < LBK) {
      fix_tail(A0);
      wait_lgkmcnt0();
      block_barrier();
    }
    frags(A0, B0, 0, a0, b0);
    int k = ks;
    for (; k + 4 <= ke; k += 4) {
      step(k, A0, B0, A1, B1, A3, B3);
      step(k + 1, A1, B1, A2, B2, A0, B0);
      step(k + 2, A2, B2, A3, B3, A1, B1);
      step(k + 3, A3, B3, A0, B0, A2, B2);
    }
    if (k < ke) step(k, A0, B0, A1, B1, A3, B3);
    if (k + 1 < ke) step(k + 1, A1, B1, A2, B2, A0, B0);
    if (k + 2 < ke) step(k + 2, A2, B2, A3, B3, A1, B1);
    // the trailing loads into unused stages have landed and every wave is
    // done with the stages
    wait_vmcnt<0>();
    wait_lgkmcnt0();
    block_barrier();
  };

  // Partial tiles keep the accumulator layout: piece (i, j, q) of wave w is
  // 1 KB at ((w NMF + JT i + j) * 4 + q) KB, lane l's four ints at 16 l.
  // (The block that finishes a tile has written its own share too, and
  // refills its accumulators with the sum of all shares read back, rather
  // than adding into them: in-place vector ALU updates would pull the
  // accumulators out of the AGPRs.)  Byte offsets into the partial area fit
  // 32 bits: it holds at most 256 tiles of at most 256 KB.
  // Partial tiles move with device-scope (sc1) buffer stores and loads,
  // which go to memory rather than staying in (or being served from) one
  // XCD's L2; a writer's vmcnt(0) before it bumps the counter then orders
  // its stores before the counter update, and the block that sees the
  // final count reads every share from memory.  This avoids writing back
  // and invalidating whole L2s, which a fence at device scope would do.
  const __amdgpu_buffer_rsrc_t prs = rsrc(part, (int64_t)T * S * TS::kTileInts * 4);
  constexpr int kSc1 = 16;  // cache-policy bit: device scope
  constexpr uint32_t kSlotBytes = TS::kTileInts * 4;
  auto write_partial = [&](uint32_t slot_bytes) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < IT; ++i)
#pragma unroll
      for (int j = 0; j < JT; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const v4i_ d = {c[i][j][4 * q], c[i][j][4 * q + 1], c[i][j][4 * q + 2],
                          c[i][j][4 * q + 3]};
          __builtin_amdgcn_raw_buffer_store_b128(
              d, prs, slot_bytes + 4 * (((wid * NMF + JT * i + j) * 4 + q) * 256 + 4 * lane), 0,
              kSc1);
        }
  };

  // Epilogue.  Element e of lane l in MFMA tile (i, j) is row 8 (e/4) +
  // 4 (l/32) + e%4, column l%32.  A wave's output goes out in pieces of one
  // MFMA row tile (32 rows) by nj = 4, 2 or 1 column tiles (W = 32 nj
  // columns), each transposed through the wave's own 16 KB of LDS, after
  // which every lane stores 16-byte pieces of rows (an instruction covers
  // 256 / W rows of W floats).  All LDS addresses are one per-lane base plus
  // constants.  Bounds are checked only in tiles on the edge of the output.
  // src(i, j0, v) fills v[jj][e] = element e of MFMA tile (i, j0 + jj).
  auto epilogue = [&](int tm, int tn, auto &&src) __attribute__((always_inline)) {
    refresh();
    {
      const int m = tm + tid;
      scale[tid] = m < M ? s[m] * bs : 0.0f;
    }
    wait_lgkmcnt0();
    block_barrier();
    float *tb = reinterpret_cast<float *>(wid == 0 ? A0 : wid == 1 ? A1 : wid == 2 ? A2 : A3);
    const bool interior = tm + LBM <= M && tn + BN <= N;
    const int rsub = lane >> 5;
    const float *sbase = scale + wm * 32 * IT + 4 * rsub;
    // one piece: MFMA row tile i, column tiles j0 .. j0 + NJ - 1
    auto piece = [&](auto inside, auto nj_tag, int i, int j0) __attribute__((always_inline)) {
      constexpr bool kInside = decltype(inside)::value;
      constexpr int NJ = decltype(nj_tag)::value;
      constexpr int W = 32 * NJ;       // columns of the piece
      constexpr int LPR = W / 4;       // lanes per row when reading back
      constexpr int RPI = 64 / LPR;    // rows per read instruction
      const int r0 = wm * 32 * IT + 32 * i;  // first row of the piece (block-relative)
      const int c0 = wn * 32 * JT + 32 * j0;
      float *wbase = tb + 4 * rsub * W + (lane & 31);
      const int rrow = lane / LPR, col4 = 4 * (lane % LPR);
      const float *rbase = tb + rrow * W + col4;
#pragma unroll
      for (int out = 0; out < 2; ++out) {
        if (out == 0 && !y) continue;
        if (out == 1 && !acc) continue;
        int v[4][16];
        src(i, j0, v);
        float sc[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) sc[e] = sbase[32 * i + 8 * (e >> 2) + (e & 3)];
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            wbase[(8 * (e >> 2) + (e & 3)) * W + 32 * jj] =
                out == 0 ? (float)v[jj][e] * sc[e] : __builtin_bit_cast(float, v[jj][e]);
        // (a wave's LDS accesses complete in order: no wait between them)
        const int64_t ld = out == 0 ? ldy : ldacc;
        float *obase = out == 0 ? y : reinterpret_cast<float *>(acc);
        // rows are 16-byte aligned: the pitch is a multiple of 4 elements
        float *orow = obase + (int64_t)(tm + r0 + rrow) * ld + tn + c0 + col4;
        // the bias of this lane's four columns, the same for every row
        float4 b4 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        const bool add_bias = out == 0 && bias != nullptr;
        if (add_bias) {
          const int n = tn + c0 + col4;
          if (kInside || n + 3 < N) {
            b4 = *reinterpret_cast<const float4 *>(__builtin_assume_aligned(bias + n, 16));
          } else {
            if (n < N) b4.x = bias[n];
            if (n + 1 < N) b4.y = bias[n + 1];
            if (n + 2 < N) b4.z = bias[n + 2];
          }
        }
#pragma unroll
        for (int pc = 0; pc < 32 / RPI; ++pc) {
          float4 o = *reinterpret_cast<const float4 *>(rbase + RPI * W * pc);
          if (add_bias) {
            o.x = o.x + b4.x;
            o.y = o.y + b4.y;
            o.z = o.z + b4.z;
            o.w = o.w + b4.w;
          }
          float *dst = orow + (int64_t)(RPI * pc) * ld;
          if (kInside) {
            *reinterpret_cast<float4 *>(__builtin_assume_aligned(dst, 16)) = o;
          } else {
            const int m = tm + r0 + RPI * pc + rrow, n = tn + c0 + col4;
            if (m < M) {
              if (n + 3 < N) {
                *reinterpret_cast<float4 *>(__builtin_assume_aligned(dst, 16)) = o;
              } else {
                const float f[4] = {o.x, o.y, o.z, o.w};
                for (int t4 = 0; t4 < 4 && n + t4 < N; ++t4) dst[t4] = f[t4];
              }
            }
          }
        }
      }
    };
    // one copy of the pass for tiles inside the output (no checks) and one
    // for tiles on its edge, so that the checks stay out of the fast path
    auto pass = [&](auto inside) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < IT; ++i) {
        if constexpr (JT >= 4) piece(inside, std::integral_constant<int, 4>(), i, 0);
        if constexpr (JT >= 8) piece(inside, std::integral_constant<int, 4>(), i, 4);
        if constexpr (JT % 4 >= 2)
          piece(inside, std::integral_constant<int, 2>(), i, JT - JT % 4);
        if constexpr (JT % 2 == 1) piece(inside, std::integral_constant<int, 1>(), i, JT - 1);
      }
    };
    if (interior)
      pass(std::integral_constant<bool, true>());
    else
      pass(std::integral_constant<bool, false>());
    // the stages may be reused after this
    wait_lgkmcnt0();
    block_barrier();
  };

  refresh();
  const int t = vb % T, split = vb / T;
  const int ks = (int)((int64_t)split * nk / S), ke = (int)((int64_t)(split + 1) * nk / S);
  const int group = t / (kGroupM * nbn), first_m = group * kGroupM;
  const int gm = min(kGroupM, nbm - first_m), r = t - group * kGroupM * nbn;
  const int tm = (first_m + r % gm) * LBM, tn = (r / gm) * BN;
  mainloop(tm, tn, ks, ke);
  bool finish = S == 1;
  if (!finish) {
    // share of split s of this tile: partial slot s T + t
    write_partial((uint32_t)vb * kSlotBytes);
    wait_vmcnt<0>();
    __syncthreads();
    if (tid == 0) {
      // Counter word: (launch epoch << 8) | arrivals.  A word carrying
      // another epoch (an earlier launch, or whatever the workspace held)
      // counts as zero arrivals, so the counters need no clearing.
      unsigned long long v = __hip_atomic_load(&cnt[t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      unsigned long long nv;
      do {
        nv = (v >> 8) == epoch ? v + 1 : (epoch << 8) | 1;
      } while (!__hip_atomic_compare_exchange_strong(&cnt[t], &v, nv, __ATOMIC_RELAXED,
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      last_flag = ((v >> 8) == epoch ? (int)(v & 255) : 0) == S - 1;
    }
    __syncthreads();
    finish = last_flag;
    if (finish) {
      // the last block in: c = sum of every share (its own included), two
      // shares in flight at a time (a missing second one reads zeros), in
      // pieces of up to 4 MFMA tiles
      // (a replay of the same launch, e.g. from a captured graph, reuses
      // the epoch: leave the word at zero arrivals)
      if (tid == 0) __hip_atomic_store(&cnt[t], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      auto refill = [&](int i, auto nj_tag, int j0) __attribute__((always_inline)) {
        constexpr int NJ = decltype(nj_tag)::value;
        const uint32_t lo = 4 * ((wid * NMF + JT * i + j0) * 1024 + 4 * lane);
        int v[NJ][16];
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
          for (int e = 0; e < 16; ++e) v[jj][e] = 0;
        for (int sp = 0; sp < S; sp += 2) {
          const uint32_t o0 = (uint32_t)(sp * T + t) * kSlotBytes + lo;
          const uint32_t o1 =
              sp + 1 < S ? (uint32_t)((sp + 1) * T + t) * kSlotBytes + lo : 0x80000000u;
          v4i_ x0[4 * NJ], x1[4 * NJ];
#pragma unroll
          for (int jq = 0; jq < 4 * NJ; ++jq) {
            x0[jq] = __builtin_amdgcn_raw_buffer_load_b128(prs, o0 + 1024 * jq, 0, kSc1);
            x1[jq] = __builtin_amdgcn_raw_buffer_load_b128(prs, o1 + 1024 * jq, 0, kSc1);
          }
#pragma unroll
          for (int jq = 0; jq < 4 * NJ; ++jq)
#pragma unroll
            for (int e = 0; e < 4; ++e) v[jq >> 2][4 * (jq & 3) + e] += x0[jq][e] + x1[jq][e];
        }
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
          for (int e = 0; e < 16; ++e) c[i][j0 + jj][e] = v[jj][e];
      };
#pragma unroll
      for (int i = 0; i < IT; ++i) {
        if constexpr (JT >= 4) refill(i, std::integral_constant<int, 4>(), 0);
        if constexpr (JT >= 8) refill(i, std::integral_constant<int, 4>(), 4);
        if constexpr (JT % 4 >= 2) refill(i, std::integral_constant<int, 2>(), JT - JT % 4);
        if constexpr (JT % 2 == 1) refill(i, std::integral_constant<int, 1>(), JT - 1);
      }
    }
  }
  if (finish)
    epilogue(tm, tn, [&](int i, int j0, int(&v)[4][16]) __attribute__((always_inline)) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int e = 0; e < 16; ++e) v[jj][e] = j0 + jj < JT ? c[i][j0 + jj][e] : 0;
    });
}

}  // namespace

namespace {

constexpr int kSplitMaxBlocks = 256;  // blocks (and partial tiles) of a split launch
constexpr int kSplitCounterBytes = 8 * kSplitMaxBlocks;
static_assert(kSplitCounterBytes == (int)kGemmCounterBytes, "counter area size");

// the large tiles pay off once there are enough of them; they address the
// operands with 32-bit buffer offsets
bool large_tiles(int64_t M, int64_t N, int64_t ldx, int64_t ldw) {
  return M >= 512 && N >= 512 && M * ldx < (INT64_C(1) << 31) &&
         N * ldw < (INT64_C(1) << 31) && M <= INT32_MAX && N <= INT32_MAX;
}

}  // namespace

// compute units of the current device (cached per device)
int device_cus() {
  // a value per device; threads that race to fill it store the same value
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

namespace {

// Launch epochs of split launches: 56-bit, never 0, one per launch.  They
// start at a random point per process, so counter words left in a
// workspace by another process, by an earlier run, or by unrelated data
// (which would have to equal epoch << 8 | arrivals in all 56 upper bits)
// match a live launch with odds of about 2^-56.
unsigned long long epoch_base() {
  unsigned long long b = 0;
  try {
    std::random_device rd;
    b = ((unsigned long long)rd() << 32) ^ (unsigned long long)rd();
  } catch (...) {
  }
  // mixed with the clock and the address of a local, in case the device
  // above is deterministic
  b ^= (unsigned long long)std::chrono::steady_clock::now().time_since_epoch().count() *
       0x9E3779B97F4A7C15ull;
  b ^= (unsigned long long)(uintptr_t)&b;
  return b;
}
unsigned long long next_epoch() {
  static std::atomic<unsigned long long> e{epoch_base()};
  unsigned long long v = (e.fetch_add(1) + 1) & ((1ull << 56) - 1);
  return v == 0 ? 1 : v;
}

// The large-tile shapes: waves along M, MFMA column tiles of the block,
// and measured costs on MI355X at full load: cycles per K step and
// microseconds per output pass of a tile.
struct LargeShape {
  int wm, nt;
  double step_cycles, epi_us;
};
constexpr LargeShape kShapes[2] = {{2, 8, 1316, 6.5}, {4, 5, 1104, 4.1}};  // 256 x 256, 160
constexpr int kNumShapes = 2;
constexpr int64_t kMaxSlotBytes = (int64_t)LBM * 256 * 4;  // largest partial tile

// Tile shape and K splits: the (shape, S) with the least estimated time (in
// microseconds, at the 1.8 GHz the matrix cores hold under full load):
// rounds of blocks x (K steps per block + output pass), plus, when split,
// moving the partial tiles (each written once and read once by the
// finishing block, at ~4 TB/s) and ~3 us of hand-over.  Ties keep the wider
// tile and fewer splits.
struct LargePlan {
  int shape, S;
  int64_t T;
};
LargePlan plan_large(int64_t M, int64_t N, int64_t nk, bool can_split, int cus) {
  LargePlan best{0, 1, 0};
  double best_us = 1e300;
  for (int sh = 0; sh < kNumShapes; ++sh) {
    const int64_t nt = kShapes[sh].nt;
    const int64_t T = ceil_div(M, LBM) * ceil_div(N, 32 * nt);
    const double step_us = kShapes[sh].step_cycles / 1800.0;
    for (int64_t S = 1; S <= nk && S <= kSplitMaxBlocks; ++S) {
      if (S > 1 && (!can_split || T * S > kSplitMaxBlocks)) break;
      const int64_t rounds = ceil_div(T * S, cus);
      double us = (double)rounds * ((double)ceil_div(nk, S) * step_us + kShapes[sh].epi_us);
      if (S > 1) us += 2.0 * (double)(T * S) * (double)(LBM * 32 * nt * 4) / 4.0e6 + 3.0;
      if (us < best_us) {
        best_us = us;
        best = {sh, (int)S, T};
      }
    }
  }
  return best;
}

template <int WM, int NT>
void launch_large(const LargePlan &p, hipStream_t st, const int8_t *xq, int64_t ldx,
                  const float *s, const int8_t *w, int64_t ldw, const float *beta,
                  const float *bias, int64_t M,
                  int64_t N, int64_t K, int32_t *acc, int64_t ldacc, float *y, int64_t ldy,
                  int32_t *part, unsigned long long *cnt, unsigned long long epoch) {
  const int64_t blocks = ceil_div(p.T * p.S, kXcds) * kXcds;
  hipLaunchKernelGGL((gemm_i8_large<WM, NT>), dim3((unsigned)blocks), dim3(LTHREADS), 0, st, xq,
                     ldx, s, w, ldw, beta, bias, (int)M, (int)N, (int)K, acc, ldacc, y, ldy, p.S,
                     part,
                     cnt, epoch);
}

}  // namespace

// The area has a fixed layout (counters at offset 0, then the partial
// tiles) and size, so that calls of any shape that share a workspace agree
// on where the counters are.
size_t gemm_split_area_bytes() {
  static_assert(kSplitCounterBytes + kSplitMaxBlocks * kMaxSlotBytes ==
                    (int64_t)UG_GEMM_SPLIT_AREA,
                "split area layout and ug.h disagree");
  return (size_t)(kSplitCounterBytes + kSplitMaxBlocks * kMaxSlotBytes);
}

hipError_t launch_gemm_i8(const int8_t *xq, int64_t ldx, const float *s, const int8_t *w,
                          int64_t ldw, const float *beta, const float *bias, int64_t M, int64_t N,
                          int64_t K,
                          int32_t *acc, int64_t ldacc, float *y, int64_t ldy, void *split,
                          int tile, int splits, hipStream_t st) {
  if (large_tiles(M, N, ldx, ldw)) {
    const int64_t nk = ceil_div(K, LBK);
    const int cus = device_cus();
    LargePlan p = plan_large(M, N, nk, split != nullptr, cus > 0 ? cus : 256);
    // an explicit tile shape (0: 256 x 256, 1: 256 x 160) and split count
    // replace the model's choice where they fit
    if (tile >= 0 && tile < kNumShapes) {
      p.shape = tile;
      p.T = ceil_div(M, LBM) * ceil_div(N, 32 * kShapes[tile].nt);
      p.S = 1;
    }
    if (splits >= 1) {
      if (split != nullptr && splits <= nk && p.T * splits <= kSplitMaxBlocks)
        p.S = splits;
      else
        p.S = 1;
    }
    int32_t *part = nullptr;
    unsigned long long *cnt = nullptr;
    unsigned long long epoch = 0;
    if (p.S > 1) {
      cnt = static_cast<unsigned long long *>(split);
      part = reinterpret_cast<int32_t *>(static_cast<char *>(split) + kSplitCounterBytes);
      epoch = next_epoch();
    }
    if (p.shape == 0)
      launch_large<2, 8>(p, st, xq, ldx, s, w, ldw, beta, bias, M, N, K, acc, ldacc, y, ldy, part, cnt,
                         epoch);
    else
      launch_large<4, 5>(p, st, xq, ldx, s, w, ldw, beta, bias, M, N, K, acc, ldacc, y, ldy, part, cnt,
                         epoch);
    return hipGetLastError();
  }
  dim3 grid((unsigned)ceil_div(N, BN), (unsigned)ceil_div(M, BM));
  hipLaunchKernelGGL(gemm_i8_kernel, grid, dim3(256), 0, st, xq, ldx, s, w, ldw, beta, bias, M, N, K,
                     acc, ldacc, y, ldy);
  return hipGetLastError();
}

}  // namespace ug

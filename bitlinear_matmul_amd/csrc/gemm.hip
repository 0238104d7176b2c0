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

// ---------------------------------------------------------------------------
// Large GEMM on v_mfma_i32_32x32x32_i8 (the 16x16x64 form issues at half the
// int8 rate on gfx950).  Lane l of that MFMA holds A row l%32 and B column
// l%32 at K bytes [16 (l/32), +16), and accumulator element i of lane l is
// D[8 (i/4) + 4 (l/32) + i%4][l%32].
//
// 256 x 256 output tile per 256-thread block, 2 x 2 waves of 128 x 128
// (4 x 4 MFMA tiles, 256 int32 accumulators per lane, held in AGPRs; one
// wave per SIMD).  K step 64, four LDS stages per operand.
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
constexpr int LBM = 256, LBN = 256, LBK = 64;
constexpr int LTHREADS = 256;
constexpr int LTILE = LBM * LBK;  // bytes of one operand tile per stage
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

__global__ __launch_bounds__(LTHREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_i8_large(const int8_t *__restrict__ xq, int64_t ldx, const float *__restrict__ s,
                   const int8_t *__restrict__ w, int64_t ldw, const float *__restrict__ beta, int M,
                   int N, int K, int32_t *__restrict__ acc, int64_t ldacc, float *__restrict__ y,
                   int64_t ldy) {
  // four stages per operand, as separate arrays so that the compiler can
  // tell a load into one stage from reads of another
  __shared__ __attribute__((aligned(1024))) int8_t A0[LTILE], A1[LTILE], A2[LTILE], A3[LTILE];
  __shared__ __attribute__((aligned(1024))) int8_t B0[LTILE], B1[LTILE], B2[LTILE], B3[LTILE];
  __shared__ float scale[LBM];

  // tile of this block: XCD x takes tiles [x * per, (x + 1) * per) of the
  // grouped order (kGroupM tile rows, then along N)
  const int nbm = (M + LBM - 1) / LBM, nbn = (N + LBN - 1) / LBN, T = nbm * nbn;
  const int per = (T + kXcds - 1) / kXcds;
  const int t = (int)(blockIdx.x % kXcds) * per + (int)(blockIdx.x / kXcds);
  if (t >= T) return;
  const int group = t / (kGroupM * nbn), first_m = group * kGroupM;
  const int gm = min(kGroupM, nbm - first_m), r = t - group * kGroupM * nbn;
  const int tm = (first_m + r % gm) * LBM, tn = (r / gm) * LBN;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;  // 2 x 2 waves
  const __amdgpu_buffer_rsrc_t ar = rsrc(xq, (int64_t)M * ldx);
  const __amdgpu_buffer_rsrc_t br = rsrc(w, (int64_t)N * ldw);
  {
    const int m = tm + tid;
    scale[tid] = m < M ? s[m] * beta[0] : 0.0f;
  }

  // Loads: 16 per operand and step, 4 per wave; load j fills rows
  // 16 j + [0, 16) of the stage.  Lane l lands at row 16 j + l/4, slot l%4,
  // so it fetches chunk (l%4) ^ ((l/16)%4) of that row.
  uint32_t aoff[4], boff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 16 * (4 * wid + i) + (lane >> 2);
    const int chunk = (lane & 3) ^ ((lane >> 4) & 3);
    aoff[i] = tm + row < M ? (uint32_t)((tm + row) * ldx + 16 * chunk) : 0x80000000u;
    boff[i] = tn + row < N ? (uint32_t)((tn + row) * ldw + 16 * chunk) : 0x80000000u;
  }
  const int nk = (K + LBK - 1) / LBK;
  const int kv = K - (nk - 1) * LBK;  // valid K bytes of the last step, 1..64
  auto load = [&](int k, int8_t *As, int8_t *Bs) {
    const uint32_t k0 = (uint32_t)min(k, nk - 1) * LBK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, (lds_void *)(As + (4 * wid + i) * 1024), 16,
                                               aoff[i] + k0, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(br, (lds_void *)(Bs + (4 * wid + i) * 1024), 16,
                                               boff[i] + k0, 0, 0, 0);
    }
  };
  // zero the activation bytes at step positions >= kv (one row per thread)
  auto fix_tail = [&](int8_t *As) {
    const int sw = (tid >> 2) & 3;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      if (16 * x + 16 <= kv) continue;
      uint4 *p = reinterpret_cast<uint4 *>(As + tid * 64 + 16 * (x ^ sw));
      *p = mask_k(*p, 16 * x, kv);
    }
  };

  v16i c[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) c[i][j][e] = 0;

  // Fragment addresses: tile i of K half h of a stage is at row
  // 32 i + (l & 31), chunk 2 h + (l >> 5), in its swizzled slot.
  int fa[2], fb[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int slot = 16 * ((2 * h + (lane >> 5)) ^ ((lane >> 2) & 3));
    fa[h] = (wm * 128 + (lane & 31)) * 64 + slot;
    fb[h] = (wn * 128 + (lane & 31)) * 64 + slot;
  }
  auto frags = [&](const int8_t *As, const int8_t *Bs, int h, v4i_(&a)[4], v4i_(&b)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const v4i_ *>(As + fa[h] + 2048 * i);
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = *reinterpret_cast<const v4i_ *>(Bs + fb[h] + 2048 * j);
  };
  auto mfmas = [&](const v4i_(&a)[4], const v4i_(&b)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        c[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[j], c[i][j], 0, 0, 0);
  };

  v4i_ a0[4], b0[4], a1[4], b1[4];
  // step k reads stage (A, B); step k+1 is in (An, Bn); step k+3 goes to (Ad, Bd)
  auto step = [&](int k, const int8_t *Ac, const int8_t *Bc, int8_t *An, int8_t *Bn, int8_t *Ad,
                  int8_t *Bd) {
    mfmas(a0, b0);
    frags(Ac, Bc, 1, a1, b1);
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    wait_vmcnt<8>();  // this wave's loads of step k+1 (those of k+2 may be in flight)
    block_barrier();
    if (k + 1 == nk - 1 && kv < LBK) {
      fix_tail(An);
      wait_lgkmcnt0();
      block_barrier();
    }
    load(k + 3, Ad, Bd);
    mfmas(a1, b1);
    frags(An, Bn, 0, a0, b0);
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
    }
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM (LDS-destination loads)
    }
  };

  load(0, A0, B0);
  load(1, A1, B1);
  load(2, A2, B2);
  wait_vmcnt<16>();
  block_barrier();
  if (nk == 1 && kv < LBK) {
    fix_tail(A0);
    wait_lgkmcnt0();
    block_barrier();
  }
  frags(A0, B0, 0, a0, b0);
  int k = 0;
  for (; k + 4 <= nk; k += 4) {
    step(k, A0, B0, A1, B1, A3, B3);
    step(k + 1, A1, B1, A2, B2, A0, B0);
    step(k + 2, A2, B2, A3, B3, A1, B1);
    step(k + 3, A3, B3, A0, B0, A2, B2);
  }
  if (k < nk) step(k, A0, B0, A1, B1, A3, B3);
  if (k + 1 < nk) step(k + 1, A1, B1, A2, B2, A0, B0);
  if (k + 2 < nk) step(k + 2, A2, B2, A3, B3, A1, B1);

  // Epilogue.  Element e of lane l in tile (i, j) is row 8 (e/4) + 4 (l/32)
  // + e%4, column l%32.  Each 32 x 32 tile goes through a per-wave 32 x 36
  // LDS buffer, so that each lane stores 16-byte pieces of rows (a wave keeps
  // at most 63 memory operations in flight: 4-byte stores would leave the
  // epilogue waiting on write latency), with a compact per-tile body (this
  // code runs once per block, from a cold instruction cache).
  wait_vmcnt<0>();  // the trailing loads into unused stages have landed
  wait_lgkmcnt0();
  block_barrier();  // and every wave is done with the stages
  float *tb = reinterpret_cast<float *>(wid == 0 ? A0 : wid == 1 ? A1 : wid == 2 ? A2 : A3);
  int *tbi = reinterpret_cast<int *>(tb);
  auto put = [&](int r0, int c0, const float4 &v, bool is_acc) {
    // lane's 4 values: row r0, columns c0..c0+3 (block-relative)
    const int m = tm + r0, n = tn + c0;
    if (m >= M) return;
    if (n + 3 < N) {
      if (is_acc)
        *reinterpret_cast<int4 *>(&acc[(int64_t)m * ldacc + n]) = __builtin_bit_cast(int4, v);
      else
        *reinterpret_cast<float4 *>(&y[(int64_t)m * ldy + n]) = v;
    } else {
      const float f[4] = {v.x, v.y, v.z, v.w};
      for (int t = 0; t < 4 && n + t < N; ++t) {
        if (is_acc)
          acc[(int64_t)m * ldacc + n + t] = __builtin_bit_cast(int, f[t]);
        else
          y[(int64_t)m * ldy + n + t] = f[t];
      }
    }
  };
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r0 = wm * 128 + 32 * i;  // first row of the tile row (block-relative)
    float sc[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) sc[e] = scale[r0 + 4 * (lane >> 5) + 8 * (e >> 2) + (e & 3)];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c0 = wn * 128 + 32 * j;
      if (y) {
#pragma unroll
        for (int e = 0; e < 16; ++e)
          tb[(4 * (lane >> 5) + 8 * (e >> 2) + (e & 3)) * 36 + (lane & 31)] = (float)c[i][j][e] * sc[e];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int rr = (lane >> 3) + 8 * q;
          put(r0 + rr, c0 + 4 * (lane & 7), *reinterpret_cast<const float4 *>(&tb[rr * 36 + 4 * (lane & 7)]), false);
        }
      }
      if (acc) {
#pragma unroll
        for (int e = 0; e < 16; ++e)
          tbi[(4 * (lane >> 5) + 8 * (e >> 2) + (e & 3)) * 36 + (lane & 31)] = c[i][j][e];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int rr = (lane >> 3) + 8 * q;
          put(r0 + rr, c0 + 4 * (lane & 7), *reinterpret_cast<const float4 *>(&tb[rr * 36 + 4 * (lane & 7)]), true);
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_i8(const int8_t *xq, int64_t ldx, const float *s, const int8_t *w,
                          int64_t ldw, const float *beta, int64_t M, int64_t N, int64_t K,
                          int32_t *acc, int64_t ldacc, float *y, int64_t ldy, hipStream_t st) {
  // the large tiles pay off once there are enough of them; they address
  // the operands with 32-bit buffer offsets
  if (M >= 512 && N >= 512 && M * ldx < (INT64_C(1) << 31) && N * ldw < (INT64_C(1) << 31) &&
      M <= INT32_MAX && N <= INT32_MAX) {
    const int64_t T = ceil_div(M, LBM) * ceil_div(N, LBN);
    const int64_t blocks = ceil_div(T, kXcds) * kXcds;
    hipLaunchKernelGGL(gemm_i8_large, dim3((unsigned)blocks), dim3(LTHREADS), 0, st, xq, ldx, s,
                       w, ldw, beta, (int)M, (int)N, (int)K, acc, ldacc, y, ldy);
    return hipGetLastError();
  }
  dim3 grid((unsigned)ceil_div(N, BN), (unsigned)ceil_div(M, BM));
  hipLaunchKernelGGL(gemm_i8_kernel, grid, dim3(256), 0, st, xq, ldx, s, w, ldw, beta, M, N, K,
                     acc, ldacc, y, ldy);
  return hipGetLastError();
}

}  // namespace ug

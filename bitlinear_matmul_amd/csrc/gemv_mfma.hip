// Decode GEMV on the matrix cores (gfx950): y = (x_q W_q^T)(s beta) for up
// to 64 activation rows, one problem or a group of independent problems in
// one launch.
//
// "ultragraph - when the graph is the 1-bit LLM, part 2", section
// "autograd on a byte-graph": integer multiply-accumulate of int8
// activations against ternary weights, one rescale by s*beta.  "a 1-bit
// llm, from scratch" measures matvecs at 94.7% of a forward pass: this is
// the kernel that streams the weights.
//
// Mapping (v_mfma_i32_16x16x64_i8, A = activations, B = weights):
//   lane l = (n = l % 16, q = l / 16) owns weight row n of a 16-row group
//   and bytes [64 st + 16 q, +16) of that row at step st.
//   One trit per byte: those 16 bytes are the B operand (K positions
//   64 st + 16 q + [0,16)).
//   Five trits per byte: the 16 bytes hold 80 trits.  Byte b gives t0..t3
//   from a 256-entry table of int8x4 in LDS and d4 = floor(b / 81) = t4 + 1,
//   computed four bytes at a time in 16-bit lanes as (b * 203) >> 14.  Byte
//   i of dword j gives dword i of B operand j (j < 4); the d4 bytes of dword
//   j give dword j of B operand 4.  The activations are stored in LDS already
//   permuted the same way (each 80-position window as fragment 0..3 holding
//   x[5g .. 5g+3] of its bytes g, then fragment 4 holding the x[5g+4]), so
//   every MFMA adds products of matching K positions, and the d4 = t4 + 1
//   offset is removed at the end by subtracting sum_g x[5g+4] once per row.
//   The table is replicated 64 times (code e, replica r at e * 64 + r) and
//   lane l reads replica l: one v_perm forms each address (b * 256 + 4 l)
//   and a wave's 64 reads fall in 64 different banks.
//
// Work: one block of 8 waves per CU.  Two ways to split a launch:
//   stream: a block takes a range of items (32 weight rows over the whole
//     K); each wave walks whole items unit by unit (SC steps), keeping the
//     weights of the next two units in flight.  For groups with megabytes of
//     weights per CU.
//   fine: a block takes up to 16 items of 16 rows of one problem, and its
//     waves split the (item, step) pieces evenly, so every wave issues all
//     its weight loads at once and the K steps of one item run on several
//     waves; partial int32 sums meet in LDS.  For decode-sized groups, where
//     the launch is one HBM round trip long.
// Loads are buffer loads: lanes past the row, past N or past the work read
// zeros without touching memory, so the loops have no branches.  The 64 KB
// table and the staged activations are built once per block and shared by
// its 8 waves.  Activations may arrive as fp32: the block then quantizes the
// rows itself with ug_quant_act's arithmetic, so act quant + GEMV of a whole
// group is one launch.
#include "ug_internal.h"

namespace ug {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned short us2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kRepl = 64;          // table replicas: one per lane of a wave
constexpr int kXsBytes = 65536;    // staged activations
constexpr int kZero = kXsBytes;    // 80 zero bytes right after them
constexpr uint32_t kOOB = 0x80000000u;  // a buffer offset past every buffer used here
constexpr int kFineItems = 16;   // fine split: items (16-row groups) per block
constexpr int kFinePieces = 8;   // fine split: (item, step) pieces per wave

template <int FMT>
struct Fmt;
template <>
struct Fmt<UG_W_PACK5> {
  static constexpr int kFrag = 5;     // 16-byte B operands per 16 weight bytes
  static constexpr int kStepK = 320;  // K positions per 64-byte step of a row
  static constexpr int kLaneK = 80;   // K positions per lane per step
};
template <>
struct Fmt<UG_W_I8> {
  static constexpr int kFrag = 1;
  static constexpr int kStepK = 64;
  static constexpr int kLaneK = 16;
};

template <int FMT, int MB, bool FINE>
struct Cfg {
  // row groups per item (they share each activation read)
  static constexpr int RGW = FINE ? 1 : 2;
  // steps per unit (three units of weights are in flight per wave)
  static constexpr int SC =
      FINE ? 1 : (FMT == UG_W_PACK5 ? (MB == 1 ? 4 : (MB == 2 ? 2 : 1)) : (MB == 4 ? 2 : 4));
  // independent MFMA chains per output tile
  static constexpr int NACC = FMT == UG_W_PACK5 && MB == 4 ? 1 : 2;
};

__host__ __device__ __forceinline__ int row_bytes_of(int fmt, int K) {
  return fmt == UG_W_PACK5 ? (K + 4) / 5 : K;
}
__host__ __device__ __forceinline__ int steps_of(int fmt, int K) {
  return (row_bytes_of(fmt, K) + 63) / 64;
}
__host__ __device__ __forceinline__ int sc_of(int fmt, int mb) {
  return fmt == UG_W_PACK5
             ? (mb == 1 ? Cfg<UG_W_PACK5, 1, false>::SC
                        : (mb == 2 ? Cfg<UG_W_PACK5, 2, false>::SC : Cfg<UG_W_PACK5, 4, false>::SC))
             : (mb == 1 ? Cfg<UG_W_I8, 1, false>::SC
                        : (mb == 2 ? Cfg<UG_W_I8, 2, false>::SC : Cfg<UG_W_I8, 4, false>::SC));
}
// Staged row length of the stream split: whole units of steps, zero past K,
// so every step a wave multiplies has activations (zeros past K) inside its
// row.  The fine split stages whole steps: fine_kp.
__host__ __device__ __forceinline__ int fine_kp(int fmt, int K) {
  return steps_of(fmt, K) * (fmt == UG_W_PACK5 ? 320 : 64);
}
__host__ __device__ __forceinline__ int staged_kp(int fmt, int mb, int K) {
  const int sc = sc_of(fmt, mb);
  return ((steps_of(fmt, K) + sc - 1) / sc) * sc * (fmt == UG_W_PACK5 ? 320 : 64);
}
__host__ __device__ __forceinline__ int mb_of(int M) { return M <= 16 ? 1 : (M <= 32 ? 2 : 4); }
__host__ __device__ __forceinline__ bool stages_x(int fmt, int M, int K) {
  return (int64_t)M * staged_kp(fmt, mb_of(M), K) <= kXsBytes;
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Descriptor pointers are generic; every access through them goes through
// these global-address-space views, so the compiler emits global (not flat)
// memory instructions.  A flat access in flight makes every later wait for
// a load a wait for all loads, which would serialize the weight pipeline.
template <class T>
__device__ __forceinline__ __attribute__((address_space(1))) T *gp(T *p) {
  return (__attribute__((address_space(1))) T *)p;
}

// Raw buffer resource over [base, base + bytes): a load past the end returns
// zeros without a memory access (gfx9 descriptor word 3).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t buffer_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ float4 buffer_load16f(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// t0..t3 of code e as int8 bytes; codes 243..255 give zeros here (their d4
// is 3: matmul results for invalid codes are unspecified).
__device__ __forceinline__ uint32_t lut4_entry(int e) {
  uint32_t v = 0;
  if (e <= 242) {
    int c = e;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v |= ((uint32_t)((c % 3) - 1) & 0xffu) << (8 * j);
      c /= 3;
    }
  }
  return v;
}

__device__ __forceinline__ int q8(float v, float s) { return rint_clamp(v / s, -127.0f, 127.0f); }

__device__ __forceinline__ uint32_t pack4(int a, int b, int c, int e) {
  return (uint32_t)(a & 0xff) | ((uint32_t)(b & 0xff) << 8) | ((uint32_t)(c & 0xff) << 16) |
         ((uint32_t)(e & 0xff) << 24);
}

// Four packed bytes -> t[0..3] = t0..t3 of bytes 0..3 (table), d4 = their
// four top digits.  lr4 = 4 * lane.
__device__ __forceinline__ void decode4(uint32_t w, const char *lut, uint32_t lr4, uint32_t *t,
                                        uint32_t &d4) {
  // byte address b * 256 + 4 * lane (selector bytes: 0 = lr4 byte 0,
  // 4+i = byte i of w, 12 = zero)
  t[0] = *reinterpret_cast<const uint32_t *>(lut + __builtin_amdgcn_perm(w, lr4, 0x0c0c0400u));
  t[1] = *reinterpret_cast<const uint32_t *>(lut + __builtin_amdgcn_perm(w, lr4, 0x0c0c0500u));
  t[2] = *reinterpret_cast<const uint32_t *>(lut + __builtin_amdgcn_perm(w, lr4, 0x0c0c0600u));
  t[3] = *reinterpret_cast<const uint32_t *>(lut + __builtin_amdgcn_perm(w, lr4, 0x0c0c0700u));
  // floor(b / 81) for b < 256 is (b * 203) >> 14 (exact; b * 203 < 2^16)
  us2 e = __builtin_bit_cast(us2, w & 0x00ff00ffu);                            // b0, b2
  us2 o = __builtin_bit_cast(us2, __builtin_amdgcn_perm(0u, w, 0x0c030c01u));  // b1, b3
  e = (e * (unsigned short)203) >> (unsigned short)14;
  o = (o * (unsigned short)203) >> (unsigned short)14;
  d4 = __builtin_bit_cast(uint32_t, e) | (__builtin_bit_cast(uint32_t, o) << 8);
}

// 80 activations (20 dwords, K order) -> the five 16-byte fragments in the
// order the decoded weights use (see the file comment).
__device__ __forceinline__ void permute80(const uint32_t (&X)[20], uint32_t (&F)[20]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    F[4 * j] = X[5 * j];
    F[4 * j + 1] = __builtin_amdgcn_alignbyte(X[5 * j + 2], X[5 * j + 1], 1);
    F[4 * j + 2] = __builtin_amdgcn_alignbyte(X[5 * j + 3], X[5 * j + 2], 2);
    F[4 * j + 3] = __builtin_amdgcn_alignbyte(X[5 * j + 4], X[5 * j + 3], 3);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)  // bytes 20 i + 4, +9, +14, +19
    F[16 + i] = (X[5 * i + 1] & 0xffu) | (X[5 * i + 2] & 0xff00u) | (X[5 * i + 3] & 0xff0000u) |
                (X[5 * i + 4] & 0xff000000u);
}

__device__ __forceinline__ int byte_sum4(uint32_t v) {
  return (int)(int8_t)(v & 0xff) + (int)(int8_t)((v >> 8) & 0xff) +
         (int)(int8_t)((v >> 16) & 0xff) + (int)(int8_t)(v >> 24);
}

template <int FMT>
struct Smem {
  uint32_t lut[FMT == UG_W_PACK5 ? 256 * kRepl : 1];
  uint32_t lut_tmp[FMT == UG_W_PACK5 ? 256 : 1];
  alignas(16) int8_t xs[kXsBytes + 80];  // staged rows, then 80 zero bytes
  alignas(16) int slots[kFineItems * 256];  // fine split: [item][m][n] int32 sums
  float part[kWaves][64];                   // per-wave row maxima (fused quantization)
  float sm[64];                             // row scales s
  int cm[64];                               // five-trit correction sum_g x[5g+4]
};

// s = fl(fl(max|x| / 127) + eps) of row m from the per-wave maxima.
template <int FMT>
__device__ __forceinline__ float row_scale(const Smem<FMT> &sh, int m, float eps) {
  float a = sh.part[0][m];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) a = fmaxf(a, sh.part[w][m]);
  const float a127 = a / 127.0f;
  return a127 + eps;
}

// Block set-up for problem d, in two halves.  setup_issue() issues the
// first batch of activation loads; the caller then issues its weight loads,
// so that waiting for the activations never waits for the weights (loads
// complete in issue order).  setup_finish() builds the decode table (first
// problem of the block), the row scales (fused quantization, else the given
// s), the activation rows staged in LDS (Kp bytes per row, zeros past K;
// five trits per byte: every 80-position window permuted as the decoded
// weights are) with the d4 correction cm[m] = sum_g x[5g+4], and zeroed
// reduction slots, and ends with a barrier.
//
// Fused quantization reads x in tiles t = (row m, 256 positions c): lane l
// takes the float4 at 256 c + 4 l, a wave keeps 8 tiles in flight.
struct XBatch {
  float4 f[8];    // fused: the first 8 tiles of this wave
  uint32_t q[8];  // x_q given: the first 8 dwords of this thread
};

__device__ __forceinline__ float4 load_tile(const GemvDesc &d, __amdgpu_buffer_rsrc_t xr, int t,
                                            int T4, int nt) {
  const int m = t / T4, k = (t - m * T4) * 256 + 4 * (threadIdx.x & 63);
  // a float4 at k < K is inside the row (ldx >= round_up(K, 4))
  return buffer_load16f(xr, t < nt && k < d.K ? (uint32_t)((m * (int)d.ldx + k) * 4) : kOOB);
}

__device__ __forceinline__ uint32_t load_xq4(const GemvDesc &d, __amdgpu_buffer_rsrc_t xr, int idx,
                                             int Kp4, int n4) {
  const int m = idx / Kp4, k = 4 * (idx - m * Kp4);
  // 4 bytes at k < K are inside the row (ldxq >= round_up(K, 16))
  return buffer_load4(xr, idx < n4 && k < d.K ? (uint32_t)(m * (int)d.ldxq + k) : kOOB);
}

// Both batches are issued without a branch (the one not needed reads past
// its buffer, i.e. nothing), so every path sees the same loads in flight
// and waiting for them never has to wait for the caller's later loads.
__device__ __forceinline__ void setup_issue(const GemvDesc &d, bool staged, int Kp, XBatch &xb) {
  const int tid = threadIdx.x, wave = uniform(tid >> 6);
  const int T4 = (d.K + 255) >> 8, nt = d.x ? d.M * T4 : 0;
  const __amdgpu_buffer_rsrc_t xr =
      buffer_rsrc(d.x, d.x ? (uint32_t)((int64_t)d.M * d.ldx * 4) : 0u);
#pragma unroll
  for (int i = 0; i < 8; ++i) xb.f[i] = load_tile(d, xr, wave + i * kWaves, T4, nt);
  const int Kp4 = Kp >> 2, n4 = !d.x && staged ? d.M * Kp4 : 0;
  const __amdgpu_buffer_rsrc_t qr =
      buffer_rsrc(d.xq, n4 ? (uint32_t)((int64_t)d.M * d.ldxq) : 0u);
#pragma unroll
  for (int i = 0; i < 8; ++i) xb.q[i] = load_xq4(d, qr, tid + i * kThreads, Kp4, n4);
}

// Pass 1 on 8 tiles t0 + i * 8: per-wave row maxima.
template <int FMT>
__device__ __forceinline__ void absmax_tiles(const GemvDesc &d, Smem<FMT> &sh, const float4 (&v)[8],
                                             int t0, int T4, int nt) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int t = t0 + i * kWaves;
    if (t < nt) {
      const int m = t / T4, k = (t - m * T4) * 256 + 4 * lane;
      float a = fabsf(v[i].x);  // zero when k >= K
      if (k + 1 < d.K) a = fmaxf(a, fabsf(v[i].y));
      if (k + 2 < d.K) a = fmaxf(a, fabsf(v[i].z));
      if (k + 3 < d.K) a = fmaxf(a, fabsf(v[i].w));
      a = wave_max(a);
      if (lane == 0) sh.part[wave][m] = fmaxf(sh.part[wave][m], a);
    }
  }
}

// Pass 2 on 8 tiles: quantize into the staging rows, K order.
template <int FMT>
__device__ __forceinline__ void quant_tiles(const GemvDesc &d, Smem<FMT> &sh, const float4 (&v)[8],
                                            int t0, int T4, int nt, int Kp) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int t = t0 + i * kWaves;
    if (t < nt) {
      const int m = t / T4, k = (t - m * T4) * 256 + 4 * lane;
      const float s = row_scale(sh, m, d.eps);
      if (k < d.K)
        *reinterpret_cast<uint32_t *>(sh.xs + m * Kp + k) =
            pack4(q8(v[i].x, s), k + 1 < d.K ? q8(v[i].y, s) : 0, k + 2 < d.K ? q8(v[i].z, s) : 0,
                  k + 3 < d.K ? q8(v[i].w, s) : 0);
    }
  }
}

// 8 dwords of x_q rows into the staging rows (zeros past K).
template <int FMT>
__device__ __forceinline__ void copy_xq4(const GemvDesc &d, Smem<FMT> &sh, const uint32_t (&v)[8],
                                         int i0, int Kp4, int n4) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int idx = i0 + i * kThreads, m = idx / Kp4, k = 4 * (idx - m * Kp4);
    if (idx < n4) {
      uint32_t w = v[i];
      if (k + 4 > d.K) w &= k >= d.K ? 0u : (0xffffffffu >> (8 * (k + 4 - d.K)));
      reinterpret_cast<uint32_t *>(sh.xs + m * 4 * Kp4)[k >> 2] = w;
    }
  }
}

// PRE: the first batch is in xb (setup_issue); else every batch is loaded
// here, which keeps the registers free for a caller short of them.
template <int FMT, bool PRE>
__device__ __forceinline__ void setup_finish(const GemvDesc &d, Smem<FMT> &sh, bool staged, int Kp,
                                             bool build_table, bool zero_slots, const XBatch &xb) {
  const int tid = threadIdx.x, wave = uniform(tid >> 6), lane = tid & 63;
  if (FMT == UG_W_PACK5 && build_table && tid < 256) sh.lut_tmp[tid] = lut4_entry(tid);
  if (tid < 64) sh.cm[tid] = 0;
  if (tid < 20) reinterpret_cast<uint32_t *>(sh.xs + kZero)[tid] = 0;
  if (zero_slots)
    for (int i = tid; i < kFineItems * 64; i += kThreads)
      reinterpret_cast<uint4 *>(sh.slots)[i] = make_uint4(0, 0, 0, 0);
  const int Kp4 = Kp >> 2;  // dwords per staged row
  if (d.x) {
    const int T4 = (d.K + 255) >> 8, nt = d.M * T4;
    const __amdgpu_buffer_rsrc_t xr = buffer_rsrc(d.x, (uint32_t)((int64_t)d.M * d.ldx * 4));
    sh.part[wave][lane] = 0.0f;
    if (PRE) absmax_tiles(d, sh, xb.f, wave, T4, nt);
    for (int t0 = PRE ? wave + 8 * kWaves : wave; t0 < nt; t0 += 8 * kWaves) {
      float4 v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = load_tile(d, xr, t0 + i * kWaves, T4, nt);
      absmax_tiles(d, sh, v, t0, T4, nt);
    }
    __syncthreads();
    if (tid < d.M) sh.sm[tid] = row_scale(sh, tid, d.eps);
    if (PRE) quant_tiles(d, sh, xb.f, wave, T4, nt, Kp);
    for (int t0 = PRE ? wave + 8 * kWaves : wave; t0 < nt; t0 += 8 * kWaves) {
      float4 v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = load_tile(d, xr, t0 + i * kWaves, T4, nt);
      quant_tiles(d, sh, v, t0, T4, nt, Kp);
    }
    // zeros from the first whole dword past K to the end of the staged row
    const int kz = (d.K + 3) >> 2, nz = Kp4 - kz;
    for (int i = tid; i < d.M * nz; i += kThreads) {
      const int m = i / nz;
      reinterpret_cast<uint32_t *>(sh.xs + m * Kp)[kz + (i - m * nz)] = 0u;
    }
  } else {
    if (tid < d.M) sh.sm[tid] = gp(d.s)[tid];
    if (staged) {
      const int n4 = d.M * Kp4;
      const __amdgpu_buffer_rsrc_t xr = buffer_rsrc(d.xq, (uint32_t)((int64_t)d.M * d.ldxq));
      if (PRE) copy_xq4(d, sh, xb.q, tid, Kp4, n4);
      for (int i0 = PRE ? tid + 8 * kThreads : tid; i0 < n4; i0 += 8 * kThreads) {
        uint32_t v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = load_xq4(d, xr, i0 + i * kThreads, Kp4, n4);
        copy_xq4(d, sh, v, i0, Kp4, n4);
      }
    }
  }
  __syncthreads();
  if (FMT == UG_W_PACK5 && build_table) {  // 64 replicas in 16-byte chunks, consecutive lanes
    uint4 *chunks = reinterpret_cast<uint4 *>(sh.lut);
#pragma unroll
    for (int i = 0; i < 256 * kRepl / 4 / kThreads; ++i) {
      const int c = tid + kThreads * i;
      const uint32_t v = sh.lut_tmp[c >> 4];
      chunks[c] = make_uint4(v, v, v, v);
    }
  }
  if (FMT == UG_W_PACK5) {
    if (staged) {  // permute every 80-position window in place, one window per thread
      const int wpr = Kp / 80, nwin = d.M * wpr;
      for (int w0 = tid; w0 < nwin; w0 += kThreads) {
        const int m = w0 / wpr;
        uint4 *win = reinterpret_cast<uint4 *>(sh.xs + m * Kp + (w0 - m * wpr) * 80);
        uint32_t X[20], F[20];
#pragma unroll
        for (int i = 0; i < 5; ++i) {
          const uint4 q = win[i];
          X[4 * i] = q.x; X[4 * i + 1] = q.y; X[4 * i + 2] = q.z; X[4 * i + 3] = q.w;
        }
        permute80(X, F);
#pragma unroll
        for (int i = 0; i < 5; ++i) win[i] = make_uint4(F[4 * i], F[4 * i + 1], F[4 * i + 2], F[4 * i + 3]);
        atomicAdd(&sh.cm[m], byte_sum4(F[16]) + byte_sum4(F[17]) + byte_sum4(F[18]) + byte_sum4(F[19]));
      }
    } else {  // correction straight from x_q
      for (int m = wave; m < d.M; m += kWaves) {
        int sum = 0;
        for (int k = 5 * lane + 4; k < d.K; k += 5 * 64) sum += gp(d.xq)[(int64_t)m * d.ldxq + k];
        sum = wave_sum_i32(sum);
        if (lane == 0) sh.cm[m] = sum;
      }
    }
    __syncthreads();
  }
}

// The quantized activations and scales as outputs (fused quantization, the
// problem's first block): undo the staging permutation per K position.
template <int FMT>
__device__ __forceinline__ void write_act_outputs(const GemvDesc &d, const Smem<FMT> &sh, int Kp) {
  const int tid = threadIdx.x;
  if (d.s)
    for (int m = tid; m < d.M; m += kThreads) gp(d.s)[m] = sh.sm[m];
  if (d.xq) {
    int8_t *xq = const_cast<int8_t *>(d.xq);
    for (int idx = tid; idx < d.M * d.K; idx += kThreads) {
      const int m = idx / d.K, k = idx - m * d.K;
      int off = k;
      if (FMT == UG_W_PACK5) {
        const int w = k / 80, r = k - 80 * w, g = r / 5, t = r - 5 * g;
        // t < 4: fragment g/4, dword g%4, byte t; t == 4: fragment 4, dword g/4, byte g%4
        off = 80 * w + (t < 4 ? 16 * (g >> 2) + 4 * (g & 3) + t : 64 + 4 * (g >> 2) + (g & 3));
      }
      gp(xq)[(int64_t)m * d.ldxq + k] = sh.xs[m * Kp + off];
    }
  }
}

template <int FMT, int MB, bool FINE>
struct Wave {
  static constexpr int F1 = Fmt<FMT>::kFrag;
  static constexpr int SC = Cfg<FMT, MB, FINE>::SC;
  static constexpr int NACC = Cfg<FMT, MB, FINE>::NACC;
  static constexpr int kRGW = Cfg<FMT, MB, FINE>::RGW;

  int S, NC;
  bool staged;
  int xbase[MB];  // staged: LDS offset of this lane's activation row (step 0)
  __amdgpu_buffer_rsrc_t wr, xr;

  __device__ __forceinline__ void init(const GemvDesc &d, bool stg, int Kp) {
    const int lane = threadIdx.x & 63, q = lane >> 4;
    S = steps_of(FMT, d.K);
    NC = (S + SC - 1) / SC;
    staged = stg;
    wr = buffer_rsrc(d.w, (uint32_t)((int64_t)d.N * d.ldw));
    xr = buffer_rsrc(d.xq, (uint32_t)((int64_t)d.M * d.ldxq));
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      // rows past M read row M-1: MFMA output row m depends only on input
      // row m, and rows past M are never stored
      const int m = min(16 * b + (lane & 15), d.M - 1);
      xbase[b] = m * Kp + q * Fmt<FMT>::kLaneK;
    }
  }

  // Weight loads of unit (item, chunk).  The whole offset is a per-lane
  // value (row offset + step offset), so the buffer's range check sees it:
  // rows past N and bytes past the end of the matrix read zeros, bytes past
  // a row's data (into the next row) meet zero activations.  ok == false
  // (past this wave's work): every offset is pushed past the buffer.
  __device__ __forceinline__ void issue(const GemvDesc &d, int item, int ch, bool ok,
                                        uint4 (&wb)[kRGW][SC]) {
    const int lane = threadIdx.x & 63, q = lane >> 4;
#pragma unroll
    for (int r = 0; r < kRGW; ++r) {
      const int n = (item * kRGW + r) * 16 + (lane & 15);
      // unsigned (wrapping) arithmetic: an offset that wraps into the buffer
      // reads real weights for a row past N, whose results are never stored
      const uint32_t voff = (uint32_t)n * (uint32_t)d.ldw + 16u * q + (ok ? 0u : kOOB);
#pragma unroll
      for (int s = 0; s < SC; ++s) wb[r][s] = buffer_load16(wr, voff + (uint32_t)(64 * (ch * SC + s)));
    }
  }

  // Activation fragments of step st for M-block b.
  __device__ __forceinline__ void xfrags(const GemvDesc &d, const int8_t *xs, int st, int b,
                                         v4i (&xf)[F1]) {
    if (FINE || staged) {
      const int off = xbase[b] + st * Fmt<FMT>::kStepK;
#pragma unroll
      for (int j = 0; j < F1; ++j) xf[j] = *reinterpret_cast<const v4i *>(xs + off + 16 * j);
      return;
    }
    // straight from x_q: 80 (or 16) positions, masked past K, permuted in
    // registers
    const int lane = threadIdx.x & 63, q = lane >> 4;
    const int m = 16 * b + (lane & 15);
    const bool ok = m < d.M && st < S;
    const int p0 = st * Fmt<FMT>::kStepK + q * Fmt<FMT>::kLaneK;
    uint32_t X[4 * F1];
#pragma unroll
    for (int c = 0; c < F1; ++c) {
      const int p = p0 + 16 * c;
      const uint4 v = buffer_load16(xr, ok && p < d.K ? (uint32_t)(m * d.ldxq + p) : kOOB);
      uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int kb = d.K - p - 4 * e;  // bytes of this dword inside the row
        X[4 * c + e] =
            w4[e] & (kb >= 4 ? 0xffffffffu : (kb <= 0 ? 0u : (0xffffffffu >> (8 * (4 - kb)))));
      }
    }
    if (FMT == UG_W_PACK5) {
      uint32_t F[20];
      permute80(reinterpret_cast<const uint32_t(&)[20]>(X), F);
#pragma unroll
      for (int j = 0; j < 5; ++j)
        xf[j] = v4i{(int)F[4 * j], (int)F[4 * j + 1], (int)F[4 * j + 2], (int)F[4 * j + 3]};
    } else {
      xf[0] = v4i{(int)X[0], (int)X[1], (int)X[2], (int)X[3]};
    }
  }

  // Multiply-accumulate one unit (SC steps of every row group of the item).
  // The table reads of the next (step, row group) pair are issued before the
  // MFMAs of the current one.
  __device__ __forceinline__ void compute(const GemvDesc &d, const int8_t *xs, const char *lut,
                                          int ch, const uint4 (&wb)[kRGW][SC],
                                          v4i (&acc)[kRGW][MB][NACC]) {
    const uint32_t lr4 = 4u * (threadIdx.x & 63);
    if (FMT == UG_W_PACK5) {
      constexpr int NP = SC * kRGW;
      uint32_t T[2][20];
      auto dec = [&](int p, uint32_t(&t)[20]) {
        const uint4 &w = wb[p % kRGW][p / kRGW];
        decode4(w.x, lut, lr4, t, t[16]);
        decode4(w.y, lut, lr4, t + 4, t[17]);
        decode4(w.z, lut, lr4, t + 8, t[18]);
        decode4(w.w, lut, lr4, t + 12, t[19]);
      };
      v4i xf[MB][F1];
      dec(0, T[0]);
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int s = p / kRGW, r = p % kRGW;
        if (r == 0)
#pragma unroll
          for (int b = 0; b < MB; ++b) xfrags(d, xs, ch * SC + s, b, xf[b]);
        if (p + 1 < NP) dec(p + 1, T[(p + 1) & 1]);
        const uint32_t(&t)[20] = T[p & 1];
#pragma unroll
        for (int j = 0; j < 5; ++j) {
          const v4i B = {(int)t[4 * j], (int)t[4 * j + 1], (int)t[4 * j + 2], (int)t[4 * j + 3]};
#pragma unroll
          for (int b = 0; b < MB; ++b)
            acc[r][b][j % NACC] =
                __builtin_amdgcn_mfma_i32_16x16x64_i8(xf[b][j], B, acc[r][b][j % NACC], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int s = 0; s < SC; ++s) {
        v4i xf[MB][F1];
#pragma unroll
        for (int b = 0; b < MB; ++b) xfrags(d, xs, ch * SC + s, b, xf[b]);
#pragma unroll
        for (int r = 0; r < kRGW; ++r) {
          const v4i B = {(int)wb[r][s].x, (int)wb[r][s].y, (int)wb[r][s].z, (int)wb[r][s].w};
#pragma unroll
          for (int b = 0; b < MB; ++b)
            acc[r][b][s % NACC] =
                __builtin_amdgcn_mfma_i32_16x16x64_i8(xf[b][0], B, acc[r][b][s % NACC], 0, 0, 0);
        }
      }
    }
  }

  // Lane (n = l%16, q = l/16) holds D[m = 16 b + 4 q + r][n].
  __device__ __forceinline__ void store(const GemvDesc &d, int item, v4i (&acc)[kRGW][MB][NACC],
                                        const float *sm, const int *cm, float beta) {
    const int lane = threadIdx.x & 63, q = lane >> 4;
#pragma unroll
    for (int rg = 0; rg < kRGW; ++rg) {
      const int n = (item * kRGW + rg) * 16 + (lane & 15);
#pragma unroll
      for (int b = 0; b < MB; ++b) {
        v4i v = acc[rg][b][0];
#pragma unroll
        for (int a = 1; a < NACC; ++a) v += acc[rg][b][a];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = 16 * b + 4 * q + r;
          if (n < d.N && m < d.M) {
            const int val = FMT == UG_W_PACK5 ? v[r] - cm[m] : v[r];
            if (d.acc) gp(d.acc)[(int64_t)m * d.ldacc + n] = val;
            if (d.y) {
              const float scale = sm[m] * beta;
              gp(d.y)[(int64_t)m * d.ldy + n] = (float)val * scale;
            }
          }
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Stream split.
//
// Items [i0, i1) of problem d: wave w takes items i0 + w, i0 + w + 8, ...,
// each NC units, with the weights of the next two units in flight.  start()
// issues the first two units' loads, so they travel while the block sets up.
template <int FMT, int MB>
struct ItemLoop {
  using W = Wave<FMT, MB, false>;
  static constexpr int SC = W::SC, NACC = W::NACC, kRGW = W::kRGW;
  W wv;
  uint4 A[kRGW][SC], B[kRGW][SC], C[kRGW][SC];
  v4i acc[kRGW][MB][NACC];
  float beta;
  int i1, U;
  // issue position (item, chunk) and process position, advanced unit by unit
  int iss_it, iss_ch, pro_it, pro_ch;

  __device__ __forceinline__ void issue(const GemvDesc &d, uint4 (&buf)[kRGW][SC]) {
    wv.issue(d, iss_it, iss_ch, iss_it < i1, buf);
    if (++iss_ch == wv.NC) {
      iss_ch = 0;
      iss_it += kWaves;
    }
  }

  __device__ __forceinline__ void process(const GemvDesc &d, const Smem<FMT> &sh,
                                          const uint4 (&buf)[kRGW][SC]) {
    if (pro_ch == 0) {
#pragma unroll
      for (int r = 0; r < kRGW; ++r)
#pragma unroll
        for (int b = 0; b < MB; ++b)
#pragma unroll
          for (int a = 0; a < NACC; ++a) acc[r][b][a] = v4i{0, 0, 0, 0};
    }
    wv.compute(d, sh.xs, reinterpret_cast<const char *>(sh.lut), pro_ch, buf, acc);
    if (pro_ch == wv.NC - 1) wv.store(d, pro_it, acc, sh.sm, sh.cm, beta);
    if (++pro_ch == wv.NC) {
      pro_ch = 0;
      pro_it += kWaves;
    }
  }

  __device__ __forceinline__ void start(const GemvDesc &d, bool staged, int Kp, int i0, int i1_) {
    wv.init(d, staged, Kp);
    const int wave = uniform(threadIdx.x >> 6);
    const int my_items = i0 + wave < i1_ ? (i1_ - i0 - wave + kWaves - 1) / kWaves : 0;
    U = uniform(my_items * wv.NC);
    i1 = i1_;
    iss_it = pro_it = i0 + wave;
    iss_ch = pro_ch = 0;
    issue(d, A);
    issue(d, B);
    beta = gp(d.beta)[0];
  }

  // Needs the block's set-up (table, staged rows) to be complete.
  __device__ __forceinline__ void run(const GemvDesc &d, const Smem<FMT> &sh) {
    for (int u = 0; u < U;) {
      issue(d, C);
      process(d, sh, A);
      if (++u >= U) break;
      issue(d, A);
      process(d, sh, B);
      if (++u >= U) break;
      issue(d, B);
      process(d, sh, C);
      ++u;
    }
  }
};

// The block takes the global items [g0, g1) of the plan (problem p holds
// item g0; problem q owns [item_begin, +items)), crossing into the next
// problem when its range does.
template <int FMT, int MB>
__device__ __forceinline__ void stream_block(const GemvDesc *plan, int count, int p, int g0,
                                             int g1) {
  __shared__ Smem<FMT> sh;
  bool first = true;
  for (int g = g0; g < g1 && p < count; ++p) {
    const GemvDesc d = plan[p];
    const int e = min(g1, d.item_begin + d.items);
    if (e <= g) continue;
    const bool staged = stages_x(FMT, d.M, d.K);
    const int Kp = staged_kp(FMT, MB, d.K);
    XBatch xb;  // unused: the set-up loads its own batches here
    ItemLoop<FMT, MB> loop;
    loop.start(d, staged, Kp, g - d.item_begin, e - d.item_begin);
    if (!first) __syncthreads();  // the previous problem's staged rows are done
    setup_finish<FMT, false>(d, sh, staged, Kp, first, false, xb);
    first = false;
    loop.run(d, sh);
    if (d.x && g == d.item_begin) write_act_outputs<FMT>(d, sh, Kp);
    g = e;
  }
}

template <int FMT, int MB>
__global__ __launch_bounds__(kThreads) void gemv_stream_single(GemvDesc d) {
  const int64_t T = d.items;
  const int g0 = (int)(T * blockIdx.x / gridDim.x), g1 = (int)(T * (blockIdx.x + 1) / gridDim.x);
  if (g0 < g1) stream_block<FMT, MB>(&d, 1, 0, g0, g1);
}

template <int FMT, int MB>
__global__ __launch_bounds__(kThreads) void gemv_stream_grouped(const GemvDesc *__restrict__ plan,
                                                                const GemvBlock *__restrict__ blocks,
                                                                int count) {
  const GemvBlock bl = blocks[blockIdx.x];
  if (bl.i0 < bl.i1) stream_block<FMT, MB>(plan, count, bl.p, bl.i0, bl.i1);
}

// ---------------------------------------------------------------------------
// Fine split (M <= 16, staged activations).
//
// A decode-sized launch is one chain of dependent steps per wave, and a wave
// issues at most one instruction every four cycles, so this path keeps the
// instruction count of every step small: no lane divides by a run-time
// value, and the problem's kind (fp32 activations or x_q) is a template
// parameter instead of a branch.

// A wave's share of the tiles of the staged rows: tiles [t, te) of the M * T
// tiles (row m = t / T, chunk c = t % T), taken 8 at a time with (m, c)
// advanced by increments: one division per wave.
struct TileWalk {
  int t, te, m, c, T;
  __device__ __forceinline__ void init(int nt, int T_) {
    const int wave = uniform(threadIdx.x >> 6);
    T = T_;
    t = (wave * nt) / kWaves;
    te = ((wave + 1) * nt) / kWaves;
    m = t / T;
    c = t - m * T;
  }
};
struct TileBatch {
  bool ok[8];
  int m[8], c[8];
};
__device__ __forceinline__ void next8(TileWalk &w, TileBatch &b) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    b.ok[i] = w.t + i < w.te;
    b.m[i] = w.m;
    b.c[i] = w.c;
    if (++w.c == w.T) {
      w.c = 0;
      ++w.m;
    }
  }
  w.t += 8;
}

// fp32 tiles: 256 positions, lane l the float4 at 256 c + 4 l (a float4 at
// k < K is inside the row: ldx >= round_up(K, 4)).  x_q tiles: 1024 bytes,
// lane l the 16 bytes at 1024 c + 16 l (inside the row when k < K: ldxq >=
// round_up(K, 16)).
template <bool FUSED>
__device__ __forceinline__ void load_batch(const GemvDesc &d, __amdgpu_buffer_rsrc_t xr,
                                           const TileBatch &b, uint4 (&u)[8]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (FUSED) {
      const int k = b.c[i] * 256 + 4 * lane;
      u[i] = buffer_load16(xr, b.ok[i] && k < d.K ? (uint32_t)((b.m[i] * (int)d.ldx + k) * 4) : kOOB);
    } else {
      const int k = b.c[i] * 1024 + 16 * lane;
      u[i] = buffer_load16(xr, b.ok[i] && k < d.K ? (uint32_t)(b.m[i] * (int)d.ldxq + k) : kOOB);
    }
  }
}

template <bool FUSED>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t x_rsrc(const GemvDesc &d) {
  return FUSED ? buffer_rsrc(d.x, (uint32_t)((int64_t)d.M * d.ldx * 4))
               : buffer_rsrc(d.xq, (uint32_t)((int64_t)d.M * d.ldxq));
}

template <bool FUSED>
__device__ __forceinline__ int tiles_per_row(int Kp) {
  return FUSED ? (Kp + 255) >> 8 : (Kp + 1023) >> 10;  // the tiles cover whole staged rows
}

// Pass 1 of fused quantization: per-wave row maxima.
template <int FMT>
__device__ __forceinline__ void fine_absmax(const GemvDesc &d, Smem<FMT> &sh, const TileBatch &b,
                                            const uint4 (&u)[8]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (b.ok[i]) {
      const float4 v = __builtin_bit_cast(float4, u[i]);
      const int k = b.c[i] * 256 + 4 * lane;
      float a = fabsf(v.x);  // zero when k >= K
      if (k + 1 < d.K) a = fmaxf(a, fabsf(v.y));
      if (k + 2 < d.K) a = fmaxf(a, fabsf(v.z));
      if (k + 3 < d.K) a = fmaxf(a, fabsf(v.w));
      a = wave_max(a);
      if (lane == 0) sh.part[wave][b.m[i]] = fmaxf(sh.part[wave][b.m[i]], a);
    }
  }
}

// Pass 2: quantized dwords into the staged rows (zeros past K), and into x_q
// when the block writes the outputs.
template <int FMT>
__device__ __forceinline__ void fine_quant(const GemvDesc &d, Smem<FMT> &sh, const TileBatch &b,
                                           const uint4 (&u)[8], int Kp, bool outputs) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int m = b.m[i], k = b.c[i] * 256 + 4 * lane;
    if (b.ok[i] && k < Kp) {
      const float4 v = __builtin_bit_cast(float4, u[i]);
      const float s = row_scale(sh, m, d.eps);
      const uint32_t w = k < d.K ? pack4(q8(v.x, s), k + 1 < d.K ? q8(v.y, s) : 0,
                                         k + 2 < d.K ? q8(v.z, s) : 0, k + 3 < d.K ? q8(v.w, s) : 0)
                                 : 0u;
      *reinterpret_cast<uint32_t *>(sh.xs + m * Kp + k) = w;
      if (outputs && k < d.K) {
        int8_t *row = const_cast<int8_t *>(d.xq) + (int64_t)m * d.ldxq;
        if (k + 4 <= d.K) {
          *gp(reinterpret_cast<uint32_t *>(row + k)) = w;  // rows are 16-byte aligned
        } else {
          for (int j = 0; k + j < d.K; ++j) gp(row)[k + j] = (int8_t)(w >> (8 * j));
        }
      }
    }
  }
}

// x_q tiles into the staged rows, bytes past K zeroed.
template <int FMT>
__device__ __forceinline__ void fine_copy(const GemvDesc &d, Smem<FMT> &sh, const TileBatch &b,
                                          const uint4 (&u)[8], int Kp) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int k = b.c[i] * 1024 + 16 * lane;
    if (b.ok[i] && k < Kp) {
      uint32_t w4[4] = {u[i].x, u[i].y, u[i].z, u[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int kb = d.K - k - 4 * e;  // bytes of this dword inside the row
        w4[e] &= kb >= 4 ? 0xffffffffu : (kb <= 0 ? 0u : (0xffffffffu >> (8 * (4 - kb))));
      }
      *reinterpret_cast<uint4 *>(sh.xs + b.m[i] * Kp + k) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
    }
  }
}

// The first batch of a wave's activation tiles, issued by the caller before
// its weight loads: loads complete in issue order, so waiting for these
// never waits for the weights.
template <bool FUSED>
__device__ __forceinline__ void fine_issue_x(const GemvDesc &d, int Kp, TileWalk &walk,
                                             TileBatch &b0, uint4 (&u0)[8]) {
  walk.init(d.M * tiles_per_row<FUSED>(Kp), tiles_per_row<FUSED>(Kp));
  next8(walk, b0);
  load_batch<FUSED>(d, x_rsrc<FUSED>(d), b0, u0);
}

// Block set-up of the fine split: decode table, row scales, staged rows
// from the wave's tiles (the first batch already loaded), the five-trit
// permutation with the correction cm, zeroed slots.  s_in: with x_q given,
// thread m < M holds s[m].  Ends with a barrier.
template <int FMT, bool FUSED>
__device__ __forceinline__ void fine_setup(const GemvDesc &d, Smem<FMT> &sh, int Kp,
                                           bool first_block, const TileWalk &walk,
                                           const TileBatch &b0, const uint4 (&u0)[8],
                                           float s_in) {
  const int tid = threadIdx.x, wave = uniform(tid >> 6), lane = tid & 63;
  if (FMT == UG_W_PACK5 && tid < 256) sh.lut_tmp[tid] = lut4_entry(tid);
  if (tid < 64) sh.cm[tid] = 0;
  if (tid < 20) reinterpret_cast<uint32_t *>(sh.xs + kZero)[tid] = 0;
#pragma unroll
  for (int i = 0; i < kFineItems * 64 / kThreads; ++i)
    reinterpret_cast<uint4 *>(sh.slots)[tid + i * kThreads] = make_uint4(0, 0, 0, 0);
  const __amdgpu_buffer_rsrc_t xr = x_rsrc<FUSED>(d);
  if (FUSED) {
    sh.part[wave][lane] = 0.0f;
    fine_absmax(d, sh, b0, u0);
    TileWalk w = walk;
    while (w.t < w.te) {
      TileBatch b;
      uint4 u[8];
      next8(w, b);
      load_batch<true>(d, xr, b, u);
      fine_absmax(d, sh, b, u);
    }
    __syncthreads();
    const bool outputs = first_block && d.xq;
    if (tid < d.M) {
      const float s = row_scale(sh, tid, d.eps);
      sh.sm[tid] = s;
      if (first_block && d.s) gp(d.s)[tid] = s;
    }
    fine_quant(d, sh, b0, u0, Kp, outputs);
    w = walk;
    while (w.t < w.te) {
      TileBatch b;
      uint4 u[8];
      next8(w, b);
      load_batch<true>(d, xr, b, u);
      fine_quant(d, sh, b, u, Kp, outputs);
    }
  } else {
    if (tid < d.M) sh.sm[tid] = s_in;
    fine_copy(d, sh, b0, u0, Kp);
    TileWalk w = walk;
    while (w.t < w.te) {
      TileBatch b;
      uint4 u[8];
      next8(w, b);
      load_batch<false>(d, xr, b, u);
      fine_copy(d, sh, b, u, Kp);
    }
  }
  __syncthreads();
  if (FMT == UG_W_PACK5) {
    uint4 *chunks = reinterpret_cast<uint4 *>(sh.lut);  // 64 replicas, 16-byte chunks
#pragma unroll
    for (int i = 0; i < 256 * kRepl / 4 / kThreads; ++i) {
      const int c = tid + kThreads * i;
      const uint32_t v = sh.lut_tmp[c >> 4];
      chunks[c] = make_uint4(v, v, v, v);
    }
    // every 80-position window permuted in place: thread per window, the
    // windows of one row on consecutive threads
    const int wpr = Kp / 80;
    int m = 0, w0 = tid;
    while (w0 >= wpr && m < d.M) {  // row of this thread's first window (few steps: wpr >= 1)
      w0 -= wpr;
      ++m;
    }
    for (; m < d.M; ) {
      uint4 *win = reinterpret_cast<uint4 *>(sh.xs + m * Kp + w0 * 80);
      uint32_t X[20], F[20];
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        const uint4 q = win[i];
        X[4 * i] = q.x; X[4 * i + 1] = q.y; X[4 * i + 2] = q.z; X[4 * i + 3] = q.w;
      }
      permute80(X, F);
#pragma unroll
      for (int i = 0; i < 5; ++i) win[i] = make_uint4(F[4 * i], F[4 * i + 1], F[4 * i + 2], F[4 * i + 3]);
      atomicAdd(&sh.cm[m], byte_sum4(F[16]) + byte_sum4(F[17]) + byte_sum4(F[18]) + byte_sum4(F[19]));
      w0 += kThreads;
      while (w0 >= wpr && m < d.M) {
        w0 -= wpr;
        ++m;
      }
    }
    __syncthreads();
  }
}

// Items [i0, i1) of problem d (16 rows each), S steps per item: piece
// p = (item i0 + p / S, step p % S).  Wave w takes pieces [w P / 8,
// (w + 1) P / 8) of the block's P, issues all their weight loads first (the
// set-up's activation loads follow them), and adds its partial sums to the
// item's LDS slot whenever its next piece belongs to another item.  After a
// barrier the block writes every item's outputs.
template <int FMT, bool FUSED>
__device__ __forceinline__ void fine_block(const GemvDesc &d, int i0, int i1) {
  using W = Wave<FMT, 1, true>;
  constexpr int NACC = W::NACC;
  __shared__ Smem<FMT> sh;
  const int tid = threadIdx.x, wave = uniform(tid >> 6), lane = tid & 63;
  const int S = steps_of(FMT, d.K), Kp = fine_kp(FMT, d.K);
  const int P = (i1 - i0) * S;
  const int p0 = uniform(wave * P / kWaves), p1 = uniform((wave + 1) * P / kWaves);
  const int it0 = p0 / S, st0 = p0 - it0 * S;
  const float s_in = !FUSED && tid < d.M ? gp(d.s)[tid] : 0.0f;
  TileWalk walk;
  TileBatch b0;
  uint4 x0[8];
  fine_issue_x<FUSED>(d, Kp, walk, b0, x0);
  W wv;
  wv.init(d, true, Kp);
  uint4 wb[kFinePieces][1][1];
  {
    int it = it0, st = st0;
#pragma unroll
    for (int j = 0; j < kFinePieces; ++j) {
      wv.issue(d, i0 + it, st, p0 + j < p1, wb[j]);
      if (++st == S) {
        st = 0;
        ++it;
      }
    }
  }
  const float beta = gp(d.beta)[0];
  fine_setup<FMT, FUSED>(d, sh, Kp, i0 == 0, walk, b0, x0, s_in);
  const char *lut = reinterpret_cast<const char *>(sh.lut);
  v4i acc[1][1][NACC];
#pragma unroll
  for (int a = 0; a < NACC; ++a) acc[0][0][a] = v4i{0, 0, 0, 0};
  int it = it0, st = st0;
#pragma unroll
  for (int j = 0; j < kFinePieces; ++j) {
    if (p0 + j < p1) {
      wv.compute(d, sh.xs, lut, st, wb[j], acc);
      if (p0 + j + 1 == p1 || st + 1 == S) {  // last piece of this item here
        v4i v = acc[0][0][0];
#pragma unroll
        for (int a = 1; a < NACC; ++a) v += acc[0][0][a];
        const int n = lane & 15, q = lane >> 4;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (4 * q + r < d.M) atomicAdd(&sh.slots[it * 256 + (4 * q + r) * 16 + n], v[r]);
#pragma unroll
        for (int a = 0; a < NACC; ++a) acc[0][0][a] = v4i{0, 0, 0, 0};
      }
      if (++st == S) {
        st = 0;
        ++it;
      }
    }
  }
  __syncthreads();
  if (tid < (i1 - i0) * 16) {  // thread (item, n) writes column n of the item, every row
    const int li = tid >> 4, n = tid & 15, ng = (i0 + li) * 16 + n;
    if (ng < d.N) {
      for (int m = 0; m < d.M; ++m) {
        const int val = sh.slots[li * 256 + m * 16 + n] - (FMT == UG_W_PACK5 ? sh.cm[m] : 0);
        if (d.acc) gp(d.acc)[(int64_t)m * d.ldacc + ng] = val;
        if (d.y) gp(d.y)[(int64_t)m * d.ldy + ng] = (float)val * (sh.sm[m] * beta);
      }
    }
  }
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void gemv_fine_single(GemvDesc d, int ipb) {
  const int i0 = blockIdx.x * ipb, i1 = min(d.items, i0 + ipb);
  if (i0 < i1) fine_block<FMT, false>(d, i0, i1);
}

template <int FMT, bool FUSED>
__global__ __launch_bounds__(kThreads) void gemv_fine_grouped(const GemvBlock *__restrict__ blocks) {
  const GemvBlock bl = blocks[blockIdx.x];
  if (bl.i0 < bl.i1) fine_block<FMT, FUSED>(bl.d, bl.i0, bl.i1);
}

// ---------------------------------------------------------------------------
// Host side.

// Fine split of a group: items per block for every problem, or false when
// the group is too large for it (then the stream split runs).  Blocks of
// about T / 256 pieces each, at most kFineItems items, one problem each.
bool plan_fine(GemvDesc *descs, int count, std::vector<GemvBlock> &blocks) {
  int64_t T = 0;
  for (int i = 0; i < count; ++i) {
    const GemvDesc &d = descs[i];
    if (d.M > 16 || (int64_t)d.M * fine_kp(d.wfmt, d.K) > kXsBytes) return false;
    if ((d.x != nullptr) != (descs[0].x != nullptr)) return false;  // one kind per launch
    T += (int64_t)((d.N + 15) / 16) * steps_of(d.wfmt, d.K);
  }
  if (T > (int64_t)kGemvBlocks * kWaves * kFinePieces) return false;
  std::vector<int> ipb((size_t)count);
  for (int64_t target = (T + kGemvBlocks - 1) / kGemvBlocks;; ++target) {
    if (target > (int64_t)kWaves * kFinePieces) return false;
    int64_t nb = 0;
    bool fits = true;
    for (int i = 0; i < count; ++i) {
      const int S = steps_of(descs[i].wfmt, descs[i].K), items = (descs[i].N + 15) / 16;
      int k = (int)(target / S);
      k = k < 1 ? 1 : (k > kFineItems ? kFineItems : k);
      k = k > items ? items : k;
      // every wave's share of a block's pieces must fit its registers
      if ((k * S + kWaves - 1) / kWaves > kFinePieces) fits = false;
      ipb[(size_t)i] = k;
      nb += (items + k - 1) / k;
    }
    if (!fits) return false;
    if (nb <= kGemvBlocks) break;
  }
  blocks.clear();
  for (int i = 0; i < count; ++i) {
    const int items = (descs[i].N + 15) / 16;
    descs[i].mb = 1;
    descs[i].items = items;
    for (int a = 0; a < items; a += ipb[(size_t)i])
      blocks.push_back(GemvBlock{descs[i], i, a, std::min(items, a + ipb[(size_t)i]), 0});
  }
  return true;
}

}  // namespace

// Blocks for T items of the stream split: one per CU when there are enough
// items, else one per 4 items.
int gemv_grid(int64_t total_items) {
  const int64_t by_items = (total_items + 3) / 4;
  return (int)(by_items < kGemvBlocks ? (by_items < 1 ? 1 : by_items) : kGemvBlocks);
}

int gemv_plan(GemvDesc *descs, int count, std::vector<GemvBlock> &blocks) {
  const int fmt = descs[0].wfmt;
  for (int i = 1; i < count; ++i)
    if (descs[i].wfmt != fmt) return -1;
  int64_t total = 0;
  if (plan_fine(descs, count, blocks)) {
    for (int i = 0; i < count; ++i) {
      descs[i].item_begin = (int32_t)total;
      total += descs[i].items;
    }
    return (descs[0].x ? 512 : 0) + 256 + 16 * fmt + 1;
  }
  const int mb = mb_of(descs[0].M);
  for (int i = 0; i < count; ++i) {
    GemvDesc &d = descs[i];
    d.mb = mb_of(d.M);
    if (d.mb != mb) return -1;
    const int rg = (d.N + 15) / 16;
    d.items = (rg + 1) / 2;  // two row groups per item
    d.item_begin = (int32_t)total;
    total += d.items;
  }
  if (total > INT32_MAX) return -1;
  const int grid = gemv_grid(total);
  blocks.clear();
  int p = 0;
  for (int b = 0; b < grid; ++b) {
    const int g0 = (int)(total * b / grid), g1 = (int)(total * (b + 1) / grid);
    while (p + 1 < count && descs[p + 1].item_begin <= g0) ++p;
    blocks.push_back(GemvBlock{descs[p], p, g0, g1, 0});
  }
  return 16 * fmt + mb;
}

bool gemv_stages_x(int wfmt, int64_t M, int64_t K) {
  return K <= UG_MAX_K && M <= 64 && stages_x(wfmt, (int)M, (int)K);
}

hipError_t launch_gemv_grouped(const GemvDesc *plan_dev, const GemvBlock *blocks_dev, int32_t count,
                               int32_t grid, int32_t variant, hipStream_t st) {
  const bool fine = (variant >> 8) & 1, fused = (variant >> 9) & 1;
  const int fmt = (variant >> 4) & 15, mb = variant & 15;
  dim3 g(grid), b(kThreads);
  if (fine) {
    if (fmt == UG_W_PACK5) {
      if (fused) hipLaunchKernelGGL((gemv_fine_grouped<UG_W_PACK5, true>), g, b, 0, st, blocks_dev);
      else hipLaunchKernelGGL((gemv_fine_grouped<UG_W_PACK5, false>), g, b, 0, st, blocks_dev);
    } else {
      if (fused) hipLaunchKernelGGL((gemv_fine_grouped<UG_W_I8, true>), g, b, 0, st, blocks_dev);
      else hipLaunchKernelGGL((gemv_fine_grouped<UG_W_I8, false>), g, b, 0, st, blocks_dev);
    }
    return hipGetLastError();
  }
#define UG_GROUPED(F, MBV) \
  hipLaunchKernelGGL((gemv_stream_grouped<F, MBV>), g, b, 0, st, plan_dev, blocks_dev, count)
  if (fmt == UG_W_PACK5) {
    if (mb == 1) UG_GROUPED(UG_W_PACK5, 1);
    else if (mb == 2) UG_GROUPED(UG_W_PACK5, 2);
    else UG_GROUPED(UG_W_PACK5, 4);
  } else {
    if (mb == 1) UG_GROUPED(UG_W_I8, 1);
    else if (mb == 2) UG_GROUPED(UG_W_I8, 2);
    else UG_GROUPED(UG_W_I8, 4);
  }
#undef UG_GROUPED
  return hipGetLastError();
}

hipError_t launch_gemv(const int8_t *xq, int64_t ldx, const float *s, const void *w, int wfmt,
                       int64_t ldw, const float *beta, int64_t M, int64_t N, int64_t K,
                       int32_t *acc, int64_t ldacc, float *y, int64_t ldy, hipStream_t st) {
  GemvDesc d{};
  d.x = nullptr;
  d.xq = xq;
  d.ldxq = ldx;
  d.s = const_cast<float *>(s);
  d.w = (const uint8_t *)w;
  d.ldw = ldw;
  d.beta = beta;
  d.acc = acc;
  d.ldacc = ldacc;
  d.y = y;
  d.ldy = ldy;
  d.wfmt = wfmt;
  d.M = (int32_t)M;
  d.N = (int32_t)N;
  d.K = (int32_t)K;
  std::vector<GemvBlock> blocks;
  const int variant = gemv_plan(&d, 1, blocks);
  if (variant < 0) return hipErrorInvalidValue;
  const int grid = (int)blocks.size();
  dim3 g(grid), b(kThreads);
  if ((variant >> 8) & 1) {
    const int ipb = blocks[0].i1 - blocks[0].i0;  // one problem: equal blocks, the last maybe short
    if (wfmt == UG_W_PACK5)
      hipLaunchKernelGGL((gemv_fine_single<UG_W_PACK5>), g, b, 0, st, d, ipb);
    else
      hipLaunchKernelGGL((gemv_fine_single<UG_W_I8>), g, b, 0, st, d, ipb);
    return hipGetLastError();
  }
#define UG_SINGLE(F, MBV) hipLaunchKernelGGL((gemv_stream_single<F, MBV>), g, b, 0, st, d)
  if (wfmt == UG_W_PACK5) {
    if (d.mb == 1) UG_SINGLE(UG_W_PACK5, 1);
    else if (d.mb == 2) UG_SINGLE(UG_W_PACK5, 2);
    else UG_SINGLE(UG_W_PACK5, 4);
  } else {
    if (d.mb == 1) UG_SINGLE(UG_W_I8, 1);
    else if (d.mb == 2) UG_SINGLE(UG_W_I8, 2);
    else UG_SINGLE(UG_W_I8, 4);
  }
#undef UG_SINGLE
  return hipGetLastError();
}

}  // namespace ug

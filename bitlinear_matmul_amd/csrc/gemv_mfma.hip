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
// Work: a block of 8 waves (one block per CU) takes a range of items of one
// problem; an item is 2 or 4 row groups (32 or 64 weight rows) over the whole K, split
// into units of SC steps.  Each wave walks its items' units keeping the
// weights of the next two units in flight (buffer loads: lanes past the row,
// past N or past the work read zeros without touching memory, so the loop
// has no branches).  The 64 KB table and the staged activations are built
// once per block and shared by its 8 waves.  Activations may arrive as fp32:
// the block then quantizes the rows itself with ug_quant_act's arithmetic,
// so act quant + GEMV of a whole group is one launch.
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

template <int FMT, int MB>
struct Cfg {
  static constexpr int RGW = 2;  // row groups per item (they share each activation read)
  // steps per unit (three units of weights are in flight per wave)
  static constexpr int SC = FMT == UG_W_PACK5 ? (MB == 1 ? 4 : (MB == 2 ? 2 : 1)) : (MB == 4 ? 2 : 4);
  // independent MFMA chains per output tile
  static constexpr int NACC = FMT == UG_W_PACK5 ? (MB == 1 ? 2 : (MB == 2 ? 2 : 1)) : 2;
};

__host__ __device__ __forceinline__ int row_bytes_of(int fmt, int K) {
  return fmt == UG_W_PACK5 ? (K + 4) / 5 : K;
}
__host__ __device__ __forceinline__ int steps_of(int fmt, int K) {
  return (row_bytes_of(fmt, K) + 63) / 64;
}
__host__ __device__ __forceinline__ int sc_of(int fmt, int mb) {
  return fmt == UG_W_PACK5 ? (mb == 1 ? Cfg<UG_W_PACK5, 1>::SC : (mb == 2 ? Cfg<UG_W_PACK5, 2>::SC : Cfg<UG_W_PACK5, 4>::SC))
                           : (mb == 1 ? Cfg<UG_W_I8, 1>::SC : (mb == 2 ? Cfg<UG_W_I8, 2>::SC : Cfg<UG_W_I8, 4>::SC));
}
// Staged row length: whole units of steps, zero past K, so every step a
// wave multiplies has activations (zeros past K) inside its row.
__host__ __device__ __forceinline__ int staged_kp(int fmt, int mb, int K) {
  const int sc = sc_of(fmt, mb);
  return ((steps_of(fmt, K) + sc - 1) / sc) * sc * (fmt == UG_W_PACK5 ? 320 : 64);
}
__host__ __device__ __forceinline__ int mb_of(int M) { return M <= 16 ? 1 : (M <= 32 ? 2 : 4); }
__host__ __device__ __forceinline__ bool stages_x(int fmt, int M, int K) {
  return (int64_t)M * staged_kp(fmt, mb_of(M), K) <= kXsBytes;
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

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
  float sm[64];
  int cm[64];
};

// Block set-up: decode table, row scales (fused quantization), staged and
// permuted activations with the d4 correction cm[m] = sum_g x[5g+4], and the
// quantized activations / scales as outputs when this is the problem's
// first block.  Ends with a barrier.
template <int FMT>
__device__ __forceinline__ void setup(const GemvDesc &d, Smem<FMT> &sh, bool staged,
                                      bool write_outputs, bool build_table) {
  const int tid = threadIdx.x, wave = uniform(tid >> 6), lane = tid & 63;
  if (FMT == UG_W_PACK5 && build_table && tid < 256) sh.lut_tmp[tid] = lut4_entry(tid);
  if (tid < 64) sh.cm[tid] = 0;
  if (tid < 20) reinterpret_cast<uint32_t *>(sh.xs + kZero)[tid] = 0;
  if (d.x) {  // row scales s = fl(fl(max|x| / 127) + eps), one wave per row
    for (int m = wave; m < d.M; m += kWaves) {
      const float *xr = d.x + (int64_t)m * d.ldx;
      float a = 0.0f;
      for (int k = 4 * lane; k < d.K; k += 256) {
        const float4 v = *reinterpret_cast<const float4 *>(xr + k);
        a = fmaxf(a, fabsf(v.x));
        if (k + 1 < d.K) a = fmaxf(a, fabsf(v.y));
        if (k + 2 < d.K) a = fmaxf(a, fabsf(v.z));
        if (k + 3 < d.K) a = fmaxf(a, fabsf(v.w));
      }
      a = wave_max(a);
      const float a127 = a / 127.0f;
      if (lane == 0) sh.sm[m] = a127 + d.eps;
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
  if (staged) {
    // window = 80 (five trits per byte) or 16 (one per byte) K positions;
    // every thread stages whole windows, all its loads issued first
    constexpr int WIN = FMT == UG_W_PACK5 ? 80 : 16;
    const int Kp = staged_kp(FMT, mb_of(d.M), d.K);
    const int wpr = Kp / WIN;  // windows per row
    const int nwin = d.M * wpr;
    const __amdgpu_buffer_rsrc_t xr = buffer_rsrc(d.xq, (uint32_t)((int64_t)d.M * d.ldxq));
    for (int w0 = tid; w0 < nwin; w0 += kThreads) {
      const int m = w0 / wpr, k0 = (w0 - m * wpr) * WIN;
      uint32_t X[WIN / 4];
      if (d.x) {
        const float *xrow = d.x + (int64_t)m * d.ldx;
        const float s = sh.sm[m];
        float4 f[WIN / 4];
#pragma unroll
        for (int i = 0; i < WIN / 4; ++i)  // float4 at k < K is in-bounds (ldx >= round_up(K,4))
          f[i] = k0 + 4 * i < d.K ? *reinterpret_cast<const float4 *>(xrow + k0 + 4 * i)
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int i = 0; i < WIN / 4; ++i) {
          const int k = k0 + 4 * i;
          X[i] = pack4(k < d.K ? q8(f[i].x, s) : 0, k + 1 < d.K ? q8(f[i].y, s) : 0,
                       k + 2 < d.K ? q8(f[i].z, s) : 0, k + 3 < d.K ? q8(f[i].w, s) : 0);
        }
      } else {
#pragma unroll
        for (int i = 0; i < WIN / 4; ++i) {
          const int k = k0 + 4 * i;  // 4 bytes at k < K are in-bounds (ldxq >= round_up(K,16))
          uint32_t v = buffer_load4(xr, k < d.K ? (uint32_t)(m * d.ldxq + k) : kOOB);
          if (k + 4 > d.K) v &= k >= d.K ? 0u : (0xffffffffu >> (8 * (k + 4 - d.K)));
          X[i] = v;
        }
      }
      uint4 *dst = reinterpret_cast<uint4 *>(sh.xs + m * Kp + k0);
      if (FMT == UG_W_PACK5) {
        uint32_t F[20];
        permute80(reinterpret_cast<const uint32_t(&)[20]>(X), F);
#pragma unroll
        for (int i = 0; i < 5; ++i) dst[i] = make_uint4(F[4 * i], F[4 * i + 1], F[4 * i + 2], F[4 * i + 3]);
        atomicAdd(&sh.cm[m], byte_sum4(F[16]) + byte_sum4(F[17]) + byte_sum4(F[18]) + byte_sum4(F[19]));
      } else {
        dst[0] = make_uint4(X[0], X[1], X[2], X[3]);
      }
    }
  } else if (FMT == UG_W_PACK5) {  // correction straight from x_q
    for (int m = wave; m < d.M; m += kWaves) {
      int sum = 0;
      for (int k = 5 * lane + 4; k < d.K; k += 5 * 64) sum += d.xq[(int64_t)m * d.ldxq + k];
      sum = wave_sum_i32(sum);
      if (lane == 0) sh.cm[m] = sum;
    }
  }
  __syncthreads();
  if (write_outputs && d.x) {
    if (d.s)
      for (int m = tid; m < d.M; m += kThreads) d.s[m] = sh.sm[m];
    if (d.xq) {  // undo the staging permutation: read back per K position
      int8_t *xq = const_cast<int8_t *>(d.xq);
      const int Kp = staged_kp(FMT, mb_of(d.M), d.K);
      for (int idx = tid; idx < d.M * d.K; idx += kThreads) {
        const int m = idx / d.K, k = idx - m * d.K;
        int off = k;
        if (FMT == UG_W_PACK5) {
          const int w = k / 80, r = k - 80 * w, g = r / 5, t = r - 5 * g;
          // t < 4: fragment g/4, dword g%4, byte t; t == 4: fragment 4, dword g/4, byte g%4
          off = 80 * w + (t < 4 ? 16 * (g >> 2) + 4 * (g & 3) + t : 64 + 4 * (g >> 2) + (g & 3));
        }
        xq[(int64_t)m * d.ldxq + k] = sh.xs[m * Kp + off];
      }
    }
  }
}

template <int FMT, int MB>
struct Wave {
  static constexpr int F1 = Fmt<FMT>::kFrag;
  static constexpr int SC = Cfg<FMT, MB>::SC;
  static constexpr int NACC = Cfg<FMT, MB>::NACC;
  static constexpr int kRGW = Cfg<FMT, MB>::RGW;

  int S, NC, Kp;
  bool staged;
  int xbase[MB];  // staged: LDS offset of this lane's activation row (step 0)
  __amdgpu_buffer_rsrc_t wr, xr;

  __device__ __forceinline__ void init(const GemvDesc &d, bool stg) {
    const int lane = threadIdx.x & 63, q = lane >> 4;
    S = steps_of(FMT, d.K);
    NC = (S + SC - 1) / SC;
    Kp = staged_kp(FMT, MB, d.K);
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
    if (staged) {
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
            if (d.acc) d.acc[(int64_t)m * d.ldacc + n] = val;
            if (d.y) {
              const float sv = d.x ? sm[m] : d.s[m];
              const float scale = sv * beta;
              d.y[(int64_t)m * d.ldy + n] = (float)val * scale;
            }
          }
        }
      }
    }
  }
};

// Items [i0, i1) of problem d: wave w takes items i0 + w, i0 + w + 8, ...,
// each NC units, with the weights of the next two units in flight.
template <int FMT, int MB>
__device__ __forceinline__ void gemv_items(const GemvDesc &d, Smem<FMT> &sh, bool staged,
                                           int i0, int i1) {
  using W = Wave<FMT, MB>;
  constexpr int SC = W::SC, NACC = W::NACC, kRGW = W::kRGW;
  W wv;
  wv.init(d, staged);
  const int wave = uniform(threadIdx.x >> 6);
  const int my_items = i0 + wave < i1 ? (i1 - i0 - wave + kWaves - 1) / kWaves : 0;
  const int U = uniform(my_items * wv.NC);
  const float beta = d.beta[0];
  const char *lut = reinterpret_cast<const char *>(sh.lut);

  uint4 A[kRGW][SC], B[kRGW][SC], C[kRGW][SC];
  v4i acc[kRGW][MB][NACC];
  const int NC = wv.NC;
  // issue position (item, chunk) and process position, advanced unit by unit
  int iss_it = i0 + wave, iss_ch = 0, pro_it = i0 + wave, pro_ch = 0;
  auto issue = [&](uint4(&buf)[kRGW][SC]) {
    wv.issue(d, iss_it, iss_ch, iss_it < i1, buf);
    if (++iss_ch == NC) {
      iss_ch = 0;
      iss_it += kWaves;
    }
  };
  auto process = [&](const uint4(&buf)[kRGW][SC]) {
    if (pro_ch == 0) {
#pragma unroll
      for (int r = 0; r < kRGW; ++r)
#pragma unroll
        for (int b = 0; b < MB; ++b)
#pragma unroll
          for (int a = 0; a < NACC; ++a) acc[r][b][a] = v4i{0, 0, 0, 0};
    }
    wv.compute(d, sh.xs, lut, pro_ch, buf, acc);
    if (pro_ch == NC - 1) wv.store(d, pro_it, acc, sh.sm, sh.cm, beta);
    if (++pro_ch == NC) {
      pro_ch = 0;
      pro_it += kWaves;
    }
  };
  issue(A);
  issue(B);
  for (int u = 0; u < U;) {
    issue(C);
    process(A);
    if (++u >= U) break;
    issue(A);
    process(B);
    if (++u >= U) break;
    issue(B);
    process(C);
    ++u;
  }
}

// Block b of nb takes the global items [b T / nb, (b + 1) T / nb) of the
// plan (T items over all problems, problem p owning [item_begin, +items)),
// crossing into the next problem when its range does.
template <int FMT, int MB>
__device__ __forceinline__ void gemv_block(const GemvDesc *plan, int count, int64_t T, int b,
                                           int nb) {
  __shared__ Smem<FMT> sh;
  const int g0 = (int)(T * b / nb), g1 = (int)(T * (b + 1) / nb);
  if (g0 >= g1) return;
  int lo = 0, hi = count - 1;  // problem holding item g0
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (plan[mid].item_begin <= g0)
      lo = mid;
    else
      hi = mid - 1;
  }
  bool first = true;
  for (int p = lo, g = g0; g < g1 && p < count; ++p) {
    const GemvDesc d = plan[p];
    const int e = min(g1, d.item_begin + d.items);
    if (e <= g) continue;
    if (!first) __syncthreads();  // the previous problem's staged rows are done
    const bool staged = stages_x(FMT, d.M, d.K);
    setup<FMT>(d, sh, staged, g == d.item_begin, first);
    first = false;
    gemv_items<FMT, MB>(d, sh, staged, g - d.item_begin, e - d.item_begin);
    g = e;
  }
}

template <int FMT, int MB>
__global__ __launch_bounds__(kThreads) void gemv_single_kernel(GemvDesc d) {
  gemv_block<FMT, MB>(&d, 1, d.items, blockIdx.x, gridDim.x);
}

template <int FMT, int MB>
__global__ __launch_bounds__(kThreads) void gemv_grouped_kernel(const GemvDesc *__restrict__ plan,
                                                                int count, int total) {
  gemv_block<FMT, MB>(plan, count, total, blockIdx.x, gridDim.x);
}

template <int FMT>
hipError_t launch_single_fmt(const GemvDesc &d, int grid, hipStream_t st) {
  switch (d.mb) {
    case 1: hipLaunchKernelGGL((gemv_single_kernel<FMT, 1>), dim3(grid), dim3(kThreads), 0, st, d); break;
    case 2: hipLaunchKernelGGL((gemv_single_kernel<FMT, 2>), dim3(grid), dim3(kThreads), 0, st, d); break;
    default: hipLaunchKernelGGL((gemv_single_kernel<FMT, 4>), dim3(grid), dim3(kThreads), 0, st, d); break;
  }
  return hipGetLastError();
}

}  // namespace

// Blocks for T items: one per CU when there are enough items, else one per
// 4 items (a small group is latency-bound: more CUs, shorter waits).
int gemv_grid(int64_t total_items) {
  const int64_t by_items = (total_items + 3) / 4;
  return (int)(by_items < kGemvBlocks ? (by_items < 1 ? 1 : by_items) : kGemvBlocks);
}

void gemv_mfma_plan(GemvDesc &d) {
  d.mb = d.M <= 16 ? 1 : (d.M <= 32 ? 2 : 4);
  const int rgw = d.wfmt == UG_W_PACK5 ? (d.mb == 1 ? Cfg<UG_W_PACK5, 1>::RGW : Cfg<UG_W_PACK5, 2>::RGW)
                                       : Cfg<UG_W_I8, 1>::RGW;
  const int RG = (d.N + 15) / 16;
  d.items = (RG + rgw - 1) / rgw;
}

bool gemv_stages_x(int wfmt, int64_t M, int64_t K) {
  return K <= UG_MAX_K && M <= 64 && stages_x(wfmt, (int)M, (int)K);
}

hipError_t launch_gemv_grouped(const GemvDesc *plan_dev, int32_t count, int32_t total_items,
                               int32_t grid, int32_t fmt_mb, hipStream_t st) {
  // fmt_mb = 16 * wfmt + mb (every problem of a plan shares both)
  const int fmt = fmt_mb >> 4, mb = fmt_mb & 15;
  dim3 g(grid), b(kThreads);
#define UG_GROUPED(F, MBV) \
  hipLaunchKernelGGL((gemv_grouped_kernel<F, MBV>), g, b, 0, st, plan_dev, count, total_items)
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
  gemv_mfma_plan(d);
  d.item_begin = 0;
  const int grid = gemv_grid(d.items);
  if (wfmt == UG_W_PACK5) return launch_single_fmt<UG_W_PACK5>(d, grid, st);
  return launch_single_fmt<UG_W_I8>(d, grid, st);
}

}  // namespace ug

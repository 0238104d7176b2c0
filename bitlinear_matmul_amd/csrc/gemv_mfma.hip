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
//   as int8x4 from a 256-entry table in LDS, and t4 = floor(b / 81) - 1:
//   fine split, from the same (wide) table entry; stream split, computed
//   four bytes at a time (the quotient in 16-bit lanes as (b * 203) >> 14,
//   the -1 borrow-free in every byte), since it keeps more weights in
//   registers.  Byte i of dword j gives dword i of B operand j (j < 4); the
//   t4 bytes of dword j give dword j of B operand 4.  The activations are stored in LDS already permuted
//   the same way (each 80-position window as fragment 0..3 holding
//   x[5g .. 5g+3] of its bytes g, then fragment 4 holding the x[5g+4]), so
//   every MFMA adds products of matching K positions.
//   Stream split with one 16-row activation block (when the rows fit the
//   stream split's 80 KB staging area; given x_q, the spread rows are built
//   straight from it): spread staging instead.  Each packed byte's five
//   activations take 8 staged bytes [x0 x1 x2 x3 x4 0 0 0], and B operand
//   j is the two wide table entries of bytes 2j and 2j+1 as they come from
//   LDS (t0..t3, then t4 in all four bytes, three of which meet zero
//   activations): 8 MFMAs per 16 weight bytes instead of 5, but 16 instead
//   of ~48 vector instructions, and no register moves, per 16 bytes.
//   The table fills 64 KB: wide (t0..t3, then t4 in all four bytes), 32
//   replicas of each 8-byte entry (code e, replica r at byte e * 256 + 8 r),
//   lane l reads replica l % 32, and each half wave's 32 eight-byte reads
//   (an LDS pass) fall in 64 different banks; narrow (t0..t3), 64 replicas
//   at e * 256 + 4 r, lane l reads replica l.  Either way one v_perm forms
//   each address.
//
// Work: one block of 8 waves per CU.  Two ways to split a launch:
//   stream: a block takes a range of items (32 weight rows over the whole
//     K); each wave walks whole items unit by unit (SC steps), keeping the
//     weights of the next two units (spread staging: the next one) in
//     flight.  For groups with megabytes of weights per CU.
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
// The fine split's blocks: 8 waves.  (16 are slower: every wave's uniform
// bookkeeping runs on the CU's one scalar unit.)
constexpr int kFineThreads = 512;
constexpr int kFineWaves = kFineThreads / 64;
constexpr int kFineWaveShift = 3;  // work splits by wave: (w * P) >> 3
static_assert(kFineWaves == kGemvFineWaves && kFineWaves == 1 << kFineWaveShift, "fine waves");
constexpr int kTableBytes = 65536;  // the decode table in LDS (wide or narrow)
constexpr int kXsBytes = 65536;    // staged activations (fine split)
// The stream and chunked splits use no reduction slots, so their staging
// area is larger.
constexpr int kXsStream = 81920;
constexpr uint32_t kOOB = 0x80000000u;  // a buffer offset past every buffer used here
constexpr int kFineItems = 16;   // fine split: items (16-row groups) per block
constexpr int kFinePieces = 8;   // fine split: (item, step) pieces per wave
// The short variant of the fine split: at most 4 pieces and (decode-sized
// activations) 2 tiles per wave, so every wave issues half the loads.
constexpr int kShortPieces = 4;
constexpr int kShortTiles = 2;
constexpr int kTinyPieces = 3;  // the tiny variant: at most 3 pieces and 1 tile per wave
constexpr int kTinyTiles = 1;

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
      FINE ? 1 : (FMT == UG_W_PACK5 ? (MB == 4 ? 1 : 2) : (MB == 4 ? 2 : 4));
  // independent MFMA chains per output tile
  static constexpr int NACC = FMT == UG_W_PACK5 && MB == 4 ? 1 : 2;
  // decode table with 8-byte entries (fewer instructions per packed byte,
  // more registers): one 16-row activation block leaves room for it
  static constexpr bool WIDE = MB == 1;
};

__host__ __device__ __forceinline__ int row_bytes_of(int fmt, int K) {
  return fmt == UG_W_PACK5 ? (K + 4) / 5 : K;
}
__host__ __device__ __forceinline__ int steps_of(int fmt, int K) {
  return (row_bytes_of(fmt, K) + 63) / 64;
}
__host__ __device__ __forceinline__ int rgw_of(int fmt, int mb) {  // row groups per stream item
  return fmt == UG_W_PACK5
             ? (mb == 1 ? Cfg<UG_W_PACK5, 1, false>::RGW
                        : (mb == 2 ? Cfg<UG_W_PACK5, 2, false>::RGW : Cfg<UG_W_PACK5, 4, false>::RGW))
             : (mb == 1 ? Cfg<UG_W_I8, 1, false>::RGW
                        : (mb == 2 ? Cfg<UG_W_I8, 2, false>::RGW : Cfg<UG_W_I8, 4, false>::RGW));
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
// LDS row pitch of M staged rows of Kp bytes: 16 bytes more when they
// still fit, so that the 16 rows one fragment load reads (a multiple of 64
// bytes apart otherwise) fall in different banks.
__host__ __device__ __forceinline__ int stage_pitch(int M, int Kp, int xs) {
  return M > 1 && M * (Kp + 16) <= xs ? Kp + 16 : Kp;
}
__host__ __device__ __forceinline__ int mb_of(int M) { return M <= 16 ? 1 : (M <= 32 ? 2 : 4); }
// The K-order rows of a problem fit the stream split's staging area.
__host__ __device__ __forceinline__ bool stages_x(int fmt, int M, int K) {
  return (int64_t)M * staged_kp(fmt, mb_of(M), K) <= kXsStream;
}
// Spread staging (stream split, five trits per byte, at most 16 rows): the
// five codes of every packed weight byte take 8 staged bytes,
// [x0 x1 x2 x3 x4 0 0 0], so one wide table entry (t0..t3, then t4 in all
// four bytes) is half of a B operand as it leaves LDS.  A 16-byte weight
// piece is then 8 matrix instructions instead of 5, with no byte permutes
// between the table reads and the matrix instructions.  The spread rows
// (512 bytes per step) sit after the K-order rows, which stay intact, when
// the launch quantizes fp32 activations; given x_q, the spread rows are
// built straight from it and are the only staged rows.
constexpr int kSpreadStep = 512;  // spread bytes per row and 64-byte step
__host__ __device__ __forceinline__ int spread_base(int M, int pitch) {
  return (M * pitch + 15) & ~15;
}
__host__ __device__ __forceinline__ int spread_pitch(int M, int Kp) {
  return (Kp / 320) * kSpreadStep + (M > 1 ? 16 : 0);
}
__host__ __device__ __forceinline__ bool stages_spread(int M, int K, bool fused) {
  const int Kp = staged_kp(UG_W_PACK5, 1, K), pitch = stage_pitch(M, Kp, kXsStream);
  return M <= 16 && (int64_t)M * Kp <= kXsStream &&
         (fused ? (int64_t)spread_base(M, pitch) : 0) + (int64_t)M * spread_pitch(M, Kp) <=
             kXsStream;
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// A descriptor in scalar registers after one memory round trip: lane i
// fetches dword i, then each dword is read from its lane.  (Scalar loads of
// the fields would be issued at their first uses, several round trips apart
// where a branch depends on an earlier field.)
template <typename T>
__device__ __forceinline__ T fetch_uniform(const T *src) {
  static_assert(sizeof(T) % 4 == 0 && sizeof(T) <= 256, "whole dwords, one per lane");
  constexpr int N = sizeof(T) / 4;
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<T *>(src), (short)0, (int)sizeof(T), 0x00020000);
  const uint32_t v = __builtin_amdgcn_raw_buffer_load_b32(r, 4u * (threadIdx.x & 63), 0, 0);
  uint32_t out[N];
#pragma unroll
  for (int i = 0; i < N; ++i) out[i] = __builtin_amdgcn_readlane(v, i);
  T t;
  __builtin_memcpy(&t, out, sizeof(T));
  return t;
}

// x kept in a vector register: arithmetic on the result runs on the wave's
// SIMD instead of the CU's one scalar unit, which every wave of the block
// shares (uniform bookkeeping repeated by 8 waves queues up there).
__device__ __forceinline__ int in_vgpr(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

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
// The weights: each byte is read once per launch, so the loads carry the
// non-temporal hint (aux bit 1): the L2 keeps them only briefly.
__device__ __forceinline__ uint4 buffer_load16_stream(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
}
__device__ __forceinline__ uint32_t buffer_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ float4 buffer_load16f(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Table entry of code e: t0..t3 as int8 bytes, and t4 in every byte of
// the second dword.  Codes 243..255 give zeros (matmul results for invalid
// codes are unspecified).
constexpr uint32_t lut_t0123(int e) {
  uint32_t v = 0;
  if (e <= 242) {
    int c = e;
    for (int j = 0; j < 4; ++j) {
      v |= ((uint32_t)((c % 3) - 1) & 0xffu) << (8 * j);
      c /= 3;
    }
  }
  return v;
}
constexpr uint32_t lut_t4(int e) {
  return e <= 242 ? ((uint32_t)(e / 81 - 1) & 0xffu) * 0x01010101u : 0u;
}
// All 256 entries, computed by the compiler: a block fills its LDS replicas
// with loads from this table instead of per-lane arithmetic.
struct LutTable {
  uint2 v[256];
  constexpr LutTable() : v() {
    for (int e = 0; e < 256; ++e) {
      v[e].x = lut_t0123(e);
      v[e].y = lut_t4(e);
    }
  }
};
__constant__ const LutTable kLut{};

__device__ __forceinline__ uint32_t pack4(int a, int b, int c, int e) {
  return (uint32_t)(a & 0xff) | ((uint32_t)(b & 0xff) << 8) | ((uint32_t)(c & 0xff) << 16) |
         ((uint32_t)(e & 0xff) << 24);
}

// Four packed bytes -> t[0..3] = t0..t3 of bytes 0..3, t4 = their four top
// trits, from the wide table.  lr8 = 8 * (lane % 32).
__device__ __forceinline__ void decode4_wide(uint32_t w, const char *lut, uint32_t lr8, uint32_t *t,
                                             uint32_t &t4) {
  // byte address b * 256 + 8 * (lane % 32) (selector bytes: 0 = lr8 byte 0,
  // 4+i = byte i of w, 12 = zero)
  const uint2 e0 = *reinterpret_cast<const uint2 *>(lut + __builtin_amdgcn_perm(w, lr8, 0x0c0c0400u));
  const uint2 e1 = *reinterpret_cast<const uint2 *>(lut + __builtin_amdgcn_perm(w, lr8, 0x0c0c0500u));
  const uint2 e2 = *reinterpret_cast<const uint2 *>(lut + __builtin_amdgcn_perm(w, lr8, 0x0c0c0600u));
  const uint2 e3 = *reinterpret_cast<const uint2 *>(lut + __builtin_amdgcn_perm(w, lr8, 0x0c0c0700u));
  t[0] = e0.x;
  t[1] = e1.x;
  t[2] = e2.x;
  t[3] = e3.x;
  // byte i from entry i's t4 dword: bytes 0, 1 of (e0, e1), bytes 2, 3 of (e2, e3)
  t4 = __builtin_amdgcn_perm(e1.y, e0.y, 0x0c0c0500u) | __builtin_amdgcn_perm(e3.y, e2.y, 0x07020c0cu);
}

// The same from the narrow table, t4 computed.  lr4 = 4 * lane.
__device__ __forceinline__ void decode4_narrow(uint32_t w, const char *lut, uint32_t lr4,
                                               uint32_t *t, uint32_t &t4) {
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
  const uint32_t d4 = __builtin_bit_cast(uint32_t, e) | (__builtin_bit_cast(uint32_t, o) << 8);
  // d4 - 1 in every byte: each byte of d4 ^ 0x80.. is 0x80 + d4 >= 1, so
  // subtracting 1 per byte borrows across no byte boundary
  t4 = ((d4 ^ 0x80808080u) - 0x01010101u) ^ 0x80808080u;
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

// STREAM: the stream and chunked splits' layout (no reduction slots, a
// larger staging area).
template <int FMT, int NW = kWaves, bool STREAM = false>
struct Smem {
  static constexpr int kXs = STREAM ? kXsStream : kXsBytes;  // staging bytes
  static constexpr int kNW = NW;
  uint4 lut[FMT == UG_W_PACK5 ? kTableBytes / 16 : 1];    // the decode table
  alignas(16) int8_t xs[kXs + 80];                       // staged rows, then 80 zero bytes
  alignas(16) int slots[STREAM ? 4 : kFineItems * 256];  // fine split: [item][m][n] int32 sums
  float part[NW][64];                                    // per-wave row maxima (fused quantization)
  float sm[64];                                          // row scales s
};
template <int FMT>
using SmemS = Smem<FMT, kWaves, true>;
static_assert(sizeof(SmemS<UG_W_PACK5>) <= 163840, "stream layout fits LDS");

// The decode table in 16-byte chunks, chunk j of code e at e * 16 + j
// (256 bytes per code): wide, entries for lanes 2j and 2j + 1 (mod 32);
// narrow, for lanes 4j .. 4j + 3.  Thread t writes chunks t + 512 i, i < 8
// (consecutive lanes, consecutive chunks: no bank conflicts), i.e. code
// 4 (w + 8 i) + r for wave w and 16-lane row r.  One table load per thread:
// lane p of row r loads the code its row writes at step p % 8, and at step
// i every lane of the row takes lane i's value (DPP row broadcast).
static_assert(kThreads == 512 && kFineThreads == 512, "8 waves write the table");
__device__ __forceinline__ uint2 table_load() {
  const int t = threadIdx.x;
  return kLut.v[4 * ((t >> 6) + 8 * (t & 7)) + ((t >> 4) & 3)];
}
template <int I>
__device__ __forceinline__ uint32_t row_broadcast(uint32_t v) {  // lane I of each 16-lane row
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x150 + I, 0xf, 0xf, false);
}
template <bool WIDE, int I, class SM>
__device__ __forceinline__ void table_store_step(SM &sh, uint2 v) {
  const uint32_t lo = row_broadcast<I>(v.x), hi = row_broadcast<I>(v.y);
  sh.lut[threadIdx.x + 512 * I] = WIDE ? make_uint4(lo, hi, lo, hi) : make_uint4(lo, lo, lo, lo);
}
// (with every lane active: the broadcasts read other lanes)
template <bool WIDE, class SM>
__device__ __forceinline__ void table_store(SM &sh, uint2 v) {
  table_store_step<WIDE, 0>(sh, v);
  table_store_step<WIDE, 1>(sh, v);
  table_store_step<WIDE, 2>(sh, v);
  table_store_step<WIDE, 3>(sh, v);
  table_store_step<WIDE, 4>(sh, v);
  table_store_step<WIDE, 5>(sh, v);
  table_store_step<WIDE, 6>(sh, v);
  table_store_step<WIDE, 7>(sh, v);
}

// s = fl(fl(max|x| / 127) + eps) of row m from the per-wave maxima.
template <class SM>
__device__ __forceinline__ float row_scale(const SM &sh, int m, float eps) {
  float a = sh.part[0][m];
#pragma unroll
  for (int w = 1; w < SM::kNW; ++w) a = fmaxf(a, sh.part[w][m]);
  const float a127 = a / 127.0f;
  return a127 + eps;
}

// Block set-up for problem d, in two halves.  pre_issue() issues the loads
// the set-up needs (decode table entry, first batch of x_q dwords, row
// scale, beta); the caller then issues its weight loads, so that waiting
// for the set-up's data never waits for the weights (loads complete in
// issue order).  setup_finish() builds the decode table (first problem of
// the block), the row scales (fused quantization, else the given s), the
// activation rows staged in LDS (Kp bytes per row, zeros past K; five trits
// per byte: every 80-position window permuted as the decoded weights are)
// and zeroed reduction slots, and ends with a barrier.
//
// Fused quantization reads x in tiles t = (row m, 256 positions c): lane l
// takes the float4 at 256 c + 4 l, a wave keeps 8 tiles in flight.
template <int NQ>
struct PreLoads {
  static_assert(NQ == 0 || NQ == 8, "x_q dwords come in batches of 8");
  uint2 lut;                 // this thread's decode table entry (table_load)
  uint32_t q[NQ ? NQ : 1];   // x_q given and staged: the first NQ dwords of this thread
  float s;                   // x_q given: the scale of row tid (tid < M)
  float beta;
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

// Every load but the table's is issued without a branch (one not needed
// reads past its buffer, i.e. nothing).
template <int FMT, int NQ>
__device__ __forceinline__ void pre_issue(const GemvDesc &d, bool staged, int Kp, bool table,
                                          PreLoads<NQ> &pl) {
  const int tid = threadIdx.x;
  pl.lut = uint2{0, 0};
  if (FMT == UG_W_PACK5 && table) pl.lut = table_load();
  if (NQ) {
    const int Kp4 = Kp >> 2, n4 = !d.x && staged ? d.M * Kp4 : 0;
    const __amdgpu_buffer_rsrc_t qr =
        buffer_rsrc(d.xq, n4 ? (uint32_t)((int64_t)d.M * d.ldxq) : 0u);
#pragma unroll
    for (int i = 0; i < NQ; ++i) pl.q[i] = load_xq4(d, qr, tid + i * kThreads, Kp4, n4);
  }
  const __amdgpu_buffer_rsrc_t sr = buffer_rsrc(d.s, d.x ? 0u : 4u * (uint32_t)d.M);
  pl.s = __builtin_bit_cast(float, buffer_load4(sr, tid < d.M ? 4u * tid : kOOB));
  pl.beta = __builtin_bit_cast(float, buffer_load4(buffer_rsrc(d.beta, 4), 0));
}

// Pass 1 on 8 tiles t0 + i * 8: per-wave row maxima.
template <int FMT, class SM>
__device__ __forceinline__ void absmax_tiles(const GemvDesc &d, SM &sh, const float4 (&v)[8],
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
template <int FMT, class SM>
__device__ __forceinline__ void quant_tiles(const GemvDesc &d, SM &sh, const float4 (&v)[8],
                                            int t0, int T4, int nt, int pitch) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int t = t0 + i * kWaves;
    if (t < nt) {
      const int m = t / T4, k = (t - m * T4) * 256 + 4 * lane;
      const float s = row_scale(sh, m, d.eps);
      if (k < d.K)
        *reinterpret_cast<uint32_t *>(sh.xs + m * pitch + k) =
            pack4(q8(v[i].x, s), k + 1 < d.K ? q8(v[i].y, s) : 0, k + 2 < d.K ? q8(v[i].z, s) : 0,
                  k + 3 < d.K ? q8(v[i].w, s) : 0);
    }
  }
}

// 8 dwords of x_q rows into the staging rows (zeros past K).
template <int FMT, class SM>
__device__ __forceinline__ void copy_xq4(const GemvDesc &d, SM &sh, const uint32_t (&v)[8],
                                         int i0, int Kp4, int n4, int pitch) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int idx = i0 + i * kThreads, m = idx / Kp4, k = 4 * (idx - m * Kp4);
    if (idx < n4) {
      uint32_t w = v[i];
      if (k + 4 > d.K) w &= k >= d.K ? 0u : (0xffffffffu >> (8 * (k + 4 - d.K)));
      reinterpret_cast<uint32_t *>(sh.xs + m * pitch)[k >> 2] = w;
    }
  }
}

// One 80-position window of codes (20 dwords, K order) -> its 128 spread
// bytes: weight byte b's codes 5b .. 5b+3 in dword 2b, code 5b+4 in the low
// byte of dword 2b+1.
__device__ __forceinline__ void spread_window(const uint32_t (&X)[20], uint4 *dst) {
  uint32_t F[32];
#pragma unroll
  for (int b = 0; b < 16; ++b) {
    const int o = 5 * b, o4 = o + 4;
    F[2 * b] = (o & 3) ? __builtin_amdgcn_alignbyte(X[(o >> 2) + 1], X[o >> 2], o & 3) : X[o >> 2];
    F[2 * b + 1] = (X[o4 >> 2] >> (8 * (o4 & 3))) & 0xffu;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) dst[i] = make_uint4(F[4 * i], F[4 * i + 1], F[4 * i + 2], F[4 * i + 3]);
}

// NQ: the first batch of x_q dwords is in pl (0: every batch is loaded
// here, which keeps the registers free for a caller short of them).
template <int FMT, int NQ, bool WIDE, bool SPREAD = false, class SM>
__device__ __forceinline__ void setup_finish(const GemvDesc &d, SM &sh, bool staged, int Kp,
                                             int pitch, bool table, bool zero_slots,
                                             const PreLoads<NQ> &pl, int sbase = 0,
                                             int spitch = 0) {
  const int tid = threadIdx.x, wave = uniform(tid >> 6), lane = tid & 63;
  if (FMT == UG_W_PACK5 && table) table_store<WIDE>(sh, pl.lut);
  if (tid < 20) reinterpret_cast<uint32_t *>(sh.xs + SM::kXs)[tid] = 0;
  if (zero_slots)
    for (int i = tid; i < kFineItems * 64; i += kThreads)
      reinterpret_cast<uint4 *>(sh.slots)[i] = make_uint4(0, 0, 0, 0);
  const int Kp4 = Kp >> 2;  // dwords per staged row
  if (d.x) {
    const int T4 = (d.K + 255) >> 8, nt = d.M * T4;
    const __amdgpu_buffer_rsrc_t xr = buffer_rsrc(d.x, (uint32_t)((int64_t)d.M * d.ldx * 4));
    sh.part[wave][lane] = 0.0f;
    for (int t0 = wave; t0 < nt; t0 += 8 * kWaves) {
      float4 v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = load_tile(d, xr, t0 + i * kWaves, T4, nt);
      absmax_tiles<FMT>(d, sh, v, t0, T4, nt);
    }
    __syncthreads();
    if (tid < d.M) sh.sm[tid] = row_scale(sh, tid, d.eps);
    for (int t0 = wave; t0 < nt; t0 += 8 * kWaves) {
      float4 v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = load_tile(d, xr, t0 + i * kWaves, T4, nt);
      quant_tiles<FMT>(d, sh, v, t0, T4, nt, pitch);
    }
    // zeros from the first whole dword past K to the end of the staged row
    const int kz = (d.K + 3) >> 2, nz = Kp4 - kz;
    for (int i = tid; i < d.M * nz; i += kThreads) {
      const int m = i / nz;
      reinterpret_cast<uint32_t *>(sh.xs + m * pitch)[kz + (i - m * nz)] = 0u;
    }
  } else if (SPREAD) {
    // x_q given: every 80-position window straight from memory into its
    // 128 spread bytes (16-byte loads: a load at k < K is inside the row,
    // ldxq >= round_up(K, 16); bytes past K zeroed)
    if (tid < d.M) sh.sm[tid] = pl.s;
    const __amdgpu_buffer_rsrc_t xr = buffer_rsrc(d.xq, (uint32_t)((int64_t)d.M * d.ldxq));
    const int wpr = Kp / 80, nwin = d.M * wpr;
    for (int w0 = tid; w0 < nwin; w0 += kThreads) {
      const int m = w0 / wpr, w = w0 - m * wpr, k0 = 80 * w;
      uint32_t X[20];
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        const int k = k0 + 16 * i;
        const uint4 v = buffer_load16(xr, k < d.K ? (uint32_t)(m * (int)d.ldxq + k) : kOOB);
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int kb = d.K - k - 4 * e;  // bytes of this dword inside the row
          X[4 * i + e] =
              w4[e] & (kb >= 4 ? 0xffffffffu : (kb <= 0 ? 0u : (0xffffffffu >> (8 * (4 - kb)))));
        }
      }
      spread_window(X, reinterpret_cast<uint4 *>(sh.xs + sbase + m * spitch + w * 128));
    }
  } else {
    if (tid < d.M) sh.sm[tid] = pl.s;
    if (staged) {
      const int n4 = d.M * Kp4;
      const __amdgpu_buffer_rsrc_t xr = buffer_rsrc(d.xq, (uint32_t)((int64_t)d.M * d.ldxq));
      if constexpr (NQ > 0) copy_xq4<FMT>(d, sh, pl.q, tid, Kp4, n4, pitch);
      for (int i0 = NQ ? tid + NQ * kThreads : tid; i0 < n4; i0 += 8 * kThreads) {
        uint32_t v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = load_xq4(d, xr, i0 + i * kThreads, Kp4, n4);
        copy_xq4<FMT>(d, sh, v, i0, Kp4, n4, pitch);
      }
    }
  }
  __syncthreads();
  // every 80-position window, one per thread: permuted in place, or spread
  // into its 128-byte window of the spread rows (x_q given and spread: done)
  if (FMT == UG_W_PACK5 && staged && !(SPREAD && !d.x)) {
    const int wpr = Kp / 80, nwin = d.M * wpr;
    for (int w0 = tid; w0 < nwin; w0 += kThreads) {
      const int m = w0 / wpr, w = w0 - m * wpr;
      uint4 *win = reinterpret_cast<uint4 *>(sh.xs + m * pitch + w * 80);
      uint32_t X[20], F[20];
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        const uint4 q = win[i];
        X[4 * i] = q.x; X[4 * i + 1] = q.y; X[4 * i + 2] = q.z; X[4 * i + 3] = q.w;
      }
      if constexpr (SPREAD) {
        spread_window(X, reinterpret_cast<uint4 *>(sh.xs + sbase + m * spitch + w * 128));
      } else {
        permute80(X, F);
#pragma unroll
        for (int i = 0; i < 5; ++i) win[i] = make_uint4(F[4 * i], F[4 * i + 1], F[4 * i + 2], F[4 * i + 3]);
      }
    }
    __syncthreads();
  }
}

// The quantized activations and scales as outputs (fused quantization, the
// problem's first block): undo the staging permutation per K position.
template <int FMT, bool SPREAD = false, class SM>
__device__ __forceinline__ void write_act_outputs(const GemvDesc &d, const SM &sh, int pitch) {
  const int tid = threadIdx.x;
  if (d.s)
    for (int m = tid; m < d.M; m += kThreads) gp(d.s)[m] = sh.sm[m];
  if (d.xq) {
    int8_t *xq = const_cast<int8_t *>(d.xq);
    for (int idx = tid; idx < d.M * d.K; idx += kThreads) {
      const int m = idx / d.K, k = idx - m * d.K;
      int off = k;
      if (FMT == UG_W_PACK5 && !SPREAD) {  // (spread staging keeps the K-order rows)
        const int w = k / 80, r = k - 80 * w, g = r / 5, t = r - 5 * g;
        // t < 4: fragment g/4, dword g%4, byte t; t == 4: fragment 4, dword g/4, byte g%4
        off = 80 * w + (t < 4 ? 16 * (g >> 2) + 4 * (g & 3) + t : 64 + 4 * (g >> 2) + (g & 3));
      }
      gp(xq)[(int64_t)m * d.ldxq + k] = sh.xs[m * pitch + off];
    }
  }
}

// SPREAD: the spread staging (five trits per byte, MB == 1, stream split).
template <int FMT, int MB, bool FINE, bool SPREAD = false>
struct Wave {
  static_assert(!SPREAD || (FMT == UG_W_PACK5 && MB == 1 && !FINE), "spread staging");
  static constexpr int F1 = SPREAD ? 8 : Fmt<FMT>::kFrag;
  static constexpr int SC = Cfg<FMT, MB, FINE>::SC;
  static constexpr int NACC = Cfg<FMT, MB, FINE>::NACC;
  static constexpr int kRGW = Cfg<FMT, MB, FINE>::RGW;

  int S, NC;
  bool staged;
  int xbase[MB];  // staged: LDS offset of this lane's activation row (step 0)
  __amdgpu_buffer_rsrc_t wr, xr;

  // (spread staging: row m of the spread rows at sbase + m * spitch)
  __device__ __forceinline__ void init(const GemvDesc &d, bool stg, int pitch, int sbase = 0,
                                       int spitch = 0) {
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
      xbase[b] = SPREAD ? sbase + m * spitch + q * 128 : m * pitch + q * Fmt<FMT>::kLaneK;
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
      // (no non-temporal hint: a row that is not a multiple of 128 bytes
      // long shares cache lines with its neighbours, which read them later)
      for (int s = 0; s < SC; ++s) wb[r][s] = buffer_load16(wr, voff + (uint32_t)(64 * (ch * SC + s)));
    }
  }

  // Activation fragments of step st for M-block b.
  __device__ __forceinline__ void xfrags(const GemvDesc &d, const int8_t *xs, int st, int b,
                                         v4i (&xf)[F1]) {
    if (SPREAD || FINE || staged) {
      const int off = xbase[b] + st * (SPREAD ? kSpreadStep : Fmt<FMT>::kStepK);
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
    if constexpr (SPREAD) {
      // piece p: byte i of the 16 weight bytes -> its table entry; matrix
      // instruction j takes the entries of bytes 2j and 2j+1 as its B
      // operand and spread fragment j (their codes) as its A operand
      constexpr int NP = SC * kRGW;
      uint2 E[2][16];
      auto dec = [&](int p, uint2(&e)[16]) {
        const uint4 &w = wb[p % kRGW][p / kRGW];
        const uint32_t lr8 = 8u * (threadIdx.x & 31);
        const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 16; ++i)
          e[i] = *reinterpret_cast<const uint2 *>(
              lut + __builtin_amdgcn_perm(wd[i >> 2], lr8, 0x0c0c0400u + ((uint32_t)(i & 3) << 8)));
      };
      v4i xf[MB][F1];
      dec(0, E[0]);
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int s = p / kRGW, r = p % kRGW;
        if (r == 0) xfrags(d, xs, ch * SC + s, 0, xf[0]);
        if (p + 1 < NP) dec(p + 1, E[(p + 1) & 1]);
        const uint2(&e)[16] = E[p & 1];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const v4i B = {(int)e[2 * j].x, (int)e[2 * j].y, (int)e[2 * j + 1].x, (int)e[2 * j + 1].y};
          acc[r][0][j % NACC] =
              __builtin_amdgcn_mfma_i32_16x16x64_i8(xf[0][j], B, acc[r][0][j % NACC], 0, 0, 0);
        }
      }
    } else if (FMT == UG_W_PACK5) {
      constexpr int NP = SC * kRGW;
      uint32_t T[2][20];
      auto dec = [&](int p, uint32_t(&t)[20]) {
        const uint4 &w = wb[p % kRGW][p / kRGW];
        if (Cfg<FMT, MB, FINE>::WIDE) {
          const uint32_t lr8 = 8u * (threadIdx.x & 31);
          decode4_wide(w.x, lut, lr8, t, t[16]);
          decode4_wide(w.y, lut, lr8, t + 4, t[17]);
          decode4_wide(w.z, lut, lr8, t + 8, t[18]);
          decode4_wide(w.w, lut, lr8, t + 12, t[19]);
        } else {
          const uint32_t lr4 = 4u * (threadIdx.x & 63);
          decode4_narrow(w.x, lut, lr4, t, t[16]);
          decode4_narrow(w.y, lut, lr4, t + 4, t[17]);
          decode4_narrow(w.z, lut, lr4, t + 8, t[18]);
          decode4_narrow(w.w, lut, lr4, t + 12, t[19]);
        }
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
                                        const float *sm, float beta) {
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
            const int val = v[r];
            if (d.acc) gp(d.acc)[(int64_t)m * d.ldacc + n] = val;
            if (d.y) {
              const float scale = sm[m] * beta;
              const float v = (float)val * scale;
              gp(d.y)[(int64_t)m * d.ldy + n] = d.bias ? v + gp(d.bias)[n] : v;
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
// each NC units, with the weights of the next two units (spread staging:
// the next unit) in flight.  start() issues those loads, so they travel
// while the block sets up.
template <int FMT, int MB, bool SPREAD = false>
struct ItemLoop {
  using W = Wave<FMT, MB, false, SPREAD>;
  static constexpr int SC = W::SC, NACC = W::NACC, kRGW = W::kRGW;
  // Spread staging: one unit of weights in flight while the wave decodes
  // the current one (its decode is short; 32 KB in flight per compute unit
  // streams faster on this GPU than 64 KB, as the read probe also shows);
  // otherwise two.
  static constexpr bool kShallow = SPREAD;
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

  __device__ __forceinline__ void process(const GemvDesc &d, const SmemS<FMT> &sh,
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
    if (pro_ch == wv.NC - 1) wv.store(d, pro_it, acc, sh.sm, beta);
    if (++pro_ch == wv.NC) {
      pro_ch = 0;
      pro_it += kWaves;
    }
  }

  __device__ __forceinline__ void start(const GemvDesc &d, bool staged, int pitch, int i0, int i1_,
                                        int sbase = 0, int spitch = 0) {
    wv.init(d, staged, pitch, sbase, spitch);
    const int wave = uniform(threadIdx.x >> 6);
    const int my_items = i0 + wave < i1_ ? (i1_ - i0 - wave + kWaves - 1) / kWaves : 0;
    U = uniform(my_items * wv.NC);
    i1 = i1_;
    iss_it = pro_it = i0 + wave;
    iss_ch = pro_ch = 0;
    issue(d, A);
    if (!kShallow) issue(d, B);
  }

  // Needs the block's set-up (table, staged rows) to be complete.  (Issuing
  // the third unit before the set-up too measured slower, and so did a
  // fourth buffer keeping three units in flight: 37.3 against 34.0 us for
  // 37 problems of 2560 -> 6912 at M = 1.)
  __device__ __forceinline__ void run(const GemvDesc &d, const SmemS<FMT> &sh) {
    if constexpr (kShallow) {
      for (int u = 0; u < U;) {
        issue(d, B);
        process(d, sh, A);
        if (++u >= U) break;
        issue(d, A);
        process(d, sh, B);
        ++u;
      }
      return;
    }
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

// ---------------------------------------------------------------------------
// Chunked stream: for launches with problems whose activation rows do not
// fit the staging area (x_q input; M * Kp > 80 KB), where the stream split
// would read every activation fragment from memory once per piece.  Waves
// take a problem's items in rounds (wave w: item i0 + w + 8 r); each round
// walks K in chunks of CH steps.  The block stages a chunk's activations
// (all rows, permuted like the staged rows) once in LDS for its 8 waves,
// loading the next chunk's activations and weights while it computes the
// current one.  Its own kernels, so its registers are its own.
template <int FMT, int MB>
struct Chunk {
  static constexpr int RG = Cfg<FMT, MB, false>::RGW;  // row groups per item
  static constexpr int CH = FMT == UG_W_PACK5 && MB == 4 ? 2 : 4;  // steps per chunk
  static constexpr int ROWS = 16 * MB;
  static constexpr int SB = FMT == UG_W_PACK5 ? 320 : 64;  // staged bytes per row and step
  static constexpr int CB = CH * SB;                        // staged bytes per row and chunk
  // row pitch in LDS: 16 bytes more, so the 16 rows read by one fragment
  // load (a multiple of 128 bytes apart otherwise) fall in different banks
  static constexpr int CBP = CB + 16;
  static constexpr int UB = FMT == UG_W_PACK5 ? 80 : 16;    // staging unit (bytes)
  static constexpr int UPR = CB / UB;                        // units per row and chunk
  static constexpr int NU = (ROWS * UPR + kThreads - 1) / kThreads;  // units per thread
  static constexpr int UV = UB / 16;                         // 16-byte loads per unit
  static_assert(ROWS * CBP <= kXsBytes, "a chunk fits the staging area");
};

// Loads (issue) this thread's staging units of chunk c: unit u = tid + 512 i
// is row u / UPR, unit u % UPR of the chunk (K positions from c * CH * step).
template <int FMT, int MB>
__device__ __forceinline__ void chunk_load(const GemvDesc &d, __amdgpu_buffer_rsrc_t xr, int c,
                                           uint4 (&v)[Chunk<FMT, MB>::NU][Chunk<FMT, MB>::UV]) {
  using C = Chunk<FMT, MB>;
#pragma unroll
  for (int i = 0; i < C::NU; ++i) {
    const int u = threadIdx.x + kThreads * i, m = u / C::UPR;
    const int k = c * C::CB + (u - m * C::UPR) * C::UB;  // K position (int8 byte) of the unit
#pragma unroll
    for (int j = 0; j < C::UV; ++j) {
      const int kj = k + 16 * j;
      // a 16-byte load at kj < K is inside the row (ldxq >= round_up(K, 16))
      v[i][j] = buffer_load16(xr, m < d.M && kj < d.K ? (uint32_t)(m * (int)d.ldxq + kj) : kOOB);
    }
  }
}

// Stores the loaded units into the staged chunk: bytes past K zeroed,
// five trits per byte: every 80-position window permuted as the weights
// decode.
template <int FMT, int MB>
__device__ __forceinline__ void chunk_store(const GemvDesc &d, int8_t *xs, int c,
                                            const uint4 (&v)[Chunk<FMT, MB>::NU][Chunk<FMT, MB>::UV]) {
  using C = Chunk<FMT, MB>;
#pragma unroll
  for (int i = 0; i < C::NU; ++i) {
    const int u = threadIdx.x + kThreads * i, m = u / C::UPR, w = u - m * C::UPR;
    if (m < d.M) {
      const int k = c * C::CB + w * C::UB;
      uint32_t X[4 * C::UV];
#pragma unroll
      for (int j = 0; j < C::UV; ++j) {
        const uint32_t w4[4] = {v[i][j].x, v[i][j].y, v[i][j].z, v[i][j].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int kb = d.K - k - 16 * j - 4 * e;  // bytes of this dword inside the row
          X[4 * j + e] = w4[e] & (kb >= 4 ? 0xffffffffu : (kb <= 0 ? 0u : (0xffffffffu >> (8 * (4 - kb)))));
        }
      }
      uint4 *dst = reinterpret_cast<uint4 *>(xs + m * C::CBP + w * C::UB);
      if (FMT == UG_W_PACK5) {
        uint32_t F[20];
        permute80(reinterpret_cast<const uint32_t(&)[20]>(X), F);
#pragma unroll
        for (int j = 0; j < 5; ++j) dst[j] = make_uint4(F[4 * j], F[4 * j + 1], F[4 * j + 2], F[4 * j + 3]);
      } else {
        dst[0] = make_uint4(X[0], X[1], X[2], X[3]);
      }
    }
  }
}

template <int FMT, int MB>
__device__ __forceinline__ void chunked_items(const GemvDesc &d, SmemS<FMT> &sh, int i0, int i1) {
  using C = Chunk<FMT, MB>;
  constexpr int RG = C::RG, CH = C::CH, F1 = Fmt<FMT>::kFrag;
  const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63, q = lane >> 4;
  const int S = steps_of(FMT, d.K), NCH = (S + CH - 1) / CH;
  const int rounds = (i1 - i0 + kWaves - 1) / kWaves, T = rounds * NCH;
  const __amdgpu_buffer_rsrc_t xr = buffer_rsrc(d.xq, (uint32_t)((int64_t)d.M * d.ldxq));
  const __amdgpu_buffer_rsrc_t wr = buffer_rsrc(d.w, (uint32_t)((int64_t)d.N * d.ldw));
  const float beta = gp(d.beta)[0];
  const char *lut = reinterpret_cast<const char *>(sh.lut);
  const uint32_t lr4 = 4u * (uint32_t)lane;
  // this lane's staged row (rows past M read row M-1: MFMA row m depends
  // only on input row m, and rows past M are never stored)
  int xrow[MB];
#pragma unroll
  for (int b = 0; b < MB; ++b) xrow[b] = min(16 * b + (lane & 15), d.M - 1) * C::CBP;

  // weights of (round r, chunk c): row group g of the wave's item, the
  // chunk's steps; steps past S and items past i1 read nothing
  auto wload = [&](int r, int c, uint4 (&w)[RG][CH]) __attribute__((always_inline)) {
    const int item = i0 + wave + kWaves * r;
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      const uint32_t n = (uint32_t)((item * RG + g) * 16 + (lane & 15));
      const uint32_t base = n * (uint32_t)d.ldw + 16u * q;
#pragma unroll
      for (int s = 0; s < CH; ++s) {
        const int st = c * CH + s;
        w[g][s] = buffer_load16(wr, item < i1 && st < S ? base + 64u * st : kOOB);
      }
    }
  };

  uint4 xv[C::NU][C::UV];
  uint4 wcur[RG][CH], wnext[RG][CH];
  chunk_load<FMT, MB>(d, xr, 0, xv);
  wload(0, 0, wcur);
  v4i acc[RG][MB];
#pragma unroll
  for (int g = 0; g < RG; ++g)
#pragma unroll
    for (int b = 0; b < MB; ++b) acc[g][b] = v4i{0, 0, 0, 0};
  int r = 0, c = 0;
  for (int t = 0; t < T; ++t) {
    __syncthreads();  // the previous chunk's reads of the staging area are done
    chunk_store<FMT, MB>(d, sh.xs, c, xv);
    const int c1 = c + 1 == NCH ? 0 : c + 1, r1 = c + 1 == NCH ? r + 1 : r;
    if (t + 1 < T) {  // the next chunk's activations and weights travel meanwhile
      chunk_load<FMT, MB>(d, xr, c1, xv);
      wload(r1, c1, wnext);
    }
    __syncthreads();  // the staged chunk is complete
    if (i0 + wave + kWaves * r < i1) {
#pragma unroll
      for (int s = 0; s < CH; ++s) {
        if (c * CH + s < S) {
          uint32_t tdec[RG][4 * F1];
#pragma unroll
          for (int g = 0; g < RG; ++g) {
            if (FMT == UG_W_PACK5) {
              decode4_narrow(wcur[g][s].x, lut, lr4, tdec[g], tdec[g][16]);
              decode4_narrow(wcur[g][s].y, lut, lr4, tdec[g] + 4, tdec[g][17]);
              decode4_narrow(wcur[g][s].z, lut, lr4, tdec[g] + 8, tdec[g][18]);
              decode4_narrow(wcur[g][s].w, lut, lr4, tdec[g] + 12, tdec[g][19]);
            } else {
              tdec[g][0] = wcur[g][s].x;
              tdec[g][1] = wcur[g][s].y;
              tdec[g][2] = wcur[g][s].z;
              tdec[g][3] = wcur[g][s].w;
            }
          }
#pragma unroll
          for (int j = 0; j < F1; ++j) {
            v4i xf[MB];
#pragma unroll
            for (int b = 0; b < MB; ++b)
              xf[b] = *reinterpret_cast<const v4i *>(sh.xs + xrow[b] + s * C::SB + q * Fmt<FMT>::kLaneK + 16 * j);
#pragma unroll
            for (int g = 0; g < RG; ++g) {
              const v4i B = {(int)tdec[g][4 * j], (int)tdec[g][4 * j + 1], (int)tdec[g][4 * j + 2],
                             (int)tdec[g][4 * j + 3]};
#pragma unroll
              for (int b = 0; b < MB; ++b)
                acc[g][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xf[b], B, acc[g][b], 0, 0, 0);
            }
          }
        }
      }
      if (c + 1 == NCH) {  // the item is complete: lane (n, q) holds rows 16 b + 4 q + e of column n
        const int item = i0 + wave + kWaves * r;
#pragma unroll
        for (int g = 0; g < RG; ++g) {
          const int n = (item * RG + g) * 16 + (lane & 15);
#pragma unroll
          for (int b = 0; b < MB; ++b) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int m = 16 * b + 4 * q + e;
              if (n < d.N && m < d.M) {
                const int val = acc[g][b][e];
                if (d.acc) gp(d.acc)[(int64_t)m * d.ldacc + n] = val;
                if (d.y) {
                  const float v = (float)val * (sh.sm[m] * beta);
                  gp(d.y)[(int64_t)m * d.ldy + n] = d.bias ? v + gp(d.bias)[n] : v;
                }
              }
            }
            acc[g][b] = v4i{0, 0, 0, 0};
          }
        }
      }
    }
#pragma unroll
    for (int g = 0; g < RG; ++g)
#pragma unroll
      for (int s = 0; s < CH; ++s) wcur[g][s] = wnext[g][s];
    r = r1;
    c = c1;
  }
}

// The block's global items [g0, g1) of the plan, problem by problem.
template <int FMT, int MB>
__device__ __forceinline__ void chunked_block(const GemvDesc *plan, int count, const GemvDesc &d0,
                                              int p0, int g0, int g1) {
  __shared__ SmemS<FMT> sh;
  bool first = true;
  GemvDesc d = d0;
  for (int g = g0, p = p0; g < g1 && p < count;) {
    const int e = min(g1, d.item_begin + d.items);
    if (e > g) {
      PreLoads<0> pl;
      pre_issue<FMT>(d, false, 0, first, pl);
      if (!first) __syncthreads();  // the previous problem is done with the staging area
      setup_finish<FMT, 0, false>(d, sh, false, 0, 0, first, false, pl);  // table, scales
      first = false;
      chunked_items<FMT, MB>(d, sh, g - d.item_begin, e - d.item_begin);
      g = e;
    }
    if (++p < count && g < g1) d = fetch_uniform(plan + p);
  }
}

template <int FMT, int MB>
__global__ __launch_bounds__(kThreads) void gemv_chunked_single(GemvDesc d) {
  const int64_t T = d.items;
  const int g0 = (int)(T * blockIdx.x / gridDim.x), g1 = (int)(T * (blockIdx.x + 1) / gridDim.x);
  if (g0 < g1) chunked_block<FMT, MB>(&d, 1, d, 0, g0, g1);
}

template <int FMT, int MB>
__global__ __launch_bounds__(kThreads) void gemv_chunked_grouped(const GemvDesc *__restrict__ plan,
                                                                 const GemvBlock *__restrict__ blocks,
                                                                 int count) {
  const GemvBlock bl = fetch_uniform(blocks + blockIdx.x);
  if (bl.i0 < bl.i1) chunked_block<FMT, MB>(plan, count, bl.d, bl.p, bl.i0, bl.i1);
}

// Items [g, e) of problem d (global item numbers).  first: the block's first
// problem (it builds the decode table, and no earlier problem's waves still
// read the staging area).
template <int FMT, int MB, bool SPREAD>
__device__ __forceinline__ void stream_problem(SmemS<FMT> &sh, const GemvDesc &d, int g, int e,
                                               bool first) {
  const bool staged = SPREAD || stages_x(FMT, d.M, d.K);
  const int Kp = staged_kp(FMT, MB, d.K), pitch = stage_pitch(d.M, Kp, kXsStream);
  // (spread rows after the K-order rows when the launch quantizes them)
  const int sbase = SPREAD && d.x ? spread_base(d.M, pitch) : 0;
  const int spitch = SPREAD ? spread_pitch(d.M, Kp) : 0;
  // (the set-up's loads leave before the weights': the first units of
  // weights stay in flight while the block sets up)
  constexpr int NQ = MB <= 2 && !SPREAD ? 8 : 0;
  PreLoads<NQ> pl;
  pre_issue<FMT>(d, staged, Kp, first, pl);
  __builtin_amdgcn_sched_barrier(0);
  ItemLoop<FMT, MB, SPREAD> loop;
  loop.start(d, staged, pitch, g - d.item_begin, e - d.item_begin, sbase, spitch);
  __builtin_amdgcn_sched_barrier(0);
  if (!first) __syncthreads();  // the previous problem's staged rows are done
  setup_finish<FMT, NQ, Cfg<FMT, MB, false>::WIDE, SPREAD>(d, sh, staged, Kp, pitch, first, false,
                                                          pl, sbase, spitch);
  // in a scalar register: a use in the loop then waits for no load
  loop.beta = __builtin_bit_cast(float, uniform(__builtin_bit_cast(int, pl.beta)));
  loop.run(d, sh);
  if (d.x && g == d.item_begin) write_act_outputs<FMT, SPREAD>(d, sh, pitch);
}

// The block takes the global items [g0, g1) of the plan (problem p0 holds
// item g0; problem q owns [item_begin, +items)), crossing into the next
// problem when its range does.  d0: problem p0's descriptor, which the
// block's entry carries (fetched with g0 and g1).
template <int FMT, int MB, bool SPREAD>
__device__ __forceinline__ void stream_block(const GemvDesc *plan, int count, const GemvDesc &d0,
                                             int p0, int g0, int g1) {
  __shared__ SmemS<FMT> sh;
  bool first = true;
  GemvDesc d = d0;
  for (int g = g0, p = p0; g < g1 && p < count;) {
    const int e = min(g1, d.item_begin + d.items);
    if (e > g) {
      stream_problem<FMT, MB, SPREAD>(sh, d, g, e, first);
      first = false;
      g = e;
    }
    if (++p < count && g < g1) d = fetch_uniform(plan + p);
  }
}

template <int FMT, int MB, bool SPREAD = false>
__global__ __launch_bounds__(kThreads) void gemv_stream_single(GemvDesc d) {
  const int64_t T = d.items;
  const int g0 = (int)(T * blockIdx.x / gridDim.x), g1 = (int)(T * (blockIdx.x + 1) / gridDim.x);
  if (g0 < g1) stream_block<FMT, MB, SPREAD>(&d, 1, d, 0, g0, g1);
}

template <int FMT, int MB, bool SPREAD = false>
__global__ __launch_bounds__(kThreads) void gemv_stream_grouped(const GemvDesc *__restrict__ plan,
                                                                const GemvBlock *__restrict__ blocks,
                                                                int count) {
  const GemvBlock bl = fetch_uniform(blocks + blockIdx.x);
  if (bl.i0 < bl.i1) stream_block<FMT, MB, SPREAD>(plan, count, bl.d, bl.p, bl.i0, bl.i1);
}

// ---------------------------------------------------------------------------
// Fine split (M <= 16, staged activations).
//
// A decode-sized launch is one chain of dependent steps per block: fetch the
// block's descriptor, issue the activation and weight loads, stage the
// activations, multiply, reduce, store.  This path keeps that chain short:
// the descriptor (FineBlock) is one round trip of scalar loads that holds every derived
// value (no lane divides by a run-time value), the decode table and the
// zeroed slots are written while it is in flight, the weight loads leave as
// soon as it arrives, and the activations are quantized (or copied) straight
// into their permuted LDS positions, so the set-up has one barrier (two
// with fp32 activations, whose row maxima need one).  The problem's kind
// (fp32 activations or x_q) is a template parameter instead of a branch.

// Four activation codes (the bytes of v) of positions k .. k+3 (k % 4 == 0)
// into the staged row at `row`.  Five trits per byte: inside its 80-position
// window x[5g + e] goes to byte 4g + e (e < 4) or 64 + g (e == 4), the order
// of the decoded weight fragments; one trit per byte: K order.
template <int FMT>
__device__ __forceinline__ void stage4(int8_t *row, int k, uint32_t v) {
  if (FMT != UG_W_PACK5) {
    *reinterpret_cast<uint32_t *>(row + k) = v;
    return;
  }
  const int win = k / 80, r = k - 80 * win;  // the four share a window (80 % 4 == 0)
  int g = r / 5, e = r - 5 * g;
  int8_t *base = row + 80 * win;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    base[e < 4 ? 4 * g + e : 64 + g] = (int8_t)(v >> (8 * j));
    if (++e == 5) {
      e = 0;
      ++g;
    }
  }
}

// A wave's activation tiles: [t, te) of the block's M * T tiles (row m =
// t / T, chunk c = t % T), taken NB at a time, (m, c) advanced by
// increments from the start the planner computed.  Batches: fp32 tiles 4
// (a decode-sized problem gives a wave at most 4), x_q tiles 8 (8 waves
// times 8 KB cover the whole staging area: always one batch).
template <bool FUSED>
constexpr int kTileBatch = FUSED ? 4 : 8;
struct TileWalk {
  int t, te, m, c, T;
};
template <int NB>
struct TileBatch {
  bool ok[NB];
  int m[NB], c[NB];
};
template <int NB>
__device__ __forceinline__ void next_batch(TileWalk &w, TileBatch<NB> &b) {
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    b.ok[i] = w.t + i < w.te;
    b.m[i] = w.m;
    b.c[i] = w.c;
    if (++w.c == w.T) {
      w.c = 0;
      ++w.m;
    }
  }
  w.t += NB;
}

// fp32 tiles: 256 positions, lane l the float4 at 256 c + 4 l (a float4 at
// k < K is inside the row: the row pitch is at least round_up(K, 4) floats).
// x_q tiles: 1024 bytes, lane l the 16 bytes at 1024 c + 16 l (inside the
// row when k < K: pitch >= round_up(K, 16)).  ldx in bytes.
template <bool FUSED, int NB>
__device__ __forceinline__ void load_batch(__amdgpu_buffer_rsrc_t xr, int ldx, int K,
                                           const TileBatch<NB> &b, uint4 (&u)[NB]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int k = FUSED ? b.c[i] * 256 + 4 * lane : b.c[i] * 1024 + 16 * lane;
    // a tile past the wave's share starts past the buffer (selects, no
    // branch: every offset below 2^31 + 2^18 reads nothing past it)
    const uint32_t row = b.ok[i] ? (uint32_t)(b.m[i] * ldx) : kOOB;
    u[i] = buffer_load16(xr, k < K ? row + (uint32_t)(FUSED ? 4 * k : k) : kOOB);
  }
}

// Pass 1 of fused quantization: per-wave row maxima.
template <int FMT, int NB>
__device__ __forceinline__ void fine_absmax(Smem<FMT, kFineWaves> &sh, const TileBatch<NB> &b, const uint4 (&u)[NB],
                                            int K) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    if (b.ok[i]) {
      const float4 v = __builtin_bit_cast(float4, u[i]);
      const int k = b.c[i] * 256 + 4 * lane;
      float a = fabsf(v.x);  // zero when k >= K
      if (k + 1 < K) a = fmaxf(a, fabsf(v.y));
      if (k + 2 < K) a = fmaxf(a, fabsf(v.z));
      if (k + 3 < K) a = fmaxf(a, fabsf(v.w));
      a = wave_max(a);
      if (lane == 0) sh.part[wave][b.m[i]] = fmaxf(sh.part[wave][b.m[i]], a);
    }
  }
}

// Pass 2: codes into the staged rows (zeros past K), and into x_q when the
// block writes it.  The codes are ug_quant_act's, bit for bit.
template <int FMT, int NB>
__device__ __forceinline__ void fine_quant(Smem<FMT, kFineWaves> &sh, const TileBatch<NB> &b, const uint4 (&u)[NB],
                                           int K, int Kp, int pitch, float eps, int8_t *xq_out,
                                           int ldxq_out) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int m = b.m[i], k = b.c[i] * 256 + 4 * lane;
    if (b.ok[i] && k < Kp) {
      const float4 v = __builtin_bit_cast(float4, u[i]);
      const float s = row_scale(sh, m, eps);
      int c0, c1, c2, c3;
      q8x4(v, s, c0, c1, c2, c3);
      const uint32_t w = pack4(k < K ? c0 : 0, k + 1 < K ? c1 : 0, k + 2 < K ? c2 : 0,
                               k + 3 < K ? c3 : 0);
      stage4<FMT>(sh.xs + m * pitch, k, w);
      if (xq_out && k < K) {
        int8_t *row = xq_out + m * ldxq_out;
        if (k + 4 <= K) {
          *gp(reinterpret_cast<uint32_t *>(row + k)) = w;  // rows are 16-byte aligned
        } else {
          for (int j = 0; k + j < K; ++j) gp(row)[k + j] = (int8_t)(w >> (8 * j));
        }
      }
    }
  }
}

// x_q tiles into the staged rows, bytes past K zeroed.
template <int FMT, int NB>
__device__ __forceinline__ void fine_copy(Smem<FMT, kFineWaves> &sh, const TileBatch<NB> &b, const uint4 (&u)[NB],
                                          int K, int Kp, int pitch) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int k = b.c[i] * 1024 + 16 * lane;
    if (b.ok[i] && k < Kp) {  // Kp % 16 == 0: the 16 bytes are all inside or all past
      const uint32_t w4[4] = {u[i].x, u[i].y, u[i].z, u[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int kb = K - k - 4 * e;  // bytes of this dword inside the row
        stage4<FMT>(sh.xs + b.m[i] * pitch, k + 4 * e,
                    w4[e] & (kb >= 4 ? 0xffffffffu : (kb <= 0 ? 0u : (0xffffffffu >> (8 * (4 - kb))))));
      }
    }
  }
}

// The activation fragments of one step from the staged rows (xoff: this
// lane's row and K offset of the step).
template <int FMT>
__device__ __forceinline__ void fine_xfrags(const int8_t *xs, int xoff,
                                            v4i (&xf)[Fmt<FMT>::kFrag]) {
#pragma unroll
  for (int j = 0; j < Fmt<FMT>::kFrag; ++j) xf[j] = *reinterpret_cast<const v4i *>(xs + xoff + 16 * j);
}

// One (item, step) piece: the step's activation fragments times the decoded
// weights, into acc (two independent chains).
template <int FMT>
__device__ __forceinline__ void fine_piece(const v4i (&xf)[Fmt<FMT>::kFrag], const char *lut,
                                           const uint4 &w, v4i (&acc)[2]) {
  acc[0] = acc[1] = v4i{0, 0, 0, 0};
  if (FMT == UG_W_PACK5) {
    const uint32_t lr8 = 8u * (threadIdx.x & 31);
    uint32_t t[20];
    decode4_wide(w.x, lut, lr8, t, t[16]);
    decode4_wide(w.y, lut, lr8, t + 4, t[17]);
    decode4_wide(w.z, lut, lr8, t + 8, t[18]);
    decode4_wide(w.w, lut, lr8, t + 12, t[19]);
#pragma unroll
    for (int j = 0; j < 5; ++j) {
      const v4i B = {(int)t[4 * j], (int)t[4 * j + 1], (int)t[4 * j + 2], (int)t[4 * j + 3]};
      acc[j & 1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xf[j], B, acc[j & 1], 0, 0, 0);
    }
  } else {
    const v4i B = {(int)w.x, (int)w.y, (int)w.z, (int)w.w};
    acc[0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xf[0], B, acc[0], 0, 0, 0);
  }
}

// Adds a piece's sums (lane (n, q) holds rows 4q .. 4q+3 of column n) to
// the item's LDS slot.  The test is uniform (r < M, not 4q + r < M): the
// slot has room for 16 rows, and rows past M are never read.
__device__ __forceinline__ void fine_flush(int *slots, int it, int M, const v4i (&acc)[2]) {
  const v4i v = acc[0] + acc[1];
  const int lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (r < M) atomicAdd(&slots[it * 256 + (4 * q + r) * 16 + n], v[r]);
}

// The block of descriptor b; ws = this wave's wave_start word; lut = this
// thread's decode table entry (table_load, five trits per byte).  Pieces
// in step-major order, p = (step p / items, item p % items), of the block's
// P = items * S: wave w takes [w P / 8, (w + 1) P / 8) and issues all their
// weight loads at once (after the activation loads).  Consecutive pieces of
// a wave share their step, so the wave reads a step's activation fragments
// from LDS once for all its items; each piece's sums go to its item's LDS
// slot (flushed one piece later, when its MFMAs are done).  After a barrier
// the block writes every item's outputs.
// LEVEL: the loads each wave issues whether or not its share needs them
// (each costs the CU's texture path about as much as a real one): 0, up to
// kFinePieces weight loads and a batch of activation tiles; 1 (short),
// kShortPieces and kShortTiles; 2 (tiny), kTinyPieces and kTinyTiles.
template <int FMT, bool FUSED, int LEVEL>
__device__ __forceinline__ void fine_block(const FineBlock &b, uint32_t ws,
                                           uint2 lut_entry) {
  constexpr int MP = LEVEL == 2 ? kTinyPieces : (LEVEL == 1 ? kShortPieces : kFinePieces);
  __shared__ Smem<FMT, kFineWaves> sh;
  const int tid = threadIdx.x, wave = uniform(tid >> 6), lane = tid & 63;
  // the table's and the descriptor's loads (the caller's) leave first
  __builtin_amdgcn_sched_barrier(0);

  const int M = b.shape & 0xff, items = (b.shape >> 8) & 0xff, S = b.shape >> 16, K = b.K;
  const int Kp = S * Fmt<FMT>::kStepK;  // staged row: whole steps, zeros past K
  const int pitch = stage_pitch(M, Kp, kXsBytes);
  const int P = items * S;
  const int p0 = (wave * P) >> kFineWaveShift, p1 = ((wave + 1) * P) >> kFineWaveShift;
  const int T = FUSED ? (Kp + 255) >> 8 : (Kp + 1023) >> 10;  // tiles cover whole staged rows
  const int nt = M * T;
  const float s_in = !FUSED && tid < M ? gp(b.s)[tid] : 0.0f;

  // activation loads, then weight loads: loads complete in issue order, so
  // waiting for the activations never waits for the weights
  const __amdgpu_buffer_rsrc_t xr = buffer_rsrc(b.x, (uint32_t)(M * b.ldx));
  TileWalk walk{(wave * nt) >> kFineWaveShift, ((wave + 1) * nt) >> kFineWaveShift,
                in_vgpr((ws >> 16) & 0xff), in_vgpr(ws >> 24), T};
  constexpr int NB = LEVEL == 2 ? kTinyTiles : (LEVEL == 1 ? kShortTiles : kTileBatch<FUSED>);
  TileBatch<NB> b0;
  uint4 x0[NB];
  next_batch(walk, b0);
  const TileWalk rest = walk;  // the tiles after the first batch
  load_batch<FUSED>(xr, b.ldx, K, b0, x0);
  __builtin_amdgcn_sched_barrier(0);  // the activation loads leave first
  const __amdgpu_buffer_rsrc_t wr = buffer_rsrc(b.w, (uint32_t)(b.N * b.ldw));
  uint4 wb[MP];
  {
    // unsigned (wrapping) offsets: an offset that wraps into the buffer
    // reads real weights for a row past N, whose results are never stored;
    // pieces past the wave's share read past the buffer (nothing)
    // (the pieces' bookkeeping in vector registers, see in_vgpr)
    const uint32_t ldw = (uint32_t)b.ldw, item_step = 16u * ldw;
    const uint32_t wrap_step = 64u - (uint32_t)(items - 1) * item_step;  // to item 0 of the next step
    int it = in_vgpr(ws & 0xff);
    uint32_t voff = (uint32_t)(b.i0 * 16 + (lane & 15)) * ldw + 16u * (lane >> 4) +
                    (uint32_t)it * item_step + 64u * ((ws >> 8) & 0xff);
#pragma unroll
    for (int j = 0; j < MP; ++j) {
      wb[j] = buffer_load16_stream(wr, p0 + j < p1 ? voff : kOOB);
      const bool wrap = ++it == items;
      it = wrap ? 0 : it;
      voff += wrap ? wrap_step : item_step;
    }
  }
  // a vector load (after the weights, used after them): a scalar one would
  // make the set-up's first LDS wait also wait for it
  const float beta = __builtin_bit_cast(float, buffer_load4(buffer_rsrc(b.beta, 4), 0));

  // LDS set-up that needs nothing from the activations: the table (its
  // loads were issued first, so waiting for them waits for nothing later)
  // and zeroed slots
  if (FMT == UG_W_PACK5) table_store<true>(sh, lut_entry);
#pragma unroll
  for (int i = 0; i < kFineItems * 64 / kFineThreads; ++i)
    reinterpret_cast<uint4 *>(sh.slots)[tid + i * kFineThreads] = make_uint4(0, 0, 0, 0);
  if (FUSED) sh.part[wave][lane] = 0.0f;  // this wave's own row maxima

  // staged rows
  if (FUSED) {
    fine_absmax(sh, b0, x0, K);
    for (TileWalk w = rest; w.t < w.te;) {
      TileBatch<NB> bb;
      uint4 u[NB];
      next_batch(w, bb);
      load_batch<true>(xr, b.ldx, K, bb, u);
      fine_absmax(sh, bb, u, K);
    }
    __syncthreads();  // row maxima
    if (tid < M) {
      const float s = row_scale(sh, tid, b.eps);
      sh.sm[tid] = s;
      if (b.s) gp(b.s)[tid] = s;
    }
    fine_quant(sh, b0, x0, K, Kp, pitch, b.eps, b.xq_out, b.ldxq_out);
    for (TileWalk w = rest; w.t < w.te;) {
      TileBatch<NB> bb;
      uint4 u[NB];
      next_batch(w, bb);
      load_batch<true>(xr, b.ldx, K, bb, u);
      fine_quant(sh, bb, u, K, Kp, pitch, b.eps, b.xq_out, b.ldxq_out);
    }
  } else {
    if (tid < M) sh.sm[tid] = s_in;
    fine_copy(sh, b0, x0, K, Kp, pitch);
    for (TileWalk w = rest; w.t < w.te;) {
      TileBatch<NB> bb;
      uint4 u[NB];
      next_batch(w, bb);
      load_batch<false>(xr, b.ldx, K, bb, u);
      fine_copy(sh, bb, u, K, Kp, pitch);
    }
  }
  __syncthreads();  // table, slots, scales and staged rows

  const char *lut = reinterpret_cast<const char *>(sh.lut);
  // rows past M read row M-1: MFMA output row m depends only on input row m,
  // and rows past M are never stored
  const int xoff = min(lane & 15, M - 1) * pitch + (lane >> 4) * Fmt<FMT>::kLaneK;
  v4i xf[Fmt<FMT>::kFrag];
  v4i acc[2], prev[2];
  int it = ws & 0xff, st = (ws >> 8) & 0xff, xst = -1, prev_it = 0;
#pragma unroll
  for (int j = 0; j < MP; ++j) {
    if (p0 + j < p1) {
      if (st != xst) {  // a new step: its fragments serve the following pieces too
        fine_xfrags<FMT>(sh.xs, xoff + st * Fmt<FMT>::kStepK, xf);
        xst = st;
      }
      fine_piece<FMT>(xf, lut, wb[j], acc);
      if (j > 0) fine_flush(sh.slots, prev_it, M, prev);
      prev[0] = acc[0];
      prev[1] = acc[1];
      prev_it = it;
      if (++it == items) {
        it = 0;
        ++st;
      }
    }
  }
  if (p0 < p1) fine_flush(sh.slots, prev_it, M, prev);
  __syncthreads();
  if (tid < items * 16) {  // thread (item, n) writes column n of the item, every row
    const int li = tid >> 4, n = tid & 15, ng = (b.i0 + li) * 16 + n;
    if (ng < b.N) {
      const float bn = b.bias ? gp(b.bias)[ng] : 0.0f;
      for (int m = 0; m < M; ++m) {
        const int val = sh.slots[li * 256 + m * 16 + n];
        if (b.acc) gp(b.acc)[(int64_t)m * b.ldacc + ng] = val;
        if (b.y) {
          const float v = (float)val * (sh.sm[m] * beta);
          gp(b.y)[(int64_t)m * b.ldy + ng] = b.bias ? v + bn : v;
        }
      }
    }
  }
}

// One problem: every block but the last takes the items of b.shape from
// blockIdx.x times that count (b.wave_start); the last takes last.items
// (last.wave_start).
struct FineTail {
  uint32_t wave_start[kFineWaves];
  int32_t items;
};

template <int FMT, int LEVEL>
__global__ __launch_bounds__(kFineThreads) void gemv_fine_single(const FineBlock b, const FineTail last) {
  const uint2 lut = FMT == UG_W_PACK5 ? table_load() : uint2{0, 0};
  const bool is_last = blockIdx.x + 1 == gridDim.x;
  const int wave = uniform(threadIdx.x >> 6);
  // indexed in the argument segment itself (a modified copy would be
  // indexed in scratch memory)
  const uint32_t ws = is_last ? last.wave_start[wave] : b.wave_start[wave];
  FineBlock mine = b;
  mine.i0 = blockIdx.x * ((b.shape >> 8) & 0xff);
  if (is_last) mine.shape = (b.shape & 0xffff00ffu) | ((uint32_t)last.items << 8);
  fine_block<FMT, false, LEVEL>(mine, ws, lut);
}

template <int FMT, bool FUSED, int LEVEL>
__global__ __launch_bounds__(kFineThreads) void gemv_fine_grouped(const FineBlock *__restrict__ blocks) {
  // the table's load first: both fetches travel together
  const uint2 lut = FMT == UG_W_PACK5 ? table_load() : uint2{0, 0};
  const FineBlock b = blocks[blockIdx.x];
  fine_block<FMT, FUSED, LEVEL>(b, blocks[blockIdx.x].wave_start[uniform(threadIdx.x >> 6)], lut);
}

// ---------------------------------------------------------------------------
// Host side.

// The FineBlock of items [i0, i1) of problem d; `first`: the problem's
// first block (the one that writes the fused quantization's outputs).
FineBlock fine_block_of(const GemvDesc &d, int i0, int i1, bool first) {
  const bool fused = d.x != nullptr;
  FineBlock f{};
  f.x = fused ? (const void *)d.x : (const void *)d.xq;
  f.w = d.w;
  f.beta = d.beta;
  f.bias = d.bias;
  f.y = d.y;
  f.acc = d.acc;
  f.s = fused ? (first ? d.s : nullptr) : d.s;
  f.xq_out = fused && first ? const_cast<int8_t *>(d.xq) : nullptr;
  f.ldx = (int32_t)(fused ? 4 * d.ldx : d.ldxq);
  f.ldw = (int32_t)d.ldw;
  f.ldy = (int32_t)d.ldy;
  f.ldacc = (int32_t)d.ldacc;
  f.ldxq_out = fused ? (int32_t)d.ldxq : 0;
  f.eps = d.eps;
  f.N = d.N;
  f.K = d.K;
  f.i0 = i0;
  const int S = steps_of(d.wfmt, d.K), P = (i1 - i0) * S, Kp = fine_kp(d.wfmt, d.K);
  const int T = fused ? (Kp + 255) >> 8 : (Kp + 1023) >> 10, nt = d.M * T;
  f.shape = (uint32_t)d.M | ((uint32_t)(i1 - i0) << 8) | ((uint32_t)S << 16);
  for (int w = 0; w < kFineWaves; ++w) {
    const int p0 = (w * P) >> kFineWaveShift, t0 = (w * nt) >> kFineWaveShift;
    // pieces in step-major order: p = step * items + item
    const int items = i1 - i0;
    f.wave_start[w] = (uint32_t)(p0 % items) | ((uint32_t)(p0 / items) << 8) |
                      ((uint32_t)(t0 / T) << 16) | ((uint32_t)(t0 % T) << 24);
  }
  return f;
}

// Fine split of a group: items per block for every problem, or false when
// the group is too large for it (then the stream split runs).  Blocks of
// about T / 256 pieces each, at most kFineItems items, one problem each.
bool plan_fine(GemvDesc *descs, int count, std::vector<FineBlock> &blocks) {
  int64_t T = 0;
  for (int i = 0; i < count; ++i) {
    const GemvDesc &d = descs[i];
    if (d.M > 16 || (int64_t)d.M * fine_kp(d.wfmt, d.K) > kXsBytes) return false;
    if ((d.x != nullptr) != (descs[0].x != nullptr)) return false;  // one kind per launch
    // the block descriptor holds 32-bit pitches
    if (d.ldy >= (INT64_C(1) << 31) || d.ldacc >= (INT64_C(1) << 31) ||
        d.ldxq >= (INT64_C(1) << 31) || 4 * d.ldx >= (INT64_C(1) << 31))
      return false;
    T += (int64_t)((d.N + 15) / 16) * steps_of(d.wfmt, d.K);
  }
  if (T > (int64_t)kGemvBlocks * kFineWaves * kFinePieces) return false;
  std::vector<int> ipb((size_t)count);
  for (int64_t target = (T + kGemvBlocks - 1) / kGemvBlocks;; ++target) {
    if (target > (int64_t)kFineWaves * kFinePieces) return false;
    int64_t nb = 0;
    bool fits = true;
    for (int i = 0; i < count; ++i) {
      const int S = steps_of(descs[i].wfmt, descs[i].K), items = (descs[i].N + 15) / 16;
      int k = (int)(target / S);
      k = k < 1 ? 1 : (k > kFineItems ? kFineItems : k);
      k = k > items ? items : k;
      // every wave's share of a block's pieces must fit its registers (so
      // a block has at most 64 pieces and an item at most 64 steps)
      if ((k * S + kFineWaves - 1) / kFineWaves > kFinePieces) fits = false;
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
      blocks.push_back(fine_block_of(descs[i], a, std::min(items, a + ipb[(size_t)i]), a == 0));
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

namespace {

// A stream block pays a set-up for every problem it works on: the
// descriptor's round trip, staging the problem's activation rows, and its
// weight pipeline draining at the switch.  Measured, one switch costs about
// as long as streaming this many weight bytes on one CU.
constexpr int64_t kSwitchBytes = 64 << 10;

// Item ranges of the stream split: ends[b] = the end of block b's range
// (block b takes [ends[b-1], ends[b]), ends[grid-1] = every item).  Blocks
// are cut so that the largest cost (weight bytes of the block's items plus
// kSwitchBytes for every problem after its first) is as small as it can be:
// the least cap for which a greedy fill in problem order needs at most
// `grid` blocks (a binary search on the cap).  Equal item counts instead put
// the blocks whose range crosses into the next problem on the launch's
// critical path.
void stream_ranges(const GemvDesc *descs, int count, int grid, std::vector<int32_t> &ends) {
  std::vector<int64_t> item_cost(count);
  int64_t total_cost = 0, max_item = 1;
  for (int i = 0; i < count; ++i) {
    const GemvDesc &d = descs[i];
    item_cost[i] = (int64_t)16 * rgw_of(d.wfmt, d.mb) * row_bytes_of(d.wfmt, d.K);
    max_item = std::max(max_item, item_cost[i]);
    total_cost += item_cost[i] * d.items;
  }
  // greedy fill under `cap`: the block ends (as item numbers), or false
  // when more than `grid` blocks are needed
  auto fill = [&](int64_t cap, std::vector<int32_t> *out) {
    int blocks = 1;
    int64_t cost = 0;  // of the open block
    bool open_has_items = false;
    int32_t g = 0;
    for (int i = 0; i < count; ++i) {
      int64_t left = descs[i].items;
      bool entered = false;  // the open block already pays for problem i
      while (left > 0) {
        const int64_t enter = open_has_items && !entered ? kSwitchBytes : 0;
        int64_t fits = cap - cost - enter;
        fits = fits > 0 ? fits / item_cost[i] : 0;
        if (fits <= 0) {
          if (!open_has_items) return false;  // the cap is below one item
          if (out) out->push_back(g);
          if (++blocks > grid) return false;
          cost = 0;
          open_has_items = false;
          entered = false;
          continue;
        }
        const int64_t take = std::min(left, fits);
        cost += enter + take * item_cost[i];
        open_has_items = true;
        entered = true;
        left -= take;
        g += (int32_t)take;
      }
    }
    if (out) {
      out->push_back(g);
      while ((int)out->size() < grid) out->push_back(g);
    }
    return true;
  };
  int64_t lo = std::max(max_item, total_cost / grid), hi = total_cost + kSwitchBytes * count;
  while (lo < hi) {
    const int64_t mid = lo + (hi - lo) / 2;
    if (fill(mid, nullptr))
      hi = mid;
    else
      lo = mid + 1;
  }
  ends.clear();
  fill(lo, &ends);
}

}  // namespace

int gemv_plan(GemvDesc *descs, int count, std::vector<GemvBlock> &blocks,
              std::vector<FineBlock> &fine) {
  const int fmt = descs[0].wfmt;
  for (int i = 1; i < count; ++i)
    if (descs[i].wfmt != fmt) return -1;
  int64_t total = 0;
  blocks.clear();
  if (plan_fine(descs, count, fine)) {
    for (int i = 0; i < count; ++i) {
      descs[i].item_begin = (int32_t)total;
      total += descs[i].items;
    }
    // the short variant when every wave of every block fits it
    // (and the tiny one, a stricter short, when every wave fits that)
    bool short_ok = true, tiny_ok = true;
    for (const FineBlock &f : fine) {
      const int M = f.shape & 0xff, items = (f.shape >> 8) & 0xff, S = f.shape >> 16;
      const int Kp = S * (fmt == UG_W_PACK5 ? 320 : 64);
      const int T = descs[0].x ? (Kp + 255) >> 8 : (Kp + 1023) >> 10;
      const int pw = (items * S + kFineWaves - 1) / kFineWaves, tw = (M * T + kFineWaves - 1) / kFineWaves;
      if (pw > kShortPieces || tw > kShortTiles) short_ok = false;
      if (pw > kTinyPieces || tw > kTinyTiles) tiny_ok = false;
    }
    return (short_ok && tiny_ok ? 4096 : 0) + (short_ok ? 1024 : 0) + (descs[0].x ? 512 : 0) +
           256 + 16 * fmt + 1;
  }
  const int mb = mb_of(descs[0].M);
  bool chunked = false;  // some problem's activations do not fit the staging area
  for (int i = 0; i < count; ++i) {
    GemvDesc &d = descs[i];
    d.mb = mb_of(d.M);
    if (d.mb != mb) return -1;
    if (!stages_x(d.wfmt, d.M, d.K)) chunked = true;
    const int rg = (d.N + 15) / 16, rgw = rgw_of(d.wfmt, d.mb);
    d.items = (rg + rgw - 1) / rgw;  // rgw row groups per item
    d.item_begin = (int32_t)total;
    total += d.items;
  }
  if (total > INT32_MAX) return -1;
  // the chunked kernel reads x_q only: a group that needs it cannot also
  // quantize fp32 activations in the launch
  if (chunked)
    for (int i = 0; i < count; ++i)
      if (descs[i].x != nullptr) return -2;
  const int grid = gemv_grid(total);
  fine.clear();
  std::vector<int32_t> ends;
  stream_ranges(descs, count, grid, ends);
  int p = 0, g0 = 0;
  for (int b = 0; b < grid; ++b) {
    const int g1 = ends[b];
    while (p + 1 < count && descs[p + 1].item_begin <= g0) ++p;
    blocks.push_back(GemvBlock{descs[p], p, g0, g1, 0});
    g0 = g1;
  }
  // the spread staging when every problem's rows fit it
  bool spread = !chunked && fmt == UG_W_PACK5 && mb == 1;
  for (int i = 0; i < count && spread; ++i)
    if (!stages_spread(descs[i].M, descs[i].K, descs[i].x != nullptr)) spread = false;
  return (spread ? 8192 : 0) + (chunked ? 2048 : 0) + 16 * fmt + mb;
}

void fine_xcd_order(std::vector<FineBlock> &fine) {
  // block b runs on XCD b % 8 (blocks are dealt to the XCDs round-robin):
  // the table's i-th block goes to the i-th slot in XCD-major order, so
  // each problem's consecutive blocks land on one XCD (or two, at a seam)
  constexpr int kXcd = 8;
  const int nb = (int)fine.size();
  if (nb <= kXcd) return;
  std::vector<FineBlock> out((size_t)nb);
  int src = 0;
  for (int x = 0; x < kXcd; ++x)
    for (int i = x; i < nb; i += kXcd) out[(size_t)i] = fine[(size_t)src++];
  fine.swap(out);
}

bool gemv_stages_x(int wfmt, int64_t M, int64_t K) {
  // (the documented limit for activations quantized in the launch: 64 KB of
  // staged rows, inside the stream split's larger area)
  return K <= UG_MAX_K && M <= 64 && (int64_t)M * staged_kp(wfmt, mb_of((int)M), (int)K) <= kXsBytes;
}

hipError_t launch_gemv_grouped(const GemvDesc *plan_dev, const void *table, int32_t count,
                               int32_t grid, int32_t variant, hipStream_t st) {
  const bool fine = (variant >> 8) & 1, fused = (variant >> 9) & 1;
  const int level = (variant >> 12) & 1 ? 2 : ((variant >> 10) & 1);
  const int fmt = (variant >> 4) & 15, mb = variant & 15;
  dim3 g(grid), b(kThreads);
  if (fine) {
    const FineBlock *fb = static_cast<const FineBlock *>(table);
    b = dim3(kFineThreads);
#define UG_FINE(F, FU, LV) hipLaunchKernelGGL((gemv_fine_grouped<F, FU, LV>), g, b, 0, st, fb)
#define UG_FINE_LV(F, FU) \
  do { if (level == 2) UG_FINE(F, FU, 2); else if (level == 1) UG_FINE(F, FU, 1); else UG_FINE(F, FU, 0); } while (0)
    if (fmt == UG_W_PACK5) {
      if (fused) UG_FINE_LV(UG_W_PACK5, true); else UG_FINE_LV(UG_W_PACK5, false);
    } else {
      if (fused) UG_FINE_LV(UG_W_I8, true); else UG_FINE_LV(UG_W_I8, false);
    }
#undef UG_FINE_LV
#undef UG_FINE
    return hipGetLastError();
  }
  const GemvBlock *blocks_dev = static_cast<const GemvBlock *>(table);
  if ((variant >> 11) & 1) {
#define UG_CHUNKED(F, MBV) \
  hipLaunchKernelGGL((gemv_chunked_grouped<F, MBV>), g, b, 0, st, plan_dev, blocks_dev, count)
    if (fmt == UG_W_PACK5) {
      if (mb == 1) UG_CHUNKED(UG_W_PACK5, 1);
      else if (mb == 2) UG_CHUNKED(UG_W_PACK5, 2);
      else UG_CHUNKED(UG_W_PACK5, 4);
    } else {
      if (mb == 1) UG_CHUNKED(UG_W_I8, 1);
      else if (mb == 2) UG_CHUNKED(UG_W_I8, 2);
      else UG_CHUNKED(UG_W_I8, 4);
    }
#undef UG_CHUNKED
    return hipGetLastError();
  }
#define UG_GROUPED(F, MBV) \
  hipLaunchKernelGGL((gemv_stream_grouped<F, MBV>), g, b, 0, st, plan_dev, blocks_dev, count)
  if ((variant >> 13) & 1) {
    hipLaunchKernelGGL((gemv_stream_grouped<UG_W_PACK5, 1, true>), g, b, 0, st, plan_dev,
                       blocks_dev, count);
  } else if (fmt == UG_W_PACK5) {
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
                       int64_t ldw, const float *beta, const float *bias, int64_t M, int64_t N,
                       int64_t K,
                       int32_t *acc, int64_t ldacc, float *y, int64_t ldy, hipStream_t st) {
  GemvDesc d{};
  d.x = nullptr;
  d.xq = xq;
  d.ldxq = ldx;
  d.s = const_cast<float *>(s);
  d.w = (const uint8_t *)w;
  d.ldw = ldw;
  d.beta = beta;
  d.bias = bias;
  d.acc = acc;
  d.ldacc = ldacc;
  d.y = y;
  d.ldy = ldy;
  d.wfmt = wfmt;
  d.M = (int32_t)M;
  d.N = (int32_t)N;
  d.K = (int32_t)K;
  std::vector<GemvBlock> blocks;
  std::vector<FineBlock> fine;
  const int variant = gemv_plan(&d, 1, blocks, fine);
  if (variant < 0) return hipErrorInvalidValue;
  if ((variant >> 8) & 1) {
    // one problem: equal blocks, the last maybe shorter
    FineTail last{};
    std::copy(fine.back().wave_start, fine.back().wave_start + kFineWaves, last.wave_start);
    last.items = (int32_t)((fine.back().shape >> 8) & 0xff);
    dim3 g((unsigned)fine.size()), b(kFineThreads);
    const int level = (variant >> 12) & 1 ? 2 : ((variant >> 10) & 1);
#define UG_SINGLE(F, LV) hipLaunchKernelGGL((gemv_fine_single<F, LV>), g, b, 0, st, fine[0], last)
    if (wfmt == UG_W_PACK5) {
      if (level == 2) UG_SINGLE(UG_W_PACK5, 2); else if (level == 1) UG_SINGLE(UG_W_PACK5, 1); else UG_SINGLE(UG_W_PACK5, 0);
    } else {
      if (level == 2) UG_SINGLE(UG_W_I8, 2); else if (level == 1) UG_SINGLE(UG_W_I8, 1); else UG_SINGLE(UG_W_I8, 0);
    }
#undef UG_SINGLE
    return hipGetLastError();
  }
  const int grid = (int)blocks.size();
  dim3 g(grid), b(kThreads);
  if ((variant >> 11) & 1) {
#define UG_CHUNKED(F, MBV) hipLaunchKernelGGL((gemv_chunked_single<F, MBV>), g, b, 0, st, d)
    if (wfmt == UG_W_PACK5) {
      if (d.mb == 1) UG_CHUNKED(UG_W_PACK5, 1);
      else if (d.mb == 2) UG_CHUNKED(UG_W_PACK5, 2);
      else UG_CHUNKED(UG_W_PACK5, 4);
    } else {
      if (d.mb == 1) UG_CHUNKED(UG_W_I8, 1);
      else if (d.mb == 2) UG_CHUNKED(UG_W_I8, 2);
      else UG_CHUNKED(UG_W_I8, 4);
    }
#undef UG_CHUNKED
    return hipGetLastError();
  }
#define UG_SINGLE(F, MBV) hipLaunchKernelGGL((gemv_stream_single<F, MBV>), g, b, 0, st, d)
  if ((variant >> 13) & 1) {
    hipLaunchKernelGGL((gemv_stream_single<UG_W_PACK5, 1, true>), g, b, 0, st, d);
  } else if (wfmt == UG_W_PACK5) {
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

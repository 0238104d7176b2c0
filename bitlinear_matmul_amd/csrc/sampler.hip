// Top-k sampling of the next token (gfx950).
//
// "a 1-bit llm, from scratch", section "the interesting bit": the sampler
// picks the next token from the k largest of 4096 logits, and finding them
// with a size-k heap instead of sorting every logit halved the time per
// token.  "ultragraph-1bit 0.12.0" README, "A whole ternary GPT": generate()
// takes a temperature and top_k.
//
// One 256-thread block per row, nothing sorted but the k kept logits.  The
// kept set is the k largest (key, ~index) pairs, where every logit becomes
// an order-preserving 32-bit key (larger logit, larger key; -0 and +0 the
// same) and equal keys rank by lower index: k distinct 64-bit values.
//   1. a threshold x with at least k keys at or above it: each wave sorts
//      its 64 threads' largest keys (a bitonic network across the lanes)
//      and takes the ceil(k/4)-th; x is the least of the four, so at least
//      4 ceil(k/4) >= k threads hold a key >= x.  On rows whose large
//      logits are spread over the threads few keys pass (about 1.25 k for
//      independent logits);
//   2. the pairs of keys >= x go to LDS (a wave scan and one LDS atomic
//      per wave place them); if at most 256 did, each one's rank is the
//      number of candidates above it and the k lowest ranks move to their
//      slots — no histograms, six block barriers in all;
//   3. otherwise (many keys tied or packed into few threads) the k-th
//      largest key t comes from four passes of an 8-bit radix select (an
//      LDS histogram of the digit among the keys that match the digits
//      chosen so far; one wave scans it from the top digit down), one
//      block scan places every key above t, then the lowest-index keys
//      equal to t, and each kept pair moves to the slot of its rank;
//   4. rank r gets the weight e_r = expf(fl(fl(l_r - l_1) / T)); an
//      inclusive fp32 scan in one fixed order gives C_r; the token is rank
//      min(#{r : C_r <= fl(u * C_k)}, k - 1).
// Both selections give the same kept pairs in the same order.  Rows of at
// most 4096 logits stay in registers (16 per thread) throughout; longer
// rows are read again from memory (L2) for each pass.
#include "ug_internal.h"

namespace ug {
namespace {

constexpr int kThreads = 256;
constexpr int kRegPer = 16;  // logits per thread held in registers

__device__ inline uint32_t rank_key(float x) {
  const uint32_t b = __float_as_uint(x == 0.0f ? 0.0f : x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ inline float key_logit(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Inclusive sum over a wave's 64 lanes, in one fixed order: within each
// 16-lane row by shifted reads (lane l adds lane l - h for h = 1, 2, 4, 8,
// in that order; a read from before the row gives 0), then lane 15's sum
// is added into rows 1 and 3 (lane 47's, the sum of row 2, into row 3),
// then lane 31's into rows 2 and 3.  Register moves (DPP) only, no LDS
// round trip.  (int or float; for an fp32 sum this order is the order.)
template <int CTRL, int ROWS, typename T>
__device__ inline T dpp_t(T v) {
  return __builtin_bit_cast(
      T, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROWS, 0xf, true));
}
template <typename T>
__device__ inline T wave_incl_scan(T v) {
  v = v + dpp_t<0x111, 0xf>(v);  // row_shr:1
  v = v + dpp_t<0x112, 0xf>(v);  // row_shr:2
  v = v + dpp_t<0x114, 0xf>(v);  // row_shr:4
  v = v + dpp_t<0x118, 0xf>(v);  // row_shr:8
  v = v + dpp_t<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v = v + dpp_t<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// Lane l ^ S's value: strides 1, 2 and 8 by DPP (quad permutations, a
// rotation by 8 within 16-lane rows), 4 and 16 by a lane swizzle (xor mask,
// no memory access), 32 through ds_bpermute.
template <int S>
__device__ inline uint32_t xor_lane(uint32_t v) {
  if constexpr (S == 1)
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xb1, 0xf, 0xf, false);
  else if constexpr (S == 2)
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4e, 0xf, 0xf, false);
  else if constexpr (S == 8)
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xf, 0xf, false);
  else if constexpr (S == 4)
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x1f | (4 << 10));
  else if constexpr (S == 16)
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x1f | (16 << 10));
  else
    return (uint32_t)__shfl_xor((int)v, S, 64);
}

// Bitonic network over the 64 lanes (descending at the end): merge blocks
// of SIZE lanes, compare-exchange at STRIDE; blocks alternate direction.
template <int SIZE, int STRIDE>
__device__ inline uint32_t bitonic_steps(uint32_t v, int lane) {
  const uint32_t o = xor_lane<STRIDE>(v);
  const bool desc = (lane & SIZE) == 0, first = (lane & STRIDE) == 0;
  v = first == desc ? max(v, o) : min(v, o);
  if constexpr (STRIDE > 1)
    return bitonic_steps<SIZE, STRIDE / 2>(v, lane);
  else if constexpr (SIZE < 64)
    return bitonic_steps<SIZE * 2, SIZE>(v, lane);
  else
    return v;
}

// Inclusive sum over the block's 256 threads in thread order (a scan within
// each wave, then the waves' totals in order); *total gets the block sum.
// 32-bit values scan by DPP (wave_incl_scan's order); 64-bit ones lane
// l adds lane l - h for h = 1, 2, 4, .., 32.
template <typename T>
__device__ inline T block_scan(T v, T *wsum, T *total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if constexpr (sizeof(T) == 4) {
    v = wave_incl_scan(v);
  } else {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const T y = __shfl_up(v, off, 64);
      if (lane >= off) v = v + y;
    }
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  T pre = T(0);
  for (int w = 0; w < wave; ++w) pre = pre + wsum[w];
  *total = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
  __syncthreads();
  return wave ? pre + v : v;
}

template <bool REG>
__global__ __launch_bounds__(kThreads) void topk_sample(
    const float *__restrict__ logits, int64_t ld, int V, int k, float temp,
    const float *__restrict__ u, int32_t *__restrict__ tok, int32_t *__restrict__ idx_out,
    int64_t ldi, float *__restrict__ val_out, int64_t ldv, float *__restrict__ prob_out,
    int64_t ldp) {
  __shared__ int hist[2][256];  // pass p counts into hist[p % 2]
  __shared__ int iws[4];
  __shared__ float fws[4];
  __shared__ unsigned long long lws[4];
  // kept pairs, in index order (the fast path's candidates, in any order,
  // then zeros up to a whole number of 32-pair blocks)
  __shared__ __attribute__((aligned(16))) unsigned long long sel[kThreads + 32];
  __shared__ unsigned long long srt[kThreads];  // kept pairs, by rank
  __shared__ uint32_t s_digit;
  __shared__ int s_above;
  __shared__ uint32_t xs[4];
  __shared__ int s_count;
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float *row = logits + (int64_t)b * ld;
  const int per = (V + kThreads - 1) / kThreads;  // this thread: [tid * per, tid * per + per)
  const int i0 = tid * per;

  uint32_t kr[REG ? kRegPer : 1];
  if (REG) {
    if (per == kRegPer && i0 + kRegPer <= V) {
      // all 16 inside the row: four 16-byte loads (rows and i0 are
      // 16-byte aligned: the pitch is a multiple of 4 floats)
      const float4 *q = reinterpret_cast<const float4 *>(row + i0);
#pragma unroll
      for (int j = 0; j < kRegPer / 4; ++j) {
        const float4 f = q[j];
        kr[4 * j] = rank_key(f.x);
        kr[4 * j + 1] = rank_key(f.y);
        kr[4 * j + 2] = rank_key(f.z);
        kr[4 * j + 3] = rank_key(f.w);
      }
    } else {
#pragma unroll
      for (int j = 0; j < kRegPer; ++j) {
        const int i = i0 + j;
        kr[j] = j < per && i < V ? rank_key(row[i]) : 0u;
      }
    }
  }
  // f(i, key) for every logit of this thread's span, in index order
  auto each = [&](auto &&f) __attribute__((always_inline)) {
    if (REG) {
#pragma unroll
      for (int j = 0; j < kRegPer; ++j)
        if (j < per && i0 + j < V) f(i0 + j, kr[j]);
    } else {
      const int e = min(i0 + per, V);
      for (int i = i0; i < e; ++i) f(i, rank_key(row[i]));
    }
  };

  // 1. the threshold: this wave's ceil(k/4)-th largest thread maximum
  // (threads without logits hold 0, below every key but a negative NaN's)
  uint32_t v = 0;
  each([&](int, uint32_t key) __attribute__((always_inline)) { v = max(v, key); });
  v = bitonic_steps<2, 1>(v, lane);
  // (cross-lane reads stay outside lane-dependent branches: inside one,
  // the compiler may compute their operands in the branch's lanes only)
  const uint32_t xw = __builtin_amdgcn_readlane(v, ((k + 3) >> 2) - 1);
  if (tid == 0) s_count = 0;
  if (lane == 0) xs[wave] = xw;
  // zeros: a pair that no candidate is below (every kept key is >= 1)
  sel[tid] = 0ull;
  if (tid < 32) sel[kThreads + tid] = 0ull;
  __syncthreads();
  const uint32_t x = min(min(xs[0], xs[1]), min(xs[2], xs[3]));
  // 2. candidates: the pairs of keys >= x, in any order
  {
    int n = 0;
    each([&](int, uint32_t key) __attribute__((always_inline)) { n += key >= x; });
    const int incl = wave_incl_scan(n);
    int base = 0;
    if (lane == 63) base = atomicAdd(&s_count, incl);
    int pos = __shfl(base, 63, 64) + incl - n;
    each([&](int i, uint32_t key) __attribute__((always_inline)) {
      if (key >= x) {
        if (pos < kThreads) sel[pos] = ((unsigned long long)key << 32) | (uint32_t)~(uint32_t)i;
        ++pos;
      }
    });
  }
  __syncthreads();
  const int ncand = s_count;
  if (ncand <= kThreads) {
    if (tid < ncand) {
      const unsigned long long c = sel[tid];
      int r = 0;
      // 32 pairs per round, their 16 reads in flight together (the zeros
      // past ncand count for nothing)
      const ulonglong2 *s2 = reinterpret_cast<const ulonglong2 *>(sel);
      for (int j = 0; j < ncand; j += 32) {
        ulonglong2 p[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) p[u] = s2[(j >> 1) + u];
#pragma unroll
        for (int u = 0; u < 16; ++u) r += (p[u].x > c) + (p[u].y > c);
      }
      if (r < k) srt[r] = c;
    }
    __syncthreads();
  } else {
    // 3. radix select of the k-th largest key.  Pass p counts into hist[p % 2]
    // (cleared during pass p - 1, after every read of pass p - 2); wave 0
    // then finds the digit: lane l holds the counts of digits 255 - 4 l ..
    // 252 - 4 l, and a scan over the lanes gives, for each digit, the number
    // of matching keys whose digit is at least it.
    hist[0][tid] = 0;
    hist[1][tid] = 0;
    __syncthreads();
    uint32_t prefix = 0, pmask = 0;
    int need = k;  // keys still to keep among those matching the prefix
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int sh = 24 - 8 * p;
      int *H = hist[p & 1];
      each([&](int, uint32_t key) __attribute__((always_inline)) {
        if ((key & pmask) == prefix) atomicAdd(&H[(key >> sh) & 255], 1);
      });
      __syncthreads();
      if (wave == 0) {
        const int c0 = H[255 - 4 * lane], c1 = H[254 - 4 * lane], c2 = H[253 - 4 * lane],
                  c3 = H[252 - 4 * lane];
        const int t3 = c0 + c1 + c2 + c3;
        int incl = t3;  // inclusive scan of the lane totals
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int y = __shfl_up(incl, off, 64);
          if (lane >= off) incl += y;
        }
        const int ge0 = incl - t3 + c0, ge1 = ge0 + c1, ge2 = ge1 + c2, ge3 = ge2 + c3;
        // the digit where the count of keys at or above it first reaches need
        if (ge0 >= need && ge0 - c0 < need) { s_digit = 255 - 4 * lane; s_above = ge0 - c0; }
        if (ge1 >= need && ge1 - c1 < need) { s_digit = 254 - 4 * lane; s_above = ge1 - c1; }
        if (ge2 >= need && ge2 - c2 < need) { s_digit = 253 - 4 * lane; s_above = ge2 - c2; }
        if (ge3 >= need && ge3 - c3 < need) { s_digit = 252 - 4 * lane; s_above = ge3 - c3; }
      }
      hist[(p + 1) & 1][tid] = 0;
      __syncthreads();
      prefix |= s_digit << sh;
      pmask |= 0xffu << sh;
      need -= s_above;
    }
    const uint32_t t = prefix;  // the k-th largest key; `need` kept keys equal it

    // compaction: keys above t, then the lowest-index keys equal to t (one
    // scan of both counts, packed in 32-bit halves)
    unsigned long long cnt = 0;
    each([&](int, uint32_t key) __attribute__((always_inline)) {
      cnt += key > t ? (1ull << 32) : (key == t ? 1ull : 0ull);
    });
    unsigned long long tot;
    const unsigned long long ex = block_scan(cnt, lws, &tot) - cnt;
    const int gtot = (int)(tot >> 32);
    int pg = (int)(ex >> 32), pe = (int)(ex & 0xffffffffu);
    each([&](int i, uint32_t key) __attribute__((always_inline)) {
      const unsigned long long c = ((unsigned long long)key << 32) | (uint32_t)~(uint32_t)i;
      if (key > t) {
        sel[pg++] = c;
      } else if (key == t) {
        if (pe < need) sel[gtot + pe] = c;
        ++pe;
      }
    });
    __syncthreads();

    // rank of each kept pair = how many kept pairs are larger (all distinct)
    if (tid < k) {
      const unsigned long long c = sel[tid];
      int r = 0;
      for (int j = 0; j < k; ++j) r += sel[j] > c;
      srt[r] = c;
    }
    __syncthreads();
  }

  // weights, their running sum and the draw
  const unsigned long long mine = tid < k ? srt[tid] : 0ull;
  const float l1 = key_logit((uint32_t)(srt[0] >> 32));
  const float lr = key_logit((uint32_t)(mine >> 32));
  const float e = tid < k ? expf((lr - l1) / temp) : 0.0f;
  float total;
  const float C = block_scan(e, fws, &total);
  const float thr = u[b] * total;
  // #{r < k : C_r <= thr}: a ballot per wave
  const unsigned long long bal = __ballot(tid < k && C <= thr);
  if (lane == 0) iws[wave] = __popcll(bal);
  __syncthreads();
  const int below = ((iws[0] + iws[1]) + iws[2]) + iws[3];
  const int pick = min(below, k - 1);
  if (tid == pick) tok[b] = (int32_t)~(uint32_t)mine;
  if (tid < k) {
    const int32_t ix = (int32_t)~(uint32_t)mine;
    if (idx_out) idx_out[(int64_t)b * ldi + tid] = ix;
    if (val_out) val_out[(int64_t)b * ldv + tid] = lr;
    if (prob_out) prob_out[(int64_t)b * ldp + tid] = e / total;
  }
}

}  // namespace

hipError_t launch_sample_topk(const float *logits, int64_t ld, int64_t B, int64_t V, int64_t k,
                              float temp, const float *u, int32_t *tok, int32_t *idx_out,
                              int64_t ldi, float *val_out, int64_t ldv, float *prob_out,
                              int64_t ldp, hipStream_t st) {
  if (V <= kThreads * kRegPer)
    hipLaunchKernelGGL(topk_sample<true>, dim3((unsigned)B), dim3(kThreads), 0, st, logits, ld,
                       (int)V, (int)k, temp, u, tok, idx_out, ldi, val_out, ldv, prob_out, ldp);
  else
    hipLaunchKernelGGL(topk_sample<false>, dim3((unsigned)B), dim3(kThreads), 0, st, logits, ld,
                       (int)V, (int)k, temp, u, tok, idx_out, ldi, val_out, ldv, prob_out, ldp);
  return hipGetLastError();
}

}  // namespace ug

// Causal attention over a key/value cache (gfx950).
//
// "ultragraph - when the graph is the 1-bit LLM, part 2", section "attention,
// as graph ops": per head, scores = Q K^T / sqrt(d_h), a causal mask,
// A = softmax(scores + mask), ctx = A V.  "ultragraph-1bit 0.12.0" README,
// "A whole ternary GPT": decoding keeps every earlier position's K and V rows
// in a cache, and a cached step gives the same bits as the full forward at
// that position.
//
// A decode step reads the whole cache once (2 * positions * H * d_h * 4
// bytes) for a few hundred flops per key: HBM-bound.  The keys are split in
// chunks of 64 so that one query row still spreads over the chip
// ("flash-decoding"): attn_partial, one wave per (chunk, head, row), computes
// the chunk's score maximum m_c, its sum l_c of exp(score - m_c) and its
// unnormalized context o_c, with no barrier and at most 17 KB of LDS, so
// that a decode step at 4096 positions with 20 heads is 1280 small blocks
// resident at once; every cache load moves 1 KB (16 bytes a lane: 256 / d_h
// rows).  attn_combine rescales the chunks to their common maximum and
// divides (a row of at most 64 chunks, 4096 positions, in one round trip
// for its records).  Every reduction has one fixed order, the same for
// every query row whatever the number of rows in the call, so row t of a
// call over many rows is bit for bit the single-row call at position t:
//   score_j = fl(dot_j / fl(sqrt(d_h))), dot_j = the d_h / 4 partials
//             of dims 4i .. 4i+3 (each the four products added in dim
//             order from +0) added in order of i from +0;
//   m_c     = max over the chunk (exact);
//   p_j     = expf(score_j - m_c);
//   l_c     = the 64 p_j summed by a butterfly (lane l adds lane l ^ h for
//             h = 32, 16, ..., 1: every lane ends with the same bits);
//   o_c[d]  = with R = 256 / d_h rows per 1 KB load: for each r < R the
//             chunk's fl(p_j v_jd) over keys j = r mod R added in key order
//             from +0, then the R sums folded pairwise (sum r takes sum
//             r + R/2, then r + R/4, ...);
//   out[d]  = fl(o[d] / l) with M = max_c m_c, e_c = expf(m_c - M);
//             for w = 0..3, l_w = sum of fl(e_c l_c) and o_w[d] = sum of
//             fl(e_c o_c[d]) over the chunks c = w, w+4, w+8, ... added in
//             that order from +0; l = (l_0 + l_1) + (l_2 + l_3), and o[d]
//             the same way.
#include "ug_internal.h"

namespace ug {
namespace {

constexpr int kChunk = 64;  // keys per partial (one wave)
constexpr int kBatch = 32;  // keys whose loads travel together

template <int DH>
struct AttnDims {
  static constexpr int R = DH >= 64 ? DH / 64 : 1;  // dims per lane in the combine
  static constexpr int kRec = DH + 4;               // floats per partial: o[DH], m, l, pad
  // partials: lane l holds dims 4 (l % LPR) .. + 3 of row l / LPR of a
  // load, which moves RPI key or value rows (1 KB)
  static constexpr int LPR = DH / 4;
  static constexpr int RPI = 64 / LPR;
};

template <int DH>
__global__ __launch_bounds__(64) void attn_partial(const float *__restrict__ q, int64_t ldq,
                                                   const float *__restrict__ kc, int64_t ldk,
                                                   const float *__restrict__ vc, int64_t ldv,
                                                   int pos0, int H, int nck, float root,
                                                   float *__restrict__ part) {
  constexpr int LPR = AttnDims<DH>::LPR, RPI = AttnDims<DH>::RPI;
  const int c = blockIdx.x, h = blockIdx.y, m = blockIdx.z;
  const int p = pos0 + m;  // the row's position: it sees keys 0 .. p
  const int j0 = c * kChunk;
  if (j0 > p) return;  // a chunk wholly after the row's position
  const int nk = min(kChunk, p + 1 - j0);  // keys of the chunk the row sees
  const int lane = threadIdx.x, col = lane % LPR, sub = lane / LPR;

  __shared__ float T[LPR * 65];  // key partials, transposed (odd pitch: no bank conflicts)
  __shared__ float pw[kChunk];

  const float4 q4 = *reinterpret_cast<const float4 *>(q + (int64_t)m * ldq + h * DH + 4 * col);

  // Loads in flight together when d_h <= 128: every key row of the chunk,
  // and the first 32 value rows, which do not depend on the scores.  (With
  // d_h = 256 the registers hold 32 key rows, then 32 value rows.)
  constexpr bool kWide = DH <= 128;
  constexpr int KB = kWide ? kChunk : kBatch;
  const float *kbase = kc + (int64_t)j0 * ldk + h * DH + 4 * col;
  const float *vbase = vc + (int64_t)j0 * ldv + h * DH + 4 * col;
  // row b0 + RPI u + sub of the chunk for u < n (zeros past the keys the row sees)
  auto load_rows = [&](const float *base, int64_t ld, int b0, auto &dst)
                       __attribute__((always_inline)) {
    constexpr int n = sizeof(dst) / sizeof(dst[0]);
#pragma unroll
    for (int u = 0; u < n; ++u) {
      const int j = b0 + RPI * u + sub;
      dst[u] = j < nk ? *reinterpret_cast<const float4 *>(base + (int64_t)j * ld)
                      : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  float4 kv[KB / RPI], vv[kBatch / RPI];
  load_rows(kbase, ldk, 0, kv);
  if (kWide) load_rows(vbase, ldv, 0, vv);

  // Scores: lane l's partial product of its four dims with every key it
  // holds, transposed through LDS so that lane t then adds key t's LPR
  // partials in dimension order.
  for (int b0 = 0; b0 < kChunk; b0 += KB) {
    if (b0 >= nk) break;  // wave-uniform
    if (b0 > 0) load_rows(kbase, ldk, b0, kv);
#pragma unroll
    for (int u = 0; u < KB / RPI; ++u) {
      float a = 0.0f;
      a = a + q4.x * kv[u].x;
      a = a + q4.y * kv[u].y;
      a = a + q4.z * kv[u].z;
      a = a + q4.w * kv[u].w;
      T[col * 65 + b0 + RPI * u + sub] = a;
    }
  }
  __syncthreads();  // (one wave) the transposed partials are in LDS
  float dot = 0.0f;
#pragma unroll 8
  for (int l = 0; l < LPR; ++l) dot = dot + T[l * 65 + lane];
  const bool valid = lane < nk;
  const float s = dot / root;

  // chunk maximum, p_j and l_c
  const float mc = wave_max(valid ? s : -INFINITY);
  const float pj = valid ? expf(s - mc) : 0.0f;
  pw[lane] = pj;
  float lc = pj;
#pragma unroll
  for (int hh = 32; hh >= 1; hh >>= 1) lc = lc + __shfl_xor(lc, hh, 64);
  __syncthreads();  // p_j are in LDS

  // unnormalized context: each lane adds fl(p_j v_jd) over its rows j (those
  // with j % RPI = sub) in increasing j from +0; then the RPI row partials
  // of each dim are folded (lane l takes lane l + f for f = 32, 16, .., LPR)
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int b0 = 0; b0 < kChunk; b0 += kBatch) {
    if (b0 >= nk) break;
    if (b0 > 0 || !kWide) load_rows(vbase, ldv, b0, vv);
#pragma unroll
    for (int u = 0; u < kBatch / RPI; ++u) {
      const int j = b0 + RPI * u + sub;
      if (j < nk) {
        const float w = pw[j];
        o.x = o.x + w * vv[u].x;
        o.y = o.y + w * vv[u].y;
        o.z = o.z + w * vv[u].z;
        o.w = o.w + w * vv[u].w;
      }
    }
  }
#pragma unroll
  for (int f = 32; f >= LPR; f >>= 1) {
    o.x = o.x + __shfl_down(o.x, f, 64);
    o.y = o.y + __shfl_down(o.y, f, 64);
    o.z = o.z + __shfl_down(o.z, f, 64);
    o.w = o.w + __shfl_down(o.w, f, 64);
  }
  float *rec = part + (((int64_t)m * H + h) * nck + c) * AttnDims<DH>::kRec;
  if (lane < LPR) *reinterpret_cast<float4 *>(rec + 4 * col) = o;
  if (lane == 0) {
    rec[DH] = mc;
    rec[DH + 1] = lc;
  }
}

template <int DH>
__global__ __launch_bounds__(256) void attn_combine(const float *__restrict__ part, int pos0,
                                                    int H, int nck, float *__restrict__ out,
                                                    int64_t ldo) {
  constexpr int R = AttnDims<DH>::R, REC = AttnDims<DH>::kRec, NB = 8, NB1 = 16;
  const int h = blockIdx.x, m = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nc = (pos0 + m) / kChunk + 1;
  const float *base = part + ((int64_t)m * H + h) * nck * REC;
  __shared__ float wmax[4], wl[4];
  __shared__ float wo[4][DH];
  float l = 0.0f, o[R];
#pragma unroll
  for (int i = 0; i < R; ++i) o[i] = 0.0f;
  if (nc <= 4 * NB1) {
    // Up to 4 * NB1 chunks: each wave loads all of its records at once (one
    // round trip), and the waves' maxima meet in LDS.  Same order of sums
    // as below.
    float mc[NB1], lc[NB1], oc[NB1][R];
#pragma unroll
    for (int u = 0; u < NB1; ++u) {
      const int c = wave + 4 * u;
      const float *rec = base + (int64_t)min(c, nc - 1) * REC;
      mc[u] = c < nc ? rec[DH] : -INFINITY;
      lc[u] = rec[DH + 1];
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int d = lane + 64 * i;
        oc[u][i] = d < DH ? rec[d] : 0.0f;
      }
    }
    float wm = mc[0];
#pragma unroll
    for (int u = 1; u < NB1; ++u) wm = fmaxf(wm, mc[u]);
    if (lane == 0) wmax[wave] = wm;
    __syncthreads();
    const float mx = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
#pragma unroll
    for (int u = 0; u < NB1; ++u) {
      if (wave + 4 * u < nc) {
        const float e = expf(mc[u] - mx);
        l = l + e * lc[u];
#pragma unroll
        for (int i = 0; i < R; ++i) o[i] = o[i] + e * oc[u][i];
      }
    }
  } else {
    // M = the largest chunk maximum (exact in any order)
    float mx = -INFINITY;
    for (int c = tid; c < nc; c += 256) mx = fmaxf(mx, base[(int64_t)c * REC + DH]);
    mx = wave_max(mx);
    if (lane == 0) wmax[wave] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    // wave w: chunks w, w + 4, ... in increasing order, NB at a time in flight
    for (int c0 = wave; c0 < nc; c0 += 4 * NB) {
      float mc[NB], lc[NB], oc[NB][R];
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int c = c0 + 4 * u;
        const float *rec = base + (int64_t)min(c, nc - 1) * REC;
        mc[u] = rec[DH];
        lc[u] = rec[DH + 1];
#pragma unroll
        for (int i = 0; i < R; ++i) {
          const int d = lane + 64 * i;
          oc[u][i] = d < DH ? rec[d] : 0.0f;
        }
      }
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        if (c0 + 4 * u < nc) {
          const float e = expf(mc[u] - mx);
          l = l + e * lc[u];
#pragma unroll
          for (int i = 0; i < R; ++i) o[i] = o[i] + e * oc[u][i];
        }
      }
    }
  }
  if (lane == 0) wl[wave] = l;
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int d = lane + 64 * i;
    if (d < DH) wo[wave][d] = o[i];
  }
  __syncthreads();
  const float lt = (wl[0] + wl[1]) + (wl[2] + wl[3]);
  float *orow = out + (int64_t)m * ldo + h * DH;
  for (int d = tid; d < DH; d += 256)
    orow[d] = ((wo[0][d] + wo[1][d]) + (wo[2][d] + wo[3][d])) / lt;
}

template <int DH>
hipError_t launch_dh(const float *q, int64_t ldq, const float *kc, int64_t ldk, const float *vc,
                     int64_t ldv, int M, int pos0, int H, float *out, int64_t ldo, float *part,
                     hipStream_t st) {
  const int nck = (pos0 + M + kChunk - 1) / kChunk;
  const float root = sqrtf((float)DH);
  hipLaunchKernelGGL(attn_partial<DH>, dim3(nck, H, M), dim3(64), 0, st, q, ldq, kc, ldk, vc,
                     ldv, pos0, H, nck, root, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_combine<DH>, dim3(H, M), dim3(256), 0, st, part, pos0, H, nck, out, ldo);
  return hipGetLastError();
}

}  // namespace

size_t attention_workspace_bytes(int64_t M, int64_t pos0, int64_t H, int64_t dh) {
  const int64_t nck = ceil_div(pos0 + M, kChunk);
  return (size_t)(4 * M * H * nck * (dh + 4));
}

hipError_t launch_attention(const float *q, int64_t ldq, const float *kc, int64_t ldk,
                            const float *vc, int64_t ldv, int64_t M, int64_t pos0, int64_t H,
                            int64_t dh, float *out, int64_t ldo, float *part, hipStream_t st) {
  const int m = (int)M, p0 = (int)pos0, h = (int)H;
  switch (dh) {
    case 32: return launch_dh<32>(q, ldq, kc, ldk, vc, ldv, m, p0, h, out, ldo, part, st);
    case 64: return launch_dh<64>(q, ldq, kc, ldk, vc, ldv, m, p0, h, out, ldo, part, st);
    case 128: return launch_dh<128>(q, ldq, kc, ldk, vc, ldv, m, p0, h, out, ldo, part, st);
    case 256: return launch_dh<256>(q, ldq, kc, ldk, vc, ldv, m, p0, h, out, ldo, part, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ug

// extern "C" entry points of libug: argument validation, then the kernel
// launches on the caller's stream.  Every argument error is reported before
// anything is launched; no entry point allocates or synchronizes.
#include <cmath>
#include <cstdint>
#include <vector>

#include <cstring>

#include "ug_internal.h"

namespace {

thread_local int32_t g_last_hip_error = 0;

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

inline ug_status hip_status(hipError_t e) {
  if (e == hipSuccess) return UG_OK;
  g_last_hip_error = (int32_t)e;
  return UG_ERR_HIP;
}

// Pointer present and 16-byte aligned.
inline bool ptr_ok(const void *p) { return p != nullptr && aligned16(p); }
// Optional pointer: absent, or 16-byte aligned.
inline bool opt_ok(const void *p) { return p == nullptr || aligned16(p); }
// Optional 4-byte counter.
inline bool counter_ok(const void *p) { return p == nullptr || ((uintptr_t)p & 3u) == 0; }
// A present fp32 scalar/vector (s, beta): 4-byte alignment is enough.
inline bool f32_ok(const void *p) { return p != nullptr && ((uintptr_t)p & 3u) == 0; }

inline bool eps_ok(float e) { return std::isfinite(e) && e > 0.0f; }

// Pitch checks: ld >= cols and a multiple of `mult`.
inline bool pitch_ok(int64_t ld, int64_t cols, int64_t mult) {
  return ld >= cols && ld % mult == 0;
}

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

bool attention_shape_ok(int64_t M, int64_t pos0, int64_t H, int64_t dh) {
  return M >= 1 && pos0 >= 0 && H >= 1 && (dh == 32 || dh == 64 || dh == 128 || dh == 256);
}

// The block table of a plan at `plan`: the first 128-byte boundary after the
// descriptors (plan is 16-byte aligned, so at most 112 bytes of padding).
size_t plan_table_offset(const void *plan, int32_t count) {
  const uintptr_t end = (uintptr_t)plan + (size_t)count * sizeof(ug::GemvDesc);
  return (size_t)(((end + 127) & ~(uintptr_t)127) - (uintptr_t)plan);
}
}  // namespace

extern "C" {

int32_t ug_version(void) { return 10100; }

const char *ug_status_string(ug_status st) {
  switch (st) {
    case UG_OK: return "UG_OK";
    case UG_ERR_INVALID_ARG: return "UG_ERR_INVALID_ARG: invalid pointer, size, pitch, alignment or format";
    case UG_ERR_UNSUPPORTED: return "UG_ERR_UNSUPPORTED: size outside what the exact arithmetic holds";
    case UG_ERR_WORKSPACE: return "UG_ERR_WORKSPACE: workspace missing or too small";
    case UG_ERR_HIP: return "UG_ERR_HIP: HIP launch or runtime error (see ug_last_hip_error)";
    default: return "unknown ug_status";
  }
}

int32_t ug_last_hip_error(void) { return g_last_hip_error; }

ug_status ug_quant_act(const float *x, int64_t ldx, int64_t M, int64_t K, float eps, int8_t *xq,
                       int64_t ldq, float *s, void *stream) {
  if (!ptr_ok(x) || !ptr_ok(xq) || !f32_ok(s)) return UG_ERR_INVALID_ARG;
  if (M < 1 || K < 1 || M > INT32_MAX) return UG_ERR_INVALID_ARG;
  if (!pitch_ok(ldx, K, 4) || !pitch_ok(ldq, K, 16) || !eps_ok(eps)) return UG_ERR_INVALID_ARG;
  return hip_status(ug::launch_quant_act(x, ldx, M, K, eps, xq, ldq, s, as_stream(stream)));
}

ug_status ug_rmsnorm_quant_act(const float *x, int64_t ldx, const float *g, int64_t M, int64_t K,
                               float eps_norm, float eps, int8_t *xq, int64_t ldq, float *s,
                               void *stream) {
  if (!ptr_ok(x) || !opt_ok(g) || !ptr_ok(xq) || !f32_ok(s)) return UG_ERR_INVALID_ARG;
  if (M < 1 || K < 1 || M > INT32_MAX) return UG_ERR_INVALID_ARG;
  if (!pitch_ok(ldx, K, 4) || !pitch_ok(ldq, K, 16)) return UG_ERR_INVALID_ARG;
  if (!eps_ok(eps) || !eps_ok(eps_norm)) return UG_ERR_INVALID_ARG;
  if ((float)K != (double)K) return UG_ERR_UNSUPPORTED;
  return hip_status(ug::launch_rmsnorm_quant_act(x, ldx, g, M, K, eps_norm, eps, xq, ldq, s,
                                                 as_stream(stream)));
}

size_t ug_quant_weight_absmean_workspace_size(int64_t N, int64_t K) {
  if (N < 1 || K < 1 || N > INT64_MAX / K) return 0;
  const int64_t chunks = ug::ceil_div(N * K, ug::kAbsmeanChunk);
  return (size_t)(4 * ug::round_up(chunks, ug::kAbsmeanLanes));
}

ug_status ug_quant_weight_absmean(const float *W, int64_t ldw, int64_t N, int64_t K, float eps,
                                  int8_t *wq, int64_t ldq, float *beta, void *ws,
                                  size_t ws_bytes, void *stream) {
  if (!ptr_ok(W) || !ptr_ok(wq) || !f32_ok(beta)) return UG_ERR_INVALID_ARG;
  if (N < 1 || K < 1 || N > INT64_MAX / K) return UG_ERR_INVALID_ARG;
  if (!pitch_ok(ldw, K, 4) || !pitch_ok(ldq, K, 16) || !eps_ok(eps)) return UG_ERR_INVALID_ARG;
  const int64_t n = N * K;
  if ((double)(float)n != (double)n || n > (INT64_C(1) << 40)) return UG_ERR_UNSUPPORTED;
  if (ug::ceil_div(n, ug::kAbsmeanChunk) > INT32_MAX) return UG_ERR_UNSUPPORTED;
  const size_t need = ug_quant_weight_absmean_workspace_size(N, K);
  if (ws == nullptr || !aligned16(ws) || ws_bytes < need) return UG_ERR_WORKSPACE;
  return hip_status(ug::launch_absmean(W, ldw, N, K, eps, wq, ldq, beta, (float *)ws,
                                       as_stream(stream)));
}

ug_status ug_quant_weight_absmean_pack5(const float *W, int64_t ldw, int64_t N, int64_t K,
                                        float eps, uint8_t *packed, int64_t ldp, float *beta,
                                        void *ws, size_t ws_bytes, void *stream) {
  if (!ptr_ok(W) || !ptr_ok(packed) || !f32_ok(beta)) return UG_ERR_INVALID_ARG;
  if (N < 1 || K < 1 || N > INT64_MAX / K) return UG_ERR_INVALID_ARG;
  if (!pitch_ok(ldw, K, 4) || !pitch_ok(ldp, ug::ceil_div(K, 5), 16) || !eps_ok(eps))
    return UG_ERR_INVALID_ARG;
  const int64_t n = N * K;
  if ((double)(float)n != (double)n || n > (INT64_C(1) << 40)) return UG_ERR_UNSUPPORTED;
  if (ug::ceil_div(n, ug::kAbsmeanChunk) > INT32_MAX) return UG_ERR_UNSUPPORTED;
  const size_t need = ug_quant_weight_absmean_workspace_size(N, K);
  if (ws == nullptr || !aligned16(ws) || ws_bytes < need) return UG_ERR_WORKSPACE;
  return hip_status(ug::launch_absmean_pack5(W, ldw, N, K, eps, packed, ldp, beta, (float *)ws,
                                             as_stream(stream)));
}

ug_status ug_quant_weight_absmean_static(const float *W, int64_t ldw, int64_t N, int64_t K,
                                         float eps, int8_t *wq, int64_t ldq, float *beta,
                                         void *stream) {
  if (!ptr_ok(W) || !ptr_ok(wq) || !f32_ok(beta)) return UG_ERR_INVALID_ARG;
  if (N < 1 || K < 1 || N > INT64_MAX / K) return UG_ERR_INVALID_ARG;
  if (!pitch_ok(ldw, K, 4) || !pitch_ok(ldq, K, 16) || !eps_ok(eps)) return UG_ERR_INVALID_ARG;
  const int64_t n = N * K;
  if ((double)(float)n != (double)n || n > (INT64_C(1) << 40)) return UG_ERR_UNSUPPORTED;
  if (ug::ceil_div(n, ug::kAbsmeanChunk) > ug::kStaticChunks) return UG_ERR_WORKSPACE;
  float *partials = nullptr;
  hipError_t e = ug::static_scratch(&partials);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(ug::launch_absmean(W, ldw, N, K, eps, wq, ldq, beta, partials,
                                       as_stream(stream)));
}

ug_status ug_pack_trits(const int8_t *wq, int64_t ldq, int64_t N, int64_t K, uint8_t *packed,
                        int64_t ldp, int32_t *bad_count, void *stream) {
  if (!ptr_ok(wq) || !ptr_ok(packed) || !counter_ok(bad_count)) return UG_ERR_INVALID_ARG;
  if (N < 1 || K < 1) return UG_ERR_INVALID_ARG;
  if (!pitch_ok(ldq, K, 16) || !pitch_ok(ldp, ug::ceil_div(K, 5), 16)) return UG_ERR_INVALID_ARG;
  return hip_status(ug::launch_pack(wq, ldq, N, K, packed, ldp, bad_count, as_stream(stream)));
}

ug_status ug_unpack_trits(const uint8_t *packed, int64_t ldp, int64_t N, int64_t K, int8_t *wq,
                          int64_t ldq, int32_t *bad_count, void *stream) {
  if (!ptr_ok(wq) || !ptr_ok(packed) || !counter_ok(bad_count)) return UG_ERR_INVALID_ARG;
  if (N < 1 || K < 1) return UG_ERR_INVALID_ARG;
  if (!pitch_ok(ldq, K, 16) || !pitch_ok(ldp, ug::ceil_div(K, 5), 16)) return UG_ERR_INVALID_ARG;
  return hip_status(ug::launch_unpack(packed, ldp, N, K, wq, ldq, bad_count, as_stream(stream)));
}

namespace {

// Shared validation of the two matmul entry points.
ug_status check_matmul(const int8_t *xq, int64_t ldx, const float *s, const void *w, int32_t wfmt,
                       int64_t ldw, const float *beta, const float *bias, int64_t M, int64_t N,
                       int64_t K, const int32_t *acc, int64_t ldacc, const float *y, int64_t ldy) {
  if (!ptr_ok(xq) || !f32_ok(s) || !ptr_ok(w) || !f32_ok(beta)) return UG_ERR_INVALID_ARG;
  if (!opt_ok(bias)) return UG_ERR_INVALID_ARG;
  if (!opt_ok(acc) || !opt_ok(y) || (acc == nullptr && y == nullptr)) return UG_ERR_INVALID_ARG;
  if (M < 1 || N < 1 || K < 1) return UG_ERR_INVALID_ARG;
  if (wfmt != UG_W_I8 && wfmt != UG_W_PACK5) return UG_ERR_INVALID_ARG;
  if (!pitch_ok(ldx, K, 16)) return UG_ERR_INVALID_ARG;
  if (!pitch_ok(ldw, wfmt == UG_W_PACK5 ? ug::ceil_div(K, 5) : K, 16)) return UG_ERR_INVALID_ARG;
  if (acc && !pitch_ok(ldacc, N, 4)) return UG_ERR_INVALID_ARG;
  if (y && !pitch_ok(ldy, N, 4)) return UG_ERR_INVALID_ARG;
  if (K > UG_MAX_K) return UG_ERR_UNSUPPORTED;
  if (M > INT32_MAX / 2 || N > INT32_MAX / 2) return UG_ERR_UNSUPPORTED;
  return UG_OK;
}

}  // namespace

ug_status ug_bitlinear_gemv(const int8_t *xq, int64_t ldx, const float *s, const void *w,
                            int32_t wfmt, int64_t ldw, const float *beta, const float *bias,
                            int64_t M, int64_t N, int64_t K, int32_t *acc, int64_t ldacc, float *y,
                            int64_t ldy, void *stream) {
  ug_status st =
      check_matmul(xq, ldx, s, w, wfmt, ldw, beta, bias, M, N, K, acc, ldacc, y, ldy);
  if (st != UG_OK) return st;
  if (M > UG_GEMV_MAX_M) return UG_ERR_INVALID_ARG;
  // the kernel addresses weights and activations with 32-bit buffer offsets
  if (N * ldw >= (INT64_C(1) << 31) || M * ldx >= (INT64_C(1) << 31)) return UG_ERR_UNSUPPORTED;
  return hip_status(ug::launch_gemv(xq, ldx, s, w, wfmt, ldw, beta, bias, M, N, K, acc, ldacc, y,
                                    ldy, as_stream(stream)));
}

size_t ug_gemv_plan_size(int32_t count) {
  if (count < 1) return 0;
  // descriptors, up to 112 bytes of padding, then the block table at a
  // 128-byte boundary (GemvBlock entries: stream split; FineBlock: fine)
  const size_t entry = std::max(sizeof(ug::GemvBlock), sizeof(ug::FineBlock));
  return (size_t)count * sizeof(ug::GemvDesc) + 112 + ug::kGemvBlocks * entry;
}

ug_status ug_gemv_plan_init(const ug_gemv_problem *problems, int32_t count, void *plan,
                            size_t plan_bytes, ug_gemv_plan_info *info) {
  if (problems == nullptr || info == nullptr || count < 1) return UG_ERR_INVALID_ARG;
  if (plan == nullptr || !aligned16(plan) || plan_bytes < ug_gemv_plan_size(count))
    return UG_ERR_WORKSPACE;
  std::vector<ug::GemvDesc> descs((size_t)count);
  for (int32_t i = 0; i < count; ++i) {
    const ug_gemv_problem &p = problems[i];
    const bool fused = p.x != nullptr;
    const int8_t *xq_in = fused ? (p.xq ? p.xq : (const int8_t *)p.x) : p.xq;
    const float *s_in = fused ? (p.s ? p.s : (const float *)p.x) : p.s;
    const int64_t ldxq = fused && !p.xq ? ug::round_up(p.K, 16) : p.ldxq;
    ug_status st = check_matmul(xq_in, ldxq, s_in, p.w, p.wfmt, p.ldw, p.beta, p.bias, p.M, p.N,
                                p.K, p.acc, p.ldacc, p.y, p.ldy);
    if (st != UG_OK) return st;
    if (p.M > UG_GEMV_MAX_M) return UG_ERR_INVALID_ARG;
    if (fused) {
      if (!ptr_ok(p.x) || !pitch_ok(p.ldx, p.K, 4) || !eps_ok(p.eps)) return UG_ERR_INVALID_ARG;
      if (!ug::gemv_stages_x(p.wfmt, p.M, p.K)) return UG_ERR_UNSUPPORTED;
      if (p.M * p.ldx * 4 >= (INT64_C(1) << 31)) return UG_ERR_UNSUPPORTED;
    }
    if (p.N * p.ldw >= (INT64_C(1) << 31) || p.M * ldxq >= (INT64_C(1) << 31))
      return UG_ERR_UNSUPPORTED;
    ug::GemvDesc d{};
    d.x = p.x;
    d.ldx = p.ldx;
    d.xq = p.xq;
    d.ldxq = p.xq ? p.ldxq : 0;
    d.s = p.s;
    d.w = (const uint8_t *)p.w;
    d.ldw = p.ldw;
    d.beta = p.beta;
    d.bias = p.bias;
    d.acc = p.acc;
    d.ldacc = p.ldacc;
    d.y = p.y;
    d.ldy = p.ldy;
    d.eps = p.eps;
    d.wfmt = p.wfmt;
    d.M = (int32_t)p.M;
    d.N = (int32_t)p.N;
    d.K = (int32_t)p.K;
    descs[(size_t)i] = d;
  }
  // the split (fine or stream), items, and the block table: descriptors
  // first, then kGemvBlocks table entries
  std::vector<ug::GemvBlock> blocks;
  std::vector<ug::FineBlock> fine;
  const int variant = ug::gemv_plan(descs.data(), count, blocks, fine);
  if (variant == -2) return UG_ERR_UNSUPPORTED;
  if (variant < 0) return UG_ERR_INVALID_ARG;
  ug::fine_xcd_order(fine);  // (the grouped kernel takes its block by table position)
  const size_t nblocks = fine.empty() ? blocks.size() : fine.size();
  if (nblocks == 0 || nblocks > (size_t)ug::kGemvBlocks) return UG_ERR_UNSUPPORTED;
  int64_t total_items = 0;
  for (const auto &d : descs) total_items += d.items;
  if (total_items > INT32_MAX) return UG_ERR_UNSUPPORTED;
  std::vector<uint8_t> host(ug_gemv_plan_size(count), 0);
  std::memcpy(host.data(), descs.data(), descs.size() * sizeof(ug::GemvDesc));
  const size_t toff = plan_table_offset(plan, count);
  if (fine.empty())
    std::memcpy(host.data() + toff, blocks.data(), blocks.size() * sizeof(ug::GemvBlock));
  else
    std::memcpy(host.data() + toff, fine.data(), fine.size() * sizeof(ug::FineBlock));
  hipError_t e = hipMemcpy(plan, host.data(), host.size(), hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_status(e);
  info->count = count;
  info->total_items = (int32_t)total_items;
  info->variant = variant;
  info->grid = (int32_t)nblocks;
  return UG_OK;
}

ug_status ug_bitlinear_gemv_grouped(const void *plan, const ug_gemv_plan_info *info,
                                    void *stream) {
  if (plan == nullptr || !aligned16(plan) || info == nullptr) return UG_ERR_INVALID_ARG;
  if (info->count < 1 || info->total_items < 1 || info->grid < 1 ||
      info->grid > ug::kGemvBlocks)
    return UG_ERR_INVALID_ARG;
  // variant = 8192 * spread + 4096 * tiny + 2048 * chunked + 1024 * short +
  // 512 * fused + 256 * fine + 16 * wfmt + mb (short and fused only with
  // fine, tiny only with short, chunked only without fine, spread only with
  // the plain stream split of five-trit weights and one 16-row block)
  const int hi = info->variant >> 8, fine = hi & 1, fmt = (info->variant >> 4) & 15,
            mb = info->variant & 15;
  if (hi > 63 || (fine && (hi & 8)) || (!fine && (hi & 6)) || ((hi & 16) && !(hi & 4)) ||
      ((hi & 32) && (fine || (hi & 8) || fmt != UG_W_PACK5 || mb != 1)) ||
      (fmt != UG_W_I8 && fmt != UG_W_PACK5) || (mb != 1 && mb != 2 && mb != 4) ||
      (fine && mb != 1))
    return UG_ERR_INVALID_ARG;
  const ug::GemvDesc *descs = (const ug::GemvDesc *)plan;
  const void *table = (const char *)plan + plan_table_offset(plan, info->count);
  return hip_status(ug::launch_gemv_grouped(descs, table, info->count, info->grid, info->variant,
                                            as_stream(stream)));
}

size_t ug_bitlinear_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int32_t wfmt) {
  if (M < 1 || N < 1 || K < 1 || (wfmt != UG_W_I8 && wfmt != UG_W_PACK5)) return 0;
  const size_t dec = wfmt == UG_W_PACK5 ? (size_t)(N * ug::round_up(K, 16)) : 0;
  if (M >= 512 && N >= 512) return ug::gemm_split_area_bytes() + dec;
  return dec ? ug::kGemmCounterBytes + dec : 0;
}

namespace {

ug_status gemm_common(const int8_t *xq, int64_t ldx, const float *s, const void *w, int32_t wfmt,
                      int64_t ldw, const float *beta, const float *bias, int64_t M, int64_t N,
                      int64_t K, int32_t *acc, int64_t ldacc, float *y, int64_t ldy, void *ws,
                      size_t ws_bytes, int tile, int splits, void *stream) {
  ug_status st =
      check_matmul(xq, ldx, s, w, wfmt, ldw, beta, bias, M, N, K, acc, ldacc, y, ldy);
  if (st != UG_OK) return st;
  hipStream_t hs = as_stream(stream);
  const size_t dec = wfmt == UG_W_PACK5 ? (size_t)(N * ug::round_up(K, 16)) : 0;
  const size_t cnt = ug::kGemmCounterBytes;
  if (ws != nullptr && !aligned16(ws)) return UG_ERR_WORKSPACE;
  if (wfmt == UG_W_PACK5 && (ws == nullptr || ws_bytes < cnt + dec)) return UG_ERR_WORKSPACE;
  // Layout, decided by the workspace size alone (so that calls of any shape
  // sharing one workspace agree): the first kGemmCounterBytes always belong
  // to the K-split counters.  With room for the whole split area and the
  // decoded weights, the split area starts the workspace and the decoded
  // weights follow it; otherwise the decoded weights follow the counter
  // bytes and no block shares a tile.  Decoded weights never land on a
  // counter word.
  void *split = nullptr;
  size_t dec_off = cnt;
  const size_t area = ug::gemm_split_area_bytes();
  if (ws != nullptr && ws_bytes >= area + dec) {
    split = ws;
    dec_off = area;
  }
  if (wfmt == UG_W_PACK5) {
    const int64_t ldu = ug::round_up(K, 16);
    int8_t *wu = static_cast<int8_t *>(ws) + dec_off;
    hipError_t e = ug::launch_unpack((const uint8_t *)w, ldw, N, K, wu, ldu, nullptr, hs);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(ug::launch_gemm_i8(xq, ldx, s, wu, ldu, beta, bias, M, N, K, acc, ldacc, y,
                                         ldy, split, tile, splits, hs));
  }
  return hip_status(ug::launch_gemm_i8(xq, ldx, s, (const int8_t *)w, ldw, beta, bias, M, N, K,
                                       acc, ldacc, y, ldy, split, tile, splits, hs));
}

}  // namespace

ug_status ug_bitlinear_gemm(const int8_t *xq, int64_t ldx, const float *s, const void *w,
                            int32_t wfmt, int64_t ldw, const float *beta, const float *bias,
                            int64_t M, int64_t N, int64_t K, int32_t *acc, int64_t ldacc, float *y,
                            int64_t ldy, void *ws, size_t ws_bytes, void *stream) {
  return gemm_common(xq, ldx, s, w, wfmt, ldw, beta, bias, M, N, K, acc, ldacc, y, ldy, ws,
                     ws_bytes, -1, -1, stream);
}

ug_status ug_bitlinear_gemm_tiled(const int8_t *xq, int64_t ldx, const float *s, const void *w,
                                  int32_t wfmt, int64_t ldw, const float *beta, const float *bias,
                                  int64_t M, int64_t N, int64_t K, int32_t *acc, int64_t ldacc,
                                  float *y, int64_t ldy, void *ws, size_t ws_bytes, int32_t tile,
                                  int32_t k_splits, void *stream) {
  if (tile < -1 || tile > 1 || k_splits == 0 || k_splits < -1) return UG_ERR_INVALID_ARG;
  return gemm_common(xq, ldx, s, w, wfmt, ldw, beta, bias, M, N, K, acc, ldacc, y, ldy, ws,
                     ws_bytes, tile, k_splits, stream);
}

size_t ug_bitlinear_backward_workspace_size(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || N < 1 || K < 1 || M >= (INT64_C(1) << 21) || N > (INT64_C(1) << 30) ||
      K > (INT64_C(1) << 30))
    return 0;
  return ug::backward_workspace_bytes(M, N, K);
}

ug_status ug_bitlinear_backward(const float *g, int64_t ldg, const float *x, int64_t ldx,
                                const float *W, int64_t ldw, int64_t M, int64_t N, int64_t K,
                                float *dx, int64_t lddx, float *dW, int64_t lddw, float *db,
                                void *ws, size_t ws_bytes, void *stream) {
  if (!ptr_ok(g) || !opt_ok(dx) || !opt_ok(dW) || !opt_ok(db)) return UG_ERR_INVALID_ARG;
  if (dx == nullptr && dW == nullptr && db == nullptr) return UG_ERR_INVALID_ARG;
  if (M < 1 || N < 1 || K < 1) return UG_ERR_INVALID_ARG;
  if (!pitch_ok(ldg, N, 4)) return UG_ERR_INVALID_ARG;
  if (dx && (!ptr_ok(W) || !pitch_ok(ldw, K, 4) || !pitch_ok(lddx, K, 4)))
    return UG_ERR_INVALID_ARG;
  if (dW && (!ptr_ok(x) || !pitch_ok(ldx, K, 4) || !pitch_ok(lddw, K, 4)))
    return UG_ERR_INVALID_ARG;
  // 32-bit tile indices and the column-sum grid
  if (M >= (INT64_C(1) << 21) || N > (INT64_C(1) << 30) || K > (INT64_C(1) << 30))
    return UG_ERR_UNSUPPORTED;
  const size_t need = ug::backward_workspace_bytes(M, N, K);
  if (ws == nullptr || !aligned16(ws) || ws_bytes < need) return UG_ERR_WORKSPACE;
  return hip_status(ug::launch_backward(g, ldg, x, ldx, W, ldw, M, N, K, dx, lddx, dW, lddw, db,
                                        static_cast<float *>(ws), as_stream(stream)));
}

ug_status ug_sample_topk(const float *logits, int64_t ld, int64_t B, int64_t V, int64_t k,
                         float temperature, const float *u, int32_t *tokens, int32_t *topk_index,
                         int64_t ldi, float *topk_logit, int64_t ldl, float *topk_prob,
                         int64_t ldp, void *stream) {
  if (!ptr_ok(logits) || !f32_ok(u) || !counter_ok(tokens) || tokens == nullptr)
    return UG_ERR_INVALID_ARG;
  if (!counter_ok(topk_index) || !counter_ok(topk_logit) || !counter_ok(topk_prob))
    return UG_ERR_INVALID_ARG;
  if (B < 1 || V < 1 || k < 1 || k > V || k > UG_SAMPLE_MAX_K) return UG_ERR_INVALID_ARG;
  if (!pitch_ok(ld, V, 4)) return UG_ERR_INVALID_ARG;
  if ((topk_index && ldi < k) || (topk_logit && ldl < k) || (topk_prob && ldp < k))
    return UG_ERR_INVALID_ARG;
  if (!std::isfinite(temperature) || !(temperature > 0.0f)) return UG_ERR_INVALID_ARG;
  if (B > INT32_MAX || V > INT32_MAX - 256) return UG_ERR_UNSUPPORTED;
  return hip_status(ug::launch_sample_topk(logits, ld, B, V, k, temperature, u, tokens,
                                           topk_index, ldi, topk_logit, ldl, topk_prob, ldp,
                                           as_stream(stream)));
}

ug_status ug_mfma_rate_probe(int32_t kind, int32_t blocks, int32_t iters, int32_t *sink,
                             void *stream) {
  if ((kind != 0 && kind != 1) || blocks < 1 || iters < 1 || !counter_ok(sink) || sink == nullptr)
    return UG_ERR_INVALID_ARG;
  return hip_status(ug::launch_mfma_rate(kind, blocks, iters, sink, as_stream(stream)));
}

ug_status ug_hbm_read_probe(const void *buf, size_t bytes, int32_t blocks, int32_t walk,
                            uint32_t *sink, void *stream) {
  if (buf == nullptr || !aligned16(buf) || bytes == 0 || bytes % 16 != 0 || blocks < 1 ||
      blocks > 65535 || (walk != 0 && walk != 1) || sink == nullptr || !counter_ok(sink))
    return UG_ERR_INVALID_ARG;
  return hip_status(
      ug::launch_hbm_read(buf, (uint64_t)bytes, blocks, walk, sink, as_stream(stream)));
}

size_t ug_attention_workspace_size(int64_t M, int64_t pos0, int64_t H, int64_t dh) {
  if (!attention_shape_ok(M, pos0, H, dh) || pos0 + M > (INT64_C(1) << 24) || H > 65535 ||
      M > 65535)
    return 0;
  return ug::attention_workspace_bytes(M, pos0, H, dh);
}

ug_status ug_attention_cached(const float *q, int64_t ldq, const float *kc, int64_t ldk,
                              const float *vc, int64_t ldv, int64_t M, int64_t pos0, int64_t H,
                              int64_t dh, float *out, int64_t ldo, void *ws, size_t ws_bytes,
                              void *stream) {
  if (!ptr_ok(q) || !ptr_ok(kc) || !ptr_ok(vc) || !ptr_ok(out)) return UG_ERR_INVALID_ARG;
  if (!attention_shape_ok(M, pos0, H, dh)) return UG_ERR_INVALID_ARG;
  if (H > INT64_MAX / dh) return UG_ERR_INVALID_ARG;
  const int64_t HD = H * dh;
  if (!pitch_ok(ldq, HD, 4) || !pitch_ok(ldk, HD, 4) || !pitch_ok(ldv, HD, 4) ||
      !pitch_ok(ldo, HD, 4))
    return UG_ERR_INVALID_ARG;
  // grid dimensions and 32-bit positions
  if (pos0 + M > (INT64_C(1) << 24) || H > 65535 || M > 65535) return UG_ERR_UNSUPPORTED;
  const size_t need = ug::attention_workspace_bytes(M, pos0, H, dh);
  if (ws == nullptr || !aligned16(ws) || ws_bytes < need) return UG_ERR_WORKSPACE;
  return hip_status(ug::launch_attention(q, ldq, kc, ldk, vc, ldv, M, pos0, H, dh, out, ldo,
                                         static_cast<float *>(ws), as_stream(stream)));
}

}  // extern "C"

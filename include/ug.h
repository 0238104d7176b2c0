/*
 * ug.h -- C ABI of libug, the BitLinear forward pass on AMD Instinct MI355X
 * (gfx950): per-token int8 activation quantization, absmean ternary weight
 * quantization, 5-trits-per-byte weight packing, and the int8 x ternary
 * matmul with int32 accumulation and the s*beta rescale.
 *
 * What is computed follows "ultragraph - when the graph is the 1-bit LLM,
 * part 2" (sections "the bytes", "autograd on a byte-graph", "attention, as
 * graph ops") and the "ultragraph-1bit 0.12.0" README (sections "A whole
 * ternary GPT" and "Layout", pack.py).  Every floating-point step is one
 * IEEE-754 binary32 operation, round to nearest even, no FMA contraction,
 * no flush-to-zero; round() is round-half-to-even.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every data pointer is a DEVICE pointer owned by the caller.  The
 *    library keeps no reference after the call returns and never allocates
 *    device memory; scratch comes from a caller workspace whose size a
 *    *_workspace_size() query returns.
 *  - Every call is asynchronous on `stream` (a hipStream_t passed as void*;
 *    NULL is the null stream).  Nothing synchronizes with the host; outputs
 *    are valid once the stream reaches the call.
 *  - Matrices are row-major.  A matrix of R rows with pitch ld occupies
 *    R*ld elements (every row, the last included, owns its full pitch; the
 *    library may READ pad elements [cols, ld) of any row but never writes
 *    them and never lets their values change a result).
 *  - Alignment: every matrix base pointer is 16-byte aligned; the fp32
 *    vectors s and beta and the int32 counters need 4-byte alignment; fp32
 *    and int32 pitches are multiples of 4 elements; int8/uint8 pitches are
 *    multiples of 16 bytes.
 *  - Weights are stored [N][K] (out x in, K contiguous): y = x W^T.
 *  - Scalars s and beta live in device memory, so the quantizers chain into
 *    the matmul without a host round trip.
 *  - Inputs must be finite (NaN/Inf are outside the contract); subnormals
 *    are inside it and are never flushed.
 *  - Errors in the arguments are returned before anything is launched.
 *    Data-dependent problems (bad trits, bad codes) are counted into an
 *    optional caller device counter instead.
 *  - Calls are thread-safe.  The library's mutable state is: a per-thread
 *    copy of the last HIP error; a per-device cache of the compute-unit
 *    count (atomic, filled on first use); and the GEMM's counter of K-split
 *    launches (atomic, seeded at random per process).  None of it changes
 *    a result.
 */
#ifndef UG_H
#define UG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t ug_status;

enum {
    UG_OK = 0,
    UG_ERR_INVALID_ARG = 1, /* null pointer, bad size/pitch/alignment/format */
    UG_ERR_UNSUPPORTED = 2, /* a size the exact arithmetic cannot hold      */
    UG_ERR_WORKSPACE = 3,   /* workspace missing or too small               */
    UG_ERR_HIP = 4          /* a HIP launch/runtime error; see ug_last_hip_error() */
};

/* Weight storage formats. */
enum {
    UG_W_I8 = 0,   /* one trit per byte: int8 two's complement -1, 0, +1
                      ("the bytes": each ternary value in a full byte)     */
    UG_W_PACK5 = 1 /* five trits per byte (README "A whole ternary GPT"):
                      byte g of a row holds K positions 5g..5g+4 as
                      121 + t0 + 3 t1 + 9 t2 + 27 t3 + 81 t4 (t0 = lowest K);
                      trits past K are 0; row bytes [ceil(K/5), ld) are pad.
                      Codes 243..255 are invalid: ug_unpack_trits counts them
                      and writes five 0 trits; the matmuls' results for a
                      row holding one are unspecified (other rows are exact,
                      no access leaves the buffers).                        */
};

/* Largest K the matmuls accept: 127*K < 2^24 keeps (float)acc exact. */
#define UG_MAX_K 132104

/* Largest activation row count of the decode GEMV. */
#define UG_GEMV_MAX_M 64

/* Library version as 10000*major + 100*minor + patch. */
int32_t ug_version(void);

/* Static description of a status code. */
const char *ug_status_string(ug_status st);

/* hipError_t of the last UG_ERR_HIP returned on the calling thread. */
int32_t ug_last_hip_error(void);

/*
 * Per-token (per-row) absmax int8 activation quantization
 * ("the bytes" and "attention, as graph ops": one scale per row):
 *     a_m = max_k |x[m][k]|,   s[m] = fl(fl(a_m / 127) + eps),
 *     xq[m][k] = clamp(rint(fl(x[m][k] / s[m])), -127, 127).
 *  x   fp32 [M][ldx] in;  xq int8 [M][ldq] out;  s fp32 [M] out.
 *  M, K >= 1; ldx >= K; ldq >= K; eps > 0 and finite.
 * Rows are independent: row m's outputs depend only on row m.
 */
ug_status ug_quant_act(const float *x, int64_t ldx, int64_t M, int64_t K,
                       float eps, int8_t *xq, int64_t ldq, float *s,
                       void *stream);

/*
 * RMSNorm with fp32 gain g ("attention, as graph ops") fused with the
 * activation quantizer above.  Per row:
 *     T  = sum_k fl(x_k * x_k), added in the fixed order: element k goes to
 *          slot floor(k/4) mod 256, each slot sums its terms from +0 in
 *          increasing k, then slots fold pairwise (t += t+h, h = 128..1);
 *     r  = sqrt(fl(fl(T / K) + eps_norm))   (correctly rounded);
 *     xn = fl(fl(x_k / r) * g[k])          (g == NULL: xn = fl(x_k / r));
 * then ug_quant_act's steps on xn.  xn itself is not stored.
 *  g fp32 [K] or NULL; eps_norm > 0, eps > 0, finite.
 */
ug_status ug_rmsnorm_quant_act(const float *x, int64_t ldx, const float *g,
                               int64_t M, int64_t K, float eps_norm,
                               float eps, int8_t *xq, int64_t ldq, float *s,
                               void *stream);

/* Bytes of workspace ug_quant_weight_absmean needs for an N x K weight:
 * 4 * ceil(ceil(N*K / 8192) / 256) * 256.  Returns 0 for invalid sizes. */
size_t ug_quant_weight_absmean_workspace_size(int64_t N, int64_t K);

/*
 * Absmean ternary weight quantization ("the bytes"):
 *     T    = sum |W| over all n = N*K elements in the fixed two-stage order:
 *            flatten row-major, split into chunks of 8192 (the last padded
 *            with +0); in chunk c lane t in [0,256) keeps four sums acc_j
 *            and adds element 8192c + 1024i + 4t + j to acc_j for
 *            i = 0..7; lane value fl(fl(acc0+acc1) + fl(acc2+acc3)); lanes
 *            fold pairwise (t += t+h, h = 128..1).  Then lane t sums chunk
 *            sums t, t+256, ... from +0 and the lanes fold the same way;
 *     beta = fl(fl(T / (float)n) + eps)   (written to *beta, device);
 *     wq   = clamp(rint(fl(W / beta)), -1, 1)   (UG_W_I8).
 *  W fp32 [N][ldw] in; wq int8 [N][ldq] out; beta fp32 [1] out;
 *  ws: device workspace of ws_bytes >= the size query.
 *  UG_ERR_UNSUPPORTED if n is not exactly representable in fp32.
 */
ug_status ug_quant_weight_absmean(const float *W, int64_t ldw, int64_t N,
                                  int64_t K, float eps, int8_t *wq,
                                  int64_t ldq, float *beta, void *ws,
                                  size_t ws_bytes, void *stream);

/*
 * Requantization straight to the deployed format: the beta and W_q of
 * ug_quant_weight_absmean (same summation order, same bits), with W_q
 * written as UG_W_PACK5 rows instead of one trit per byte ("ultragraph ...
 * part 2", "training the thing": the fp32 masters are requantized after
 * every optimizer step; README "A whole ternary GPT": deployed weights hold
 * five ternary values per byte).  The bytes equal ug_pack_trits applied to
 * ug_quant_weight_absmean's output: packed uint8 [N][ldp], ldp >= ceil(K/5)
 * and a multiple of 16, row bytes [ceil(K/5), ldp) written as 121.
 * ws as for ug_quant_weight_absmean (the same size query).
 */
ug_status ug_quant_weight_absmean_pack5(const float *W, int64_t ldw, int64_t N,
                                        int64_t K, float eps, uint8_t *packed,
                                        int64_t ldp, float *beta, void *ws,
                                        size_t ws_bytes, void *stream);

/*
 * ug_quant_weight_absmean without a workspace argument and without any
 * allocation: for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  The stage-1 chunk sums go to a static 64 KB array in the
 * library's device code (one per GPU, held until the process ends), so the
 * tensor may hold at most UG_ABSMEAN_STATIC_MAX_ELEMS elements, else
 * UG_ERR_WORKSPACE before anything is launched.  Same arguments, results
 * (bit for bit) and errors as ug_quant_weight_absmean otherwise.  Every
 * call on a GPU shares that GPU's array: calls that overlap in time on one
 * GPU (different streams, or different host threads) race and may return
 * wrong results; serialize them.  The first call on a device looks the
 * array up (hipGetSymbolAddress) and may return UG_ERR_HIP if that fails.
 */
#define UG_ABSMEAN_STATIC_MAX_ELEMS (16384LL * 8192LL)
ug_status ug_quant_weight_absmean_static(const float *W, int64_t ldw,
                                         int64_t N, int64_t K, float eps,
                                         int8_t *wq, int64_t ldq, float *beta,
                                         void *stream);

/*
 * Pack one-trit-per-byte weights into UG_W_PACK5 (README "A whole ternary
 * GPT"; "Layout": pack.py).  wq int8 [N][ldq] in; packed uint8 [N][ldp]
 * out, ldp >= ceil(K/5); bytes [ceil(K/5), ldp) of every row are written as
 * 121.  An entry outside {-1,0,1} is packed as its value clamped to [-1,1]
 * and, if bad_count != NULL, added to *bad_count (device int32, not reset).
 */
ug_status ug_pack_trits(const int8_t *wq, int64_t ldq, int64_t N, int64_t K,
                        uint8_t *packed, int64_t ldp, int32_t *bad_count,
                        void *stream);

/*
 * Inverse of ug_pack_trits: writes wq[n][k] for k < K.  A code above 242
 * among the first ceil(K/5) bytes of a row decodes to five 0 trits and, if
 * bad_count != NULL, is added to *bad_count.  Pad bytes are not read.
 */
ug_status ug_unpack_trits(const uint8_t *packed, int64_t ldp, int64_t N,
                          int64_t K, int8_t *wq, int64_t ldq,
                          int32_t *bad_count, void *stream);

/*
 * Decode GEMV: the integer forward y = (x_q W_q^T)(s beta) + b ("autograd
 * on a byte-graph") for a few activation rows:
 *     acc[m][n] = sum_k xq[m][k] * W_q[n][k]      (int32, exact),
 *     y[m][n]   = fl((float)acc[m][n] * fl(s[m] * beta))          (bias NULL)
 *     y[m][n]   = fl(fl((float)acc[m][n] * fl(s[m] * beta)) + bias[n]).
 *  xq int8 [M][ldx]; s fp32 [M]; beta fp32 [1] (device);
 *  bias fp32 [N] (device, 16-byte aligned) or NULL; acc never includes it;
 *  w: wfmt == UG_W_I8: int8 [N][ldw]; UG_W_PACK5: uint8 [N][ldw] bytes,
 *     ldw >= ceil(K/5);
 *  acc int32 [M][ldacc] out or NULL; y fp32 [M][ldy] out or NULL (not both
 *  NULL).  1 <= M <= UG_GEMV_MAX_M; 1 <= K <= UG_MAX_K.
 */
ug_status ug_bitlinear_gemv(const int8_t *xq, int64_t ldx, const float *s,
                            const void *w, int32_t wfmt, int64_t ldw,
                            const float *beta, const float *bias, int64_t M,
                            int64_t N, int64_t K, int32_t *acc, int64_t ldacc,
                            float *y, int64_t ldy, void *stream);

/*
 * Grouped decode GEMV: several independent ug_bitlinear_gemv problems (for
 * example every matrix of a batch-1 decode pass) in ONE launch, each with
 * its own activations, weights, beta and outputs.  A problem may hand over
 * fp32 activations instead of x_q: then the launch also performs
 * ug_quant_act's per-row absmax quantization of them (same arithmetic, same
 * bits), so quantization + GEMV of the whole group is a single kernel.
 *
 * ug_gemv_problem (host struct; all pointers device pointers):
 *   x, ldx, eps  fp32 [M][ldx] activations to quantize in the launch, or
 *                x == NULL to use xq/s as inputs;
 *   xq, ldxq     int8 [M][ldxq]: input when x == NULL, else optional output
 *                of the quantized activations (NULL: not written);
 *   s            fp32 [M]: input when x == NULL, else optional output;
 *   w, wfmt, ldw, beta, bias, M, N, K, acc, ldacc, y, ldy: as
 *                ug_bitlinear_gemv.
 * Every problem of a group has the same wfmt and the same activation-row
 * class (M <= 16, 17..32 or 33..64).  With x != NULL the quantized rows
 * must fit the kernel's 64 KB staging area: M * Kp <= 65536, else
 * UG_ERR_UNSUPPORTED.  Kp = S * U * ceil(ceil(B / 64) / U) with B the packed
 * row length (ceil(K/5) for UG_W_PACK5, K for UG_W_I8), S = 320 (UG_W_PACK5)
 * or 64 (UG_W_I8), and U the steps per unit of the row class: UG_W_PACK5
 * U = 2, 2, 1 for M <= 16, 17..32, 33..64; UG_W_I8 U = 4, 4, 2.  Rows
 * given as x_q may take up to 80 KB (M * Kp <= 81920); a group in which
 * some problem's x_q rows do not fit that either runs a kernel that takes
 * x_q only; such a group cannot also hold a problem with x != NULL:
 * UG_ERR_UNSUPPORTED (launch those separately).  Weights of
 * N * ldw >= 2^31 bytes or
 * activations of M * ldxq >= 2^31 bytes are UG_ERR_UNSUPPORTED (32-bit
 * offsets), here and in ug_bitlinear_gemv.
 */
typedef struct ug_gemv_problem {
    const float *x;
    int64_t ldx;
    float eps;
    int8_t *xq;
    int64_t ldxq;
    float *s;
    const void *w;
    int32_t wfmt;
    int64_t ldw;
    const float *beta;
    const float *bias;
    int64_t M, N, K;
    int32_t *acc;
    int64_t ldacc;
    float *y;
    int64_t ldy;
} ug_gemv_problem;

/* What the launch needs besides the device plan (filled by plan_init). */
typedef struct ug_gemv_plan_info {
    int32_t count;        /* problems                                  */
    int32_t total_items;  /* work items over all problems              */
    int32_t variant;      /* kernel variant (format and row class)     */
    int32_t grid;         /* blocks to launch                          */
} ug_gemv_plan_info;

/* Device bytes a plan of `count` problems occupies (0 if count < 1). */
size_t ug_gemv_plan_size(int32_t count);

/*
 * Validates `count` host problems, lays out their tiling and copies the
 * plan to the device buffer `plan` (16-byte aligned, >= ug_gemv_plan_size).
 * A set-up call: it blocks until the plan is on the device.  The plan stays
 * valid as long as the buffers it names do, at the address it was written
 * to (its block table sits at a 128-byte boundary inside the buffer, so a
 * copy elsewhere is not a plan); replaying the grouped launch (for example
 * from a captured HIP graph) needs no further host work.
 */
ug_status ug_gemv_plan_init(const ug_gemv_problem *problems, int32_t count,
                            void *plan, size_t plan_bytes,
                            ug_gemv_plan_info *info);

/* One launch of every problem of a plan on `stream`. */
ug_status ug_bitlinear_gemv_grouped(const void *plan,
                                    const ug_gemv_plan_info *info,
                                    void *stream);

/*
 * Bytes of workspace ug_bitlinear_gemm can use: for M, N >= 512 the K-split
 * area (UG_GEMM_SPLIT_AREA bytes), plus, for UG_W_PACK5, N*round_up(K,16)
 * bytes of decoded weights.  Below 512 x 512: 0 for UG_W_I8, and
 * UG_GEMM_COUNTER_BYTES + the decoded bytes for UG_W_PACK5.
 */
size_t ug_bitlinear_gemm_workspace_size(int64_t M, int64_t N, int64_t K,
                                        int32_t wfmt);

/* Size of the K-split area: 2 KB of tile counters, then 256 partial tiles of
 * 256 x 256 int32. */
#define UG_GEMM_COUNTER_BYTES 2048
#define UG_GEMM_SPLIT_AREA (UG_GEMM_COUNTER_BYTES + 256 * 256 * 256 * 4)

/*
 * Prefill GEMM: the same result as ug_bitlinear_gemv (bias included) for
 * any M >= 1, as a dense int8 contraction on the matrix cores (ternary
 * values are exact in int8).  Same arguments, plus the workspace ws (device memory, 16-byte
 * aligned, any contents; NULL allowed for UG_W_I8).  Its first
 * UG_GEMM_COUNTER_BYTES only ever hold K-split tile counters:
 *   - ws_bytes >= UG_GEMM_SPLIT_AREA + decoded bytes: the split area starts
 *     ws and the decoded weights (UG_W_PACK5) follow it.  Problems with few
 *     output tiles may then share a tile's K steps between blocks ("K
 *     split"; integer partial sums, so the result is the same bits).
 *   - otherwise the decoded weights follow the counter bytes and every
 *     block computes whole tiles.
 * UG_ERR_WORKSPACE if UG_W_PACK5 gets less than UG_GEMM_COUNTER_BYTES + the
 * decoded bytes, or ws is misaligned.  Calls that run at the same time must
 * not share a workspace.
 */
ug_status ug_bitlinear_gemm(const int8_t *xq, int64_t ldx, const float *s,
                            const void *w, int32_t wfmt, int64_t ldw,
                            const float *beta, const float *bias, int64_t M,
                            int64_t N, int64_t K, int32_t *acc, int64_t ldacc,
                            float *y, int64_t ldy, void *ws, size_t ws_bytes,
                            void *stream);

/*
 * ug_bitlinear_gemm with the tiling chosen by the caller instead of the
 * library's time model: tile = -1 (model), 0 (256 x 256 output tiles) or 1
 * (256 x 160), and k_splits = -1 (model) or >= 1 K splits per tile.  Both
 * apply to problems of at least 512 x 512 only; a split count that does not
 * fit (more than the K steps, more than 256 blocks, no split area in ws)
 * runs unsplit.  The result is the same bits whatever the tiling.  For
 * tests and tuning.  UG_ERR_INVALID_ARG for other tile or k_splits values.
 */
ug_status ug_bitlinear_gemm_tiled(const int8_t *xq, int64_t ldx, const float *s,
                                  const void *w, int32_t wfmt, int64_t ldw,
                                  const float *beta, const float *bias,
                                  int64_t M, int64_t N, int64_t K,
                                  int32_t *acc, int64_t ldacc, float *y,
                                  int64_t ldy, void *ws, size_t ws_bytes,
                                  int32_t tile, int32_t k_splits, void *stream);

/* Bytes of workspace ug_bitlinear_backward needs on the current device: the
 * larger of 4 * ceil(M / 32) * N (db's chunk sums) and, for each product,
 * 64 KB per piece of the 128 x 128 output tiles it cuts along the
 * contraction (the rem tiles beyond its last whole round of B = 4 x CUs
 * blocks, each in ceil(B / rem) pieces or fewer: under 2B pieces, 128 MB
 * on 256 CUs).  0 for invalid sizes. */
size_t ug_bitlinear_backward_workspace_size(int64_t M, int64_t N, int64_t K);

/*
 * Straight-through backward of the BitLinear layer ("ultragraph ... part
 * 2", "autograd on a byte-graph": the estimator treats the quantizers and
 * the per-row scale as the identity and sends the gradient to the fp32
 * master weights).  With g = dL/dy fp32 [M][ldg] (N used), the layer's
 * fp32 input x [M][ldx] (K used) and the fp32 masters W [N][ldw]:
 *     dx[m][k] = sum_n g[m][n] W[n][k]     (dL/dx = g W),
 *     dW[n][k] = sum_m g[m][n] x[m][k]     (dL/dW = g^T x),
 *     db[n]    = sum_m g[m][n]             (dL/db = sum g).
 *  dx fp32 [M][lddx], dW fp32 [N][lddw], db fp32 [N]: each may be NULL
 *  (not computed; not all three).  x is read only for dW, W only for dx.
 *  Pitches >= the row length and multiples of 4; matrix pointers 16-byte
 *  aligned.  ws: device workspace of ws_bytes >= the size query.
 * Arithmetic: fp32 products and sums on the fp32 matrix cores (dx, dW; the
 * tiles beyond the last whole round of blocks may be computed in pieces
 * along the contraction, added in piece order) and a fixed-order fp32 column sum
 * (db: 32-row chunks added in order, then the chunk sums in order); the
 * same bits on every run on a given device (the cut into pieces depends on
 * the shape and the CU count), each result within the fp32 rounding bound
 * gamma_(n+8) * sum |terms| of the exact sum.  Calls that share ws must not
 * overlap.  UG_ERR_UNSUPPORTED for
 * M >= 2^21 or N, K > 2^30.
 */
ug_status ug_bitlinear_backward(const float *g, int64_t ldg, const float *x,
                                int64_t ldx, const float *W, int64_t ldw,
                                int64_t M, int64_t N, int64_t K, float *dx,
                                int64_t lddx, float *dW, int64_t lddw,
                                float *db, void *ws, size_t ws_bytes,
                                void *stream);

/* Largest k of ug_sample_topk. */
#define UG_SAMPLE_MAX_K 256

/*
 * Top-k sampling of the next token, one row of logits per sequence ("a
 * 1-bit llm, from scratch", "the interesting bit": the next token comes from
 * the k largest logits, found without sorting the vocabulary; README "A
 * whole ternary GPT": generate() with temperature and top_k).  Per row b:
 *   rank the V logits, larger first, equal values (-0 == +0) by lower index;
 *   keep ranks 1..k; weight rank r by e_r = expf(fl(fl(l_r - l_1) / T));
 *   C_r = e_1 + ... + e_r (fp32, one fixed order);
 *   tokens[b] = the index of rank min(#{r : C_r <= fl(u[b] * C_k)}, k - 1)
 *   (the first rank whose running weight exceeds u[b] times the total).
 *  logits fp32 [B][ld] (16-byte aligned, ld >= V, ld % 4 == 0);
 *  u fp32 [B] uniform draws in [0, 1), supplied by the caller;
 *  tokens int32 [B] out;  optional outputs (NULL: not written), row pitch
 *  >= k: topk_index int32 [B][ldi] (the kept indices in rank order),
 *  topk_logit fp32 [B][ldl] (their logits), topk_prob fp32 [B][ldp]
 *  (e_r / C_k).  1 <= k <= min(V, UG_SAMPLE_MAX_K); T > 0 and finite.
 * Logits must be finite.  Which indices are kept, and their order, is exact
 * (comparisons only); the draw depends on expf and fp32 sums, so a u within
 * a few ulps of a boundary C_r / C_k may land on either neighbouring rank.
 */
ug_status ug_sample_topk(const float *logits, int64_t ld, int64_t B, int64_t V,
                         int64_t k, float temperature, const float *u,
                         int32_t *tokens, int32_t *topk_index, int64_t ldi,
                         float *topk_logit, int64_t ldl, float *topk_prob,
                         int64_t ldp, void *stream);

/* Bytes of workspace ug_attention_cached needs:
 * 4 * M * H * ceil((pos0 + M) / 64) * (dh + 4).  0 for invalid shapes. */
size_t ug_attention_workspace_size(int64_t M, int64_t pos0, int64_t H,
                                   int64_t dh);

/*
 * Causal multi-head attention of M query rows over a key/value cache
 * ("ultragraph ... part 2", "attention, as graph ops": per head,
 * scores = Q K^T / sqrt(d_h), a causal mask, A = softmax(scores + mask),
 * ctx = A V; README "A whole ternary GPT": decoding keeps the earlier
 * positions' K and V rows in a cache).  Query row m is at position
 * p = pos0 + m and attends to cache rows 0 .. p; head h uses columns
 * h*dh .. h*dh + dh - 1 of q, kc, vc and out.  A decode step is M = 1 with
 * pos0 = the new token's position (its K and V rows already in the cache);
 * a full forward over T tokens is M = T, pos0 = 0.
 *  q   fp32 [M][ldq];  kc, vc fp32 [pos0 + M][ldk / ldv] (rows past the
 *      last query's position are not read);  out fp32 [M][ldo];
 *  dh in {32, 64, 128, 256}; every pitch >= H*dh, a multiple of 4;
 *  ws: device workspace of ws_bytes >= ug_attention_workspace_size.
 * Arithmetic: fp32 with one fixed reduction order for every row whatever
 * M is, so row m equals, bit for bit, the call with M = 1 at position
 * pos0 + m (cached decoding reproduces the full forward); exp is the
 * device's expf.  UG_ERR_UNSUPPORTED if pos0 + M > 2^24, H > 65535 or
 * M > 65535.  Inputs must be finite.
 */
ug_status ug_attention_cached(const float *q, int64_t ldq, const float *kc,
                              int64_t ldk, const float *vc, int64_t ldv,
                              int64_t M, int64_t pos0, int64_t H, int64_t dh,
                              float *out, int64_t ldo, void *ws,
                              size_t ws_bytes, void *stream);

/*
 * Measurement helper beside the forward path (not a step of it): the rate
 * the matrix cores sustain when every CU runs them.  Launches `blocks`
 * blocks of four waves (one per SIMD; blocks = the CU count loads every
 * CU once); each wave issues iters x 16 back-to-back matrix instructions on
 * register operands that change from one instruction to the next, with no
 * memory traffic:
 *   kind 0: v_mfma_i32_32x32x32_i8 (65536 int8 ops each),
 *   kind 1: v_mfma_f32_16x16x4f32 (2048 fp32 flops each).
 * Each wave writes one int32 derived from its accumulators to sink[w]
 * (device memory, 4 * blocks words), which keeps every instruction in the
 * program.  The caller times the call on `stream`: the sustained rate is
 * 4 * blocks * iters * 16 * (ops per instruction) / time.
 * UG_ERR_INVALID_ARG for another kind, blocks < 1, iters < 1 or a sink
 * that is NULL or not 4-byte aligned.
 */
ug_status ug_mfma_rate_probe(int32_t kind, int32_t blocks, int32_t iters,
                             int32_t *sink, void *stream);

/*
 * Measurement helper beside the forward path (not a step of it): the rate
 * a plain streaming read reaches on this GPU, the measured ceiling for the
 * bandwidth-bound kernels.  Reads the `bytes` bytes at `buf` (device
 * memory, 16-byte aligned, bytes a positive multiple of 16) once, with
 * `blocks` blocks of four waves walking its 16-byte words (every load
 * instruction of a wave reads 1 KB contiguous, eight in flight per thread):
 * walk 0, one grid stride over the whole buffer; walk 1, block b reads the
 * b-th of `blocks` contiguous ranges.  Writes to sink (device memory,
 * 4 * blocks uint32 words) one word per wave such that the XOR of all sink
 * words is the XOR of every 32-bit word of the buffer.  The caller times
 * the call on `stream`: the read rate is bytes / time.  UG_ERR_INVALID_ARG
 * for a NULL or misaligned pointer, bytes not a positive multiple of 16,
 * blocks outside [1, 65535] or another walk.
 */
ug_status ug_hbm_read_probe(const void *buf, size_t bytes, int32_t blocks, int32_t walk,
                            uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* UG_H */

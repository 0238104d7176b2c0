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
 *  - Calls are thread-safe: the library holds no mutable global state
 *    except a per-thread copy of the last HIP error.
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
 * Decode GEMV: the integer forward y = (x_q W_q^T)(s beta) ("autograd on a
 * byte-graph", no bias) for a few activation rows:
 *     acc[m][n] = sum_k xq[m][k] * W_q[n][k]      (int32, exact),
 *     y[m][n]   = fl((float)acc[m][n] * fl(s[m] * beta)).
 *  xq int8 [M][ldx]; s fp32 [M]; beta fp32 [1] (device);
 *  w: wfmt == UG_W_I8: int8 [N][ldw]; UG_W_PACK5: uint8 [N][ldw] bytes,
 *     ldw >= ceil(K/5);
 *  acc int32 [M][ldacc] out or NULL; y fp32 [M][ldy] out or NULL (not both
 *  NULL).  1 <= M <= UG_GEMV_MAX_M; 1 <= K <= UG_MAX_K.
 */
ug_status ug_bitlinear_gemv(const int8_t *xq, int64_t ldx, const float *s,
                            const void *w, int32_t wfmt, int64_t ldw,
                            const float *beta, int64_t M, int64_t N,
                            int64_t K, int32_t *acc, int64_t ldacc, float *y,
                            int64_t ldy, void *stream);

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
 *   w, wfmt, ldw, beta, M, N, K, acc, ldacc, y, ldy: as ug_bitlinear_gemv.
 * Every problem of a group has the same wfmt and the same activation-row
 * class (M <= 16, 17..32 or 33..64).  With x != NULL the quantized rows
 * must fit the kernel's 64 KB staging area: M * Kp <= 65536, else
 * UG_ERR_UNSUPPORTED.  Kp = S * U * ceil(ceil(B / 64) / U) with B the packed
 * row length (ceil(K/5) for UG_W_PACK5, K for UG_W_I8), S = 320 (UG_W_PACK5)
 * or 64 (UG_W_I8), and U the steps per unit of the row class: UG_W_PACK5
 * U = 2, 2, 1 for M <= 16, 17..32, 33..64; UG_W_I8 U = 4, 4, 2.  Weights of N * ldw >= 2^31 bytes or
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
 * bytes of decoded weights.  0 for UG_W_I8 below 512 x 512.
 */
size_t ug_bitlinear_gemm_workspace_size(int64_t M, int64_t N, int64_t K,
                                        int32_t wfmt);

/* Size of the K-split area: 2 KB of tile counters, then 256 partial tiles of
 * 256 x 256 int32. */
#define UG_GEMM_SPLIT_AREA (2048 + 256 * 256 * 256 * 4)

/*
 * Prefill GEMM: the same result as ug_bitlinear_gemv for any M >= 1, as a
 * dense int8 contraction on the matrix cores (ternary values are exact in
 * int8).  Same arguments, plus the workspace ws (device memory, 16-byte
 * aligned, any contents; NULL allowed for UG_W_I8):
 *   - ws_bytes >= UG_GEMM_SPLIT_AREA + decoded bytes: the split area starts
 *     ws and the decoded weights (UG_W_PACK5) follow it.  Problems with few
 *     output tiles may then share a tile's K steps between blocks ("K
 *     split"; integer partial sums, so the result is the same bits).
 *   - otherwise the decoded weights start ws and every block computes whole
 *     tiles.
 * UG_ERR_WORKSPACE if UG_W_PACK5 gets less than the decoded bytes or ws is
 * misaligned.  Calls that run at the same time must not share a workspace.
 */
ug_status ug_bitlinear_gemm(const int8_t *xq, int64_t ldx, const float *s,
                            const void *w, int32_t wfmt, int64_t ldw,
                            const float *beta, int64_t M, int64_t N,
                            int64_t K, int32_t *acc, int64_t ldacc, float *y,
                            int64_t ldy, void *ws, size_t ws_bytes,
                            void *stream);

#ifdef __cplusplus
}
#endif

#endif /* UG_H */

/*
 * ugref -- the CPU oracle for the BitLinear forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or
 * calls this file; only the tests, the smoke check and the benchmark's CPU
 * baseline do.  It shares no code, header, table or helper with the HIP
 * library: everything below is written out as plain scalar loops so that a
 * reader can check it against the pages by eye.
 *
 * Sources (the pages are the authority on what is computed):
 *   - "ultragraph - when the graph is the 1-bit LLM, part 2", section
 *     "the bytes": absmean ternary weight quantization (beta = mean|W| + eps,
 *     W_q = clip(round(W/beta), -1, 1)), dequantization as one scalar
 *     multiply, and per-row absmax int8 activation quantization
 *     (s = max|x|/127 + eps, x_q = clip(round(x/s), -127, 127)), with the
 *     symmetric range [-127, 127].
 *   - same page, section "autograd on a byte-graph": the integer forward
 *     y = (x_q W_q^T)(s beta) + b (the bias optional).
 *   - same page, section "attention, as graph ops": RMSNorm with a learnable
 *     fp32 gain, and the per-token (per-row) scale.
 *   - "ultragraph-1bit 0.12.0" README, sections "A whole ternary GPT" and
 *     "Layout" (pack.py): weights stored 5 ternary values per byte.
 *
 * Readings where the pages leave a step open (each is listed in the design
 * document):
 *   - every floating-point step is one IEEE-754 binary32 operation with
 *     round-to-nearest-even; no FMA contraction (built with
 *     -ffp-contract=off), no flush-to-zero;
 *   - round() is round-half-to-even (rintf in the default rounding mode);
 *   - s = fl(fl(a / 127) + eps) and beta = fl(fl(T / n) + eps), divisions
 *     correctly rounded, never a reciprocal multiply;
 *   - the whole-tensor sum of |W| and the per-row sum of squares are
 *     added in the fixed orders spelled out at absmean_sum() and
 *     rmsnorm_row() below;
 *   - the 5-trits-per-byte code of trits t_0..t_4 (t_0 at the lowest K) is
 *     121 + sum_j t_j 3^j; trits past K are 0; row bytes past ceil(K/5) are
 *     121; codes 243..255 are invalid and decode to five zero trits;
 *   - y = fl((float)acc * fl(s * beta)), plus fl(. + b[n]) with a bias.
 *
 * OpenMP runs only over independent rows or independent chunks, so every
 * result is bit-identical at any thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

/* ------------------------------------------------------------------ */
/* Activation quantization (per-token absmax)                           */
/* ------------------------------------------------------------------ */

/* One row: a = max|x_k|; s = fl(fl(a/127) + eps);
 * x_q[k] = clamp(rint(fl(x_k / s)), -127, 127). */
static float quant_act_row(const float *x, int64_t K, float eps, int8_t *xq)
{
    float a = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
        float v = fabsf(x[k]);
        if (v > a)
            a = v;
    }
    float a_over = a / 127.0f;
    float s = a_over + eps;
    for (int64_t k = 0; k < K; ++k) {
        float q = x[k] / s;
        float r = rintf(q);
        if (r > 127.0f)
            r = 127.0f;
        if (r < -127.0f)
            r = -127.0f;
        xq[k] = (int8_t)r;
    }
    return s;
}

void ugref_quant_act(const float *x, int64_t ldx, int64_t M, int64_t K,
                     float eps, int8_t *xq, int64_t ldq, float *s)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        s[m] = quant_act_row(x + m * ldx, K, eps, xq + m * ldq);
}

/* ------------------------------------------------------------------ */
/* RMSNorm (fp32 gain) feeding the activation quantizer                */
/* ------------------------------------------------------------------ */

/* Sum of squares of one row in the fixed order used throughout:
 * element k belongs to slot t = floor(k/4) mod 256; each slot adds its
 * fl(x_k * x_k) from +0 in increasing k; then the 256 slots are folded
 * pairwise, slot t += slot t+h for h = 128, 64, ..., 1. */
static float row_sum_squares(const float *x, int64_t K)
{
    float p[256];
    for (int t = 0; t < 256; ++t)
        p[t] = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
        int t = (int)((k / 4) % 256);
        float sq = x[k] * x[k];
        p[t] = p[t] + sq;
    }
    for (int h = 128; h >= 1; h /= 2)
        for (int t = 0; t < h; ++t)
            p[t] = p[t] + p[t + h];
    return p[0];
}

/* RMSNorm(x) = x / sqrt(mean(x^2) + eps_n) * g, with
 * ms = fl(T / K), r = sqrt(fl(ms + eps_n)) correctly rounded,
 * x_n = fl(fl(x / r) * g).  g == NULL means a gain of ones. */
static void rmsnorm_row(const float *x, const float *g, int64_t K,
                        float eps_n, float *xn)
{
    float T = row_sum_squares(x, K);
    float ms = T / (float)K;
    float r = sqrtf(ms + eps_n);
    for (int64_t k = 0; k < K; ++k) {
        float v = x[k] / r;
        xn[k] = g ? v * g[k] : v;
    }
}

void ugref_rmsnorm(const float *x, int64_t ldx, const float *g, int64_t M,
                   int64_t K, float eps_n, float *xn, int64_t ldn)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        rmsnorm_row(x + m * ldx, g, K, eps_n, xn + m * ldn);
}

float ugref_row_sum_squares(const float *x, int64_t K)
{
    return row_sum_squares(x, K);
}

void ugref_rmsnorm_quant_act(const float *x, int64_t ldx, const float *g,
                             int64_t M, int64_t K, float eps_n, float eps,
                             int8_t *xq, int64_t ldq, float *s)
{
#pragma omp parallel
    {
        float *xn = (float *)malloc((size_t)(K > 0 ? K : 1) * sizeof(float));
#pragma omp for schedule(static)
        for (int64_t m = 0; m < M; ++m) {
            rmsnorm_row(x + m * ldx, g, K, eps_n, xn);
            s[m] = quant_act_row(xn, K, eps, xq + m * ldq);
        }
        free(xn);
    }
}

/* ------------------------------------------------------------------ */
/* Absmean ternary weight quantization                                 */
/* ------------------------------------------------------------------ */

#define UGREF_CHUNK 8192

/* |W| of flat element e of the row-major [N, K] matrix (pitch ldw);
 * elements at or past n = N*K are +0. */
static float abs_at(const float *W, int64_t ldw, int64_t K, int64_t n,
                    int64_t e)
{
    if (e >= n)
        return 0.0f;
    int64_t row = e / K, col = e % K;
    return fabsf(W[row * ldw + col]);
}

/* Stage 1 of the fixed summation order: chunk c holds flat elements
 * [8192c, 8192c + 8192).  Lane t in [0,256) keeps four running sums
 * acc_j, j in [0,4); for i = 0..7 it adds element 8192c + 1024i + 4t + j
 * to acc_j.  Lane t's value is fl(fl(acc_0+acc_1) + fl(acc_2+acc_3));
 * the 256 lane values are folded pairwise (t += t+h, h = 128..1). */
static float chunk_sum(const float *W, int64_t ldw, int64_t K, int64_t n,
                       int64_t c)
{
    float p[256];
    for (int t = 0; t < 256; ++t) {
        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int i = 0; i < 8; ++i)
            for (int j = 0; j < 4; ++j) {
                int64_t e = c * UGREF_CHUNK + 1024 * (int64_t)i + 4 * t + j;
                acc[j] = acc[j] + abs_at(W, ldw, K, n, e);
            }
        float lo = acc[0] + acc[1];
        float hi = acc[2] + acc[3];
        p[t] = lo + hi;
    }
    for (int h = 128; h >= 1; h /= 2)
        for (int t = 0; t < h; ++t)
            p[t] = p[t] + p[t + h];
    return p[0];
}

/* Stage 2: lane t in [0,256) adds the chunk sums t, t+256, t+512, ...
 * from +0 in that order; the lanes are folded pairwise as above. */
static float combine_chunks(const float *S, int64_t nchunks)
{
    float p[256];
    for (int t = 0; t < 256; ++t) {
        float acc = 0.0f;
        for (int64_t c = t; c < nchunks; c += 256)
            acc = acc + S[c];
        p[t] = acc;
    }
    for (int h = 128; h >= 1; h /= 2)
        for (int t = 0; t < h; ++t)
            p[t] = p[t] + p[t + h];
    return p[0];
}

/* T = sum |W| over the whole N x K tensor in the order above.  The
 * per-chunk sums are also returned through S when S is not NULL. */
float ugref_absmean_sum(const float *W, int64_t ldw, int64_t N, int64_t K,
                        float *S_out)
{
    int64_t n = N * K;
    int64_t nchunks = (n + UGREF_CHUNK - 1) / UGREF_CHUNK;
    float *S = (float *)malloc((size_t)(nchunks > 0 ? nchunks : 1) * sizeof(float));
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < nchunks; ++c)
        S[c] = chunk_sum(W, ldw, K, n, c);
    float T = combine_chunks(S, nchunks);
    if (S_out)
        for (int64_t c = 0; c < nchunks; ++c)
            S_out[c] = S[c];
    free(S);
    return T;
}

/* beta = fl(fl(T / (float)n) + eps);
 * W_q = clamp(rint(fl(W / beta)), -1, 1), one byte per trit. */
void ugref_quant_weight_absmean(const float *W, int64_t ldw, int64_t N,
                                int64_t K, float eps, int8_t *wq, int64_t ldq,
                                float *beta_out)
{
    float T = ugref_absmean_sum(W, ldw, N, K, NULL);
    float mean = T / (float)(N * K);
    float beta = mean + eps;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < N; ++r)
        for (int64_t k = 0; k < K; ++k) {
            float q = W[r * ldw + k] / beta;
            float t = rintf(q);
            if (t > 1.0f)
                t = 1.0f;
            if (t < -1.0f)
                t = -1.0f;
            wq[r * ldq + k] = (int8_t)t;
        }
    *beta_out = beta;
}

/* ------------------------------------------------------------------ */
/* Five trits per byte                                                 */
/* ------------------------------------------------------------------ */

/* Row n, byte g holds the trits of K positions 5g .. 5g+4:
 * code = 121 + t_0 + 3 t_1 + 9 t_2 + 27 t_3 + 81 t_4 (trits past K are 0).
 * Bytes g in [ceil(K/5), ldp) are 121.  An entry outside {-1,0,1} is
 * counted and packed as its value clamped to [-1, 1].  Returns the count. */
int64_t ugref_pack_trits(const int8_t *wq, int64_t ldq, int64_t N, int64_t K,
                         uint8_t *packed, int64_t ldp)
{
    int64_t groups = (K + 4) / 5;
    int64_t bad = 0;
#pragma omp parallel for schedule(static) reduction(+ : bad)
    for (int64_t r = 0; r < N; ++r) {
        for (int64_t g = 0; g < ldp; ++g) {
            int code = 121;
            if (g < groups) {
                int pow3 = 1;
                for (int j = 0; j < 5; ++j) {
                    int64_t k = 5 * g + j;
                    int t = 0;
                    if (k < K) {
                        t = wq[r * ldq + k];
                        if (t < -1 || t > 1) {
                            ++bad;
                            t = t < -1 ? -1 : 1;
                        }
                    }
                    code += t * pow3;
                    pow3 *= 3;
                }
            }
            packed[r * ldp + g] = (uint8_t)code;
        }
    }
    return bad;
}

/* Inverse of ugref_pack_trits for the first K positions of each row.
 * A code above 242 among the first ceil(K/5) bytes of a row is counted and
 * decodes to five zero trits.  Returns the count. */
int64_t ugref_unpack_trits(const uint8_t *packed, int64_t ldp, int64_t N,
                           int64_t K, int8_t *wq, int64_t ldq)
{
    int64_t groups = (K + 4) / 5;
    int64_t bad = 0;
#pragma omp parallel for schedule(static) reduction(+ : bad)
    for (int64_t r = 0; r < N; ++r) {
        for (int64_t g = 0; g < groups; ++g) {
            int code = packed[r * ldp + g];
            if (code > 242) {
                ++bad;
                code = 121;
            }
            int digits = code; /* base-3 digits d_j = t_j + 1 */
            for (int j = 0; j < 5; ++j) {
                int64_t k = 5 * g + j;
                int d = digits % 3;
                digits /= 3;
                if (k < K)
                    wq[r * ldq + k] = (int8_t)(d - 1);
            }
        }
    }
    return bad;
}

/* ------------------------------------------------------------------ */
/* Integer matmul and the rescale                                      */
/* ------------------------------------------------------------------ */

/* acc[m][n] = sum_k x_q[m][k] * W_q[n][k], exact in integers. */
void ugref_matmul_i32(const int8_t *xq, int64_t ldx, const int8_t *wq,
                      int64_t ldw, int64_t M, int64_t N, int64_t K,
                      int32_t *acc, int64_t ldacc)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            int64_t sum = 0;
            for (int64_t k = 0; k < K; ++k)
                sum += (int64_t)xq[m * ldx + k] * (int64_t)wq[n * ldw + k];
            acc[m * ldacc + n] = (int32_t)sum;
        }
}

/* The same sums for a list of (m, n) pairs only. */
void ugref_matmul_i32_pairs(const int8_t *xq, int64_t ldx, const int8_t *wq,
                            int64_t ldw, int64_t K, const int64_t *mi,
                            const int64_t *ni, int64_t count, int32_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < count; ++p) {
        int64_t sum = 0;
        for (int64_t k = 0; k < K; ++k)
            sum += (int64_t)xq[mi[p] * ldx + k] * (int64_t)wq[ni[p] * ldw + k];
        out[p] = (int32_t)sum;
    }
}

/* y[m][n] = fl((float)acc[m][n] * fl(s[m] * beta)), then, with a bias,
 * y[m][n] = fl(that + b[n]): the deployed forward y = (x_q W_q^T)(s beta) + b
 * ("autograd on a byte-graph"), rescale first, one rounding per operation.
 * b == NULL: no bias. */
void ugref_epilogue(const int32_t *acc, int64_t ldacc, const float *s,
                    float beta, const float *b, int64_t M, int64_t N, float *y,
                    int64_t ldy)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        float scale = s[m] * beta;
        for (int64_t n = 0; n < N; ++n) {
            float v = (float)acc[m * ldacc + n] * scale;
            if (b)
                v = v + b[n];
            y[m * ldy + n] = v;
        }
    }
}

/* ------------------------------------------------------------------ */
/* Causal attention over a key/value cache                             */
/* ------------------------------------------------------------------ */

/* "ultragraph - when the graph is the 1-bit LLM, part 2", section
 * "attention, as graph ops": per head h (columns h*dh .. h*dh+dh-1 of
 * q, K, V), scores = Q K^T / sqrt(d_h), a causal mask that removes keys
 * after the query's position, A = softmax(scores + mask), ctx = A V.
 * "ultragraph-1bit 0.12.0" README, "A whole ternary GPT": decoding keeps
 * every earlier position's K and V rows in a cache.
 *
 * Query row m sits at position p = pos0 + m and sees cache rows 0..p.
 * Computed in double precision straight from the definition (the exact
 * softmax up to double rounding), rounded to fp32 once at the end. */
void ugref_attention(const float *q, int64_t ldq, const float *kc, int64_t ldk,
                     const float *vc, int64_t ldv, int64_t M, int64_t pos0,
                     int64_t H, int64_t dh, float *out, int64_t ldo)
{
#pragma omp parallel for schedule(dynamic) collapse(2)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t h = 0; h < H; ++h) {
            int64_t n = pos0 + m + 1; /* keys 0 .. pos0 + m */
            double *sc = (double *)malloc((size_t)n * sizeof(double));
            const float *qr = q + m * ldq + h * dh;
            double root = sqrt((double)dh);
            double mx = -INFINITY;
            for (int64_t j = 0; j < n; ++j) {
                const float *kr = kc + j * ldk + h * dh;
                double dot = 0.0;
                for (int64_t d = 0; d < dh; ++d)
                    dot += (double)qr[d] * (double)kr[d];
                sc[j] = dot / root;
                if (sc[j] > mx)
                    mx = sc[j];
            }
            double sum = 0.0;
            for (int64_t j = 0; j < n; ++j) {
                sc[j] = exp(sc[j] - mx);
                sum += sc[j];
            }
            for (int64_t d = 0; d < dh; ++d) {
                double o = 0.0;
                for (int64_t j = 0; j < n; ++j)
                    o += sc[j] * (double)vc[j * ldv + h * dh + d];
                out[m * ldo + h * dh + d] = (float)(o / sum);
            }
            free(sc);
        }
}

/* ------------------------------------------------------------------ */
/* Top-k sampling                                                      */
/* ------------------------------------------------------------------ */

/* "a 1-bit llm, from scratch", section "the interesting bit": the next
 * token is drawn from the k largest logits (the page keeps them in a size-k
 * min-heap instead of sorting the whole vocabulary); "ultragraph-1bit
 * 0.12.0" README, "A whole ternary GPT": generate() takes a temperature and
 * top_k.  Reading: rank the logits by value, larger first, equal values by
 * lower index; keep ranks 1..k; weight rank r by exp((l_r - l_1) / T) (the
 * softmax with temperature T over the kept logits); with the caller's
 * uniform u in [0, 1), the token is the first rank whose cumulative weight
 * exceeds u times the total.  Double precision for the weights.  The sort is
 * the C library's qsort on (value, index) pairs. */
typedef struct {
    float v;
    int32_t i;
} ugref_vi;

static int ugref_rank_cmp(const void *a, const void *b)
{
    const ugref_vi *x = (const ugref_vi *)a, *y = (const ugref_vi *)b;
    if (x->v > y->v)
        return -1;
    if (x->v < y->v)
        return 1;
    return (x->i > y->i) - (x->i < y->i);
}

void ugref_sample_topk(const float *logits, int64_t ld, int64_t B, int64_t V,
                       int64_t k, float temp, const float *u, int32_t *tok,
                       int32_t *idx_out, float *val_out, double *cdf_out)
{
#pragma omp parallel for schedule(dynamic)
    for (int64_t b = 0; b < B; ++b) {
        ugref_vi *e = (ugref_vi *)malloc((size_t)V * sizeof(ugref_vi));
        for (int64_t i = 0; i < V; ++i) {
            e[i].v = logits[b * ld + i];
            e[i].i = (int32_t)i;
        }
        qsort(e, (size_t)V, sizeof(ugref_vi), ugref_rank_cmp);
        double *c = cdf_out + b * k;
        double run = 0.0;
        for (int64_t r = 0; r < k; ++r) {
            run += exp(((double)e[r].v - (double)e[0].v) / (double)temp);
            c[r] = run;
        }
        for (int64_t r = 0; r < k; ++r)
            c[r] /= run;
        int64_t pick = k - 1;
        for (int64_t r = 0; r < k; ++r)
            if ((double)u[b] < c[r]) {
                pick = r;
                break;
            }
        tok[b] = e[pick].i;
        for (int64_t r = 0; r < k; ++r) {
            idx_out[b * k + r] = e[r].i;
            val_out[b * k + r] = e[r].v;
        }
        free(e);
    }
}

/* ------------------------------------------------------------------ */
/* Straight-through backward of the BitLinear layer                    */
/* ------------------------------------------------------------------ */

/* "ultragraph - when the graph is the 1-bit LLM, part 2", section "autograd
 * on a byte-graph": the straight-through estimator treats the quantizers
 * and the per-row scale as the identity, so with g = dL/dy [M][N], the
 * fp32 master weights W [N][K] and the layer's fp32 input x [M][K]:
 *     dL/dx = g W        dx[m][k] = sum_n g[m][n] W[n][k]
 *     dL/dW = g^T x      dW[n][k] = sum_m g[m][n] x[m][k]
 *     dL/db = sum_m g    db[n]    = sum_m g[m][n]
 * Double-precision sums, rounded to fp32 once.  Any output may be NULL. */
void ugref_bitlinear_backward(const float *g, int64_t ldg, const float *x,
                              int64_t ldx, const float *W, int64_t ldw,
                              int64_t M, int64_t N, int64_t K, float *dx,
                              int64_t lddx, float *dW, int64_t lddw, float *db)
{
    if (dx) {
#pragma omp parallel for schedule(static)
        for (int64_t m = 0; m < M; ++m) {
            double *row = (double *)calloc((size_t)K, sizeof(double));
            for (int64_t n = 0; n < N; ++n) {
                double gv = g[m * ldg + n];
                for (int64_t k = 0; k < K; ++k)
                    row[k] += gv * (double)W[n * ldw + k];
            }
            for (int64_t k = 0; k < K; ++k)
                dx[m * lddx + k] = (float)row[k];
            free(row);
        }
    }
    if (dW) {
#pragma omp parallel for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            double *row = (double *)calloc((size_t)K, sizeof(double));
            for (int64_t m = 0; m < M; ++m) {
                double gv = g[m * ldg + n];
                for (int64_t k = 0; k < K; ++k)
                    row[k] += gv * (double)x[m * ldx + k];
            }
            for (int64_t k = 0; k < K; ++k)
                dW[n * lddw + k] = (float)row[k];
            free(row);
        }
    }
    if (db) {
#pragma omp parallel for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            double s = 0.0;
            for (int64_t m = 0; m < M; ++m)
                s += (double)g[m * ldg + n];
            db[n] = (float)s;
        }
    }
}

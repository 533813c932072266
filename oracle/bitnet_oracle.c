/*
 * Plain CPU oracle for the ternary-weight x int8-activation projection.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg do.  It shares no code with the HIP library: it has its own layout code,
 * its own rounding and its own loops, written straight from the definitions.
 *
 * Build: gcc -O2 -std=c11 -fno-fast-math -ffp-contract=off -fopenmp -shared -fPIC
 * (no FMA contraction, IEEE float, default round-to-nearest-even mode).
 *
 * What is computed, and where the pages define it:
 *
 *  - Ternarization (BitNet b1.58, per tensor).  Every LM projection weight
 *    becomes -1, 0 or +1 (blog "The Paper Says ARM Support. I Might Be the First
 *    to Actually Compile It", section "What the model is trying to do"); the
 *    scale is one number per tensor built from the mean absolute weight (ONNX
 *    model card "multimodalart/VibeVoice-ASR-BitNet-ONNX", Quantization table,
 *    row "LM projections"), applied to QAT master weights right before export
 *    (same card, paragraph under the Quantization table).
 *    Reading used here: m = mean|W| (fp64 sum, fixed order, rounded once to
 *    fp32), code = clamp(rint(fl32(W / m)), -1, 1), stored scale = m.
 *
 *  - Packing.  Codes are stored at 2 bits in units of 128 consecutive inputs
 *    (blog above, section "Postscript two": the format packs 128 elements per
 *    unit and a 64-element reading scrambles the weights).  The bit placement
 *    inside a unit is not on the pages; this oracle follows the layout that the
 *    library header specifies (field value u = code + 1; unit-column-major).
 *
 *  - Activation quantization: per row, absmax int8: s = fl32(127 / max|x|),
 *    xq = clamp(rint(fl32(x * s)), -127, 127); an all-zero row gives xq = 0 and
 *    s = 1.  int8 activations appear on the pages for the audio encoder's I8_S
 *    path (ONNX card, Quantization table, row "VAE encoders"); the LM formula
 *    is this reading's.
 *
 *  - Contraction: with ternary codes the products become additions and
 *    subtractions of activations (xujun.org article, section on heterogeneous
 *    quantization; aitrends.kr summary, sections on technical features and
 *    differentiators).  acc[m,n] = sum_{q=+1} xq - sum_{q=-1} xq in int32.
 *
 *  - Dequantization: y = acc * w_scale / x_scale, computed in fp64 and rounded
 *    once to fp32 (the pages are silent on the epilogue; this is the plain
 *    reading of "dequantize both factors").
 *
 *  - Embeddings and lm_head: an 8-bit table with one scale per row (ONNX
 *    card, Quantization table, row "Embeddings / lm_head"); see the section
 *    of that name below.
 *
 * Parity pins for every function live in the CPU tests; none is "parity
 * unpinned" except the correspondence of the packed bit layout to the original
 * GGUF I2_S files, and of the 8-bit table to the GGUF build's Q6_K blocks,
 * neither of which is available (the layouts here are our own spec).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_UNIT 128

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ---------------------------------------------------------------------- */
/* Ternarization                                                           */
/* ---------------------------------------------------------------------- */

/* mean|W| over all N*K entries.  Each row is summed in fp64 with k ascending,
 * then the row sums are added in fp64 with n ascending; the quotient by N*K is
 * taken in fp64 and rounded once to fp32.  The order is fixed because one ulp
 * of m can move a code that sits on the rounding threshold. */
float oracle_absmean(const float *W, int64_t N, int64_t K) {
    double total = 0.0;
    for (int64_t n = 0; n < N; ++n) {
        double row = 0.0;
        for (int64_t k = 0; k < K; ++k) row += fabs((double)W[n * K + k]);
        total += row;
    }
    return (float)(total / (double)(N * K));
}

/* One code from one weight, given the tensor's m (m > 0). */
static int8_t ternary_code(float w, float m) {
    float r = w / m;          /* IEEE fp32 division, correctly rounded */
    float t = rintf(r);       /* round half to even (default mode) */
    if (t > 1.0f) return 1;
    if (t < -1.0f) return -1;
    return (int8_t)t;
}

/* codes q[N,K] in {-1,0,+1} and the stored scale m.  m == 0 (all-zero W)
 * gives all-zero codes and scale 0. */
void oracle_ternarize(const float *W, int64_t N, int64_t K, int8_t *q, float *w_scale) {
    float m = oracle_absmean(W, N, K);
    *w_scale = m;
    int64_t total = N * K;
    if (m == 0.0f) {
        memset(q, 0, (size_t)total);
        return;
    }
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < total; ++i) q[i] = ternary_code(W[i], m);
}

/* ---------------------------------------------------------------------- */
/* 2-bit packing in 128-code units                                          */
/* ---------------------------------------------------------------------- */

/* Position of code (n,k) in the packed buffer: unit t = k/128 of row n is the
 * 32-byte block number t*N + n; inside it, offset r = k%128 sits in byte r%32
 * at bit 2*(r/32). */
static int64_t packed_byte(int64_t N, int64_t n, int64_t k) {
    int64_t t = k / ORACLE_UNIT, r = k % ORACLE_UNIT;
    return (t * N + n) * 32 + (r % 32);
}
static int packed_shift(int64_t k) { return 2 * (int)((k % ORACLE_UNIT) / 32); }

void oracle_pack(const int8_t *q, int64_t N, int64_t K, uint8_t *packed) {
    memset(packed, 0, (size_t)(N * K / 4));
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            unsigned u = (unsigned)(q[n * K + k] + 1);   /* 0,1,2 */
            packed[packed_byte(N, n, k)] |= (uint8_t)(u << packed_shift(k));
        }
}

/* Inverse of oracle_pack.  Returns the number of fields holding the value 3,
 * which no valid buffer contains (those codes are written as 0). */
int64_t oracle_unpack(const uint8_t *packed, int64_t N, int64_t K, int8_t *q) {
    int64_t bad = 0;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            unsigned u = (packed[packed_byte(N, n, k)] >> packed_shift(k)) & 3u;
            if (u == 3u) { ++bad; u = 1u; }
            q[n * K + k] = (int8_t)((int)u - 1);
        }
    return bad;
}

/* One code read straight from the packed buffer. */
int oracle_code_at(const uint8_t *packed, int64_t N, int64_t n, int64_t k) {
    unsigned u = (packed[packed_byte(N, n, k)] >> packed_shift(k)) & 3u;
    return (int)u - 1;
}

void oracle_ternarize_pack(const float *W, int64_t N, int64_t K, uint8_t *packed,
                           float *w_scale) {
    int8_t *q = (int8_t *)malloc((size_t)(N * K));
    oracle_ternarize(W, N, K, q, w_scale);
    oracle_pack(q, N, K, packed);
    free(q);
}

/* ---------------------------------------------------------------------- */
/* Activation quantization, one scale per row                               */
/* ---------------------------------------------------------------------- */

void oracle_quant_act(const float *x, int64_t M, int64_t K, int8_t *xq, float *x_scale) {
    for (int64_t m = 0; m < M; ++m) {
        const float *row = x + m * K;
        float a = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float v = fabsf(row[k]);
            if (v > a) a = v;
        }
        if (a == 0.0f) {
            memset(xq + m * K, 0, (size_t)K);
            x_scale[m] = 1.0f;
            continue;
        }
        float s = 127.0f / a;            /* fp32, correctly rounded */
        x_scale[m] = s;
        for (int64_t k = 0; k < K; ++k) {
            float p = row[k] * s;        /* fp32 product */
            float t = rintf(p);          /* half to even */
            if (t > 127.0f) t = 127.0f;
            if (t < -127.0f) t = -127.0f;
            xq[m * K + k] = (int8_t)t;
        }
    }
}

/* ---------------------------------------------------------------------- */
/* Ternary contraction and dequantization                                   */
/* ---------------------------------------------------------------------- */

/* acc[m,n] = (sum of xq[m,k] over k with q[n,k] = +1)
 *          - (sum of xq[m,k] over k with q[n,k] = -1). */
void oracle_matmul_i32(const int8_t *xq, const int8_t *q, int64_t M, int64_t N, int64_t K,
                       int32_t *acc) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            int32_t plus = 0, minus = 0;
            for (int64_t k = 0; k < K; ++k) {
                int8_t c = q[n * K + k];
                if (c == 1) plus += xq[m * K + k];
                else if (c == -1) minus += xq[m * K + k];
            }
            acc[m * N + n] = plus - minus;
        }
}

void oracle_dequant(const int32_t *acc, float w_scale, const float *x_scale, int64_t M,
                    int64_t N, float *y) {
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            y[m * N + n] = (float)((double)acc[m * N + n] * (double)w_scale /
                                   (double)x_scale[m]);
}

/* The whole projection: quantize x, decode the packed codes, contract, dequantize.
 * xq_out / x_scale_out / acc_out may be NULL. */
void oracle_ternary_matmul(int64_t M, int64_t N, int64_t K, const float *x,
                           const uint8_t *packed, float w_scale, float *y,
                           int8_t *xq_out, float *x_scale_out, int32_t *acc_out) {
    int8_t *xq = (int8_t *)malloc((size_t)(M * K));
    float *xs = (float *)malloc(sizeof(float) * (size_t)M);
    int8_t *q = (int8_t *)malloc((size_t)(N * K));
    int32_t *acc = (int32_t *)malloc(sizeof(int32_t) * (size_t)(M * N));
    oracle_quant_act(x, M, K, xq, xs);
    oracle_unpack(packed, N, K, q);
    oracle_matmul_i32(xq, q, M, N, K, acc);
    oracle_dequant(acc, w_scale, xs, M, N, y);
    if (xq_out) memcpy(xq_out, xq, (size_t)(M * K));
    if (x_scale_out) memcpy(x_scale_out, xs, sizeof(float) * (size_t)M);
    if (acc_out) memcpy(acc_out, acc, sizeof(int32_t) * (size_t)(M * N));
    free(xq); free(xs); free(q); free(acc);
}

/* Selected outputs only: for each pair (ms[i], ns[i]) the accumulator and the
 * dequantized output, reading codes one by one from the packed buffer.  xq and
 * x_scale are the oracle's own quantized activations for all M rows. */
void oracle_matmul_sampled(int64_t N, int64_t K, const int8_t *xq, const float *x_scale,
                           const uint8_t *packed, float w_scale, const int64_t *ms,
                           const int64_t *ns, int64_t count, int32_t *acc, float *y) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        int64_t m = ms[i], n = ns[i];
        int32_t plus = 0, minus = 0;
        for (int64_t k = 0; k < K; ++k) {
            int c = oracle_code_at(packed, N, n, k);
            if (c == 1) plus += xq[m * K + k];
            else if (c == -1) minus += xq[m * K + k];
        }
        acc[i] = plus - minus;
        y[i] = (float)((double)acc[i] * (double)w_scale / (double)x_scale[m]);
    }
}

/* ---------------------------------------------------------------------- */
/* I8_S: int8 weights x int8 activations (the audio encoders' path)         */
/* ---------------------------------------------------------------------- */
/*
 * The audio tokenizer's encoders run as I8_S: int8 weights and int8
 * activations, with ReLU in place of GELU (ONNX model card
 * "multimodalart/VibeVoice-ASR-BitNet-ONNX", Quantization table, row "VAE
 * encoders"), in fused conv / depthwise conv / matmul+bias+ReLU routines
 * (aitrends.kr summary, technical-features section).  The pages give no scale
 * granularity or formula.  Readings used here:
 *  - one scale per weight tensor, as in I2_S: a = max|W|, s = fl32(a / 127)
 *    (the dequant multiplier), q = clamp(rint(fl32(W / s)), -127, 127); a
 *    zero tensor gives s = 0 and q = 0;
 *  - activations per row exactly as oracle_quant_act;
 *  - y = relu?(acc * s / x_scale + bias) with acc = sum_k xq * q in int32,
 *    computed in fp64 and rounded once to fp32; relu(v) = v > 0 ? v : 0.
 */

void oracle_i8_quant_weights(const float *W, int64_t N, int64_t K, int8_t *q, float *w_scale) {
    float a = 0.0f;
    for (int64_t i = 0; i < N * K; ++i) {
        float v = fabsf(W[i]);
        if (v > a) a = v;
    }
    if (a == 0.0f) {
        memset(q, 0, (size_t)(N * K));
        *w_scale = 0.0f;
        return;
    }
    float s = a / 127.0f;                 /* fp32, correctly rounded */
    *w_scale = s;
    for (int64_t i = 0; i < N * K; ++i) {
        float t = rintf(W[i] / s);        /* fp32 quotient, half to even */
        if (t > 127.0f) t = 127.0f;
        if (t < -127.0f) t = -127.0f;
        q[i] = (int8_t)t;
    }
}

/* acc[m,n] = sum_k xq[m,k] * q[n,k], exactly (int64, stored as int32). */
void oracle_i8_matmul(const int8_t *xq, const int8_t *q, int64_t M, int64_t N, int64_t K,
                      int32_t *acc) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            int64_t s = 0;
            for (int64_t k = 0; k < K; ++k) s += (int64_t)xq[m * K + k] * (int64_t)q[n * K + k];
            acc[m * N + n] = (int32_t)s;
        }
}

/* The whole I8_S linear layer.  bias may be NULL (no bias); relu != 0 applies
 * ReLU.  xq_out / x_scale_out / acc_out may be NULL. */
void oracle_i8_linear(int64_t M, int64_t N, int64_t K, const float *x, const int8_t *q,
                      float w_scale, const float *bias, int relu, float *y, int8_t *xq_out,
                      float *x_scale_out, int32_t *acc_out) {
    int8_t *xq = (int8_t *)malloc((size_t)(M * K));
    float *xs = (float *)malloc(sizeof(float) * (size_t)M);
    int32_t *acc = (int32_t *)malloc(sizeof(int32_t) * (size_t)(M * N));
    oracle_quant_act(x, M, K, xq, xs);
    oracle_i8_matmul(xq, q, M, N, K, acc);
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double v = (double)acc[m * N + n] * (double)w_scale / (double)xs[m];
            if (bias) v += (double)bias[n];
            if (relu && !(v > 0.0)) v = 0.0;
            y[m * N + n] = (float)v;
        }
    if (xq_out) memcpy(xq_out, xq, (size_t)(M * K));
    if (x_scale_out) memcpy(x_scale_out, xs, sizeof(float) * (size_t)M);
    if (acc_out) memcpy(acc_out, acc, sizeof(int32_t) * (size_t)(M * N));
    free(xq); free(xs); free(acc);
}

/* Selected outputs of the I8_S linear layer from the oracle's own quantized
 * rows: for each pair (ms[i], ns[i]), acc[i] and the fp64 value before ReLU
 * and bias (d[i] = acc * w_scale / x_scale) and the output y[i]. */
void oracle_i8_linear_sampled(int64_t N, int64_t K, const int8_t *xq, const float *x_scale,
                              const int8_t *q, float w_scale, const float *bias, int relu,
                              const int64_t *ms, const int64_t *ns, int64_t count,
                              int32_t *acc, double *d, float *y) {
    (void)N;   /* q is [N, K]; only the selected rows are read */
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        int64_t m = ms[i], n = ns[i], s = 0;
        for (int64_t k = 0; k < K; ++k) s += (int64_t)xq[m * K + k] * (int64_t)q[n * K + k];
        acc[i] = (int32_t)s;
        d[i] = (double)acc[i] * (double)w_scale / (double)x_scale[m];
        double v = d[i] + (bias ? (double)bias[n] : 0.0);
        if (relu && !(v > 0.0)) v = 0.0;
        y[i] = (float)v;
    }
}

/* ---------------------------------------------------------------------- */
/* 8-bit weights with one scale per row: embeddings and lm_head             */
/* ---------------------------------------------------------------------- */
/*
 * The decoder's token embeddings and its lm_head are stored at 8 bits with
 * one scale per row (per vocabulary entry) in the ONNX build, Q6_K in the
 * GGUF build (ONNX model card "multimodalart/VibeVoice-ASR-BitNet-ONNX",
 * Quantization table, row "Embeddings / lm_head": "8-bit per-row /
 * per-column"; xujun.org article, heterogeneous-quantization section: I2_S
 * plus Q6_K embeddings).  The table is [V, K] (vocabulary x hidden); a row
 * of it is one token's embedding, and, read as the lm_head weight, one output
 * column's weights, so the same per-row scale serves both readings of the
 * card's cell.  The card gives no formula.  Readings used here:
 *  - per row n: a = max_k |W[n,k]|, s[n] = fl32(a / 127) (the dequant
 *    multiplier), q = clamp(rint(fl32(W / s[n])), -127, 127); a zero row
 *    gives s[n] = 0 and q = 0 (the same formula as the I8_S weights above,
 *    applied to each row on its own);
 *  - embedding lookup: e[t,k] = fl32(q[id_t,k] * s[id_t]); an id outside
 *    [0, V) gives a zero row;
 *  - lm_head: activations quantized per row exactly as oracle_quant_act,
 *    acc = sum_k xq * q in int32, y[m,n] = acc * s[n] / x_scale[m] in fp64,
 *    rounded once to fp32.
 */

void oracle_rowq_quant_weights(const float *W, int64_t N, int64_t K, int8_t *q,
                               float *w_scale) {
    for (int64_t n = 0; n < N; ++n) {
        const float *row = W + n * K;
        float a = 0.0f;                       /* max |W| over row n */
        for (int64_t k = 0; k < K; ++k) a = fabsf(row[k]) > a ? fabsf(row[k]) : a;
        if (a == 0.0f) {
            memset(q + n * K, 0, (size_t)K);
            w_scale[n] = 0.0f;
            continue;
        }
        float s = a / 127.0f;                 /* row scale: fp32, correctly rounded */
        w_scale[n] = s;
        for (int64_t k = 0; k < K; ++k) {
            float t = rintf(row[k] / s);      /* fp32 quotient, half to even */
            if (t > 127.0f) t = 127.0f;
            if (t < -127.0f) t = -127.0f;
            q[n * K + k] = (int8_t)t;
        }
    }
}

void oracle_rowq_embed(const int32_t *ids, int64_t T, const int8_t *q, const float *w_scale,
                       int64_t N, int64_t K, float *out) {
    for (int64_t t = 0; t < T; ++t) {
        int64_t id = ids[t];
        for (int64_t k = 0; k < K; ++k)
            out[t * K + k] = (id >= 0 && id < N)
                                 ? (float)((double)q[id * K + k] * (double)w_scale[id])
                                 : 0.0f;
    }
}

/* The whole lm_head: y[m,n] = (sum_k xq[m,k] * q[n,k]) * s[n] / x_scale[m].
 * xq_out / x_scale_out / acc_out may be NULL. */
void oracle_rowq_linear(int64_t M, int64_t N, int64_t K, const float *x, const int8_t *q,
                        const float *w_scale, float *y, int8_t *xq_out, float *x_scale_out,
                        int32_t *acc_out) {
    int8_t *xq = (int8_t *)malloc((size_t)(M * K));
    float *xs = (float *)malloc(sizeof(float) * (size_t)M);
    int32_t *acc = (int32_t *)malloc(sizeof(int32_t) * (size_t)(M * N));
    oracle_quant_act(x, M, K, xq, xs);
    oracle_i8_matmul(xq, q, M, N, K, acc);
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            y[m * N + n] = (float)((double)acc[m * N + n] * (double)w_scale[n] /
                                   (double)xs[m]);
    if (xq_out) memcpy(xq_out, xq, (size_t)(M * K));
    if (x_scale_out) memcpy(x_scale_out, xs, sizeof(float) * (size_t)M);
    if (acc_out) memcpy(acc_out, acc, sizeof(int32_t) * (size_t)(M * N));
    free(xq); free(xs); free(acc);
}

/* Selected outputs of the lm_head from the oracle's own quantized rows. */
void oracle_rowq_linear_sampled(int64_t K, const int8_t *xq, const float *x_scale,
                                const int8_t *q, const float *w_scale, const int64_t *ms,
                                const int64_t *ns, int64_t count, int32_t *acc, float *y) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        int64_t m = ms[i], n = ns[i], dot = 0;
        for (int64_t k = 0; k < K; ++k) dot += (int64_t)q[n * K + k] * (int64_t)xq[m * K + k];
        acc[i] = (int32_t)dot;
        y[i] = (float)((double)acc[i] * (double)w_scale[n] / (double)x_scale[m]);
    }
}

/* ---------------------------------------------------------------------- */
/* I8_S with one weight scale per output channel                            */
/* ---------------------------------------------------------------------- */
/*
 * The ONNX build of the audio encoders stores "int8 per-channel weights"
 * (ONNX model card "multimodalart/VibeVoice-ASR-BitNet-ONNX", Quantization
 * table, row "VAE encoders").  Per output channel n the weights are
 * quantized exactly as a table row above (oracle_rowq_quant_weights), the
 * activations per row as oracle_quant_act, and
 *   y[m,n] = relu?(acc[m,n] * w_scale[n] / x_scale[m] + bias[n])
 * in fp64, rounded once to fp32.
 */
void oracle_i8_linear_rows(int64_t M, int64_t N, int64_t K, const float *x, const int8_t *q,
                           const float *w_scale, const float *bias, int relu, float *y,
                           int8_t *xq_out, float *x_scale_out, int32_t *acc_out) {
    int8_t *xq = (int8_t *)malloc((size_t)(M * K));
    float *xs = (float *)malloc(sizeof(float) * (size_t)M);
    int32_t *acc = (int32_t *)malloc(sizeof(int32_t) * (size_t)(M * N));
    oracle_quant_act(x, M, K, xq, xs);
    oracle_i8_matmul(xq, q, M, N, K, acc);
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double v = (double)acc[m * N + n] * (double)w_scale[n] / (double)xs[m];
            if (bias) v += (double)bias[n];          /* channel bias */
            if (relu && v <= 0.0) v = 0.0;
            y[m * N + n] = (float)v;
        }
    if (xq_out) memcpy(xq_out, xq, (size_t)(M * K));
    if (x_scale_out) memcpy(x_scale_out, xs, sizeof(float) * (size_t)M);
    if (acc_out) memcpy(acc_out, acc, sizeof(int32_t) * (size_t)(M * N));
    free(xq); free(xs); free(acc);
}

/* Selected outputs of the per-channel layer from the oracle's own quantized
 * rows: acc[i], d[i] = acc * w_scale[n] / x_scale[m] (fp64, before bias and
 * ReLU) and y[i]. */
void oracle_i8_linear_rows_sampled(int64_t K, const int8_t *xq, const float *x_scale,
                                   const int8_t *q, const float *w_scale, const float *bias,
                                   int relu, const int64_t *ms, const int64_t *ns,
                                   int64_t count, int32_t *acc, double *d, float *y) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        int64_t m = ms[i], n = ns[i], dot = 0;
        for (int64_t k = 0; k < K; ++k) dot += (int64_t)q[n * K + k] * (int64_t)xq[m * K + k];
        acc[i] = (int32_t)dot;
        d[i] = (double)acc[i] * (double)w_scale[n] / (double)x_scale[m];
        double v = d[i] + (bias ? (double)bias[n] : 0.0);
        if (relu && v <= 0.0) v = 0.0;
        y[i] = (float)v;
    }
}

/* ---------------------------------------------------------------------- */
/* Storage layout of the 8-bit table (the library's own)                    */
/* ---------------------------------------------------------------------- */
/*
 * The pages fix only "8-bit per-row" for the table; its byte order in
 * memory is this library's.  Rows are grouped by 16 and inputs by 256; each
 * 16-row x 256-input tile is 4096 contiguous bytes, tiles ordered by row
 * group, then by input chunk.  Inside a tile, input k = 64j + 16h + e
 * (j, h < 4, e < 16) of tile row r sits at byte 1024j + 256h + 16r + e.
 * The table is padded with zero codes to Vp = 16*ceil(V/16) rows and
 * Kp = 256*ceil(K/256) inputs.
 */
int64_t oracle_table_bytes(int64_t V, int64_t K) {
    int64_t Vp = (V + 15) / 16 * 16, Kp = (K + 255) / 256 * 256;
    return Vp * Kp;
}

static int64_t table_offset(int64_t K, int64_t v, int64_t k) {
    int64_t chunks = (K + 255) / 256;            /* 256-input chunks per row group */
    int64_t tile = (v / 16) * chunks + k / 256;
    int64_t j = (k % 256) / 64, h = (k % 64) / 16, e = k % 16;
    return tile * 4096 + j * 1024 + h * 256 + (v % 16) * 16 + e;
}

void oracle_table_pack(const int8_t *q, int64_t V, int64_t K, int8_t *table) {
    memset(table, 0, (size_t)oracle_table_bytes(V, K));
    for (int64_t v = 0; v < V; ++v)
        for (int64_t k = 0; k < K; ++k) table[table_offset(K, v, k)] = q[v * K + k];
}

/* Inverse of oracle_table_pack.  Returns the number of padding bytes that are
 * not zero (a valid table has none). */
int64_t oracle_table_unpack(const int8_t *table, int64_t V, int64_t K, int8_t *q) {
    int64_t Vp = (V + 15) / 16 * 16, Kp = (K + 255) / 256 * 256, bad = 0;
    for (int64_t v = 0; v < Vp; ++v)
        for (int64_t k = 0; k < Kp; ++k) {
            int8_t b = table[table_offset(K, v, k)];
            if (v < V && k < K) q[v * K + k] = b;
            else if (b != 0) ++bad;
        }
    return bad;
}

/* ---------------------------------------------------------------------- */
/* I8_S depthwise convolution over time (the encoders' token mixer)         */
/* ---------------------------------------------------------------------- */
/*
 * The encoders run fused int8 convolution and depthwise convolution routines
 * with bias (aitrends.kr summary, technical-features section: fused conv,
 * depthwise conv and matmul+bias+ReLU over permuted layouts); their ONNX
 * export pads the convolutions causally (ONNX model card
 * "multimodalart/VibeVoice-ASR-BitNet-ONNX", Provenance: static causal
 * padding of the tokenizer encoders); the weights are int8 per channel (same
 * card, Quantization table, row "VAE encoders").  Readings used here:
 *  - x is [B, T, C] (sequences, frames, channels; channels innermost, the
 *    layout of the pointwise layers' rows), the kernel w is [C, k];
 *  - y[b,t,c] = sum_{j<k} w[c,j] * x[b, t-(k-1)+j, c], frames before 0 are 0;
 *  - weights quantized per channel as the table rows above
 *    (oracle_rowq_quant_weights on [C, k]);
 *  - activations quantized with one scale per (sequence, channel): the
 *    convolution sums over frames within a channel, so one scale per channel
 *    keeps that sum exact in int32 (as one scale per row does for the
 *    pointwise layers, which sum over channels within a frame):
 *    s[b,c] = fl32(127 / max_t |x[b,t,c]|), xq = clamp(rint(fl32(x * s)),
 *    -127, 127); an all-zero column gives xq = 0 and s = 1;
 *  - y = relu?(acc * w_scale[c] / s[b,c] + bias[c]) in fp64, rounded once.
 */
void oracle_i8_col_quant(const float *x, int64_t B, int64_t T, int64_t C, int8_t *xq,
                         float *x_scale) {
    for (int64_t b = 0; b < B; ++b)
        for (int64_t c = 0; c < C; ++c) {
            const float *col = x + b * T * C + c;     /* stride C */
            float a = 0.0f;
            for (int64_t t = 0; t < T; ++t) {
                float v = fabsf(col[t * C]);
                if (v > a) a = v;
            }
            int8_t *dst = xq + b * T * C + c;
            if (a == 0.0f) {
                for (int64_t t = 0; t < T; ++t) dst[t * C] = 0;
                x_scale[b * C + c] = 1.0f;
                continue;
            }
            float s = 127.0f / a;                    /* fp32, correctly rounded */
            x_scale[b * C + c] = s;
            for (int64_t t = 0; t < T; ++t) {
                float u = rintf(col[t * C] * s);     /* fp32 product, half to even */
                if (u > 127.0f) u = 127.0f;
                if (u < -127.0f) u = -127.0f;
                dst[t * C] = (int8_t)u;
            }
        }
}

void oracle_i8_dwconv(int64_t B, int64_t T, int64_t C, int64_t k, const float *x,
                      const int8_t *q, const float *w_scale, const float *bias, int relu,
                      float *y, int8_t *xq_out, float *x_scale_out, int32_t *acc_out) {
    int8_t *xq = (int8_t *)malloc((size_t)(B * T * C));
    float *xs = (float *)malloc(sizeof(float) * (size_t)(B * C));
    oracle_i8_col_quant(x, B, T, C, xq, xs);
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < B; ++b)
        for (int64_t t = 0; t < T; ++t)
            for (int64_t c = 0; c < C; ++c) {
                int32_t acc = 0;
                for (int64_t j = 0; j < k; ++j) {
                    int64_t src = t - (k - 1) + j;   /* causal: earlier frames only */
                    if (src >= 0) acc += (int32_t)xq[(b * T + src) * C + c] * (int32_t)q[c * k + j];
                }
                int64_t o = (b * T + t) * C + c;
                if (acc_out) acc_out[o] = acc;
                double v = (double)acc * (double)w_scale[c] / (double)xs[b * C + c];
                if (bias) v += (double)bias[c];
                if (relu && v <= 0.0) v = 0.0;
                y[o] = (float)v;
            }
    if (xq_out) memcpy(xq_out, xq, (size_t)(B * T * C));
    if (x_scale_out) memcpy(x_scale_out, xs, sizeof(float) * (size_t)(B * C));
    free(xq); free(xs);
}

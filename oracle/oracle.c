/*
 * oracle.c -- plain, slow, single-threaded CPU oracle of the neuron-sparse FFN.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no source, header,
 * table or helper with the GPU library, and the GPU library never calls it.
 *
 * Conventions used by every function below:
 *   - all sums run over ascending indices and accumulate in IEEE binary64;
 *   - weights are read exactly: fp32 and fp16 values widen exactly to fp64,
 *     a 4-bit block value (q - 8) * s is exact in fp64;
 *   - matrices are row-major; W_down is held transposed as W_downT [d_ffn, d],
 *     so row i of W_downT is column i of W_down;
 *   - activations x are given as fp64 (the callers widen fp32 inputs exactly).
 *
 * Sources (page titles abbreviated):
 *   [Guide]  "PowerInfer Guide: Exploiting Activation Sparsity for LLM AI"
 *   [x64]    "PowerInfer_x64: Neuron-Level Sparse Inference Makes Large Models
 *             Fly on Consumer GPUs"
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_F32 0
#define OR_F16 1
#define OR_Q4_0 2
#define OR_FP8_E4M3 3

#define OR_RELU 0
#define OR_REGLU 1
#define OR_SWIGLU 2

#define Q4_0_BLOCK 32
#define Q4_0_BYTES 18

/* IEEE 754 binary16 -> binary64, from the format's definition: 1 sign bit,
 * 5 exponent bits with bias 15, 10 fraction bits; exponent 0 holds zeros and
 * subnormals (f * 2^-24), exponent 31 holds infinities and NaNs. */
double oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return sign ? -v : v;
}

/* One 4-bit block (the GGUF "Q4_0" layout, the 4-bit weights named by [x64]'s
 * throughput table): bytes 0..1 hold an fp16 scale s (little-endian), bytes
 * 2..17 hold 32 codes; byte 2+k keeps code k in its low nibble and code k+16
 * in its high nibble.  Weight k of the block is (code_k - 8) * s. */
static double q4_0_value(const uint8_t *blk, int k)
{
    uint16_t sbits = (uint16_t)(blk[0] | ((uint16_t)blk[1] << 8));
    uint8_t byte = blk[2 + (k & 15)];
    int q = (k < 16) ? (byte & 0x0f) : (byte >> 4);
    return (double)(q - 8) * oracle_f16_to_f64(sbits);
}

/* OCP 8-bit floating point, E4M3 format (the OCP 8-bit Floating Point
 * Specification): bit 7 is the sign, bits 6..3 the exponent e with bias 7,
 * bits 2..0 the mantissa m.  e = 0 holds zero and the subnormals m * 2^-9;
 * otherwise the value is (1 + m/8) * 2^(e-7); the format has no infinities and
 * S.1111.111 is NaN (so the largest finite magnitude is 1.75 * 2^8 = 448). */
double oracle_e4m3_to_f64(uint8_t c)
{
    int sign = c >> 7;
    int e = (c >> 3) & 0xf;
    int m = c & 7;
    double v;
    if (e == 15 && m == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp((double)(8 + m), e - 10);
    return sign ? -v : v;
}

/* Row `row` of a [rows, cols] weight matrix stored as `dtype`, widened to fp64.
 * An fp8 (E4M3) matrix is one buffer: rows * cols code bytes, row-major, then
 * one fp32 scale per row; weight (i, k) = e4m3(code[i][k]) * scale[i], exact
 * in fp64 (a 4-bit significand times a 24-bit one). */
int oracle_deq_row(const void *w, int dtype, int64_t rows, int64_t cols, int64_t row,
                   double *out)
{
    int64_t k;
    if (dtype == OR_F32) {
        const float *p = (const float *)w + row * cols;
        for (k = 0; k < cols; ++k)
            out[k] = (double)p[k];
    } else if (dtype == OR_F16) {
        const uint16_t *p = (const uint16_t *)w + row * cols;
        for (k = 0; k < cols; ++k)
            out[k] = oracle_f16_to_f64(p[k]);
    } else if (dtype == OR_FP8_E4M3) {
        const uint8_t *p = (const uint8_t *)w + row * cols;
        float scale;
        memcpy(&scale, (const uint8_t *)w + rows * cols + row * 4, sizeof scale);
        for (k = 0; k < cols; ++k)
            out[k] = oracle_e4m3_to_f64(p[k]) * (double)scale;
    } else if (dtype == OR_Q4_0) {
        if (cols % Q4_0_BLOCK)
            return -1;
        const uint8_t *p = (const uint8_t *)w + row * (cols / Q4_0_BLOCK) * Q4_0_BYTES;
        for (k = 0; k < cols; ++k)
            out[k] = q4_0_value(p + (k / Q4_0_BLOCK) * Q4_0_BYTES, (int)(k % Q4_0_BLOCK));
    } else {
        return -1;
    }
    return 0;
}

static double dot(const double *a, const double *b, int64_t n)
{
    double s = 0.0;
    int64_t k;
    for (k = 0; k < n; ++k)
        s += a[k] * b[k];
    return s;
}

/* Two-layer MLP predictor ([x64] "Prediction and Caching": a 2-layer MLP;
 * [Guide] section 3 "Adaptive Online Neuron Predictors": one score per FFN
 * neuron, thresholded into a binary mask):
 *   hid_j   = max(0, W1[j] . x + b1_j)                 j < r
 *   logit_i = W2[i] . hid + b2_i                       i < d_ffn
 *   mask_i  = logit_i > t
 * [Guide] compares sigmoid(logit) > tau strictly; sigmoid is increasing, so
 * this equals logit > t with t = ln(tau / (1 - tau)), which the caller passes.
 * The first dense_prefix neurons are not scored: they are always active
 * (the always-hot neurons of [Guide] section 2 run without the predictor)
 * and their logit is reported as +inf.
 * hid may be NULL; logits and mask may be NULL. */
int oracle_predict(int64_t d, int64_t d_ffn, int64_t r, int p_dtype,
                   const void *W1, const float *b1, const void *W2, const float *b2,
                   const double *x, double t, int64_t dense_prefix, double *hid_out,
                   double *logits, uint8_t *mask)
{
    int64_t j, i;
    double *row = (double *)malloc(sizeof(double) * (size_t)(d > r ? d : r));
    double *hid = (double *)malloc(sizeof(double) * (size_t)r);
    if (!row || !hid) {
        free(row);
        free(hid);
        return -2;
    }
    for (j = 0; j < r; ++j) {
        if (oracle_deq_row(W1, p_dtype, r, d, j, row)) {
            free(row);
            free(hid);
            return -1;
        }
        double s = dot(row, x, d) + (double)b1[j];
        hid[j] = s > 0.0 ? s : 0.0;
        if (hid_out)
            hid_out[j] = hid[j];
    }
    for (i = 0; i < d_ffn; ++i) {
        double l;
        if (i < dense_prefix) {
            l = INFINITY;
        } else {
            oracle_deq_row(W2, p_dtype, d_ffn, r, i, row);
            l = dot(row, hid, r) + (double)b2[i];
        }
        if (logits)
            logits[i] = l;
        if (mask)
            mask[i] = (uint8_t)(i < dense_prefix || l > t);
    }
    free(row);
    free(hid);
    return 0;
}

/* Threshold given logits: mask_i = logit_i > t, compared in the logits' own
 * precision (fp32 values and an fp32 threshold compare identically in fp64). */
void oracle_threshold(const float *logits, int64_t n, float t, uint8_t *mask)
{
    int64_t i;
    for (i = 0; i < n; ++i)
        mask[i] = (uint8_t)((double)logits[i] > (double)t);
}

/* Compaction ([Guide] Step 3 keeps the positions where the mask is set;
 * section 4 decodes the activation bitmask into the active indices):
 * idx = the i with mask_i != 0, ascending; returns their count. */
int64_t oracle_compact(const uint8_t *mask, int64_t n, int32_t *idx)
{
    int64_t i, c = 0;
    for (i = 0; i < n; ++i)
        if (mask[i])
            idx[c++] = (int32_t)i;
    return c;
}

/* Union over a batch of masks [B, n]: U_i = OR_b mask_{b,i}. */
void oracle_union(const uint8_t *masks, int64_t B, int64_t n, uint8_t *out)
{
    int64_t b, i;
    for (i = 0; i < n; ++i) {
        uint8_t u = 0;
        for (b = 0; b < B; ++b)
            u |= (uint8_t)(masks[b * n + i] != 0);
        out[i] = u;
    }
}

/* Pre-activations of neuron i ([Guide] "The Hidden Inefficiency", the FFN
 * equation; bias b_i only on the activated projection):
 *   ReLU  (non-gated):  z_i = W_up[i] . x + b_i,   u_i = 1 (unused)
 *   ReGLU, SwiGLU (gated): z_i = W_gate[i] . x + b_i, u_i = W_up[i] . x
 * The activation is a_i = max(z_i, 0) (ReLU), max(z_i, 0) * u_i (ReGLU) or
 * silu(z_i) * u_i (SwiGLU), silu(z) = z * sigmoid(z) = z / (1 + e^-z). */
static double neuron_act(int kind, int w_dtype, int64_t d, int64_t d_ffn,
                         const void *W_gate, const void *W_up, const float *b,
                         const double *x, int64_t i, double *row, double *z_out)
{
    double z, u = 1.0;
    if (kind != OR_RELU) {
        oracle_deq_row(W_gate, w_dtype, d_ffn, d, i, row);
        z = dot(row, x, d) + (b ? (double)b[i] : 0.0);
        oracle_deq_row(W_up, w_dtype, d_ffn, d, i, row);
        u = dot(row, x, d);
    } else {
        oracle_deq_row(W_up, w_dtype, d_ffn, d, i, row);
        z = dot(row, x, d) + (b ? (double)b[i] : 0.0);
    }
    if (z_out)
        *z_out = z;
    double a = kind == OR_SWIGLU ? z / (1.0 + exp(-z)) : (z > 0.0 ? z : 0.0);
    return kind != OR_RELU ? a * u : a;
}

static int check_layer(int kind, int w_dtype, int64_t d)
{
    if (kind != OR_RELU && kind != OR_REGLU && kind != OR_SWIGLU)
        return -1;
    if (w_dtype != OR_F32 && w_dtype != OR_F16 && w_dtype != OR_Q4_0)
        return -1;
    if (w_dtype == OR_Q4_0 && d % Q4_0_BLOCK)
        return -1;
    return 0;
}

/* Dense FFN over every neuron ([Guide] FFN equation):
 *   y = sum_{i=0}^{d_ffn-1} a_i * W_downT[i]
 * act (optional, [d_ffn]) receives every a_i. */
int oracle_ffn_dense(int kind, int w_dtype, int64_t d, int64_t d_ffn,
                     const void *W_gate, const void *W_up, const void *W_downT, const float *b,
                     const double *x, double *y, double *act)
{
    int64_t i, k;
    if (check_layer(kind, w_dtype, d))
        return -1;
    double *row = (double *)malloc(sizeof(double) * (size_t)d);
    double *a = (double *)malloc(sizeof(double) * (size_t)(d_ffn > 0 ? d_ffn : 1));
    if (!row || !a) {
        free(row);
        free(a);
        return -2;
    }
    for (i = 0; i < d_ffn; ++i)
        a[i] = neuron_act(kind, w_dtype, d, d_ffn, W_gate, W_up, b, x, i, row, NULL);
    for (k = 0; k < d; ++k)
        y[k] = 0.0;
    for (i = 0; i < d_ffn; ++i) {
        oracle_deq_row(W_downT, w_dtype, d_ffn, d, i, row);
        for (k = 0; k < d; ++k)
            y[k] += a[i] * row[k];
        if (act)
            act[i] = a[i];
    }
    free(row);
    free(a);
    return 0;
}

/* Neuron-sparse FFN ([Guide] Step 3 "Fused PowerInfer Sparse FFN Module":
 * gather the rows of the active neurons, activate, gather the matching
 * columns of W_down, sum):  y = sum_{j < count} a_{idx_j} * W_downT[idx_j],
 * with idx the active neurons in ascending order.  act (optional, [count])
 * receives a_{idx_j} in list order.  Returns count, or < 0 on error. */
int64_t oracle_ffn_sparse(int kind, int w_dtype, int64_t d, int64_t d_ffn,
                          const void *W_gate, const void *W_up, const void *W_downT,
                          const float *b, const double *x, const int32_t *idx, int64_t count,
                          double *y, double *act)
{
    int64_t j, k;
    if (check_layer(kind, w_dtype, d))
        return -1;
    for (j = 0; j < count; ++j)
        if (idx[j] < 0 || idx[j] >= d_ffn)
            return -3;
    double *row = (double *)malloc(sizeof(double) * (size_t)d);
    if (!row)
        return -2;
    for (k = 0; k < d; ++k)
        y[k] = 0.0;
    for (j = 0; j < count; ++j) {
        int64_t i = idx[j];
        double a = neuron_act(kind, w_dtype, d, d_ffn, W_gate, W_up, b, x, i, row, NULL);
        oracle_deq_row(W_downT, w_dtype, d_ffn, d, i, row);
        for (k = 0; k < d; ++k)
            y[k] += a * row[k];
        if (act)
            act[j] = a;
    }
    free(row);
    return count;
}

/* Masked FFN: compaction of the mask, then the neuron-sparse FFN on it. */
int64_t oracle_ffn_masked(int kind, int w_dtype, int64_t d, int64_t d_ffn,
                          const void *W_gate, const void *W_up, const void *W_downT,
                          const float *b, const double *x, const uint8_t *mask, double *y)
{
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)(d_ffn > 0 ? d_ffn : 1));
    if (!idx)
        return -2;
    int64_t count = oracle_compact(mask, d_ffn, idx);
    int64_t rc = oracle_ffn_sparse(kind, w_dtype, d, d_ffn, W_gate, W_up, W_downT, b, x,
                                   idx, count, y, NULL);
    free(idx);
    return rc;
}

/* Pre-activations z [d_ffn] (and u for ReGLU, may be NULL) of one token, and the
 * exact mask z_i > 0: the neurons whose post-activation is positive ([Guide]
 * Step 1 counts a neuron as active when its activation is > 0). */
int oracle_preact(int kind, int w_dtype, int64_t d, int64_t d_ffn,
                  const void *W_gate, const void *W_up, const float *b,
                  const double *x, double *z, double *u, uint8_t *exact_mask)
{
    int64_t i;
    if (check_layer(kind, w_dtype, d))
        return -1;
    double *row = (double *)malloc(sizeof(double) * (size_t)d);
    if (!row)
        return -2;
    for (i = 0; i < d_ffn; ++i) {
        double zi;
        if (kind != OR_RELU) {
            oracle_deq_row(W_gate, w_dtype, d_ffn, d, i, row);
            zi = dot(row, x, d) + (b ? (double)b[i] : 0.0);
            if (u) {
                oracle_deq_row(W_up, w_dtype, d_ffn, d, i, row);
                u[i] = dot(row, x, d);
            }
        } else {
            oracle_deq_row(W_up, w_dtype, d_ffn, d, i, row);
            zi = dot(row, x, d) + (b ? (double)b[i] : 0.0);
            if (u)
                u[i] = 1.0;
        }
        if (z)
            z[i] = zi;
        if (exact_mask)
            exact_mask[i] = (uint8_t)(zi > 0.0);
    }
    free(row);
    return 0;
}

/* Activation profile ([Guide] Step 1 "Offline Activation Profiler"): for each
 * neuron, the number of the N tokens X [N, d] on which it is active (z_i > 0). */
int oracle_profile(int kind, int w_dtype, int64_t d, int64_t d_ffn,
                   const void *W_gate, const void *W_up, const float *b,
                   const double *X, int64_t N, int32_t *counts)
{
    int64_t i, t;
    if (check_layer(kind, w_dtype, d))
        return -1;
    const void *W_act = (kind != OR_RELU) ? W_gate : W_up;
    double *row = (double *)malloc(sizeof(double) * (size_t)d);
    if (!row)
        return -2;
    for (i = 0; i < d_ffn; ++i) {
        int32_t c = 0;
        oracle_deq_row(W_act, w_dtype, d_ffn, d, i, row);
        for (t = 0; t < N; ++t) {
            double z = dot(row, X + t * d, d) + (b ? (double)b[i] : 0.0);
            c += (z > 0.0);
        }
        counts[i] = c;
    }
    free(row);
    return 0;
}

/* Gainless RMS normalisation of one vector: out = x / sqrt(mean(x^2) + eps). */
void oracle_rmsnorm(const double *x, int64_t d, double eps, double *out)
{
    int64_t k;
    double ss = 0.0;
    for (k = 0; k < d; ++k)
        ss += x[k] * x[k];
    double den = sqrt(ss / (double)d + eps);
    for (k = 0; k < d; ++k)
        out[k] = x[k] / den;
}

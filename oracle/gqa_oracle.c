/*
 * gqa_oracle.c -- plain, slow, fp64 CPU reference for grouped-query attention
 * (GQA) over a KV cache.
 *
 * TEST INFRASTRUCTURE.  Nothing in the product library calls, links or
 * includes this file.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header or constant
 * with the HIP path.
 *
 * What it computes (sources are the pages' titles and sections):
 *   - "GQA reading notes" (zhongzhuzhou.org), section "方法详解 > GQA 架构":
 *     query head h (1-indexed) belongs to group g(h) = ceil(h / (H/G)) and
 *     head_h = softmax(Q_h K_g(h)^T / sqrt(d_k)) V_g(h).  With 0-indexed heads
 *     that is g = floor(h / (H/G)): contiguous blocks of H/G query heads share
 *     one K/V head.
 *   - Same page, Algorithm 2 (GQA decode, step t), the per-query-head part:
 *     scores over every cached row of group g, softmax, weighted sum of V.
 *     Appending the new token's K/V happens before this call (the caller's
 *     seqlens[b] already counts it).
 *   - "从MHA到GQA" (gzher.com), section on why the question becomes how KV is
 *     stored: prefill attends every prompt position under a causal mask;
 *     decode attends one new query to all cached rows.
 *
 * Arithmetic: every input element is converted exactly to double (fp32 and
 * bf16 both widen exactly), all sums run in double in a fixed ascending
 * order, exp() is the C library's, and the softmax subtracts the row maximum
 * before exponentiating (equal to the plain softmax in exact arithmetic).
 *
 * Layouts (row-major, contiguous):
 *   decode : q [B,Hq,d]; k, v [B,Lmax,Hkv,d]; seqlens [B] (int32); out [rows,d]
 *   prefill: q [B,P,Hq,d]; k, v [B,P,Hkv,d]; out [rows,d]
 * dtype 0 = fp32 values, 1 = bf16 bit patterns (uint16).
 *
 * A row with zero valid keys (seqlens[b] == 0) is defined to be all zeros.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_F32 0
#define ORC_BF16 1

/* Exact widening of one stored element to double. */
static double orc_elem(const void *base, int64_t idx, int dtype)
{
    if (dtype == ORC_F32)
        return (double)((const float *)base)[idx];
    uint32_t bits = ((uint32_t)((const uint16_t *)base)[idx]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Set the OpenMP thread count of later calls (n >= 1); returns the previous one. */
int oracle_set_threads(int n)
{
    const int prev = oracle_num_threads();
#ifdef _OPENMP
    if (n >= 1)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
    return prev;
}

/*
 * Attention of one query row over n key/value rows.
 *   qrow   : element offset of the query row in q
 *   kv0    : element offset of key/value row 0 in k and v
 *   stride : element distance between consecutive key rows
 * w (length >= n) and acc (length >= d) are scratch.  Writes d values to out
 * and, if wout is not NULL, the normalised weights w_j / Z to wout.
 */
static void orc_attend(const void *q, int64_t qrow, const void *k, const void *v,
                       int64_t kv0, int64_t stride, int64_t n, int64_t d,
                       double scale, int dtype, double *w, double *acc,
                       double *out, double *wout)
{
    if (n <= 0) {
        for (int64_t c = 0; c < d; ++c)
            out[c] = 0.0;
        return;
    }
    /* scores s_j = scale * (q . k_j), dot product summed over c ascending */
    for (int64_t j = 0; j < n; ++j) {
        double dot = 0.0;
        const int64_t kr = kv0 + j * stride;
        for (int64_t c = 0; c < d; ++c)
            dot += orc_elem(q, qrow + c, dtype) * orc_elem(k, kr + c, dtype);
        w[j] = dot * scale;
    }
    /* softmax over j: subtract the maximum, exponentiate, sum j ascending */
    double m = w[0];
    for (int64_t j = 1; j < n; ++j)
        if (w[j] > m)
            m = w[j];
    double z = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        w[j] = exp(w[j] - m);
        z += w[j];
    }
    /* out_c = (sum_j w_j * v_jc) / Z, j ascending for every c */
    for (int64_t c = 0; c < d; ++c)
        acc[c] = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        const int64_t vr = kv0 + j * stride;
        for (int64_t c = 0; c < d; ++c)
            acc[c] += w[j] * orc_elem(v, vr + c, dtype);
    }
    for (int64_t c = 0; c < d; ++c)
        out[c] = acc[c] / z;
    if (wout)
        for (int64_t j = 0; j < n; ++j)
            wout[j] = w[j] / z;
}

static int orc_check_common(int64_t B, int64_t Hq, int64_t Hkv, int64_t d, int dtype)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || d <= 0)
        return -1;
    if (Hq % Hkv != 0)
        return -2; /* H must be divisible by the number of groups */
    if (dtype != ORC_F32 && dtype != ORC_BF16)
        return -3;
    return 0;
}

/*
 * Decode: one new query per sequence against that sequence's cached rows.
 * rows == NULL computes all B*Hq rows in order (nrows must be B*Hq);
 * otherwise rows[i] = b*Hq + h selects which (b, h) rows to compute.
 * Returns 0, or a negative code for invalid arguments.
 */
int oracle_decode(const void *q, const void *k, const void *v, const int32_t *seqlens,
                  int64_t B, int64_t Hq, int64_t Hkv, int64_t d, int64_t Lmax,
                  double scale, int dtype, const int64_t *rows, int64_t nrows,
                  double *out)
{
    int rc = orc_check_common(B, Hq, Hkv, d, dtype);
    if (rc)
        return rc;
    if (Lmax < 0)
        return -1;
    for (int64_t b = 0; b < B; ++b)
        if (seqlens[b] < 0 || seqlens[b] > Lmax)
            return -4;
    if (!rows && nrows != B * Hq)
        return -5;
    const int64_t gsize = Hq / Hkv;
    int err = 0;
#pragma omp parallel
    {
        double *w = (double *)malloc(sizeof(double) * (size_t)(Lmax > 0 ? Lmax : 1));
        double *acc = (double *)malloc(sizeof(double) * (size_t)d);
        if (!w || !acc) {
#pragma omp atomic write
            err = -6;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t i = 0; i < nrows; ++i) {
                const int64_t r = rows ? rows[i] : i;
                if (r < 0 || r >= B * Hq) {
#pragma omp atomic write
                    err = -5;
                    continue;
                }
                const int64_t b = r / Hq, h = r % Hq;
                const int64_t g = h / gsize; /* contiguous groups */
                const int64_t n = seqlens[b];
                orc_attend(q, (b * Hq + h) * d, k, v, ((b * Lmax) * Hkv + g) * d,
                           Hkv * d, n, d, scale, dtype, w, acc, out + i * d, NULL);
            }
        }
        free(w);
        free(acc);
    }
    return err;
}

/* Normalised softmax weights of decode row (b, h): wout[j], j < seqlens[b]. */
int oracle_decode_weights(const void *q, const void *k, const void *v, const int32_t *seqlens,
                          int64_t B, int64_t Hq, int64_t Hkv, int64_t d, int64_t Lmax,
                          double scale, int dtype, int64_t b, int64_t h, double *wout,
                          double *out)
{
    int rc = orc_check_common(B, Hq, Hkv, d, dtype);
    if (rc)
        return rc;
    if (b < 0 || b >= B || h < 0 || h >= Hq || seqlens[b] < 0 || seqlens[b] > Lmax)
        return -4;
    const int64_t g = h / (Hq / Hkv);
    const int64_t n = seqlens[b];
    double *w = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    double *acc = (double *)malloc(sizeof(double) * (size_t)d);
    if (!w || !acc) {
        free(w);
        free(acc);
        return -6;
    }
    orc_attend(q, (b * Hq + h) * d, k, v, ((b * Lmax) * Hkv + g) * d, Hkv * d, n, d,
               scale, dtype, w, acc, out, wout);
    free(w);
    free(acc);
    return 0;
}

/*
 * Prefill: every prompt position i of every sequence attends to keys
 * j in [0, i] (causal) or [0, P) (not causal).  rows == NULL computes all
 * B*P*Hq rows; otherwise rows[i] = (b*P + pos)*Hq + h.
 */
int oracle_prefill(const void *q, const void *k, const void *v, int64_t B, int64_t P,
                   int64_t Hq, int64_t Hkv, int64_t d, int causal, double scale, int dtype,
                   const int64_t *rows, int64_t nrows, double *out)
{
    int rc = orc_check_common(B, Hq, Hkv, d, dtype);
    if (rc)
        return rc;
    if (P < 0)
        return -1;
    if (!rows && nrows != B * P * Hq)
        return -5;
    const int64_t gsize = Hq / Hkv;
    int err = 0;
#pragma omp parallel
    {
        double *w = (double *)malloc(sizeof(double) * (size_t)(P > 0 ? P : 1));
        double *acc = (double *)malloc(sizeof(double) * (size_t)d);
        if (!w || !acc) {
#pragma omp atomic write
            err = -6;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t i = 0; i < nrows; ++i) {
                const int64_t r = rows ? rows[i] : i;
                if (r < 0 || r >= B * P * Hq) {
#pragma omp atomic write
                    err = -5;
                    continue;
                }
                const int64_t h = r % Hq, bp = r / Hq;
                const int64_t b = bp / P, pos = bp % P;
                const int64_t g = h / gsize;
                const int64_t n = causal ? pos + 1 : P;
                orc_attend(q, (bp * Hq + h) * d, k, v, ((b * P) * Hkv + g) * d, Hkv * d, n, d,
                           scale, dtype, w, acc, out + i * d, NULL);
            }
        }
        free(w);
        free(acc);
    }
    return err;
}

/*
 * Multi-head attention decode, written on its own: every query head h reads
 * its own K/V head h (k, v are [B,Lmax,H,d]).  No group index anywhere.
 * Same operation order as oracle_decode.
 */
int oracle_mha_decode(const void *q, const void *k, const void *v, const int32_t *seqlens,
                      int64_t B, int64_t H, int64_t d, int64_t Lmax, double scale, int dtype,
                      double *out)
{
    if (B < 0 || H <= 0 || d <= 0 || Lmax < 0 || (dtype != ORC_F32 && dtype != ORC_BF16))
        return -1;
    for (int64_t b = 0; b < B; ++b) {
        const int64_t n = seqlens[b];
        if (n < 0 || n > Lmax)
            return -4;
        for (int64_t h = 0; h < H; ++h) {
            double *o = out + (b * H + h) * d;
            if (n == 0) {
                for (int64_t c = 0; c < d; ++c)
                    o[c] = 0.0;
                continue;
            }
            double *s = (double *)malloc(sizeof(double) * (size_t)n);
            if (!s)
                return -6;
            for (int64_t j = 0; j < n; ++j) {
                double dot = 0.0;
                for (int64_t c = 0; c < d; ++c)
                    dot += orc_elem(q, (b * H + h) * d + c, dtype) *
                           orc_elem(k, ((b * Lmax + j) * H + h) * d + c, dtype);
                s[j] = dot * scale;
            }
            double m = s[0];
            for (int64_t j = 1; j < n; ++j)
                if (s[j] > m)
                    m = s[j];
            double z = 0.0;
            for (int64_t j = 0; j < n; ++j) {
                s[j] = exp(s[j] - m);
                z += s[j];
            }
            for (int64_t c = 0; c < d; ++c)
                o[c] = 0.0;
            for (int64_t j = 0; j < n; ++j)
                for (int64_t c = 0; c < d; ++c)
                    o[c] += s[j] * orc_elem(v, ((b * Lmax + j) * H + h) * d + c, dtype);
            for (int64_t c = 0; c < d; ++c)
                o[c] = o[c] / z;
            free(s);
        }
    }
    return 0;
}

/*
 * Multi-query attention decode, written on its own: all H query heads read
 * the single K/V head (k, v are [B,Lmax,1,d]).  Same operation order.
 */
int oracle_mqa_decode(const void *q, const void *k, const void *v, const int32_t *seqlens,
                      int64_t B, int64_t H, int64_t d, int64_t Lmax, double scale, int dtype,
                      double *out)
{
    if (B < 0 || H <= 0 || d <= 0 || Lmax < 0 || (dtype != ORC_F32 && dtype != ORC_BF16))
        return -1;
    for (int64_t b = 0; b < B; ++b) {
        const int64_t n = seqlens[b];
        if (n < 0 || n > Lmax)
            return -4;
        for (int64_t h = 0; h < H; ++h) {
            double *o = out + (b * H + h) * d;
            if (n == 0) {
                for (int64_t c = 0; c < d; ++c)
                    o[c] = 0.0;
                continue;
            }
            double *s = (double *)malloc(sizeof(double) * (size_t)n);
            if (!s)
                return -6;
            for (int64_t j = 0; j < n; ++j) {
                double dot = 0.0;
                for (int64_t c = 0; c < d; ++c)
                    dot += orc_elem(q, (b * H + h) * d + c, dtype) *
                           orc_elem(k, (b * Lmax + j) * d + c, dtype);
                s[j] = dot * scale;
            }
            double m = s[0];
            for (int64_t j = 1; j < n; ++j)
                if (s[j] > m)
                    m = s[j];
            double z = 0.0;
            for (int64_t j = 0; j < n; ++j) {
                s[j] = exp(s[j] - m);
                z += s[j];
            }
            for (int64_t c = 0; c < d; ++c)
                o[c] = 0.0;
            for (int64_t j = 0; j < n; ++j)
                for (int64_t c = 0; c < d; ++c)
                    o[c] += s[j] * orc_elem(v, (b * Lmax + j) * d + c, dtype);
            for (int64_t c = 0; c < d; ++c)
                o[c] = o[c] / z;
            free(s);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------
 * Extended decode: the next rows after the hot path.
 *
 *   - Several new query tokens per sequence (speculative verification, the
 *     multi-token decode step): q [B,T,Hq,d].  seqlens[b] = n counts every
 *     valid cached row, the T new ones included, so token t sits at position
 *     pos = n - T + t and attends keys j <= pos: the causal rule of prefill
 *     ("从MHA到GQA", causal mask section) applied to the new tokens.
 *   - Sliding window W > 0: only keys j in [pos - W + 1, pos].
 *   - Cache rows stored as fp32 / bf16 (kv_fmt = 0: q's dtype), or as OCP
 *     FP8 bytes, E4M3 (kv_fmt = 1) or E5M2 (kv_fmt = 2), whose value is
 *     decode(byte) * k_scale[g] for K and decode(byte) * v_scale[g] for V,
 *     one scale per KV head g.
 *   - Cache addressing: contiguous [B,Lmax,Hkv,d] (block_table == NULL), or
 *     paged: row j of sequence b is row j % bs of block
 *     block_table[b*max_blocks + j / bs] in a pool [nblocks,bs,Hkv,d].
 * rows == NULL computes all B*T*Hq rows, ordered ((b*T + t)*Hq + h);
 * otherwise rows[i] names one such index.  Same operation order as
 * oracle_decode (dot product over c ascending, maximum, exp, sums over j
 * ascending).  Returns 0 or a negative code.
 * ------------------------------------------------------------------------ */

/* OCP FP8 E4M3 (the "fn" variant: no infinities): sign, 4 exponent bits with
 * bias 7, 3 mantissa bits; exponent 0 is subnormal (m/8 * 2^-6); the all-ones
 * pattern S.1111.111 is NaN; the largest finite value is 1.75 * 2^8 = 448. */
double oracle_e4m3_value(unsigned byte)
{
    const int sgn = (byte >> 7) & 1, e = (byte >> 3) & 15, m = byte & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sgn ? -v : v;
}

/* OCP FP8 E5M2: sign, 5 exponent bits with bias 15, 2 mantissa bits, laid
 * out like the top byte of an IEEE half; exponent 0 is subnormal
 * (m/4 * 2^-14); exponent 31 holds +-infinity (m = 0) and NaN (m != 0); the
 * largest finite value is 1.75 * 2^15 = 57344. */
double oracle_e5m2_value(unsigned byte)
{
    const int sgn = (byte >> 7) & 1, e = (byte >> 2) & 31, m = byte & 3;
    double v;
    if (e == 31)
        v = m ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)m / 4.0, -14);
    else
        v = ldexp(1.0 + (double)m / 4.0, e - 15);
    return sgn ? -v : v;
}

/* Element offset of cached row j of sequence b, KV head g. */
static int64_t orc_row_ex(int64_t b, int64_t j, int64_t g, int64_t Hkv, int64_t d, int64_t Lmax,
                          const int32_t *block_table, int64_t max_blocks, int64_t bs)
{
    if (!block_table)
        return ((b * Lmax + j) * Hkv + g) * d;
    const int64_t blk = block_table[b * max_blocks + j / bs];
    return ((blk * bs + j % bs) * Hkv + g) * d;
}

static double orc_kv_elem(const void *base, int64_t idx, int dtype, int kv_fmt, double scale)
{
    if (kv_fmt == 1)
        return oracle_e4m3_value(((const uint8_t *)base)[idx]) * scale;
    if (kv_fmt == 2)
        return oracle_e5m2_value(((const uint8_t *)base)[idx]) * scale;
    return orc_elem(base, idx, dtype);
}

/*
 * Error-model terms of one output row, for the tests' derived tolerances only
 * (nothing here feeds the output).  With w_j / Z the softmax weights of the
 * row's n visible keys (w as left by the softmax above) and o its output:
 *   t[c]       = sum_j (w_j / Z) |v_jc - o_c|   (weighted spread of V about o)
 *   t[d + c]   = sum_j (w_j / Z) |v_jc|         (weighted mean magnitude of V)
 *   t[2d]      = scale * max_j sum_c |q_c| |k_jc|  (largest absolute score sum)
 * Rounding the weights by a relative e moves the output by at most e * t[c]
 * when numerator and denominator share the rounded weights, by e * t[d + c]
 * when only the numerator does; t[2d] bounds the size of a score's rounding.
 */
static void orc_error_terms(const void *q, int64_t qrow, const void *k, const void *v,
                            int64_t b, int64_t lo, int64_t n, int64_t g, int64_t Hkv, int64_t d,
                            int64_t Lmax, const int32_t *block_table, int64_t max_blocks,
                            int64_t bs, double scale, int dtype, int kv_fmt, double ks, double vs,
                            const double *w, double z, const double *o, double *t)
{
    double kappa = 0.0;
    for (int64_t c = 0; c < 2 * d; ++c)
        t[c] = 0.0;
    for (int64_t jj = 0; jj < n; ++jj) {
        const int64_t r = orc_row_ex(b, lo + jj, g, Hkv, d, Lmax, block_table, max_blocks, bs);
        const double wj = w[jj] / z;
        double sabs = 0.0;
        for (int64_t c = 0; c < d; ++c) {
            const double vc = orc_kv_elem(v, r + c, dtype, kv_fmt, vs);
            t[c] += wj * fabs(vc - o[c]);
            t[d + c] += wj * fabs(vc);
            sabs += fabs(orc_elem(q, qrow + c, dtype)) * fabs(orc_kv_elem(k, r + c, dtype, kv_fmt, ks));
        }
        if (sabs > kappa)
            kappa = sabs;
    }
    t[2 * d] = fabs(scale) * kappa;
}

int oracle_decode_ex(const void *q, const void *k, const void *v, const int32_t *seqlens,
                     int64_t B, int64_t T, int64_t Hq, int64_t Hkv, int64_t d, int64_t Lmax,
                     double scale, int dtype, int kv_fmt, const float *k_scale,
                     const float *v_scale, const int32_t *block_table, int64_t max_blocks,
                     int64_t bs, int64_t window, const int64_t *rows, int64_t nrows, double *out,
                     double *terms)
{
    int rc = orc_check_common(B, Hq, Hkv, d, dtype);
    if (rc)
        return rc;
    if (T <= 0 || Lmax < 0 || window < 0)
        return -1;
    if (kv_fmt < 0 || kv_fmt > 2 || (kv_fmt && (!k_scale || !v_scale)))
        return -1;
    if (block_table && (bs <= 0 || max_blocks <= 0 || Lmax > max_blocks * bs))
        return -1;
    for (int64_t b = 0; b < B; ++b)
        if (seqlens[b] < T || seqlens[b] > Lmax)
            return -4;
    if (!rows && nrows != B * T * Hq)
        return -5;
    const int64_t gsize = Hq / Hkv;
    int err = 0;
#pragma omp parallel
    {
        double *w = (double *)malloc(sizeof(double) * (size_t)(Lmax > 0 ? Lmax : 1));
        double *acc = (double *)malloc(sizeof(double) * (size_t)d);
        if (!w || !acc) {
#pragma omp atomic write
            err = -6;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t i = 0; i < nrows; ++i) {
                const int64_t r = rows ? rows[i] : i;
                if (r < 0 || r >= B * T * Hq) {
#pragma omp atomic write
                    err = -5;
                    continue;
                }
                const int64_t h = r % Hq, bt = r / Hq;
                const int64_t b = bt / T, t = bt % T;
                const int64_t g = h / gsize; /* contiguous groups */
                const int64_t pos = seqlens[b] - T + t;
                const int64_t lo = (window > 0 && pos - window + 1 > 0) ? pos - window + 1 : 0;
                const int64_t n = pos - lo + 1; /* keys lo .. pos */
                const double ks = kv_fmt ? (double)k_scale[g] : 1.0;
                const double vs = kv_fmt ? (double)v_scale[g] : 1.0;
                const int64_t qrow = (bt * Hq + h) * d;
                double *o = out + i * d;
                /* scores, j ascending over the visible keys */
                for (int64_t jj = 0; jj < n; ++jj) {
                    const int64_t kr = orc_row_ex(b, lo + jj, g, Hkv, d, Lmax, block_table, max_blocks, bs);
                    double dot = 0.0;
                    for (int64_t c = 0; c < d; ++c)
                        dot += orc_elem(q, qrow + c, dtype) * orc_kv_elem(k, kr + c, dtype, kv_fmt, ks);
                    w[jj] = dot * scale;
                }
                double m = w[0];
                for (int64_t jj = 1; jj < n; ++jj)
                    if (w[jj] > m)
                        m = w[jj];
                double z = 0.0;
                for (int64_t jj = 0; jj < n; ++jj) {
                    w[jj] = exp(w[jj] - m);
                    z += w[jj];
                }
                for (int64_t c = 0; c < d; ++c)
                    acc[c] = 0.0;
                for (int64_t jj = 0; jj < n; ++jj) {
                    const int64_t vr = orc_row_ex(b, lo + jj, g, Hkv, d, Lmax, block_table, max_blocks, bs);
                    for (int64_t c = 0; c < d; ++c)
                        acc[c] += w[jj] * orc_kv_elem(v, vr + c, dtype, kv_fmt, vs);
                }
                for (int64_t c = 0; c < d; ++c)
                    o[c] = acc[c] / z;
                if (terms)
                    orc_error_terms(q, qrow, k, v, b, lo, n, g, Hkv, d, Lmax, block_table,
                                    max_blocks, bs, scale, dtype, kv_fmt, ks, vs, w, z, o,
                                    terms + i * (2 * d + 1));
            }
        }
        free(w);
        free(acc);
    }
    return err;
}

/*
 * Append (Algorithm 2 of "GQA reading notes", the cache-update lines): the T
 * new K/V rows of sequence b, k_new/v_new [B,T,Hkv,d], are stored at cache
 * rows seqlens[b] - T + t (seqlens counts them already), contiguous or paged
 * as in oracle_decode_ex.  elt = bytes per stored element (4 fp32, 2 bf16,
 * 1 FP8); the rows are copied byte for byte.
 */
int oracle_append(void *k_cache, void *v_cache, const void *k_new, const void *v_new,
                  const int32_t *seqlens, int64_t B, int64_t T, int64_t Hkv, int64_t d,
                  int64_t Lmax, int64_t elt, const int32_t *block_table, int64_t max_blocks,
                  int64_t bs)
{
    if (B < 0 || T <= 0 || Hkv <= 0 || d <= 0 || Lmax < 0 || (elt != 1 && elt != 2 && elt != 4))
        return -1;
    if (block_table && (bs <= 0 || max_blocks <= 0 || Lmax > max_blocks * bs))
        return -1;
    for (int64_t b = 0; b < B; ++b)
        if (seqlens[b] < T || seqlens[b] > Lmax)
            return -4;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t t = 0; t < T; ++t)
            for (int64_t g = 0; g < Hkv; ++g) {
                const int64_t j = seqlens[b] - T + t;
                const int64_t dst = orc_row_ex(b, j, g, Hkv, d, Lmax, block_table, max_blocks, bs);
                const int64_t src = ((b * T + t) * Hkv + g) * d;
                memcpy((char *)k_cache + dst * elt, (const char *)k_new + src * elt, (size_t)(d * elt));
                memcpy((char *)v_cache + dst * elt, (const char *)v_new + src * elt, (size_t)(d * elt));
            }
    return 0;
}

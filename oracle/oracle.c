/*
 * CPU oracle for the quantized decode matvec — TEST INFRASTRUCTURE ONLY.
 * See oracle.h for the sources, the precision rules and the contract.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- O1 -- */
/* [P3] §3 "Decode FP16 control tensors", written from the IEEE 754 binary16
 * format rather than from bit surgery.  A code is a sign s (bit 15), a
 * biased exponent E (bits 10..14, bias 15) and a fraction F (bits 0..9):
 *   E = 0       value (-1)^s * F * 2^-24          (zero or subnormal)
 *   E = 1..30   value (-1)^s * (1024 + F) * 2^(E - 25)
 *   E = 31      infinity when F = 0, otherwise NaN.
 * The magnitude is formed with ldexp in double; every binary16 value is
 * exactly representable in binary32, so the final conversion is exact. */
float oracle_f16(uint16_t h)
{
    int negative = (h >> 15) & 1;
    int E = (h >> 10) & 31;
    int F = h & 1023;
    double magnitude;
    if (E == 31)
        magnitude = F == 0 ? HUGE_VAL : NAN;
    else if (E == 0)
        magnitude = ldexp((double)F, -24);
    else
        magnitude = ldexp((double)(1024 + F), E - 25);
    return (float)(negative ? -magnitude : magnitude);
}

/* ------------------------------------------------------------ O3 core -- */
/* [P1] §1: for stride = 1, 2, 4, ... < n, pair element j of each 2*stride
 * block with element j + stride and replace them by their sum and their
 * difference.  Each store rounds to fp32 (a Float32Array on the page). */
void oracle_fwht(float *x, int64_t n)
{
    for (int64_t stride = 1; stride < n; stride <<= 1) {
        for (int64_t base = 0; base < n; base += stride << 1) {
            for (int64_t j = 0; j < stride; j++) {
                float a = x[base + j];
                float b = x[base + j + stride];
                x[base + j] = a + b;
                x[base + j + stride] = a - b;
            }
        }
    }
}

static int is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

static int cq_ok(const oracle_cq *m)
{
    if (!m || !m->packed || !m->norms || !m->codebook) return 0;
    if (m->bits < 2 || m->bits > 5) return 0;
    if (!is_pow2(m->group)) return 0;
    if (m->input < 0 || m->input > m->input_padded) return 0;
    if (m->input_padded <= 0 || m->input_padded % m->group != 0) return 0;
    if (m->output < 0) return 0;
    if (m->row_bytes * 8 < m->input_padded * m->bits) return 0;
    return 1;
}

/* ---------------------------------------------------------------- O2 -- */
/* Index bit j of column col is bit (bits*col + j) of the row's byte stream,
 * where bit t lives in byte t/8 at position t%8 (least significant first).
 * For 2-bit this is the crumb rule of [P1] §3 (crumb k of a byte is
 * (byte >> 2k) & 3); for 4-bit the low nibble holds the even column. */
uint32_t oracle_cq_index(const oracle_cq *m, int64_t row, int64_t col)
{
    const uint8_t *r = m->packed + row * m->row_bytes;
    uint32_t idx = 0;
    for (int64_t j = 0; j < m->bits; j++) {
        int64_t t = m->bits * col + j;
        uint32_t bit = (r[t >> 3] >> (t & 7)) & 1u;
        idx |= bit << j;
    }
    return idx;
}

int oracle_cq_unpack_row(const oracle_cq *m, int64_t row, uint8_t *idx)
{
    if (!cq_ok(m) || row < 0 || row >= m->output) return -1;
    for (int64_t c = 0; c < m->input_padded; c++)
        idx[c] = (uint8_t)oracle_cq_index(m, row, c);
    return 0;
}

/* Multiply by 1/sqrt(group) the way the page does: the scale is a double,
 * the product is formed in double and stored back to fp32. */
static float scale_store(float v, int64_t group)
{
    double scale = 1.0 / sqrt((double)group);
    return (float)((double)v * scale);
}

/* ---------------------------------------------------------------- O3 -- */
/* [P1] §2: zero-pad to input_padded, transform every group, normalize. */
int oracle_cq_prepare(const oracle_cq *m, const float *x, float *p)
{
    if (!cq_ok(m)) return -1;
    for (int64_t k = 0; k < m->input_padded; k++) p[k] = k < m->input ? x[k] : 0.0f;
    for (int64_t start = 0; start < m->input_padded; start += m->group) {
        oracle_fwht(p + start, m->group);
        for (int64_t k = 0; k < m->group; k++) p[start + k] = scale_store(p[start + k], m->group);
    }
    return 0;
}

/* ---------------------------------------------------------------- O4 -- */
/* [P1] §3: for each row and group, the group's sum of codebook[index] times
 * prepared[column], times the fp16 norm of (row, group), added to the row
 * sum.  JavaScript sums are doubles: accumulate in fp64. */
int oracle_cq_matvec(const oracle_cq *m, const float *p, int64_t row_begin,
                     int64_t row_count, double *y, double *mag)
{
    if (!cq_ok(m) || row_begin < 0 || row_count < 0 || row_begin + row_count > m->output)
        return -1;
    int64_t n_groups = m->input_padded / m->group;
    for (int64_t i = 0; i < row_count; i++) {
        int64_t row = row_begin + i;
        double acc = 0.0, amag = 0.0;
        for (int64_t g = 0; g < n_groups; g++) {
            double part = 0.0, apart = 0.0;
            for (int64_t k = g * m->group; k < (g + 1) * m->group; k++) {
                double term = (double)m->codebook[oracle_cq_index(m, row, k)] * (double)p[k];
                part += term;
                apart += fabs(term);
            }
            double norm = (double)oracle_f16(m->norms[row * n_groups + g]);
            acc += norm * part;
            amag += fabs(norm) * apart;
        }
        if (y) y[i] = acc;
        if (mag) mag[i] = amag;
    }
    return 0;
}

/* ---------------------------------------------------------------- O5 -- */
/* [P1] "Row gather": per group, each codebook value times the group norm
 * (an fp32 product), then the normalized transform (the unnormalized
 * butterfly, then the same 1/sqrt(group) store as prepare); the columns below
 * the unpadded width are the dense row. */
int oracle_cq_dequantize_row(const oracle_cq *m, int64_t row, float *out)
{
    if (!cq_ok(m) || row < 0 || row >= m->output) return -1;
    int64_t n_groups = m->input_padded / m->group;
    float *t = (float *)malloc(sizeof(float) * (size_t)m->input_padded);
    if (!t) return -1;
    for (int64_t g = 0; g < n_groups; g++) {
        float norm = oracle_f16(m->norms[row * n_groups + g]);
        float *tg = t + g * m->group;
        for (int64_t k = 0; k < m->group; k++)
            tg[k] = m->codebook[oracle_cq_index(m, row, g * m->group + k)] * norm;
        oracle_fwht(tg, m->group);
        for (int64_t k = 0; k < m->group; k++) tg[k] = scale_store(tg[k], m->group);
    }
    memcpy(out, t, sizeof(float) * (size_t)m->input);
    free(t);
    return 0;
}

/* ---------------------------------------------------------------- O6 -- */
int oracle_cq_gather(const oracle_cq *m, const int32_t *ids, int64_t n,
                     float *out, double *gmag)
{
    if (!cq_ok(m) || n < 0) return -1;
    int64_t n_groups = m->input_padded / m->group;
    double inv = 1.0 / sqrt((double)m->group);
    for (int64_t i = 0; i < n; i++) {
        if (ids[i] < 0 || ids[i] >= m->output) return -1;
        if (oracle_cq_dequantize_row(m, ids[i], out + i * m->input) != 0) return -1;
        if (!gmag) continue;
        for (int64_t g = 0; g < n_groups; g++) {
            double norm = fabs((double)oracle_f16(m->norms[(int64_t)ids[i] * n_groups + g]));
            double s = 0.0;
            for (int64_t k = g * m->group; k < (g + 1) * m->group; k++)
                s += fabs((double)m->codebook[oracle_cq_index(m, ids[i], k)]) * norm;
            for (int64_t k = g * m->group; k < (g + 1) * m->group && k < m->input; k++)
                gmag[i * m->input + k] = s * inv;
        }
    }
    return 0;
}

/* ---------------------------------------------------------------- O7 -- */
int oracle_cq_dense_matvec(const oracle_cq *m, const float *x, int64_t row_begin,
                           int64_t row_count, double *y)
{
    if (!cq_ok(m) || row_begin < 0 || row_count < 0 || row_begin + row_count > m->output)
        return -1;
    float *row = (float *)malloc(sizeof(float) * (size_t)(m->input > 0 ? m->input : 1));
    if (!row) return -1;
    for (int64_t i = 0; i < row_count; i++) {
        if (oracle_cq_dequantize_row(m, row_begin + i, row) != 0) { free(row); return -1; }
        double acc = 0.0;
        for (int64_t c = 0; c < m->input; c++) acc += (double)row[c] * (double)x[c];
        y[i] = acc;
    }
    free(row);
    return 0;
}

/* ---------------------------------------------------------------- O8 -- */
/* [P4] Step 1 / Step 4: sign bit, 4-bit exponent e, 3-bit mantissa m.
 * e = 0 is subnormal: (m/8) * 2^(1-7); otherwise (1 + m/8) * 2^(e-7).
 * The e = 15 clamp bounds the magnitude at 448, so only mantissa 7 (which
 * would give 480) changes. */
float oracle_e4m3(uint8_t code)
{
    int s = code >> 7;
    int e = (code >> 3) & 15;
    int mant = code & 7;
    double v;
    if (e == 0)
        v = ldexp((double)mant / 8.0, 1 - 7);
    else
        v = ldexp(1.0 + (double)mant / 8.0, e - 7);
    if (v > 448.0) v = 448.0;
    return (float)(s ? -v : v);
}

/* ---------------------------------------------------------------- O9 -- */
/* [P4] Step 1: an E8M0 block scale is the power of two 2^(e-127); the byte
 * 255 has no power-of-two meaning and decodes to NaN. */
float oracle_e8m0(uint8_t e)
{
    if (e == 255) return NAN;
    return (float)ldexp(1.0, (int)e - 127);
}

/* --------------------------------------------------------------- O10 -- */
/* [P4] Step 1: element (r, c) of the weight takes the scale
 * S[floor(r*SR/R)][floor(c*SC/C)]; the dot runs over all C columns. */
int oracle_f8_matvec(const uint8_t *w, int64_t R, int64_t C, const uint8_t *s,
                     int64_t SR, int64_t SC, const float *x, int64_t row_begin,
                     int64_t row_count, double *y, double *mag)
{
    if (!w || !s || !x || R < 0 || C < 0 || SR < 1 || SC < 1 || SR > (R > 0 ? R : 1) ||
        SC > (C > 0 ? C : 1) || row_begin < 0 || row_count < 0 || row_begin + row_count > R)
        return -1;
    for (int64_t i = 0; i < row_count; i++) {
        int64_t r = row_begin + i;
        int64_t sr = (r * SR) / R;
        double acc = 0.0, amag = 0.0;
        for (int64_t c = 0; c < C; c++) {
            int64_t sc = (c * SC) / C;
            double term = (double)oracle_e4m3(w[r * C + c]) *
                          (double)oracle_e8m0(s[sr * SC + sc]) * (double)x[c];
            acc += term;
            amag += fabs(term);
        }
        if (y) y[i] = acc;
        if (mag) mag[i] = amag;
    }
    return 0;
}

/* --------------------------------------------------------------- O11 -- */
uint32_t oracle_xorshift32(uint32_t s)
{
    s ^= s << 13;
    s ^= s >> 17;
    s ^= s << 5;
    return s;
}

/* --------------------------------------------------------------- O12 -- */
/* [P4] work item 3: the k best candidates for sampling.  A plain sort of
 * all indices by (value descending, index ascending), NaNs last. */
static const float *topk_logits;

static int topk_cmp(const void *pa, const void *pb)
{
    int64_t a = *(const int64_t *)pa, b = *(const int64_t *)pb;
    float va = topk_logits[a], vb = topk_logits[b];
    int na = isnan(va), nb = isnan(vb);
    if (na != nb) return na ? 1 : -1;          /* NaN after every number */
    if (!na && va != vb) return va > vb ? -1 : 1;
    return a < b ? -1 : (a > b ? 1 : 0);       /* equal values: lower index */
}

int oracle_topk(const float *logits, int64_t n, int64_t k, int32_t *ids, float *vals)
{
    if (!logits || n < 1 || k < 1 || k > n) return -1;
    int64_t *order = (int64_t *)malloc(sizeof(int64_t) * (size_t)n);
    if (!order) return -1;
    for (int64_t i = 0; i < n; i++) order[i] = i;
    topk_logits = logits;
    qsort(order, (size_t)n, sizeof(int64_t), topk_cmp);
    for (int64_t i = 0; i < k; i++) {
        ids[i] = (int32_t)order[i];
        vals[i] = logits[order[i]];
    }
    free(order);
    return 0;
}

/* --------------------------------------------------------------- O13 -- */
/* [P4] "Step 3 done": a softmax over the candidates at the temperature,
 * then the inverse of its cumulative sum at the uniform draw. */
int32_t oracle_sample_u(const float *vals, const int32_t *ids, int64_t k,
                        double temperature, double u)
{
    if (temperature <= 0.0 || k == 1 || !isfinite(vals[0])) return ids[0];
    double S = 0.0;
    for (int64_t i = 0; i < k; i++)
        S += isnan(vals[i]) ? 0.0 : exp(((double)vals[i] - (double)vals[0]) / temperature);
    double target = u * S, run = 0.0;
    for (int64_t i = 0; i < k; i++) {
        run += isnan(vals[i]) ? 0.0 : exp(((double)vals[i] - (double)vals[0]) / temperature);
        if (target < run) return ids[i];
    }
    return ids[k - 1];
}

int32_t oracle_sample(const float *vals, const int32_t *ids, int64_t k,
                      double temperature, uint32_t *state)
{
    *state = oracle_xorshift32(*state);
    return oracle_sample_u(vals, ids, k, temperature, (double)*state / 4294967296.0);
}

/* --------------------------------------------------------------- O14 -- */
/* [P4] "Step 4 done": the I8 matvec widens int8 weights and applies one E8M0
 * scale per group of G consecutive columns of a row (G = 16 on the page).
 * Row r's scales are s[r][0 .. ceil(C/G)). */
int oracle_i8_matvec(const int8_t *w, int64_t R, int64_t C, const uint8_t *s, int64_t G,
                     const float *x, int64_t row_begin, int64_t row_count, double *y,
                     double *mag)
{
    if (!w || !s || !x || R < 0 || C < 1 || G < 1 || row_begin < 0 || row_count < 0 ||
        row_begin + row_count > R)
        return -1;
    int64_t ns = (C + G - 1) / G;
    for (int64_t i = 0; i < row_count; i++) {
        int64_t r = row_begin + i;
        double acc = 0.0, amag = 0.0;
        for (int64_t c = 0; c < C; c++) {
            double term = (double)w[r * C + c] * (double)oracle_e8m0(s[r * ns + c / G]) *
                          (double)x[c];
            acc += term;
            amag += fabs(term);
        }
        if (y) y[i] = acc;
        if (mag) mag[i] = amag;
    }
    return 0;
}

/* --------------------------------------------------------------- O15 -- */
/* [P1] §7 "Per-vector int8 quantization" (storeInt8): the largest magnitude,
 * floored at 1e-12, over 127 is the vector's scale (a JavaScript number;
 * the scale array stores it as fp32); every element divided by that scale
 * (in fp64) and rounded to the nearest integer, ties to even, is stored in
 * an Int8Array.  The page's arithmetic is JavaScript's: Math.max turns the
 * maximum into NaN when an element is NaN, and the Int8Array store turns NaN
 * into 0. */
static double js_max(double a, double b)
{
    if (isnan(a) || isnan(b)) return NAN;
    return a > b ? a : b;
}

static int8_t js_to_int8(double v)
{
    if (!isfinite(v)) return 0;
    double t = fmod(trunc(v), 256.0);        /* ToInt8: truncate, wrap mod 2^8 */
    if (t < 0) t += 256.0;
    return (int8_t)(t >= 128.0 ? t - 256.0 : t);
}

int oracle_store_int8(const float *v, int64_t n, int8_t *q, float *scale_out)
{
    if (!v || !q || !scale_out || n < 0) return -1;
    double maximum = 1e-12;
    for (int64_t i = 0; i < n; i++) maximum = js_max(maximum, fabs((double)v[i]));
    double scale = maximum / 127.0;
    *scale_out = (float)scale;
    for (int64_t i = 0; i < n; i++) q[i] = js_to_int8(nearbyint((double)v[i] / scale));
    return 0;
}

/* --------------------------------------------------------------- O16 -- */
/* [P1] §7: a key dot against an int8 cache row multiplies the cached
 * integers by the row's scale: y = scale[r] * sum_j K[r][j] * x[j]. */
int oracle_int8_dot(const int8_t *K, const float *scales, int64_t R, int64_t d,
                    const float *x, int64_t row_begin, int64_t row_count, double *y,
                    double *mag)
{
    if (!K || !scales || !x || R < 0 || d < 0 || row_begin < 0 || row_count < 0 ||
        row_begin + row_count > R)
        return -1;
    for (int64_t i = 0; i < row_count; i++) {
        int64_t r = row_begin + i;
        double acc = 0.0, amag = 0.0;
        for (int64_t j = 0; j < d; j++) {
            acc += (double)K[r * d + j] * (double)x[j];
            amag += fabs((double)K[r * d + j] * (double)x[j]);
        }
        if (y) y[i] = (double)scales[r] * acc;
        if (mag) mag[i] = fabs((double)scales[r]) * amag;
    }
    return 0;
}

/* --------------------------------------------------------------- O17 -- */
/* [P1] §8 "Hadamard MLP", from the normalized block input n[hidden] on:
 * z = n zero-padded to H; z *= d1; normalized FWHT; z = silu(d2 * z);
 * normalized FWHT; z *= d3; block output = resid + z[0 .. hidden); the update
 * subtracts u when u is given.  Float32Array stores round every array write
 * to fp32; products, silu and the 1/sqrt(H) scale are formed in fp64 first
 * (JavaScript numbers).  silu(t) = t / (1 + exp(-t)).  mag[i] bounds what
 * the output's rounding scales with: |resid| + |u| + |d3| / sqrt(H) * sum |silu|. */
static void normalized_fwht(float *z, int64_t H)
{
    oracle_fwht(z, H);
    double scale = 1.0 / sqrt((double)H);
    for (int64_t i = 0; i < H; i++) z[i] = (float)((double)z[i] * scale);
}

int oracle_hadamard_mlp(const float *n, int64_t hidden, int64_t H, const float *d1,
                        const float *d2, const float *d3, const float *resid,
                        const float *u, float *out, double *mag)
{
    if (!n || !d1 || !d2 || !d3 || !resid || !out || hidden < 0 || H < 1 || hidden > H ||
        !is_pow2(H))
        return -1;
    float *z = (float *)malloc(sizeof(float) * (size_t)H);
    if (!z) return -1;
    for (int64_t i = 0; i < H; i++) z[i] = i < hidden ? n[i] : 0.0f;
    for (int64_t i = 0; i < H; i++) z[i] = (float)((double)z[i] * (double)d1[i]);
    normalized_fwht(z, H);
    double l1 = 0.0;
    for (int64_t i = 0; i < H; i++) {
        double t = (double)d2[i] * (double)z[i];
        z[i] = (float)(t / (1.0 + exp(-t)));
        l1 += fabs((double)z[i]);
    }
    normalized_fwht(z, H);
    for (int64_t i = 0; i < H; i++) z[i] = (float)((double)z[i] * (double)d3[i]);
    for (int64_t i = 0; i < hidden; i++) {
        float block = (float)((double)resid[i] + (double)z[i]);
        out[i] = u ? (float)((double)block - (double)u[i]) : block;
        if (mag)
            mag[i] = fabs((double)resid[i]) + (u ? fabs((double)u[i]) : 0.0) +
                     fabs((double)d3[i]) / sqrt((double)H) * l1;
    }
    free(z);
    return 0;
}

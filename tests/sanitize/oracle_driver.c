/*
 * Drives every function of the CPU oracle (oracle/oracle.c) over small,
 * exactly sized heap buffers, valid and invalid shapes, and special values,
 * so that a build with AddressSanitizer and UndefinedBehaviorSanitizer sees
 * every code path.  It checks no values (the oracle's pins do that); it
 * exits 0 when it ran to the end, and the sanitizers abort it on the first
 * finding.  Built and run by tests/test_sanitizers.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static uint64_t lcg_state = 0x243F6A8885A308D3ull;

static uint32_t next32(void)
{
    lcg_state = lcg_state * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(lcg_state >> 32);
}

static float normalish(void) { return ((float)(next32() % 20001) - 10000.0f) / 3000.0f; }

static void *xmalloc(size_t n) { return malloc(n ? n : 1); }

static double sink = 0.0;

static void drive_cq(int64_t output, int64_t input, int64_t input_padded, int64_t group,
                     int64_t bits, int64_t extra_row_bytes)
{
    int64_t row_bytes = (input_padded * bits + 7) / 8 + extra_row_bytes;
    int64_t ng = input_padded / group;
    uint8_t *packed = xmalloc((size_t)(output * row_bytes));
    uint16_t *norms = xmalloc((size_t)(output * ng) * 2);
    float *cb = xmalloc(sizeof(float) << bits);
    for (int64_t i = 0; i < output * row_bytes; i++) packed[i] = (uint8_t)next32();
    for (int64_t i = 0; i < output * ng; i++) norms[i] = (uint16_t)(0x3800 + next32() % 0x800);
    for (int64_t i = 0; i < (1 << bits); i++) cb[i] = normalish();
    oracle_cq m = {output, input, input_padded, group, bits, row_bytes, packed, norms, cb};

    float *x = xmalloc(sizeof(float) * (size_t)input);
    float *p = xmalloc(sizeof(float) * (size_t)input_padded);
    for (int64_t i = 0; i < input; i++) x[i] = normalish();
    if (oracle_cq_prepare(&m, x, p) != 0) abort();

    double *y = xmalloc(sizeof(double) * (size_t)output);
    double *mag = xmalloc(sizeof(double) * (size_t)output);
    if (oracle_cq_matvec(&m, p, 0, output, y, mag) != 0) abort();
    if (output > 1 && oracle_cq_matvec(&m, p, 1, output - 1, y, NULL) != 0) abort();
    if (oracle_cq_dense_matvec(&m, x, 0, output, y) != 0) abort();
    for (int64_t r = 0; r < output; r++) sink += y[r] + mag[r];

    uint8_t *idx = xmalloc((size_t)input_padded);
    float *row = xmalloc(sizeof(float) * (size_t)input);
    for (int64_t r = 0; r < output; r++) {
        if (oracle_cq_unpack_row(&m, r, idx) != 0) abort();
        if (oracle_cq_dequantize_row(&m, r, row) != 0) abort();
    }
    int64_t n_ids = 5;
    int32_t *ids = xmalloc(sizeof(int32_t) * (size_t)n_ids);
    for (int64_t i = 0; i < n_ids; i++) ids[i] = output ? (int32_t)(next32() % output) : 0;
    float *g = xmalloc(sizeof(float) * (size_t)(n_ids * input));
    double *gmag = xmalloc(sizeof(double) * (size_t)(n_ids * input));
    if (output && oracle_cq_gather(&m, ids, n_ids, g, gmag) != 0) abort();
    if (output && oracle_cq_gather(&m, ids, n_ids, g, NULL) != 0) abort();

    /* invalid shapes and ranges are refused without reading the arrays */
    oracle_cq bad = m;
    bad.bits = 6;
    if (oracle_cq_prepare(&bad, x, p) == 0) abort();
    bad = m;
    bad.group = 3;
    if (oracle_cq_matvec(&bad, p, 0, output, y, mag) == 0) abort();
    bad = m;
    bad.row_bytes = 0;
    if (oracle_cq_unpack_row(&bad, 0, idx) == 0) abort();
    if (oracle_cq_matvec(&m, p, output, 1, y, mag) == 0) abort();
    if (oracle_cq_unpack_row(&m, output, idx) == 0) abort();
    if (oracle_cq_dequantize_row(&m, -1, row) == 0) abort();

    free(packed), free(norms), free(cb), free(x), free(p), free(y), free(mag), free(idx);
    free(row), free(ids), free(g), free(gmag);
}

static void drive_f8_i8(int64_t R, int64_t C, int64_t SR, int64_t SC, int64_t G)
{
    uint8_t *w = xmalloc((size_t)(R * C));
    uint8_t *s = xmalloc((size_t)(SR * SC));
    float *x = xmalloc(sizeof(float) * (size_t)C);
    double *y = xmalloc(sizeof(double) * (size_t)R);
    double *mag = xmalloc(sizeof(double) * (size_t)R);
    for (int64_t i = 0; i < R * C; i++) w[i] = (uint8_t)next32();
    for (int64_t i = 0; i < SR * SC; i++) s[i] = (uint8_t)(120 + next32() % 11);
    for (int64_t i = 0; i < C; i++) x[i] = normalish();
    if (oracle_f8_matvec(w, R, C, s, SR, SC, x, 0, R, y, mag) != 0) abort();
    if (oracle_f8_matvec(w, R, C, s, SR, SC, x, R - 1, 1, NULL, mag) != 0) abort();
    for (int64_t r = 0; r < R; r++) sink += y[r] + mag[r];

    int64_t ns = (C + G - 1) / G;
    uint8_t *si = xmalloc((size_t)(R * ns));
    for (int64_t i = 0; i < R * ns; i++) si[i] = (uint8_t)(120 + next32() % 11);
    if (oracle_i8_matvec((const int8_t *)w, R, C, si, G, x, 0, R, y, mag) != 0) abort();
    for (int64_t r = 0; r < R; r++) sink += y[r] + mag[r];

    float *sc = xmalloc(sizeof(float) * (size_t)R);
    for (int64_t r = 0; r < R; r++) sc[r] = normalish();
    if (oracle_int8_dot((const int8_t *)w, sc, R, C, x, 0, R, y, mag) != 0) abort();
    for (int64_t r = 0; r < R; r++) sink += y[r] + mag[r];
    free(w), free(s), free(x), free(y), free(mag), free(si), free(sc);
}

static void drive_sampling(int64_t n)
{
    float *logits = xmalloc(sizeof(float) * (size_t)n);
    for (int64_t i = 0; i < n; i++) logits[i] = (float)(next32() % 7) - 3.0f;
    if (n > 3) {
        logits[0] = NAN;
        logits[1] = -INFINITY;
        logits[2] = -0.0f;
    }
    for (int64_t k = 1; k <= n && k <= 64; k += 7) {
        int32_t *ids = xmalloc(sizeof(int32_t) * (size_t)k);
        float *vals = xmalloc(sizeof(float) * (size_t)k);
        if (oracle_topk(logits, n, k, ids, vals) != 0) abort();
        uint32_t st = 12345u;
        for (int j = 0; j < 4; j++) sink += oracle_sample(vals, ids, k, 0.8, &st);
        sink += oracle_sample_u(vals, ids, k, 0.0, 0.5) + oracle_sample_u(vals, ids, k, 2.5, 0.999);
        free(ids), free(vals);
    }
    int32_t one_id;
    float one_val;
    if (oracle_topk(logits, n, n + 1, &one_id, &one_val) == 0) abort();
    free(logits);
}

int main(void)
{
    for (uint32_t h = 0; h < 65536; h++) sink += oracle_f16((uint16_t)h) == 0.0f;
    for (int c = 0; c < 256; c++) sink += oracle_e4m3((uint8_t)c) + (double)!isnan(oracle_e8m0((uint8_t)c));
    for (int64_t n = 1; n <= 1024; n <<= 1) {
        float *v = xmalloc(sizeof(float) * (size_t)n);
        for (int64_t i = 0; i < n; i++) v[i] = normalish();
        oracle_fwht(v, n);
        sink += v[n - 1];
        free(v);
    }
    uint32_t s = 1;
    for (int i = 0; i < 1000; i++) s = oracle_xorshift32(s);
    sink += s;

    drive_cq(5, 3, 4, 4, 2, 0);
    drive_cq(7, 13, 16, 4, 3, 0);
    drive_cq(6, 30, 32, 8, 5, 3);
    drive_cq(9, 64, 64, 16, 4, 8);
    drive_cq(4, 100, 128, 32, 3, 5);
    drive_cq(3, 200, 256, 64, 2, 0);
    drive_cq(4, 250, 256, 128, 5, 1);
    drive_cq(3, 256, 256, 256, 4, 0);
    drive_cq(2, 1, 1, 1, 2, 0);
    drive_cq(0, 16, 16, 16, 4, 0);
    drive_cq(3, 0, 8, 8, 4, 0);

    drive_f8_i8(10, 7, 3, 2, 3);
    drive_f8_i8(33, 128, 33, 8, 16);
    drive_f8_i8(40, 768, 4, 3, 7);
    drive_f8_i8(1, 1, 1, 1, 1);

    drive_sampling(1);
    drive_sampling(5);
    drive_sampling(300);

    /* storeInt8 on ordinary, tied, empty-magnitude and special vectors */
    float v[9] = {0.5f, -1.5f, 2.5f, 0.0f, -63.5f, 127.0f, 1e-30f, -0.0f, 3.0f};
    int8_t q[9];
    float scale;
    if (oracle_store_int8(v, 9, q, &scale) != 0) abort();
    v[3] = NAN;
    if (oracle_store_int8(v, 9, q, &scale) != 0) abort();
    v[3] = INFINITY;
    if (oracle_store_int8(v, 9, q, &scale) != 0) abort();
    if (oracle_store_int8(v, 0, q, &scale) != 0) abort();
    sink += scale + q[0];

    /* the Hadamard MLP with and without u, hidden below H, and H = 1 */
    for (int64_t H = 1; H <= 1024; H <<= 3) {
        int64_t hidden = H > 2 ? H / 2 + 1 : H;
        float *n = xmalloc(sizeof(float) * (size_t)hidden), *resid = xmalloc(sizeof(float) * (size_t)hidden);
        float *u = xmalloc(sizeof(float) * (size_t)hidden), *out = xmalloc(sizeof(float) * (size_t)hidden);
        float *d1 = xmalloc(sizeof(float) * (size_t)H), *d2 = xmalloc(sizeof(float) * (size_t)H);
        float *d3 = xmalloc(sizeof(float) * (size_t)H);
        double *mag = xmalloc(sizeof(double) * (size_t)hidden);
        for (int64_t i = 0; i < hidden; i++) n[i] = normalish(), resid[i] = normalish(), u[i] = normalish();
        for (int64_t i = 0; i < H; i++) d1[i] = normalish(), d2[i] = normalish(), d3[i] = normalish();
        if (oracle_hadamard_mlp(n, hidden, H, d1, d2, d3, resid, u, out, mag) != 0) abort();
        if (oracle_hadamard_mlp(n, hidden, H, d1, d2, d3, resid, NULL, out, NULL) != 0) abort();
        if (oracle_hadamard_mlp(n, hidden, 3 * H, d1, d2, d3, resid, NULL, out, NULL) == 0) abort();
        sink += out[0] + mag[0];
        free(n), free(resid), free(u), free(out), free(d1), free(d2), free(d3), free(mag);
    }
    printf("oracle driver done (%g)\n", sink);
    return 0;
}

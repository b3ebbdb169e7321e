/*
 * CPU oracle for the quantized decode matvec — TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct C implementation of what the HIP path
 * computes.  Only the test suite, the smoke check and the benchmark's CPU
 * baseline leg may load it; the product library never links, loads or calls
 * it, and it shares no header, helper, table or constant with the HIP path.
 *
 * Sources (web pages, cited by title and section):
 *   [P1] "Inference engine, part 2: kernels and token step" — §1 Fast
 *        Walsh–Hadamard transform, §2 Prepare an activation for CQ, §3 Dot
 *        packed rows directly, "Row gather", §7 (per-vector int8
 *        quantization, scaled key dots), §8 (Hadamard MLP).
 *   [P3] "Inference engine, part 1: loader and tokenizer" — §3 Decode FP16
 *        control tensors, §4 Retain packed matrices.
 *   [P4] "attention + tokenizer + sampling: the path to real text
 *        (milestone 6)" — "Step 1 done: F8 kernel", "Step 4 done: I8 +
 *        F8_E4M3 SIMD matvecs", and the sampling of work item 3 and "Step 3
 *        done" (head logits, top-k / temperature sampling, a deterministic
 *        softmax + xorshift sampler).
 *
 * Precision: the pages' arrays are Float32Array (each store rounds to fp32)
 * and their scalars are JavaScript numbers (fp64).  The oracle keeps exactly
 * that: fp32 transform stages, fp64 scale multiply then one rounding, fp64
 * accumulation of dots.  Built with -O2 -ffp-contract=off, no fast-math.
 *
 * Every function has a pin in the CPU test suite (no function is "parity
 * unpinned").
 *
 * Return values: 0 on success, -1 on an invalid shape.
 */
#ifndef BQD_ORACLE_H
#define BQD_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* A CQ (codebook-quantized) matrix, as the record in [P3] §4. */
typedef struct oracle_cq {
    int64_t output;          /* rows                                        */
    int64_t input;           /* unpadded columns                            */
    int64_t input_padded;    /* stored (transform-domain) columns           */
    int64_t group;           /* transform group size, a power of two        */
    int64_t bits;            /* 2, 3, 4 or 5                                */
    int64_t row_bytes;       /* stride between packed rows                  */
    const uint8_t *packed;   /* [output][row_bytes]                         */
    const uint16_t *norms;   /* fp16 bits [output][input_padded / group]    */
    const float *codebook;   /* [1 << bits]                                 */
} oracle_cq;

/* O1: fp16 bit pattern -> fp32 value ([P3] §3). */
float oracle_f16(uint16_t h);

/* O3 core: unnormalized in-place Walsh–Hadamard butterfly over n floats,
 * stride ascending, butterflies (a + b, a - b) in fp32 ([P1] §1). */
void oracle_fwht(float *x, int64_t n);

/* O2: the codebook index of (row, col): bits [bits*col, bits*col + bits) of
 * the row's little-endian bit stream, read one bit at a time. */
uint32_t oracle_cq_index(const oracle_cq *m, int64_t row, int64_t col);

/* O2 for a whole row: idx[col] for col < input_padded. */
int oracle_cq_unpack_row(const oracle_cq *m, int64_t row, uint8_t *idx);

/* O3: prepare one activation vector ([P1] §2): zero-pad x[input] to
 * p[input_padded], FWHT each group, multiply by 1/sqrt(group). */
int oracle_cq_prepare(const oracle_cq *m, const float *x, float *p);

/* O4: the method's packed-row dot ([P1] §3) on a prepared vector, rows
 * [row_begin, row_begin + row_count).  y[i] is the row sum; mag[i] is
 * sum_g |norm| * sum_k |codebook[idx] * p[k]| (the magnitude the tolerance
 * scales with).  Either output may be NULL. */
int oracle_cq_matvec(const oracle_cq *m, const float *p, int64_t row_begin,
                     int64_t row_count, double *y, double *mag);

/* O5: dequantizeRow ([P1] "Row gather"): per group, codebook value times
 * norm (fp32), FWHT, times 1/sqrt(group); the first `input` columns. */
int oracle_cq_dequantize_row(const oracle_cq *m, int64_t row, float *out);

/* O6: gather rows ids[0..n) into out[n][input]; gmag[n][input] (may be NULL)
 * is (1/sqrt(group)) * sum over the column's group of |codebook * norm|. */
int oracle_cq_gather(const oracle_cq *m, const int32_t *ids, int64_t n,
                     float *out, double *gmag);

/* O7: the plain definition ([P1] "Row gather" identity): y[i] = sum over
 * c < input of dequantizeRow(row)[c] * x[c], in fp64. */
int oracle_cq_dense_matvec(const oracle_cq *m, const float *x, int64_t row_begin,
                           int64_t row_count, double *y);

/* O8: FP8 E4M3 code -> value ([P4] Step 1): e = 0 subnormal, values above
 * 448 clamped to 448, sign kept (0x80 is -0.0). */
float oracle_e4m3(uint8_t code);

/* O9: E8M0 exponent byte -> 2^(e - 127); 255 -> NaN. */
float oracle_e8m0(uint8_t e);

/* O10: y[i] = sum_c e4m3(W[r][c]) * e8m0(S[r*SR/R][c*SC/C]) * x[c] for
 * r = row_begin + i, indices by 64-bit floor division; mag likewise with
 * absolute values.  Either output may be NULL. */
int oracle_f8_matvec(const uint8_t *w, int64_t R, int64_t C, const uint8_t *s,
                     int64_t SR, int64_t SC, const float *x, int64_t row_begin,
                     int64_t row_count, double *y, double *mag);

/* O11: one step of the 32-bit xorshift generator (Marsaglia's (13, 17, 5)
 * triple; [P4] names only "xorshift"): s ^= s << 13; s ^= s >> 17;
 * s ^= s << 5.  Maps nonzero states to nonzero states. */
uint32_t oracle_xorshift32(uint32_t s);

/* O12: the k largest logits ([P4] work item 3, top-k): ids[0..k) and
 * vals[0..k) in order: larger value first; equal values (+0 = -0) by lower
 * index first; NaNs after every number.  1 <= k <= n. */
int oracle_topk(const float *logits, int64_t n, int64_t k, int32_t *ids, float *vals);

/* O13: temperature sampling over a top-k list given the uniform draw u in
 * [0, 1) ([P4] "Step 3 done": softmax + xorshift).  temperature <= 0, k = 1,
 * or a top value that is not finite: ids[0].  Otherwise, in fp64,
 * p_i = exp((vals[i] - vals[0]) / temperature) (NaN values weigh 0),
 * S = sum of p_i in list order, and the token is the first ids[i] whose
 * running sum exceeds u * S (ids[k-1] if rounding leaves none). */
int32_t oracle_sample_u(const float *vals, const int32_t *ids, int64_t k,
                        double temperature, double u);

/* O13 with the generator: *state advances once (O11), u = state * 2^-32,
 * then O13.  *state must be nonzero. */
int32_t oracle_sample(const float *vals, const int32_t *ids, int64_t k,
                      double temperature, uint32_t *state);

/* O14: I8 matvec ([P4] "Step 4 done"): y[i] = sum_c w[r][c] *
 * e8m0(s[r][c / G]) * x[c] for r = row_begin + i, with ceil(C / G) scale
 * bytes per row (G = 16 on the page); mag likewise with absolute values. */
int oracle_i8_matvec(const int8_t *w, int64_t R, int64_t C, const uint8_t *s, int64_t G,
                     const float *x, int64_t row_begin, int64_t row_count, double *y,
                     double *mag);

/* O15: storeInt8 ([P1] §7): scale = max(1e-12, max |v|) / 127 in fp64,
 * stored as fp32 in *scale; q[i] = v[i] / scale (fp64) rounded to the
 * nearest integer, ties to even, as an Int8Array stores it (NaN -> 0; a NaN
 * element makes the scale NaN). */
int oracle_store_int8(const float *v, int64_t n, int8_t *q, float *scale);

/* O16: scaled int8 dot ([P1] §7): y[i] = scales[r] * sum_j K[r][j] * x[j],
 * r = row_begin + i, fp64; mag = |scales[r]| * sum |K x|. */
int oracle_int8_dot(const int8_t *K, const float *scales, int64_t R, int64_t d,
                    const float *x, int64_t row_begin, int64_t row_count, double *y,
                    double *mag);

/* O17: Hadamard MLP ([P1] §8) from the normalized input n[hidden]: pad to H
 * (a power of two), times d1, normalized FWHT, silu(d2 * z), normalized FWHT,
 * times d3; out[i] = resid[i] + z[i] (minus u[i] when u is not NULL), for
 * i < hidden.  mag (may be NULL): |resid| + |u| + |d3| / sqrt(H) * sum|silu|. */
int oracle_hadamard_mlp(const float *n, int64_t hidden, int64_t H, const float *d1,
                        const float *d2, const float *d3, const float *resid,
                        const float *u, float *out, double *mag);

#ifdef __cplusplus
}
#endif
#endif

/*
 * bqd.h — C ABI of the MI355X (gfx950) quantized decode matvec library.
 *
 * The operations are those of two public write-ups:
 *   [P1] "Inference engine, part 2: kernels and token step" (needle.js
 *        tutorial): §1 "Fast Walsh–Hadamard transform", §2 "Prepare an
 *        activation for CQ", §3 "Dot packed rows directly", "Row gather",
 *        §6 (row-range matvec, one prepared activation reused for several
 *        matrices), §7 (per-vector int8 quantization, key dots), §8
 *        (Hadamard MLP);
 *   [P3] "Inference engine, part 1: loader and tokenizer": §2 "Make bounds
 *        checks boring", §3 "Decode FP16 control tensors", §4 "Retain packed
 *        matrices" (the CQ record);
 *   [P4] "attention + tokenizer + sampling: the path to real text (milestone
 *        6)": "Step 1 done: F8 kernel" (E4M3 decode, E8M0 block scales),
 *        "Step 4 done" (the vector decode, the I8 matvec), work item 3 and "Step 3 done"
 *        (head logits, top-k / temperature sampling, a deterministic
 *        softmax + xorshift sampler).
 *
 * Conventions shared by every entry point:
 *  - All data pointers are DEVICE pointers owned by the caller; the library
 *    allocates nothing, keeps no per-call state and never frees.  Host
 *    pointers (the bqd_cq_matrix descriptor itself) are read during the call
 *    only.
 *  - `stream` is a hipStream_t (NULL: the null stream).  Calls only enqueue
 *    work and return; results are valid once the stream has reached them.
 *  - Arrays are dense, C order, with the element types stated.  Pointers must
 *    be aligned to their element size (float/int32: 4 bytes, fp16: 2 bytes).
 *  - No output array may share a byte with another output or with any array
 *    the call reads (activations, weights, scales, norms, codebook, ids):
 *    workgroups read inputs while others already store outputs, so such a
 *    call is refused with BQD_EINVAL rather than giving scheduling-dependent
 *    results.  Inputs may overlap one another.
 *  - Every argument is validated on the host before anything is enqueued; a
 *    call that returns an error has enqueued nothing.  Return value: BQD_OK
 *    or one of the negative codes below.  A zero-sized problem (no rows, no
 *    vectors, no ids) is valid and enqueues nothing.
 *  - Results are deterministic: a fixed reduction order, no atomics.
 *  - Concurrent calls on different streams are safe; the library holds no
 *    mutable global state, except the static scratch of logits_sample_noalloc
 *    (whose overlapping calls on one GPU race, as stated there).
 */
#ifndef BQD_H
#define BQD_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    BQD_OK = 0,
    BQD_EINVAL = -1,    /* a shape or parameter outside the documented range */
    BQD_EOVERFLOW = -2, /* a size product does not fit in int64              */
    BQD_EALIGN = -3,    /* a pointer not aligned to its element size          */
    BQD_ENULL = -4,     /* a required pointer is NULL                         */
    BQD_EHIP = -5       /* the HIP runtime reported a launch error            */
};

/* A codebook-quantized matrix, the record of [P3] §4.  Row r, padded column
 * c (0 <= c < input_padded) holds a `bits`-wide codebook index stored at bit
 * offset bits*c of the row's little-endian bit stream (bit t of a row is bit
 * t%8 of byte t/8): for 2-bit, crumb k of a byte is (byte >> 2k) & 3 as in
 * [P1] §3; for 4-bit the low nibble is the even column.  Bits past the last
 * index of a row are ignored.  The matrix acts on the Walsh–Hadamard domain:
 * its dense row is recovered by the "Row gather" of [P1]. */
typedef struct bqd_cq_matrix {
    int64_t output;        /* rows, 0 <= output < 2^30                          */
    int64_t input;         /* unpadded columns, 0 <= input <= input_padded      */
    int64_t input_padded;  /* stored columns, > 0, < 2^28, a multiple of group  */
    int64_t group;         /* transform block, a power of two in [1, 1024]      */
    int64_t bits;          /* 2, 3, 4 or 5                                      */
    int64_t row_bytes;     /* stride of packed rows, >= ceil(input_padded*bits/8) */
    const uint8_t *packed;   /* [output][row_bytes]                               */
    const uint16_t *norms;   /* fp16 bit patterns [output][input_padded / group]  */
    const float *codebook;   /* [1 << bits] fp32                                  */
} bqd_cq_matrix;

/* [P1] §1–§2.  For each of `batch` vectors: p = x zero-padded to
 * input_padded; for each group, the unnormalized fast Walsh–Hadamard
 * transform (stride 1, 2, ..., group/2; pairs become (a + b, a - b) in fp32),
 * then every element is multiplied by 1/sqrt(group) (formed in fp64, rounded
 * once to fp32).  Bit-exact with that sequence of fp32 operations.
 *   x:        fp32 [batch][m->input]          (may be NULL when input == 0)
 *   prepared: fp32 [batch][m->input_padded]   (must not overlap x)
 * Only the shape fields of `m` are read.  One prepared vector may feed any
 * number of cq_matvec calls on matrices of the same input_padded and group.
 * Errors: BQD_EINVAL (shape fields, batch < 0), BQD_ENULL, BQD_EALIGN,
 * BQD_EOVERFLOW, BQD_EHIP. */
int cq_prepare(const bqd_cq_matrix *m, const float *x, float *prepared,
               int64_t batch, void *stream);

/* [P1] §3 with the row range of §6: for b < batch and i < row_count, with
 * r = row_begin + i,
 *   y[b][i] = sum over groups g of  f16(norms[r][g]) *
 *             sum over c in g of codebook[index(r, c)] * prepared[b][c].
 * Accumulation is fp32 (tolerance against the fp64 sum:
 * 1e-4 * sum|w*x| + 1e-6 per output).
 *   prepared: fp32 [batch][m->input_padded]   (the output of cq_prepare)
 *   y:        fp32 [batch][row_count]
 * Errors: BQD_EINVAL (shape fields, batch < 0, row range outside
 * [0, output], y overlapping prepared or the matrix's arrays), BQD_ENULL,
 * BQD_EALIGN, BQD_EOVERFLOW, BQD_EHIP. */
int cq_matvec(const bqd_cq_matrix *m, const float *prepared, float *y,
              int64_t batch, int64_t row_begin, int64_t row_count, void *stream);

/* [P1] §2 followed by §3 in one call: the page's cqMatvec(matrix, x), which
 * prepares the raw activation and then dots the packed rows.  Results are
 * those of cq_prepare(m, x, prepared, batch) followed by cq_matvec(m,
 * prepared, y, batch, row_begin, row_count), bit for bit: `prepared` receives
 * the prepared vectors (a caller buffer; reuse it for further matrices, [P1]
 * §6), y the outputs.  For one 4-bit vector with input_padded in {512, 1024,
 * 2048, 4096, 8192}, group <= 256 and 16-byte aligned rows the two steps run
 * as one kernel launch; otherwise as two.
 *   x:        fp32 [batch][m->input]
 *   prepared: fp32 [batch][m->input_padded]   (written; must not overlap x or y)
 *   y:        fp32 [batch][row_count]         (must not overlap x)
 * Errors: those of cq_prepare and cq_matvec, and BQD_EINVAL when y or
 * prepared overlaps x, each other or the matrix's arrays. */
int cq_prepare_matvec(const bqd_cq_matrix *m, const float *x, float *prepared, float *y,
                      int64_t batch, int64_t row_begin, int64_t row_count, void *stream);

/* [P1] §6: several matrices on one activation vector (phiPre, phiPost and
 * phiResidual from one normalized input), each restricted to a row range:
 * for k < n, ys[k][i] for i < row_count[k] is row row_begin[k] + i of
 * cq_matvec(&ms[k], prepared, ...) at batch 1, bit for bit.  Matrices of
 * one shape class share kernel launches (up to 4 per launch on the batch-1
 * 4-bit shapes of cq_prepare_matvec); the rest take one launch each.
 *   ms:        host array of n descriptors, equal input_padded and group
 *   row_begin, row_count: host arrays of n (NULL: 0, and the rest of each matrix)
 *   prepared:  fp32 [input_padded] (the output of cq_prepare)
 *   ys:        host array of n device pointers, ys[k] fp32 [row_count[k]]
 * Requires 1 <= n <= 64.  Errors: as cq_matvec for every matrix, BQD_EINVAL
 * for unequal shapes or an output overlapping another output, prepared or
 * any matrix's arrays, BQD_ENULL. */
int cq_matvec_multi(const bqd_cq_matrix *ms, int64_t n, const int64_t *row_begin,
                    const int64_t *row_count, const float *prepared, float *const *ys,
                    void *stream);

/* cq_matvec_multi on the raw activation x (fp32 [ms[0].input]; all
 * matrices of equal input too): prepared receives cq_prepare's output and
 * the outputs are those of cq_prepare followed by cq_matvec_multi, bit for
 * bit.  On the fused shapes of cq_prepare_matvec the prepare runs inside the
 * first launch.  Errors: those of cq_prepare and cq_matvec_multi, and
 * BQD_EINVAL when an output overlaps x. */
int cq_prepare_matvec_multi(const bqd_cq_matrix *ms, int64_t n, const int64_t *row_begin,
                            const int64_t *row_count, const float *x, float *prepared,
                            float *const *ys, void *stream);

/* [P1] "Row gather": for i < n, out[i][c] for c < input is the dense row
 * rows[i]: per group, codebook value times norm (fp32 product), the
 * unnormalized transform as in cq_prepare, times 1/sqrt(group), keeping the
 * first `input` columns.  Bit-exact with that sequence of fp32 operations.
 * Ids may repeat.  An id outside [0, output) cannot be checked on the host
 * without a synchronization: its output row is filled with quiet NaNs.
 *   rows: int32 [n]              out: fp32 [n][m->input]
 * Errors: BQD_EINVAL (shape fields, n < 0 or n >= 2^30), BQD_ENULL, BQD_EALIGN,
 * BQD_EOVERFLOW, BQD_EHIP. */
int cq_gather_rows(const bqd_cq_matrix *m, const int32_t *rows, int64_t n,
                   float *out, void *stream);

/* [P4] Step 1: y[b][r] = sum over c < C of e4m3(w[r][c]) *
 * e8m0(scale[r*SR/R][c*SC/C]) * x[b][c], with the scale indices by integer
 * floor division.  E4M3: sign, 4-bit exponent e, 3-bit mantissa m; e = 0 is
 * subnormal (m/8 * 2^-6), otherwise (1 + m/8) * 2^(e-7), magnitudes above 448
 * clamped to 448 (codes 0x7F and 0xFF are +-448).  E8M0: 2^(e-127), the byte
 * 255 is NaN.  Accumulation is fp32 (same tolerance as cq_matvec).
 *   w:     E4M3 codes [R][C]     scale: E8M0 bytes [SR][SC]
 *   x:     fp32 [batch][C]       y:     fp32 [batch][R]
 * Requires 0 <= R < 2^30, 1 <= C < 2^28, 1 <= SR <= max(R, 1), 1 <= SC <= C,
 * batch >= 0.
 * Errors: BQD_EINVAL, BQD_ENULL, BQD_EALIGN, BQD_EOVERFLOW, BQD_EHIP. */
int f8_matvec(const uint8_t *w, int64_t R, int64_t C, const uint8_t *scale,
              int64_t SR, int64_t SC, const float *x, float *y, int64_t batch,
              void *stream);

/* f8_matvec with the argmax of each vector's outputs fused into the same
 * pass ([P4] work item 3 and "Step 3 done": the logits of the head go
 * straight to token selection; this is its greedy form, the token that
 * logits_sample returns at temperature 0 or k = 1): token[b] = the row of
 * the largest y[b][r], equal values taken at the lowest row, NaN below every
 * number, -0 equal to +0.  Each workgroup of the matvec stores the largest
 * (value, row) key of the rows it computed to a slot of the workspace; one
 * small launch then reduces the slots to the token (no atomics; the result
 * does not depend on scheduling).  Shapes the streaming kernel does not take
 * fill the slots from y in a pass of their own.
 *   workspace: device scratch of f8_matvec_argmax_workspace_bytes(batch)
 *              bytes, 8-byte aligned, caller-owned; nothing in it needs
 *              clearing; calls that share it must be ordered on one stream
 *   token:     int32 [batch]
 * Other arguments as f8_matvec; requires R >= 1.
 * Errors: as f8_matvec (BQD_EINVAL also for a workspace smaller than the
 * need; BQD_EALIGN for one not 8-byte aligned; outputs y, the workspace and
 * token must not overlap one another or the inputs). */
int64_t f8_matvec_argmax_workspace_bytes(int64_t batch);
int f8_matvec_argmax(const uint8_t *w, int64_t R, int64_t C, const uint8_t *scale,
                     int64_t SR, int64_t SC, const float *x, float *y, int64_t batch,
                     void *workspace, int64_t workspace_bytes, int32_t *token, void *stream);

/* f8_matvec with top-k / temperature sampling of each vector's outputs
 * fused onto the pass ([P4] work item 3 and "Step 3 done": the head's logits
 * go straight to the sampler).  Per vector b, the results are those of
 * logits_sample on y[b] with k, temperature and state[b], bit for bit:
 * topk_ids[b][0..k) / topk_logits[b][0..k) the k best logits (larger value
 * first, equal values at the lower row, NaN after every number, -0 equal to
 * +0), state[b] advanced one xorshift32 step, token[b] drawn as logits_sample
 * draws it.  How: each workgroup of the matvec stores the largest (value,
 * row) key of its rows to its slot of the workspace (as f8_matvec_argmax);
 * then one workgroup per vector bounds the k-th largest logit from the
 * slots and reads only the rows of the workgroups whose slots pass the bound
 * (about k workgroups of 32 rows on the 246272-row head) instead of all R.
 * No device atomics: the result does not depend on scheduling.
 *   state:       uint32 [batch], read and written
 *   workspace:   f8_matvec_argmax_workspace_bytes(batch) bytes, 8-byte
 *                aligned, caller-owned, no initial contents needed; calls that
 *                share it must be ordered on one stream
 *   token:       int32 [batch]     topk_ids: int32 [batch][k]
 *   topk_logits: fp32 [batch][k]
 * Other arguments as f8_matvec.  Requires 1 <= R <= 2^20,
 * 1 <= k <= min(64, R), 0 <= temperature < inf.
 * Errors: as f8_matvec (BQD_EINVAL also for R, k, temperature or a workspace
 * smaller than the need; BQD_EALIGN for a workspace not 8-byte aligned; the
 * outputs y, workspace, state, token, topk_ids and topk_logits must not
 * overlap one another or the inputs). */
int f8_matvec_sample(const uint8_t *w, int64_t R, int64_t C, const uint8_t *scale,
                     int64_t SR, int64_t SC, const float *x, float *y, int64_t batch,
                     int64_t k, float temperature, uint32_t *state, void *workspace,
                     int64_t workspace_bytes, int32_t *token, int32_t *topk_ids,
                     float *topk_logits, void *stream);

/* [P4] "Step 4 done" (the I8 matvec: int8 weights widened, one E8M0 scale
 * per group of consecutive columns; the page's groups are 16 wide):
 *   y[b][r] = sum over c < C of w[r][c] * e8m0(scale[r][c / G]) * x[b][c],
 * with ceil(C / G) scale bytes per row and e8m0 as in f8_matvec.
 * Accumulation is fp32 (same tolerance as cq_matvec).
 *   w:     int8 [R][C]          scale: E8M0 bytes [R][ceil(C / G)]
 *   x:     fp32 [batch][C]      y:     fp32 [batch][R]
 * Requires 0 <= R < 2^30, 1 <= C < 2^28, 1 <= G <= C, batch >= 0.  Rows of
 * a multiple of 16 bytes, 16-byte aligned, with G a multiple of 16 take the
 * streaming kernel; anything else a generic one.
 * Errors: BQD_EINVAL, BQD_ENULL, BQD_EALIGN, BQD_EOVERFLOW, BQD_EHIP. */
int i8_matvec(const int8_t *w, int64_t R, int64_t C, const uint8_t *scale, int64_t G,
              const float *x, float *y, int64_t batch, void *stream);

/* [P1] §7 "Per-vector int8 quantization" (storeInt8), for each of n_vec
 * vectors of d floats: maximum = max(1e-12, largest |v|) (NaN if any
 * element is NaN), scale = maximum / 127 formed in fp64 and stored as fp32
 * in scales[i]; q[i][j] = v[i][j] / scale (fp64) rounded to the nearest
 * integer, ties to even (0 where that quotient is NaN).  Codes are bit-exact
 * with that arithmetic and lie in [-127, 127].
 *   v: fp32 [n_vec][d]    q: int8 [n_vec][d]    scales: fp32 [n_vec]
 * Requires 0 <= n_vec < 2^30, 0 <= d < 2^28.
 * Errors: BQD_EINVAL, BQD_ENULL, BQD_EALIGN, BQD_EOVERFLOW, BQD_EHIP. */
int kv_quantize_int8(const float *v, int64_t n_vec, int64_t d, int8_t *q, float *scales,
                     void *stream);

/* [P1] §7 key dot against an int8 cache: for b < batch and r < R,
 *   y[b][r] = scales[r] * sum over j < d of K[r][j] * x[b][j]
 * (fp32 accumulation; same tolerance as cq_matvec).
 *   K: int8 [R][d] (rows as kv_quantize_int8 writes them)   scales: fp32 [R]
 *   x: fp32 [batch][d]                                       y: fp32 [batch][R]
 * Requires 0 <= R < 2^30, 1 <= d < 2^28, batch >= 0.
 * Errors: BQD_EINVAL, BQD_ENULL, BQD_EALIGN, BQD_EOVERFLOW, BQD_EHIP. */
int kv_int8_dot(const int8_t *K, const float *scales, int64_t R, int64_t d, const float *x,
                float *y, int64_t batch, void *stream);

/* [P1] §8 "Hadamard MLP", from the normalized block input on (the page's
 * zcrms normalization is not defined there and stays with the caller).  For
 * each of `batch` vectors, with z of H = a power of two >= hidden elements:
 *   z = n zero-padded to H;  z *= d1;  normalized FWHT;  z = silu(d2 * z);
 *   normalized FWHT;  z *= d3;  out = resid + z[0 .. hidden)  (- u if u);
 * where the normalized FWHT is the transform of cq_prepare over all H
 * elements times 1/sqrt(H), silu(t) = t / (1 + exp(-t)), and every stored
 * value rounds to fp32 while products, silu and the scale are formed in fp64
 * (the page's Float32Array / JavaScript-number arithmetic).  The fp64 exp is
 * the device library's, so a silu value may differ from another exp's in
 * its last bit; outputs are held to 1e-5 * m + 1e-6 per element, m =
 * |resid| + |u| + |d3| / sqrt(H) * sum |silu|.
 *   n, resid, u, out: fp32 [batch][hidden] (u may be NULL)
 *   d1, d2, d3:       fp32 [H], shared by the batch
 * Requires H a power of two in [1, 16384], 0 <= hidden <= H, 0 <= batch < 2^31.
 * Errors: BQD_EINVAL, BQD_ENULL, BQD_EALIGN, BQD_EOVERFLOW, BQD_EHIP. */
int hadamard_mlp(const float *n, int64_t hidden, int64_t H, const float *d1, const float *d2,
                 const float *d3, const float *resid, const float *u, float *out, int64_t batch,
                 void *stream);

/* Bytes of device workspace logits_sample needs: ceil(n / C) * k * 8, where
 * C = 1024 for n <= 262144, 2048 for n <= 524288, else 4096 (the per-block
 * candidate lists of the first of its two launches).
 * Returns BQD_EINVAL (negative) for n or k outside logits_sample's range. */
int64_t logits_sample_workspace_bytes(int64_t n, int64_t k);

/* [P4] work item 3 and "Step 3 done": the k best logits and one token drawn
 * from them at a temperature with a seeded xorshift generator.
 *   Order: a larger value first; equal values (+0 = -0) by the lower index;
 *   NaNs after every number.  topk_ids[0..k) / topk_logits[0..k) receive the
 *   k best in that order (logits copied bit for bit).
 *   Draw: *state advances one xorshift32 step (s ^= s << 13; s ^= s >> 17;
 *   s ^= s << 5) and u = state * 2^-32.  If temperature is 0, k is 1, or the
 *   top logit is not finite, the token is topk_ids[0].  Otherwise, in fp64,
 *   p_i = exp((topk_logits[i] - topk_logits[0]) / temperature) (NaNs weigh
 *   0), S = sum of p_i in list order, and the token is the first topk_ids[i]
 *   whose running sum exceeds u * S (topk_ids[k-1] if rounding leaves none).
 *   The same state and logits give the same token; successive calls on one
 *   state continue the generator's sequence.  A zero state stays zero.
 *   logits:      fp32 [n]                 state: uint32 [1], read and written
 *   workspace:   logits_sample_workspace_bytes(n, k) bytes, 4-byte aligned,
 *                no initial contents needed; calls that share a workspace
 *                must not overlap in time.
 *   token:       int32 [1]                topk_ids: int32 [k]   topk_logits: fp32 [k]
 * All pointers are device pointers.  Requires 1 <= n <= 2^20,
 * 1 <= k <= min(64, n), 0 <= temperature < inf.
 * Errors: BQD_EINVAL (ranges, temperature, workspace_bytes too small),
 * BQD_ENULL, BQD_EALIGN, BQD_EHIP. */
int logits_sample(const float *logits, int64_t n, int64_t k, float temperature,
                  uint32_t *state, void *workspace, int64_t workspace_bytes,
                  int32_t *token, int32_t *topk_ids, float *topk_logits, void *stream);

/* logits_sample without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): the same kernels and results, bit for bit, with
 * the workspace taken from a static device array inside the library, 131,072
 * bytes (the need of the largest call: n = 2^20, k = 64) held by each GPU the
 * library runs on until the process ends.  The call allocates nothing.  Its
 * address is looked up on the first call on each device: the device of
 * `stream` (the current device for the null stream), made current for the
 * lookup and then restored.  All calls on one GPU share that array: calls that overlap in
 * time on one GPU (different streams, no ordering between them) race and
 * may return wrong results; calls ordered on one stream are safe.  Arguments
 * and errors as logits_sample (a call needing more scratch than the array
 * holds is refused with BQD_EINVAL; none can within the documented ranges),
 * plus BQD_EHIP if the array's device address cannot be found. */
int logits_sample_noalloc(const float *logits, int64_t n, int64_t k, float temperature,
                          uint32_t *state, int32_t *token, int32_t *topk_ids,
                          float *topk_logits, void *stream);

/* Test probes: run the very device decode routines the kernels use.
 * bqd_dbg_cq_unpack: idx[c] = index(row, c) for c < input_padded (uint8).
 * bqd_dbg_f16_decode: out[i] = fp16 codes[i] as fp32 (the norm decode).
 * bqd_dbg_f8_decode: out[i] = e4m3(codes[i]) (the weight decode).
 * bqd_dbg_e8m0_decode: out[i] = e8m0(codes[i]) (the scale decode).
 * Same conventions and error codes as above; n >= 0; row in [0, output). */
int bqd_dbg_cq_unpack(const bqd_cq_matrix *m, int64_t row, uint8_t *idx, void *stream);
int bqd_dbg_f16_decode(const uint16_t *codes, int64_t n, float *out, void *stream);
int bqd_dbg_f8_decode(const uint8_t *codes, int64_t n, float *out, void *stream);
int bqd_dbg_e8m0_decode(const uint8_t *codes, int64_t n, float *out, void *stream);

/* Measurement probe: reads bytes bytes of buf once (nontemporal 16-byte
 * loads, the layout of the head kernels, no other work) and writes the XOR
 * of every 32-bit word read, split over out[0 .. BQD_READ_STREAM_WORDS) (one
 * word per workgroup, zeros after the last; the XOR of all of out is the XOR
 * of the buffer's words).  Its duration is the plain-read reference for the
 * decode kernels' bandwidth.
 *   buf: device, 16-byte aligned, bytes a multiple of 16, 0 <= bytes < 2^46
 *   out: device uint32 [BQD_READ_STREAM_WORDS], 4-byte aligned
 * Errors: BQD_EINVAL (bytes), BQD_ENULL, BQD_EALIGN, BQD_EHIP.  bytes == 0
 * returns BQD_OK without a launch. */
#define BQD_READ_STREAM_WORDS 2048
int bqd_dbg_read_stream(const void *buf, int64_t bytes, uint32_t *out, void *stream);

/* A static, human-readable name for a status code. */
const char *bqd_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* BQD_H */

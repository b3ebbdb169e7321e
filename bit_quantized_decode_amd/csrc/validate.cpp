// Host-side argument validation of the C ABI ("Inference engine, part 1:
// loader and tokenizer", §2: every range is checked before anything is read,
// and size products are checked before they are used).  No HIP here.
#include "validate.h"

namespace bqd {
namespace {

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

// a * b * c must fit in int64 (all operands non-negative).
bool mul_ok(int64_t a, int64_t b, int64_t c = 1) {
  int64_t t;
  if (__builtin_mul_overflow(a, b, &t)) return false;
  if (__builtin_mul_overflow(t, c, &t)) return false;
  return true;
}

// A byte range [p, p + bytes) of a call's buffer; null or empty ranges take
// no part in the overlap test.
struct Span {
  const void* p;
  int64_t bytes;
};

bool spans_meet(const Span& a, const Span& b) {
  if (!a.p || !b.p || a.bytes <= 0 || b.bytes <= 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + (uintptr_t)b.bytes && b0 < a0 + (uintptr_t)a.bytes;
}

// Every workgroup reads its inputs while others already store outputs, so an
// output that shares a byte with another output or with any input would make
// the result depend on scheduling: such calls are refused (BQD_EINVAL).
bool outputs_overlap(const Span* outs, int n_out, const Span* ins, int n_in) {
  for (int i = 0; i < n_out; ++i) {
    for (int j = i + 1; j < n_out; ++j)
      if (spans_meet(outs[i], outs[j])) return true;
    for (int j = 0; j < n_in; ++j)
      if (spans_meet(outs[i], ins[j])) return true;
  }
  return false;
}

// The three arrays a CQ matrix reads (its shape already validated).
void cq_spans(const bqd_cq_matrix* m, Span* s) {
  s[0] = {m->packed, m->output * m->row_bytes};
  s[1] = {m->norms, m->output * (m->input_padded / m->group) * 2};
  s[2] = {m->codebook, (int64_t)4 << m->bits};
}

}  // namespace

int check_cq_shape(const bqd_cq_matrix* m) {
  if (!m) return BQD_ENULL;
  if (m->bits < 2 || m->bits > 5) return BQD_EINVAL;
  if (!is_pow2(m->group) || m->group > kMaxGroup) return BQD_EINVAL;
  if (m->input_padded <= 0 || m->input_padded >= kMaxColumns) return BQD_EINVAL;
  if (m->input_padded % m->group != 0) return BQD_EINVAL;
  if (m->input < 0 || m->input > m->input_padded) return BQD_EINVAL;
  if (m->output < 0 || m->output >= kMaxRows) return BQD_EINVAL;
  if (m->row_bytes <= 0) return BQD_EINVAL;
  const int64_t need = (m->input_padded * m->bits + 7) / 8;
  if (m->row_bytes < need) return BQD_EINVAL;
  if (!mul_ok(m->output, m->row_bytes)) return BQD_EOVERFLOW;
  if (!mul_ok(m->output, m->input_padded / m->group, 2)) return BQD_EOVERFLOW;
  return BQD_OK;
}

int check_cq(const bqd_cq_matrix* m) {
  int rc = check_cq_shape(m);
  if (rc) return rc;
  if (m->output > 0 && (!m->packed || !m->norms)) return BQD_ENULL;
  if (!m->codebook) return BQD_ENULL;
  if (!aligned(m->norms, 2) || !aligned(m->codebook, 4)) return BQD_EALIGN;
  return BQD_OK;
}

int check_prepare(const bqd_cq_matrix* m, const float* x, const float* prepared, int64_t batch) {
  int rc = check_cq_shape(m);
  if (rc) return rc;
  if (batch < 0) return BQD_EINVAL;
  if (!mul_ok(batch, m->input_padded, 4)) return BQD_EOVERFLOW;
  if (batch == 0) return BQD_OK;
  if (!prepared || (m->input > 0 && !x)) return BQD_ENULL;
  if (!aligned(x, 4) || !aligned(prepared, 4)) return BQD_EALIGN;
  const Span out[1] = {{prepared, batch * m->input_padded * 4}};
  const Span in[1] = {{x, batch * m->input * 4}};
  if (outputs_overlap(out, 1, in, 1)) return BQD_EINVAL;
  return BQD_OK;
}

int check_matvec(const bqd_cq_matrix* m, const float* prepared, const float* y, int64_t batch,
                 int64_t row_begin, int64_t row_count) {
  int rc = check_cq(m);
  if (rc) return rc;
  if (batch < 0 || row_begin < 0 || row_count < 0) return BQD_EINVAL;
  if (row_begin > m->output || row_count > m->output - row_begin) return BQD_EINVAL;
  if (!mul_ok(batch, m->input_padded, 4) || !mul_ok(batch, row_count, 4)) return BQD_EOVERFLOW;
  if (batch == 0 || row_count == 0) return BQD_OK;
  if (!prepared || !y) return BQD_ENULL;
  if (!aligned(prepared, 4) || !aligned(y, 4)) return BQD_EALIGN;
  Span in[4];
  cq_spans(m, in);
  in[3] = {prepared, batch * m->input_padded * 4};
  const Span out[1] = {{y, batch * row_count * 4}};
  if (outputs_overlap(out, 1, in, 4)) return BQD_EINVAL;
  return BQD_OK;
}

int check_prepare_matvec(const bqd_cq_matrix* m, const float* x, const float* prepared,
                         const float* y, int64_t batch, int64_t row_begin, int64_t row_count) {
  int rc = check_prepare(m, x, prepared, batch);
  if (rc) return rc;
  rc = check_matvec(m, prepared, y, batch, row_begin, row_count);
  if (rc || batch == 0) return rc;
  // the prepared vectors are an output here as well
  Span in[4];
  cq_spans(m, in);
  in[3] = {x, batch * m->input * 4};
  const Span out[2] = {{prepared, batch * m->input_padded * 4}, {y, batch * row_count * 4}};
  if (outputs_overlap(out, 2, in, 4)) return BQD_EINVAL;
  return BQD_OK;
}

int check_matvec_multi(const bqd_cq_matrix* ms, int64_t n, const int64_t* row_begin,
                       const int64_t* row_count, bool with_x, const float* x,
                       const float* prepared, float* const* ys, int64_t* rb, int64_t* rc) {
  if (!ms || !ys) return BQD_ENULL;
  if (n < 1 || n > kMaxMulti) return BQD_EINVAL;
  for (int64_t k = 0; k < n; ++k) {
    rb[k] = row_begin ? row_begin[k] : 0;
    // the begin is range-checked before the default count subtracts it
    const int rs = check_cq_shape(&ms[k]);
    if (rs) return rs;
    if (rb[k] < 0 || rb[k] > ms[k].output) return BQD_EINVAL;
    rc[k] = row_count ? row_count[k] : ms[k].output - rb[k];
    int rc_k = check_matvec(&ms[k], prepared, ys[k], 1, rb[k], rc[k]);
    if (rc_k) return rc_k;
    if (ms[k].input_padded != ms[0].input_padded || ms[k].group != ms[0].group ||
        (with_x && ms[k].input != ms[0].input))
      return BQD_EINVAL;
  }
  if (with_x) {
    int rcp = check_prepare(&ms[0], x, prepared, 1);
    if (rcp) return rcp;
  }
  if (!prepared) return BQD_ENULL;
  if (!aligned(prepared, 4)) return BQD_EALIGN;
  // No output may overlap another output or anything a launch reads: the
  // activation (with x, the raw input too) and every matrix's arrays.  With
  // x the prepared vector is an output; without it, an input.
  Span outs[kMaxMulti + 1];
  Span ins[3 * kMaxMulti + 2];
  int n_out = 0, n_in = 0;
  for (int64_t k = 0; k < n; ++k) {
    outs[n_out++] = {ys[k], rc[k] * 4};
    cq_spans(&ms[k], ins + n_in);
    n_in += 3;
  }
  const Span pspan = {prepared, ms[0].input_padded * 4};
  if (with_x) {
    outs[n_out++] = pspan;
    ins[n_in++] = {x, ms[0].input * 4};
  } else {
    ins[n_in++] = pspan;
  }
  if (outputs_overlap(outs, n_out, ins, n_in)) return BQD_EINVAL;
  return BQD_OK;
}

int check_gather(const bqd_cq_matrix* m, const int32_t* rows, int64_t n, const float* out) {
  int rc = check_cq(m);
  if (rc) return rc;
  if (n < 0 || n >= kMaxRows) return BQD_EINVAL;
  if (!mul_ok(n, m->input, 4)) return BQD_EOVERFLOW;
  if (n == 0) return BQD_OK;
  if (!rows || (m->input > 0 && !out)) return BQD_ENULL;
  if (!aligned(rows, 4) || !aligned(out, 4)) return BQD_EALIGN;
  Span in[4];
  cq_spans(m, in);
  in[3] = {rows, n * 4};
  const Span o[1] = {{out, n * m->input * 4}};
  if (outputs_overlap(o, 1, in, 4)) return BQD_EINVAL;
  return BQD_OK;
}

int check_f8(const uint8_t* w, int64_t R, int64_t C, const uint8_t* scale, int64_t SR,
             int64_t SC, const float* x, const float* y, int64_t batch) {
  if (R < 0 || R >= kMaxRows || C < 1 || C >= kMaxColumns) return BQD_EINVAL;
  if (SR < 1 || SR > (R > 0 ? R : 1) || SC < 1 || SC > C) return BQD_EINVAL;
  if (batch < 0) return BQD_EINVAL;
  if (!mul_ok(R, C) || !mul_ok(SR, SC) || !mul_ok(batch, C, 4) || !mul_ok(batch, R, 4) ||
      !mul_ok(R, SR) || !mul_ok(C, SC))
    return BQD_EOVERFLOW;
  if (batch == 0 || R == 0) return BQD_OK;
  if (!w || !scale || !x || !y) return BQD_ENULL;
  if (!aligned(x, 4) || !aligned(y, 4)) return BQD_EALIGN;
  const Span in[3] = {{w, R * C}, {scale, SR * SC}, {x, batch * C * 4}};
  const Span out[1] = {{y, batch * R * 4}};
  if (outputs_overlap(out, 1, in, 3)) return BQD_EINVAL;
  return BQD_OK;
}

int check_f8_argmax(const uint8_t* w, int64_t R, int64_t C, const uint8_t* scale, int64_t SR,
                    int64_t SC, const float* x, const float* y, int64_t batch,
                    const void* workspace, int64_t workspace_bytes, const int32_t* token) {
  if (R < 1) return BQD_EINVAL;  // every vector has a largest logit
  const int rc = check_f8(w, R, C, scale, SR, SC, x, y, batch);
  if (rc || batch == 0) return rc;
  if (!mul_ok(batch, kF8ArgmaxSlots, 8)) return BQD_EOVERFLOW;
  const int64_t need = f8_argmax_workspace_need(batch);
  if (workspace_bytes < need) return BQD_EINVAL;
  if (!workspace || !token) return BQD_ENULL;
  if (!aligned(workspace, 8) || !aligned(token, 4)) return BQD_EALIGN;
  const Span in[3] = {{w, R * C}, {scale, SR * SC}, {x, batch * C * 4}};
  const Span out[3] = {{y, batch * R * 4}, {workspace, need}, {token, batch * 4}};
  if (outputs_overlap(out, 3, in, 3)) return BQD_EINVAL;
  return BQD_OK;
}

int check_f8_sample(const uint8_t* w, int64_t R, int64_t C, const uint8_t* scale, int64_t SR,
                    int64_t SC, const float* x, const float* y, int64_t batch, int64_t k,
                    float temperature, const uint32_t* state, const void* workspace,
                    int64_t workspace_bytes, const int32_t* token, const int32_t* topk_ids,
                    const float* topk_logits) {
  if (R < 1 || R > kMaxSampleLogits || k < 1 || k > kMaxSampleK || k > R) return BQD_EINVAL;
  if (!(temperature >= 0.0f) || temperature > 3.4e38f) return BQD_EINVAL;  // NaN, < 0, inf
  const int rc = check_f8(w, R, C, scale, SR, SC, x, y, batch);
  if (rc || batch == 0) return rc;
  if (!mul_ok(batch, kF8ArgmaxSlots, 8) || !mul_ok(batch, k, 4)) return BQD_EOVERFLOW;
  const int64_t need = f8_argmax_workspace_need(batch);
  if (workspace_bytes < need) return BQD_EINVAL;
  if (!workspace || !state || !token || !topk_ids || !topk_logits) return BQD_ENULL;
  if (!aligned(workspace, 8) || !aligned(state, 4) || !aligned(token, 4) ||
      !aligned(topk_ids, 4) || !aligned(topk_logits, 4))
    return BQD_EALIGN;
  // the generator states are read and written: they count as outputs
  const Span in[3] = {{w, R * C}, {scale, SR * SC}, {x, batch * C * 4}};
  const Span out[6] = {{y, batch * R * 4},        {workspace, need},
                       {state, batch * 4},        {token, batch * 4},
                       {topk_ids, batch * k * 4}, {topk_logits, batch * k * 4}};
  if (outputs_overlap(out, 6, in, 3)) return BQD_EINVAL;
  return BQD_OK;
}

int check_i8(const int8_t* w, int64_t R, int64_t C, const uint8_t* scale, int64_t G,
             const float* x, const float* y, int64_t batch) {
  if (R < 0 || R >= kMaxRows || C < 1 || C >= kMaxColumns || G < 1 || G > C || batch < 0)
    return BQD_EINVAL;
  const int64_t ns = (C + G - 1) / G;
  if (!mul_ok(R, C) || !mul_ok(R, ns) || !mul_ok(batch, C, 4) || !mul_ok(batch, R, 4))
    return BQD_EOVERFLOW;
  if (batch == 0 || R == 0) return BQD_OK;
  if (!w || !scale || !x || !y) return BQD_ENULL;
  if (!aligned(x, 4) || !aligned(y, 4)) return BQD_EALIGN;
  const Span in[3] = {{w, R * C}, {scale, R * ns}, {x, batch * C * 4}};
  const Span out[1] = {{y, batch * R * 4}};
  if (outputs_overlap(out, 1, in, 3)) return BQD_EINVAL;
  return BQD_OK;
}

int check_kv_quantize(const float* v, int64_t n_vec, int64_t d, const int8_t* q,
                      const float* scales) {
  if (n_vec < 0 || n_vec >= kMaxRows || d < 0 || d >= kMaxColumns) return BQD_EINVAL;
  if (!mul_ok(n_vec, d, 4)) return BQD_EOVERFLOW;
  if (n_vec == 0) return BQD_OK;
  if (!scales || (d > 0 && (!v || !q))) return BQD_ENULL;
  if (!aligned(v, 4) || !aligned(scales, 4)) return BQD_EALIGN;
  const Span in[1] = {{v, n_vec * d * 4}};
  const Span out[2] = {{q, n_vec * d}, {scales, n_vec * 4}};
  if (outputs_overlap(out, 2, in, 1)) return BQD_EINVAL;
  return BQD_OK;
}

int check_kv_dot(const int8_t* K, const float* scales, int64_t R, int64_t d, const float* x,
                 const float* y, int64_t batch) {
  if (R < 0 || R >= kMaxRows || d < 1 || d >= kMaxColumns || batch < 0) return BQD_EINVAL;
  if (!mul_ok(R, d) || !mul_ok(batch, d, 4) || !mul_ok(batch, R, 4)) return BQD_EOVERFLOW;
  if (batch == 0 || R == 0) return BQD_OK;
  if (!K || !scales || !x || !y) return BQD_ENULL;
  if (!aligned(scales, 4) || !aligned(x, 4) || !aligned(y, 4)) return BQD_EALIGN;
  const Span in[3] = {{K, R * d}, {scales, R * 4}, {x, batch * d * 4}};
  const Span out[1] = {{y, batch * R * 4}};
  if (outputs_overlap(out, 1, in, 3)) return BQD_EINVAL;
  return BQD_OK;
}

int check_hadamard_mlp(const float* n, int64_t hidden, int64_t H, const float* d1,
                       const float* d2, const float* d3, const float* resid, const float* u,
                       const float* out, int64_t batch) {
  if (!is_pow2(H) || H > kMaxHadamard || hidden < 0 || hidden > H) return BQD_EINVAL;
  if (batch < 0 || batch >= kMaxBatchBlocks) return BQD_EINVAL;
  if (!mul_ok(batch, hidden, 4)) return BQD_EOVERFLOW;
  if (batch == 0) return BQD_OK;
  if (!d1 || !d2 || !d3) return BQD_ENULL;
  if (hidden > 0 && (!n || !resid || !out)) return BQD_ENULL;
  if (!aligned(n, 4) || !aligned(d1, 4) || !aligned(d2, 4) || !aligned(d3, 4) ||
      !aligned(resid, 4) || !aligned(u, 4) || !aligned(out, 4))
    return BQD_EALIGN;
  const int64_t vec = batch * hidden * 4;
  const Span in[6] = {{n, vec}, {d1, H * 4}, {d2, H * 4}, {d3, H * 4}, {resid, vec}, {u, vec}};
  const Span o[1] = {{out, vec}};
  if (outputs_overlap(o, 1, in, 6)) return BQD_EINVAL;
  return BQD_OK;
}

int check_unpack(const bqd_cq_matrix* m, int64_t row, const uint8_t* idx) {
  int rc = check_cq(m);
  if (rc) return rc;
  if (row < 0 || row >= m->output) return BQD_EINVAL;
  if (!idx) return BQD_ENULL;
  return BQD_OK;
}

int check_decode(const void* codes, int64_t n, const float* out, int code_size) {
  if (n < 0 || n >= kMaxRows) return BQD_EINVAL;
  if (n == 0) return BQD_OK;
  if (!codes || !out) return BQD_ENULL;
  if (!aligned(codes, (uintptr_t)code_size) || !aligned(out, 4)) return BQD_EALIGN;
  return BQD_OK;
}

int check_read_stream(const void* buf, int64_t bytes, const uint32_t* out) {
  if (bytes < 0 || bytes % 16 != 0 || bytes >= (int64_t(1) << 46)) return BQD_EINVAL;
  if (bytes == 0) return BQD_OK;
  if (!buf || !out) return BQD_ENULL;
  if (!aligned(buf, 16) || !aligned(out, 4)) return BQD_EALIGN;
  return BQD_OK;
}

int64_t sample_workspace_need(int64_t n, int64_t k) {
  if (n < 1 || n > kMaxSampleLogits || k < 1 || k > kMaxSampleK || k > n) return BQD_EINVAL;
  const int64_t chunk = sample_chunk(n);
  return (n + chunk - 1) / chunk * k * 8;
}

int check_sample(const float* logits, int64_t n, int64_t k, float temperature,
                 const uint32_t* state, const void* workspace, int64_t workspace_bytes,
                 const int32_t* token, const int32_t* topk_ids, const float* topk_logits) {
  const int64_t need = sample_workspace_need(n, k);
  if (need < 0) return BQD_EINVAL;
  if (!(temperature >= 0.0f) || temperature > 3.4e38f) return BQD_EINVAL;  // NaN, < 0, inf
  if (!logits || !state || !workspace || !token || !topk_ids || !topk_logits) return BQD_ENULL;
  if (workspace_bytes < need) return BQD_EINVAL;
  if (!aligned(logits, 4) || !aligned(state, 4) || !aligned(workspace, 4) || !aligned(token, 4) ||
      !aligned(topk_ids, 4) || !aligned(topk_logits, 4))
    return BQD_EALIGN;
  // the generator state is read and written: it counts as an output
  const Span in[1] = {{logits, n * 4}};
  const Span out[5] = {{state, 4}, {workspace, need}, {token, 4}, {topk_ids, k * 4},
                       {topk_logits, k * 4}};
  if (outputs_overlap(out, 5, in, 1)) return BQD_EINVAL;
  return BQD_OK;
}

int check_sample_noalloc(const float* logits, int64_t n, int64_t k, float temperature,
                         const uint32_t* state, const int32_t* token, const int32_t* topk_ids,
                         const float* topk_logits, int64_t scratch_bytes) {
  const int64_t need = sample_workspace_need(n, k);
  if (need < 0 || need > scratch_bytes) return BQD_EINVAL;
  if (!(temperature >= 0.0f) || temperature > 3.4e38f) return BQD_EINVAL;  // NaN, < 0, inf
  if (!logits || !state || !token || !topk_ids || !topk_logits) return BQD_ENULL;
  if (!aligned(logits, 4) || !aligned(state, 4) || !aligned(token, 4) || !aligned(topk_ids, 4) ||
      !aligned(topk_logits, 4))
    return BQD_EALIGN;
  const Span in[1] = {{logits, n * 4}};
  const Span out[4] = {{state, 4}, {token, 4}, {topk_ids, k * 4}, {topk_logits, k * 4}};
  if (outputs_overlap(out, 4, in, 1)) return BQD_EINVAL;
  return BQD_OK;
}

}  // namespace bqd

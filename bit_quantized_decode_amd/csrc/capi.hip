// The C ABI entry points: validate on the host (validate.cpp, HIP-free), then
// enqueue the kernels on the caller's stream.
#include "launch.h"
#include "validate.h"

using namespace bqd;

namespace {
hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
}  // namespace

extern "C" {

int cq_prepare(const bqd_cq_matrix* m, const float* x, float* prepared, int64_t batch,
               void* stream) {
  int rc = check_prepare(m, x, prepared, batch);
  if (rc || batch == 0) return rc;
  return launch_cq_prepare(m, x, prepared, batch, as_stream(stream));
}

int cq_matvec(const bqd_cq_matrix* m, const float* prepared, float* y, int64_t batch,
              int64_t row_begin, int64_t row_count, void* stream) {
  int rc = check_matvec(m, prepared, y, batch, row_begin, row_count);
  if (rc || batch == 0 || row_count == 0) return rc;
  return launch_cq_matvec(m, prepared, y, batch, row_begin, row_count, as_stream(stream));
}

int cq_prepare_matvec(const bqd_cq_matrix* m, const float* x, float* prepared, float* y,
                      int64_t batch, int64_t row_begin, int64_t row_count, void* stream) {
  int rc = check_prepare_matvec(m, x, prepared, y, batch, row_begin, row_count);
  if (rc || batch == 0) return rc;
  return launch_cq_prepare_matvec(m, x, prepared, y, batch, row_begin, row_count,
                                  as_stream(stream));
}

int cq_matvec_multi(const bqd_cq_matrix* ms, int64_t n, const int64_t* row_begin,
                    const int64_t* row_count, const float* prepared, float* const* ys,
                    void* stream) {
  int64_t rb[kMaxMulti], rc[kMaxMulti];
  int rc0 = check_matvec_multi(ms, n, row_begin, row_count, false, nullptr, prepared, ys, rb, rc);
  if (rc0) return rc0;
  return launch_cq_matvec_multi(ms, n, rb, rc, false, nullptr, const_cast<float*>(prepared), ys,
                                as_stream(stream));
}

int cq_prepare_matvec_multi(const bqd_cq_matrix* ms, int64_t n, const int64_t* row_begin,
                            const int64_t* row_count, const float* x, float* prepared,
                            float* const* ys, void* stream) {
  int64_t rb[kMaxMulti], rc[kMaxMulti];
  int rc0 = check_matvec_multi(ms, n, row_begin, row_count, true, x, prepared, ys, rb, rc);
  if (rc0) return rc0;
  return launch_cq_matvec_multi(ms, n, rb, rc, true, x, prepared, ys, as_stream(stream));
}

int cq_gather_rows(const bqd_cq_matrix* m, const int32_t* rows, int64_t n, float* out,
                   void* stream) {
  int rc = check_gather(m, rows, n, out);
  if (rc || n == 0) return rc;
  return launch_cq_gather(m, rows, n, out, as_stream(stream));
}

int f8_matvec(const uint8_t* w, int64_t R, int64_t C, const uint8_t* scale, int64_t SR,
              int64_t SC, const float* x, float* y, int64_t batch, void* stream) {
  int rc = check_f8(w, R, C, scale, SR, SC, x, y, batch);
  if (rc || batch == 0 || R == 0) return rc;
  return launch_f8_matvec(w, R, C, scale, SR, SC, x, y, batch, as_stream(stream));
}

int64_t f8_matvec_argmax_workspace_bytes(int64_t batch) {
  if (batch < 0 || batch >= kMaxRows) return BQD_EINVAL;
  return f8_argmax_workspace_need(batch);
}

int f8_matvec_argmax(const uint8_t* w, int64_t R, int64_t C, const uint8_t* scale, int64_t SR,
                     int64_t SC, const float* x, float* y, int64_t batch, void* workspace,
                     int64_t workspace_bytes, int32_t* token, void* stream) {
  int rc = check_f8_argmax(w, R, C, scale, SR, SC, x, y, batch, workspace, workspace_bytes,
                           token);
  if (rc || batch == 0) return rc;
  return launch_f8_matvec_argmax(w, R, C, scale, SR, SC, x, y, batch, workspace, token,
                                 as_stream(stream));
}

int f8_matvec_sample(const uint8_t* w, int64_t R, int64_t C, const uint8_t* scale, int64_t SR,
                     int64_t SC, const float* x, float* y, int64_t batch, int64_t k,
                     float temperature, uint32_t* state, void* workspace,
                     int64_t workspace_bytes, int32_t* token, int32_t* topk_ids,
                     float* topk_logits, void* stream) {
  int rc = check_f8_sample(w, R, C, scale, SR, SC, x, y, batch, k, temperature, state, workspace,
                           workspace_bytes, token, topk_ids, topk_logits);
  if (rc || batch == 0) return rc;
  return launch_f8_matvec_sample(w, R, C, scale, SR, SC, x, y, batch, k, temperature, state,
                                 workspace, token, topk_ids, topk_logits, as_stream(stream));
}

int i8_matvec(const int8_t* w, int64_t R, int64_t C, const uint8_t* scale, int64_t G,
              const float* x, float* y, int64_t batch, void* stream) {
  int rc = check_i8(w, R, C, scale, G, x, y, batch);
  if (rc || batch == 0 || R == 0) return rc;
  return launch_i8_matvec(w, R, C, scale, G, x, y, batch, as_stream(stream));
}

int kv_quantize_int8(const float* v, int64_t n_vec, int64_t d, int8_t* q, float* scales,
                     void* stream) {
  int rc = check_kv_quantize(v, n_vec, d, q, scales);
  if (rc || n_vec == 0) return rc;
  return launch_kv_quantize_int8(v, n_vec, d, q, scales, as_stream(stream));
}

int kv_int8_dot(const int8_t* K, const float* scales, int64_t R, int64_t d, const float* x,
                float* y, int64_t batch, void* stream) {
  int rc = check_kv_dot(K, scales, R, d, x, y, batch);
  if (rc || batch == 0 || R == 0) return rc;
  return launch_kv_int8_dot(K, scales, R, d, x, y, batch, as_stream(stream));
}

int hadamard_mlp(const float* n, int64_t hidden, int64_t H, const float* d1, const float* d2,
                 const float* d3, const float* resid, const float* u, float* out, int64_t batch,
                 void* stream) {
  int rc = check_hadamard_mlp(n, hidden, H, d1, d2, d3, resid, u, out, batch);
  if (rc || batch == 0 || hidden == 0) return rc;
  return launch_hadamard_mlp(n, hidden, H, d1, d2, d3, resid, u, out, batch, as_stream(stream));
}

int bqd_dbg_cq_unpack(const bqd_cq_matrix* m, int64_t row, uint8_t* idx, void* stream) {
  int rc = check_unpack(m, row, idx);
  if (rc) return rc;
  return launch_cq_unpack(m, row, idx, as_stream(stream));
}

int bqd_dbg_f16_decode(const uint16_t* codes, int64_t n, float* out, void* stream) {
  int rc = check_decode(codes, n, out, 2);
  if (rc || n == 0) return rc;
  return launch_f16_decode(codes, n, out, as_stream(stream));
}

int bqd_dbg_f8_decode(const uint8_t* codes, int64_t n, float* out, void* stream) {
  int rc = check_decode(codes, n, out, 1);
  if (rc || n == 0) return rc;
  return launch_f8_decode(codes, n, out, as_stream(stream));
}

int bqd_dbg_e8m0_decode(const uint8_t* codes, int64_t n, float* out, void* stream) {
  int rc = check_decode(codes, n, out, 1);
  if (rc || n == 0) return rc;
  return launch_e8m0_decode(codes, n, out, as_stream(stream));
}

int bqd_dbg_read_stream(const void* buf, int64_t bytes, uint32_t* out, void* stream) {
  int rc = check_read_stream(buf, bytes, out);
  if (rc || bytes == 0) return rc;
  return launch_read_stream(buf, bytes, out, as_stream(stream));
}

int64_t logits_sample_workspace_bytes(int64_t n, int64_t k) {
  return sample_workspace_need(n, k);
}

int logits_sample(const float* logits, int64_t n, int64_t k, float temperature, uint32_t* state,
                  void* workspace, int64_t workspace_bytes, int32_t* token, int32_t* topk_ids,
                  float* topk_logits, void* stream) {
  int rc = check_sample(logits, n, k, temperature, state, workspace, workspace_bytes, token,
                        topk_ids, topk_logits);
  if (rc) return rc;
  return launch_logits_sample(logits, n, k, temperature, state, workspace, token, topk_ids,
                              topk_logits, as_stream(stream));
}

int logits_sample_noalloc(const float* logits, int64_t n, int64_t k, float temperature,
                          uint32_t* state, int32_t* token, int32_t* topk_ids, float* topk_logits,
                          void* stream) {
  int rc = check_sample_noalloc(logits, n, k, temperature, state, token, topk_ids, topk_logits,
                                sample_scratch_bytes());
  if (rc) return rc;
  void* ws = nullptr;
  rc = sample_scratch(as_stream(stream), &ws);
  if (rc) return rc;
  return launch_logits_sample(logits, n, k, temperature, state, ws, token, topk_ids,
                              topk_logits, as_stream(stream));
}

const char* bqd_status_string(int status) {
  switch (status) {
    case BQD_OK: return "ok";
    case BQD_EINVAL: return "invalid shape or parameter";
    case BQD_EOVERFLOW: return "size product overflows int64";
    case BQD_EALIGN: return "pointer not aligned to its element size";
    case BQD_ENULL: return "required pointer is NULL";
    case BQD_EHIP: return "HIP launch error";
  }
  return "unknown status";
}

}  // extern "C"

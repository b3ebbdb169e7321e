// Host-side argument validation of the C ABI.  Compiled without any HIP
// header, so every status code can be produced and tested on a CPU-only host.
#pragma once
#include <stdint.h>

#include "../../include/bqd.h"

namespace bqd {

// Shape fields of a CQ matrix (data pointers are not looked at).
int check_cq_shape(const bqd_cq_matrix* m);
// Shape fields plus the packed / norms / codebook pointers.
int check_cq(const bqd_cq_matrix* m);

int check_prepare(const bqd_cq_matrix* m, const float* x, const float* prepared, int64_t batch);
int check_matvec(const bqd_cq_matrix* m, const float* prepared, const float* y, int64_t batch,
                 int64_t row_begin, int64_t row_count);
int check_prepare_matvec(const bqd_cq_matrix* m, const float* x, const float* prepared,
                         const float* y, int64_t batch, int64_t row_begin, int64_t row_count);
// Several matrices on one vector: n in [1, kMaxMulti]; row_begin / row_count
// may be NULL (0 / the rest of each matrix) and are resolved into rb / rc.
int check_matvec_multi(const bqd_cq_matrix* ms, int64_t n, const int64_t* row_begin,
                       const int64_t* row_count, bool with_x, const float* x,
                       const float* prepared, float* const* ys, int64_t* rb, int64_t* rc);
int check_gather(const bqd_cq_matrix* m, const int32_t* rows, int64_t n, const float* out);
int check_f8(const uint8_t* w, int64_t R, int64_t C, const uint8_t* scale, int64_t SR,
             int64_t SC, const float* x, const float* y, int64_t batch);
// f8_matvec_argmax's workspace: one 8-byte slot per workgroup of the
// widest launch (8192) per vector.
constexpr int64_t kF8ArgmaxSlots = 8192;
inline int64_t f8_argmax_workspace_need(int64_t batch) { return batch * kF8ArgmaxSlots * 8; }
// f8_matvec_argmax: check_f8's rules, R >= 1, and the workspace (8-byte
// aligned, large enough) and tokens (4-byte aligned) as two more outputs.
int check_f8_argmax(const uint8_t* w, int64_t R, int64_t C, const uint8_t* scale, int64_t SR,
                    int64_t SC, const float* x, const float* y, int64_t batch,
                    const void* workspace, int64_t workspace_bytes, const int32_t* token);
// f8_matvec_sample: check_f8's rules, 1 <= R <= kMaxSampleLogits,
// 1 <= k <= min(kMaxSampleK, R), a finite temperature >= 0, the workspace as
// f8_matvec_argmax's, and state / token [batch], topk_ids / topk_logits
// [batch][k] (4-byte aligned) as more outputs.
int check_f8_sample(const uint8_t* w, int64_t R, int64_t C, const uint8_t* scale, int64_t SR,
                    int64_t SC, const float* x, const float* y, int64_t batch, int64_t k,
                    float temperature, const uint32_t* state, const void* workspace,
                    int64_t workspace_bytes, const int32_t* token, const int32_t* topk_ids,
                    const float* topk_logits);
int check_i8(const int8_t* w, int64_t R, int64_t C, const uint8_t* scale, int64_t G,
             const float* x, const float* y, int64_t batch);
int check_kv_quantize(const float* v, int64_t n_vec, int64_t d, const int8_t* q,
                      const float* scales);
int check_kv_dot(const int8_t* K, const float* scales, int64_t R, int64_t d, const float* x,
                 const float* y, int64_t batch);
int check_hadamard_mlp(const float* n, int64_t hidden, int64_t H, const float* d1,
                       const float* d2, const float* d3, const float* resid, const float* u,
                       const float* out, int64_t batch);
int check_unpack(const bqd_cq_matrix* m, int64_t row, const uint8_t* idx);
int check_decode(const void* codes, int64_t n, const float* out, int code_size);
int check_read_stream(const void* buf, int64_t bytes, const uint32_t* out);
int64_t sample_workspace_need(int64_t n, int64_t k);  // or BQD_EINVAL
int check_sample(const float* logits, int64_t n, int64_t k, float temperature,
                 const uint32_t* state, const void* workspace, int64_t workspace_bytes,
                 const int32_t* token, const int32_t* topk_ids, const float* topk_logits);
// logits_sample_noalloc: check_sample's rules for everything but the
// workspace, which is the library's scratch of scratch_bytes (a call needing
// more is refused with BQD_EINVAL).
int check_sample_noalloc(const float* logits, int64_t n, int64_t k, float temperature,
                         const uint32_t* state, const int32_t* token, const int32_t* topk_ids,
                         const float* topk_logits, int64_t scratch_bytes);

// Largest sizes the kernels index with their 32-bit row / column counters.
constexpr int64_t kMaxRows = (int64_t)1 << 30;      // exclusive
constexpr int64_t kMaxColumns = (int64_t)1 << 28;   // exclusive
constexpr int64_t kMaxGroup = 1024;
constexpr int64_t kMaxSampleLogits = (int64_t)1 << 20;  // inclusive
constexpr int64_t kMaxSampleK = 64;
// Logits per first-stage sampler workgroup: the smallest of 1024, 2048 and
// 4096 that leaves at most 256 workgroups (256 lists of candidates for the
// second stage) for n <= kMaxSampleLogits.
constexpr int64_t sample_chunk(int64_t n) {
  return n <= 256 * 1024 ? 1024 : (n <= 256 * 2048 ? 2048 : 4096);
}
constexpr int64_t kMaxHadamard = 16384;
constexpr int64_t kMaxMulti = 64;               // inclusive
constexpr int64_t kMaxBatchBlocks = (int64_t)1 << 31;  // exclusive (one workgroup each)

}  // namespace bqd

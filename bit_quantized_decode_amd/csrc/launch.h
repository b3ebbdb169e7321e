// Kernel launchers behind the C ABI.  Arguments arrive validated.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bqd.h"

namespace bqd {

int launch_cq_prepare(const bqd_cq_matrix* m, const float* x, float* prepared, int64_t batch,
                      hipStream_t s);
int launch_cq_matvec(const bqd_cq_matrix* m, const float* prepared, float* y, int64_t batch,
                     int64_t row_begin, int64_t row_count, hipStream_t s);
int launch_cq_prepare_matvec(const bqd_cq_matrix* m, const float* x, float* prepared, float* y,
                             int64_t batch, int64_t row_begin, int64_t row_count, hipStream_t s);
int launch_cq_matvec_multi(const bqd_cq_matrix* ms, int64_t n, const int64_t* row_begin,
                           const int64_t* row_count, bool with_x, const float* x,
                           float* prepared, float* const* ys, hipStream_t s);
int launch_cq_gather(const bqd_cq_matrix* m, const int32_t* rows, int64_t n, float* out,
                     hipStream_t s);
int launch_cq_unpack(const bqd_cq_matrix* m, int64_t row, uint8_t* idx, hipStream_t s);

int launch_f8_matvec(const uint8_t* w, int64_t R, int64_t C, const uint8_t* scale, int64_t SR,
                     int64_t SC, const float* x, float* y, int64_t batch, hipStream_t s);
int launch_f8_matvec_argmax(const uint8_t* w, int64_t R, int64_t C, const uint8_t* scale,
                            int64_t SR, int64_t SC, const float* x, float* y, int64_t batch,
                            void* workspace, int32_t* token, hipStream_t s);
int launch_i8_matvec(const int8_t* w, int64_t R, int64_t C, const uint8_t* scale, int64_t G,
                     const float* x, float* y, int64_t batch, hipStream_t s);
int launch_kv_quantize_int8(const float* v, int64_t n_vec, int64_t d, int8_t* q, float* scales,
                            hipStream_t s);
int launch_kv_int8_dot(const int8_t* K, const float* scales, int64_t R, int64_t d, const float* x,
                       float* y, int64_t batch, hipStream_t s);
int launch_hadamard_mlp(const float* n, int64_t hidden, int64_t H, const float* d1,
                        const float* d2, const float* d3, const float* resid, const float* u,
                        float* out, int64_t batch, hipStream_t s);
int launch_f16_decode(const uint16_t* codes, int64_t n, float* out, hipStream_t s);
int launch_f8_decode(const uint8_t* codes, int64_t n, float* out, hipStream_t s);
int launch_e8m0_decode(const uint8_t* codes, int64_t n, float* out, hipStream_t s);
int launch_read_stream(const void* buf, int64_t bytes, uint32_t* out, hipStream_t s);
int launch_logits_sample(const float* logits, int64_t n, int64_t k, float temperature,
                         uint32_t* state, void* workspace, int32_t* token, int32_t* topk_ids,
                         float* topk_logits, hipStream_t s);

// The rows of each per-workgroup slot a matvec leaves for the fused sampling
// (sample.hip): group g owns rows g gstride + t S + i (t >= 0, i < l_valid,
// i < 2^log2_L, t 2^log2_L + i < rows_pg <= 2^log2_pg), below R; row r is in
// group (r / gstride) % G.
struct SlotRowsHost {
  int64_t R, n_slots, G, gstride;
  int log2_L;
  int64_t l_valid, S;
  int log2_pg;
  int64_t rows_pg;
};
// Top-k / temperature sampling of each vector's logits [batch][R] from the
// slots (8192 per vector) of the matvec that wrote them.
int launch_slots_sample(const float* logits, const uint64_t* slots, const SlotRowsHost& h,
                        int64_t batch, int64_t k, float temperature, uint32_t* state,
                        int32_t* token, int32_t* topk_ids, float* topk_logits, hipStream_t s);
int launch_f8_matvec_sample(const uint8_t* w, int64_t R, int64_t C, const uint8_t* scale,
                            int64_t SR, int64_t SC, const float* x, float* y, int64_t batch,
                            int64_t k, float temperature, uint32_t* state, void* workspace,
                            int32_t* token, int32_t* topk_ids, float* topk_logits,
                            hipStream_t s);

// The allocation-free sampler's device scratch: its size, and its address on
// the device of stream s (looked up once per device).
int64_t sample_scratch_bytes();
int sample_scratch(hipStream_t s, void** out);

inline int launch_status() {
  return hipGetLastError() == hipSuccess ? BQD_OK : BQD_EHIP;
}

// Grid cap of the kernels that loop over their work (grid-stride): 65536
// workgroups of at most 1024 threads keep a launch below the 2^32 work-items
// one dispatch can hold, whatever the problem size.
constexpr int64_t kMaxStrideGrid = 65536;

inline bool is_aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

inline int ilog2(int64_t v) {
  int r = 0;
  while ((int64_t(1) << (r + 1)) <= v) ++r;
  return r;
}

// The smallest r with 2^r >= v (v >= 1).
inline int ceil_log2(int64_t v) {
  int r = 0;
  while ((int64_t(1) << r) < v) ++r;
  return r;
}

}  // namespace bqd

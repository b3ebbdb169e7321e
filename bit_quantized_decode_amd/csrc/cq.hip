// CQ (codebook-quantized) kernels for gfx950: activation prepare, packed-row
// matvec and dense row gather.
//
// Method: "Inference engine, part 2: kernels and token step" — §1 (the
// unnormalized Walsh–Hadamard butterfly), §2 (prepare: zero-pad, transform
// each group, multiply by 1/sqrt(group)), §3 (dot packed rows directly: per
// row and group, the fp16 norm times the sum of codebook[index] * prepared),
// "Row gather" (decode a group's levels times its norm, normalized transform,
// keep the unpadded columns) and §6 (a row range of a matrix).  The record
// layout is that of "Inference engine, part 1: loader and tokenizer", §4.
#include <algorithm>
#include <cmath>

#include "device.h"
#include "launch.h"

namespace bqd {

constexpr int kThreads = 256;       // 4 wavefronts per workgroup
constexpr int kTransformChunk = 1024;  // floats per workgroup in prepare/gather

// ---------------------------------------------------------------------------
// Shared transform step: the butterflies of one chunk held in LDS, stride
// ascending over 1 .. group/2, each pair (a, b) -> (a + b, a - b) in fp32 —
// the same operations, operands and order as the scalar loop on the page, so
// results are bit-identical to it.  `n` is a multiple of `group`.
__device__ __forceinline__ void lds_fwht(float* buf, int n, int log2_group) {
  for (int ls = 0; ls < log2_group; ++ls) {
    const int s = 1 << ls;
    for (int t = threadIdx.x; t < (n >> 1); t += kThreads) {
      const int i = ((t >> ls) << (ls + 1)) | (t & (s - 1));
      const float a = buf[i];
      const float b = buf[i + s];
      buf[i] = a + b;
      buf[i + s] = a - b;
    }
    __syncthreads();
  }
}

// 1/sqrt(group) is applied as the page does: the scale is an fp64 value, the
// product is formed in fp64 and rounded once to fp32.
__device__ __forceinline__ float scale_store(float v, double scale) {
  return (float)((double)v * scale);
}

// ------------------------------------------------------------------ prepare
// Workgroup (vector b, chunk ch) transforms `chunk` padded columns.
__global__ __launch_bounds__(kThreads) void cq_prepare_kernel(
    const float* __restrict__ x, float* __restrict__ p, int64_t input, int64_t input_padded,
    int log2_group, int chunk, int64_t n_chunks, double scale) {
  __shared__ float buf[kTransformChunk];
  const int64_t b = blockIdx.x / n_chunks;
  const int64_t c0 = (blockIdx.x % n_chunks) * (int64_t)chunk;
  const int n = (int)min((int64_t)chunk, input_padded - c0);
  const float* xb = x + b * input;
  for (int i = threadIdx.x; i < n; i += kThreads) {
    const int64_t c = c0 + i;
    buf[i] = c < input ? xb[c] : 0.0f;
  }
  __syncthreads();
  lds_fwht(buf, n, log2_group);
  float* pb = p + b * input_padded + c0;
  for (int i = threadIdx.x; i < n; i += kThreads) pb[i] = scale_store(buf[i], scale);
}

int launch_cq_prepare(const bqd_cq_matrix* m, const float* x, float* prepared, int64_t batch,
                      hipStream_t s) {
  const int chunk = (int)std::max<int64_t>(m->group, std::min<int64_t>(kTransformChunk, m->input_padded));
  const int64_t n_chunks = (m->input_padded + chunk - 1) / chunk;
  const double scale = 1.0 / std::sqrt((double)m->group);
  hipLaunchKernelGGL(cq_prepare_kernel, dim3((unsigned)(n_chunks * batch)), dim3(kThreads), 0, s,
                     x, prepared, m->input, m->input_padded, ilog2(m->group), chunk, n_chunks,
                     scale);
  return launch_status();
}

// ------------------------------------------------------------------- gather
// Workgroup (id i, chunk ch): decode codebook value times norm (an fp32
// product), transform, scale, store the columns below `input`.
__global__ __launch_bounds__(kThreads) void cq_gather_kernel(
    const uint8_t* __restrict__ packed, const uint16_t* __restrict__ norms,
    const float* __restrict__ codebook, const int32_t* __restrict__ rows, float* __restrict__ out,
    int64_t output, int64_t input, int64_t input_padded, int64_t row_bytes, int bits,
    int log2_group, int chunk, int64_t n_chunks, double scale) {
  __shared__ float buf[kTransformChunk];
  __shared__ float cb[32];
  const int64_t i = blockIdx.x / n_chunks;
  const int64_t c0 = (blockIdx.x % n_chunks) * (int64_t)chunk;
  if (c0 >= input) return;  // no visible column in this chunk (uniform)
  const int n = (int)min((int64_t)chunk, input_padded - c0);
  const int64_t r = rows[i];
  float* o = out + i * input;
  if (r < 0 || r >= output) {  // uniform: an id outside the table gives a NaN row
    for (int k = threadIdx.x; k < n; k += kThreads)
      if (c0 + k < input) o[c0 + k] = __uint_as_float(0x7fc00000u);
    return;
  }
  if (threadIdx.x < (1 << bits)) cb[threadIdx.x] = codebook[threadIdx.x];
  __syncthreads();
  const uint8_t* prow = packed + r * row_bytes;
  const uint16_t* nrow = norms + r * (input_padded >> log2_group);
  for (int k = threadIdx.x; k < n; k += kThreads) {
    const int64_t c = c0 + k;
    const float nm = f16_to_f32(nrow[c >> log2_group]);
    buf[k] = cb[byte_index(prow, bits, c)] * nm;
  }
  __syncthreads();
  lds_fwht(buf, n, log2_group);
  for (int k = threadIdx.x; k < n; k += kThreads) {
    const int64_t c = c0 + k;
    if (c < input) o[c] = scale_store(buf[k], scale);
  }
}

int launch_cq_gather(const bqd_cq_matrix* m, const int32_t* rows, int64_t n, float* out,
                     hipStream_t s) {
  if (m->input == 0) return BQD_OK;
  const int chunk = (int)std::max<int64_t>(m->group, std::min<int64_t>(kTransformChunk, m->input_padded));
  const int64_t n_chunks = (m->input_padded + chunk - 1) / chunk;
  const double scale = 1.0 / std::sqrt((double)m->group);
  hipLaunchKernelGGL(cq_gather_kernel, dim3((unsigned)(n_chunks * n)), dim3(kThreads), 0, s,
                     m->packed, m->norms, m->codebook, rows, out, m->output, m->input,
                     m->input_padded, m->row_bytes, (int)m->bits, ilog2(m->group), chunk,
                     n_chunks, scale);
  return launch_status();
}

// ----------------------------------------------------------- generic matvec
// Any shape and alignment: one wavefront per row; lanes stride over each
// group's columns; per lane, the group partial times the norm is added to the
// row sum, then the wavefront reduces in a fixed order.
__global__ __launch_bounds__(kThreads) void cq_matvec_generic(
    const uint8_t* __restrict__ packed, const uint16_t* __restrict__ norms,
    const float* __restrict__ codebook, const float* __restrict__ prepared, float* __restrict__ y,
    int64_t input_padded, int64_t row_bytes, int bits, int log2_group, int64_t row_begin,
    int64_t row_count, int64_t batch) {
  __shared__ float cb[32];
  if (threadIdx.x < (1 << bits)) cb[threadIdx.x] = codebook[threadIdx.x];
  __syncthreads();
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int64_t group = int64_t(1) << log2_group;
  const int64_t n_groups = input_padded >> log2_group;
  for (int64_t i = (int64_t)blockIdx.x * (kThreads / kWave) + wave; i < row_count;
       i += (int64_t)gridDim.x * (kThreads / kWave)) {
    const int64_t r = row_begin + i;
    const uint8_t* prow = packed + r * row_bytes;
    for (int64_t b = 0; b < batch; ++b) {
      const float* pb = prepared + b * input_padded;
      float acc = 0.0f;
      for (int64_t g = 0; g < n_groups; ++g) {
        float part = 0.0f;
        for (int64_t c = g * group + lane; c < (g + 1) * group; c += kWave)
          part += cb[byte_index(prow, bits, c)] * pb[c];
        acc += f16_to_f32(norms[r * n_groups + g]) * part;
      }
      acc = group_sum<kWave>(acc);
      if (lane == kWave - 1) y[b * row_count + i] = acc;
    }
  }
}

// -------------------------------------------------------------- fast matvec
// Rows whose padded width is a multiple of 32 columns, groups of >= 32 and
// dword-aligned rows.  A 32-column chunk is BITS dwords; `LPR` lanes share a
// row (chunk q + LPR*j for j < NJ belongs to lane q), so one load instruction
// of a wavefront reads 64 consecutive chunks: contiguous, coalesced bytes.
// Each lane keeps the prepared activations of its chunks in registers for the
// whole kernel (the same columns for every row), looks the codebook up in LDS
// (2^BITS distinct words in distinct banks: conflict free), multiplies the
// chunk partial by its group norm, and the LPR lanes of a row reduce with DPP.
// NB activation vectors share each decoded weight.  U row steps are loaded
// before any of them is consumed, to keep loads in flight.
template <int BITS, int NJ, int LPR, int NB, int U>
__global__ __launch_bounds__(kThreads) void cq_matvec_fast(
    const uint8_t* __restrict__ packed, const uint16_t* __restrict__ norms,
    const float* __restrict__ codebook, const float* __restrict__ prepared, float* __restrict__ y,
    int64_t input_padded, int64_t row_bytes, int log2_group, int64_t row_begin, int64_t row_count,
    int nb) {
  constexpr int SLOTS = LPR <= kThreads ? kThreads / LPR : 1;  // rows per step
  constexpr int WPS = LPR > kWave ? LPR / kWave : 1;            // wavefronts per row
  constexpr int RED = LPR > kWave ? kThreads / kWave * U * NB : 1;
  __shared__ float cb[32];
  __shared__ float red[RED];
  const int tid = threadIdx.x;
  const int slot = tid / LPR;
  const int q = tid % LPR;
  if (tid < (1 << BITS)) cb[tid] = codebook[tid];

  const int64_t n_groups = input_padded >> log2_group;
  float act[NB][NJ][32];
  int gidx[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int64_t c = 32 * (int64_t)(q + LPR * j);
    gidx[j] = (int)(c >> log2_group);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      // vectors past nb reuse the last one; their sums are never stored
      const float* pb = prepared + (int64_t)(b < nb ? b : nb - 1) * input_padded + c;
#pragma unroll
      for (int k = 0; k < 32; ++k) act[b][j][k] = pb[k];
    }
  }
  __syncthreads();

  const int64_t n_steps = (row_count + SLOTS - 1) / SLOTS;
  for (int64_t s0 = (int64_t)blockIdx.x * U; s0 < n_steps; s0 += (int64_t)gridDim.x * U) {
    uint32_t d[U][NJ][BITS];
    float nrm[U][NJ];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int64_t i = (s0 + u) * SLOTS + slot;
      i = i < row_count ? i : row_count - 1;  // in-bounds load; the result is dropped
      const int64_t r = row_begin + i;
      const uint32_t* prow = reinterpret_cast<const uint32_t*>(packed + r * row_bytes);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const uint32_t* pc = prow + BITS * (q + LPR * j);
#pragma unroll
        for (int t = 0; t < BITS; ++t) d[u][j][t] = __builtin_nontemporal_load(pc + t);
        nrm[u][j] = f16_to_f32(norms[r * n_groups + gidx[j]]);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float acc[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[b] = 0.0f;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        float part[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) part[b] = 0.0f;
#pragma unroll
        for (int k = 0; k < 32; ++k) {
          const float w = cb[chunk_index<BITS>(d[u][j], k)];
#pragma unroll
          for (int b = 0; b < NB; ++b) part[b] += w * act[b][j][k];
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b] += nrm[u][j] * part[b];
      }
      const int64_t i = (s0 + u) * SLOTS + slot;
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[b] = group_sum<(LPR < kWave ? LPR : kWave)>(acc[b]);
      if constexpr (LPR <= kWave) {
        if (q == LPR - 1 && i < row_count) {
#pragma unroll
          for (int b = 0; b < NB; ++b)
            if (b < nb) y[b * row_count + i] = acc[b];
        }
      } else {
        const int w_in_slot = q / kWave;
        if ((tid & (kWave - 1)) == kWave - 1) {
#pragma unroll
          for (int b = 0; b < NB; ++b) red[((slot * WPS + w_in_slot) * U + u) * NB + b] = acc[b];
        }
      }
    }
    if constexpr (LPR > kWave) {
      __syncthreads();
      for (int t = tid; t < SLOTS * U * NB; t += kThreads) {
        const int b = t % NB;
        const int u = (t / NB) % U;
        const int sl = t / (NB * U);
        float v = 0.0f;
        for (int w = 0; w < WPS; ++w) v += red[((sl * WPS + w) * U + u) * NB + b];
        const int64_t i = (s0 + u) * SLOTS + sl;
        if (b < nb && i < row_count) y[b * row_count + i] = v;
      }
      __syncthreads();
    }
  }
}

namespace {

constexpr int kMaxGrid = 4096;

struct FastShape {
  int lpr, nj;
};

// The fast kernel's lane layout for a row of n_chunk 32-column chunks, or
// {0, 0} when no instantiation covers it.
FastShape fast_shape(int64_t n_chunk, int nb_max) {
  if (nb_max == 1) {
    if (n_chunk >= 8 && n_chunk <= 64 && (n_chunk & (n_chunk - 1)) == 0) return {(int)n_chunk, 1};
    if (n_chunk == 128) return {64, 2};
    if (n_chunk == 256) return {64, 4};
  } else {
    if (n_chunk >= 8 && n_chunk <= 256 && (n_chunk & (n_chunk - 1)) == 0) return {(int)n_chunk, 1};
  }
  return {0, 0};
}

bool fast_ok(const bqd_cq_matrix* m) {
  return m->input_padded % 32 == 0 && m->group >= 32 && m->row_bytes % 4 == 0 &&
         is_aligned(m->packed, 4);
}

template <int BITS, int NJ, int LPR, int NB>
int launch_fast(const bqd_cq_matrix* m, const float* prepared, float* y, int nb,
                int64_t row_begin, int64_t row_count, hipStream_t s) {
  constexpr int U = NB == 1 ? 4 : 2;
  constexpr int SLOTS = LPR <= kThreads ? kThreads / LPR : 1;
  const int64_t n_steps = (row_count + SLOTS - 1) / SLOTS;
  const int64_t grid = std::min<int64_t>((n_steps + U - 1) / U, kMaxGrid);
  hipLaunchKernelGGL((cq_matvec_fast<BITS, NJ, LPR, NB, U>), dim3((unsigned)grid), dim3(kThreads),
                     0, s, m->packed, m->norms, m->codebook, prepared, y, m->input_padded,
                     m->row_bytes, ilog2(m->group), row_begin, row_count, nb);
  return launch_status();
}

template <int BITS>
int dispatch_fast(const bqd_cq_matrix* m, FastShape f, int nb_max, const float* prepared, float* y,
                  int nb, int64_t row_begin, int64_t row_count, hipStream_t s) {
  if (nb_max == 1) {
    switch (f.lpr * 16 + f.nj) {
      case 8 * 16 + 1: return launch_fast<BITS, 1, 8, 1>(m, prepared, y, nb, row_begin, row_count, s);
      case 16 * 16 + 1: return launch_fast<BITS, 1, 16, 1>(m, prepared, y, nb, row_begin, row_count, s);
      case 32 * 16 + 1: return launch_fast<BITS, 1, 32, 1>(m, prepared, y, nb, row_begin, row_count, s);
      case 64 * 16 + 1: return launch_fast<BITS, 1, 64, 1>(m, prepared, y, nb, row_begin, row_count, s);
      case 64 * 16 + 2: return launch_fast<BITS, 2, 64, 1>(m, prepared, y, nb, row_begin, row_count, s);
      case 64 * 16 + 4: return launch_fast<BITS, 4, 64, 1>(m, prepared, y, nb, row_begin, row_count, s);
    }
  } else {
    switch (f.lpr) {
      case 8: return launch_fast<BITS, 1, 8, 4>(m, prepared, y, nb, row_begin, row_count, s);
      case 16: return launch_fast<BITS, 1, 16, 4>(m, prepared, y, nb, row_begin, row_count, s);
      case 32: return launch_fast<BITS, 1, 32, 4>(m, prepared, y, nb, row_begin, row_count, s);
      case 64: return launch_fast<BITS, 1, 64, 4>(m, prepared, y, nb, row_begin, row_count, s);
      case 128: return launch_fast<BITS, 1, 128, 4>(m, prepared, y, nb, row_begin, row_count, s);
      case 256: return launch_fast<BITS, 1, 256, 4>(m, prepared, y, nb, row_begin, row_count, s);
    }
  }
  return BQD_EINVAL;  // unreachable: fast_shape() only returns instantiated layouts
}

int run_fast(const bqd_cq_matrix* m, FastShape f, int nb_max, const float* prepared, float* y,
             int nb, int64_t row_begin, int64_t row_count, hipStream_t s) {
  switch (m->bits) {
    case 2: return dispatch_fast<2>(m, f, nb_max, prepared, y, nb, row_begin, row_count, s);
    case 3: return dispatch_fast<3>(m, f, nb_max, prepared, y, nb, row_begin, row_count, s);
    case 4: return dispatch_fast<4>(m, f, nb_max, prepared, y, nb, row_begin, row_count, s);
    case 5: return dispatch_fast<5>(m, f, nb_max, prepared, y, nb, row_begin, row_count, s);
  }
  return BQD_EINVAL;
}

int launch_generic(const bqd_cq_matrix* m, const float* prepared, float* y, int64_t batch,
                   int64_t row_begin, int64_t row_count, hipStream_t s) {
  const int64_t waves = kThreads / kWave;
  const int64_t grid = std::min<int64_t>((row_count + waves - 1) / waves, kMaxGrid);
  hipLaunchKernelGGL(cq_matvec_generic, dim3((unsigned)grid), dim3(kThreads), 0, s, m->packed,
                     m->norms, m->codebook, prepared, y, m->input_padded, m->row_bytes,
                     (int)m->bits, ilog2(m->group), row_begin, row_count, batch);
  return launch_status();
}

}  // namespace

int launch_cq_matvec(const bqd_cq_matrix* m, const float* prepared, float* y, int64_t batch,
                     int64_t row_begin, int64_t row_count, hipStream_t s) {
  if (!fast_ok(m)) return launch_generic(m, prepared, y, batch, row_begin, row_count, s);
  const int64_t n_chunk = m->input_padded / 32;
  if (batch == 1) {
    const FastShape f = fast_shape(n_chunk, 1);
    if (f.lpr == 0) return launch_generic(m, prepared, y, batch, row_begin, row_count, s);
    return run_fast(m, f, 1, prepared, y, 1, row_begin, row_count, s);
  }
  // Several vectors: up to four share each decoded weight per launch.
  const FastShape f4 = fast_shape(n_chunk, 4);
  const FastShape f1 = fast_shape(n_chunk, 1);
  if (f4.lpr == 0 && f1.lpr == 0) return launch_generic(m, prepared, y, batch, row_begin, row_count, s);
  for (int64_t b = 0; b < batch;) {
    const int64_t nb = f4.lpr ? std::min<int64_t>(4, batch - b) : 1;
    const int rc = f4.lpr ? run_fast(m, f4, 4, prepared + b * m->input_padded, y + b * row_count,
                                     (int)nb, row_begin, row_count, s)
                          : run_fast(m, f1, 1, prepared + b * m->input_padded, y + b * row_count,
                                     1, row_begin, row_count, s);
    if (rc) return rc;
    b += nb;
  }
  return BQD_OK;
}

// ------------------------------------------------------------- unpack probe
// idx[c] for one row through the same decode the matvec uses for this
// matrix: chunk decode from dwords on the fast layout, byte decode otherwise.
template <int BITS>
__global__ void cq_unpack_chunks(const uint8_t* __restrict__ prow, uint8_t* __restrict__ idx,
                                 int64_t n_chunk) {
  const int64_t ch = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (ch >= n_chunk) return;
  const uint32_t* pc = reinterpret_cast<const uint32_t*>(prow) + BITS * ch;
  uint32_t d[BITS];
#pragma unroll
  for (int t = 0; t < BITS; ++t) d[t] = pc[t];
#pragma unroll
  for (int k = 0; k < 32; ++k) idx[32 * ch + k] = (uint8_t)chunk_index<BITS>(d, k);
}

__global__ void cq_unpack_bytes(const uint8_t* __restrict__ prow, uint8_t* __restrict__ idx,
                                int64_t n, int bits) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c < n) idx[c] = (uint8_t)byte_index(prow, bits, c);
}

int launch_cq_unpack(const bqd_cq_matrix* m, int64_t row, uint8_t* idx, hipStream_t s) {
  const uint8_t* prow = m->packed + row * m->row_bytes;
  if (fast_ok(m)) {
    const int64_t n_chunk = m->input_padded / 32;
    const dim3 grid((unsigned)((n_chunk + 63) / 64)), block(64);
    switch (m->bits) {
      case 2: hipLaunchKernelGGL(cq_unpack_chunks<2>, grid, block, 0, s, prow, idx, n_chunk); break;
      case 3: hipLaunchKernelGGL(cq_unpack_chunks<3>, grid, block, 0, s, prow, idx, n_chunk); break;
      case 4: hipLaunchKernelGGL(cq_unpack_chunks<4>, grid, block, 0, s, prow, idx, n_chunk); break;
      case 5: hipLaunchKernelGGL(cq_unpack_chunks<5>, grid, block, 0, s, prow, idx, n_chunk); break;
    }
  } else {
    const dim3 grid((unsigned)((m->input_padded + 255) / 256)), block(256);
    hipLaunchKernelGGL(cq_unpack_bytes, grid, block, 0, s, prow, idx, m->input_padded,
                       (int)m->bits);
  }
  return launch_status();
}

}  // namespace bqd

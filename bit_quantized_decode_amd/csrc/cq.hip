// CQ (codebook-quantized) kernels for gfx950: activation prepare, packed-row
// matvec and dense row gather.
//
// Method: "Inference engine, part 2: kernels and token step" — §1 (the
// unnormalized Walsh–Hadamard butterfly), §2 (prepare: zero-pad, transform
// each group, multiply by 1/sqrt(group)), §3 (dot packed rows directly: per
// row and group, the fp16 norm times the sum of codebook[index] * prepared),
// "Row gather" (each group's codebook values scaled by the group norm, the
// normalized transform, the columns below the unpadded width) and §6 (a row range of a matrix).  The record
// layout is that of "Inference engine, part 1: loader and tokenizer", §4.
#include <algorithm>
#include <atomic>
#include <cmath>

#include "device.h"
#include "launch.h"

namespace bqd {

constexpr int kThreads = 256;  // 4 wavefronts per workgroup
constexpr int kWavesPerBlock = kThreads / kWave;

int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// 1/sqrt(group) is applied as the page does: the scale is an fp64 value, the
// product is formed in fp64 and rounded once to fp32.
__device__ __forceinline__ float scale_store(float v, double scale) {
  return (float)((double)v * scale);
}

// Elements per lane of the wavefront transform: a wavefront spans one group
// (64 * E = group) for groups of 64 and more, else 64 / group whole groups.
inline int lane_elems(int64_t group) { return group >= 64 ? (int)(group / 64) : 1; }

// ------------------------------------------------------------------ prepare
// One wavefront per (vector, span of 64*E padded columns).
template <int E>
__global__ __launch_bounds__(kThreads) void cq_prepare_kernel(
    const float* __restrict__ x, float* __restrict__ p, int64_t input, int64_t input_padded,
    int log2_group, int64_t spans, int64_t n_waves, double scale) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wv = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
  if (wv >= n_waves) return;  // whole wavefront
  const int64_t b = wv / spans;
  const int64_t c0 = (wv % spans) * (64 * E) + lane * E;
  const float* xb = x + b * input;
  float v[E];
#pragma unroll
  for (int e = 0; e < E; ++e) v[e] = c0 + e < input ? xb[c0 + e] : 0.0f;
  wave_fwht<E>(v, lane, log2_group);
  float* pb = p + b * input_padded;
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (c0 + e < input_padded) pb[c0 + e] = scale_store(v[e], scale);
}

template <int E>
int launch_prepare_e(const bqd_cq_matrix* m, const float* x, float* prepared, int64_t batch,
                     hipStream_t s) {
  const int64_t spans = (m->input_padded + 64 * E - 1) / (64 * E);
  const int64_t n_waves = spans * batch;
  const int64_t grid = (n_waves + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL((cq_prepare_kernel<E>), dim3((unsigned)grid), dim3(kThreads), 0, s, x,
                     prepared, m->input, m->input_padded, ilog2(m->group), spans, n_waves,
                     1.0 / std::sqrt((double)m->group));
  return launch_status();
}

int launch_cq_prepare(const bqd_cq_matrix* m, const float* x, float* prepared, int64_t batch,
                      hipStream_t s) {
  switch (lane_elems(m->group)) {
    case 1: return launch_prepare_e<1>(m, x, prepared, batch, s);
    case 2: return launch_prepare_e<2>(m, x, prepared, batch, s);
    case 4: return launch_prepare_e<4>(m, x, prepared, batch, s);
    case 8: return launch_prepare_e<8>(m, x, prepared, batch, s);
    case 16: return launch_prepare_e<16>(m, x, prepared, batch, s);
  }
  return BQD_EINVAL;  // unreachable: group <= 1024 is validated
}

// ------------------------------------------------------------------- gather
// One wavefront per (id, span of 64*E columns): codebook value times norm
// (an fp32 product), transform, scale, store the columns below `input`.
template <int E>
__global__ __launch_bounds__(kThreads) void cq_gather_kernel(
    const uint8_t* __restrict__ packed, const uint16_t* __restrict__ norms,
    const float* __restrict__ codebook, const int32_t* __restrict__ rows, float* __restrict__ out,
    int64_t output, int64_t input, int64_t input_padded, int64_t row_bytes, int bits,
    int log2_group, int64_t spans, int64_t n_waves, double scale) {
  __shared__ float cb[32];
  if (threadIdx.x < (1 << bits)) cb[threadIdx.x] = codebook[threadIdx.x];
  __syncthreads();
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wv = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
  if (wv >= n_waves) return;  // whole wavefront
  const int64_t i = wv / spans;
  const int64_t c0 = (wv % spans) * (64 * E) + lane * E;
  const int64_t r = rows[i];
  float* o = out + i * input;
  if (r < 0 || r >= output) {  // an id outside the table: a NaN row
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (c0 + e < input) o[c0 + e] = __uint_as_float(0x7fc00000u);
    return;
  }
  const uint8_t* prow = packed + r * row_bytes;
  const uint16_t* nrow = norms + r * (input_padded >> log2_group);
  float v[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int64_t c = c0 + e;
    v[e] = c < input_padded ? cb[byte_index(prow, bits, c)] * f16_to_f32(nrow[c >> log2_group])
                            : 0.0f;
  }
  wave_fwht<E>(v, lane, log2_group);
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (c0 + e < input) o[c0 + e] = scale_store(v[e], scale);
}

template <int E>
int launch_gather_e(const bqd_cq_matrix* m, const int32_t* rows, int64_t n, float* out,
                    hipStream_t s) {
  // spans past the last visible column store nothing and are not launched
  const int64_t spans = (m->input + 64 * E - 1) / (64 * E);
  const int64_t n_waves = spans * n;
  const int64_t grid = (n_waves + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL((cq_gather_kernel<E>), dim3((unsigned)grid), dim3(kThreads), 0, s,
                     m->packed, m->norms, m->codebook, rows, out, m->output, m->input,
                     m->input_padded, m->row_bytes, (int)m->bits, ilog2(m->group), spans,
                     n_waves, 1.0 / std::sqrt((double)m->group));
  return launch_status();
}

int launch_cq_gather(const bqd_cq_matrix* m, const int32_t* rows, int64_t n, float* out,
                     hipStream_t s) {
  if (m->input == 0) return BQD_OK;
  switch (lane_elems(m->group)) {
    case 1: return launch_gather_e<1>(m, rows, n, out, s);
    case 2: return launch_gather_e<2>(m, rows, n, out, s);
    case 4: return launch_gather_e<4>(m, rows, n, out, s);
    case 8: return launch_gather_e<8>(m, rows, n, out, s);
    case 16: return launch_gather_e<16>(m, rows, n, out, s);
  }
  return BQD_EINVAL;
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
  for (int64_t i = (int64_t)blockIdx.x * kWavesPerBlock + wave; i < row_count;
       i += (int64_t)gridDim.x * kWavesPerBlock) {
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

// ------------------------------------------------------ fast matvec, batch 1
// Rows whose padded width is a multiple of 32 columns, groups of >= 32 and
// dword-aligned rows.  A 32-column chunk is BITS dwords; LPR lanes share a
// row and each owns NJ chunks: chunks q*NJ .. q*NJ+NJ-1 when CONTIG (one
// contiguous span, so one group norm per row once groups span it), else
// chunks q + LPR*j (each load instruction of a wavefront then reads 64
// consecutive chunks).  Every lane keeps the prepared activations of its
// chunks in registers for the whole kernel (the same columns for every row).
// They are staged once per workgroup through LDS: coalesced global loads,
// then 16-byte LDS reads from a layout padded by 4 floats per lane span so
// that the 16 lanes of a read phase hit distinct banks.  The codebook is
// looked up in LDS (2^BITS distinct words in distinct banks: conflict free),
// each chunk partial is multiplied by its group norm, and the LPR lanes of a
// row reduce with DPP.  The codebook lookups are the LDS's limit and their
// latency is hidden by occupancy: the kernel is held to 128 VGPRs (4
// wavefronts per SIMD; 2 for rows of 8192 columns, whose activations alone
// take 128) and the grid is persistent, each workgroup walking steps of
// SLOTS*U rows.
template <int NJ, int LPR, bool CONTIG>
struct ActLayout {
  static constexpr int kUnit = CONTIG ? 32 * NJ : 32;  // floats read contiguously by a lane
  static constexpr int kStride = kUnit + 4;            // padded LDS stride of a unit
  // LDS float offset of float f of the padded row
  __device__ static int offset(int f) {
    const int c = f >> 5;  // chunk
    const int unit = CONTIG ? c / NJ : c;
    const int within = CONTIG ? (c % NJ) * 32 + (f & 31) : (f & 31);
    return unit * kStride + within;
  }
  static int64_t floats(int64_t input_padded) {
    const int64_t n_chunk = input_padded / 32;
    return (CONTIG ? n_chunk / NJ : n_chunk) * kStride;
  }
};

template <int BITS, int NJ, int LPR, int U, bool CONTIG>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(NJ > 2 ? 2 : 4, NJ > 2 ? 2 : 4)))
void cq_matvec_b1(const uint8_t* __restrict__ packed, const uint16_t* __restrict__ norms,
                  const float* __restrict__ codebook, const float* __restrict__ prepared,
                  float* __restrict__ y, int64_t input_padded, int64_t row_bytes, int log2_group,
                  int64_t row_begin, int64_t row_count) {
  typedef ActLayout<NJ, LPR, CONTIG> L;
  constexpr int SLOTS = kThreads / LPR;  // rows per step
  extern __shared__ float act_lds[];
  __shared__ float cb[32];
  const int tid = threadIdx.x;
  const int slot = tid / LPR;
  const int q = tid % LPR;
  const int n_groups = (int)(input_padded >> log2_group);
  const int rows = (int)row_count;  // < 2^30, validated
  const int n_steps = (rows + SLOTS - 1) / SLOTS;
  const int stride = (int)gridDim.x * U;
  auto chunk_of = [&](int j) { return CONTIG ? q * NJ + j : q + LPR * j; };
  // one norm per row when the lane's chunks lie in one group
  const bool one_norm = CONTIG && (32 * NJ) <= (1 << log2_group);
  const uint8_t* lane_base = packed + row_begin * row_bytes + 4 * BITS * chunk_of(0);
  const uint16_t* norm_base = norms + row_begin * n_groups;
  int gidx[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) gidx[j] = (32 * chunk_of(j)) >> log2_group;

  // stage the activations (coalesced float4 reads) and the codebook
  const int n4 = (int)(input_padded >> 2);
  for (int i = tid; i < n4; i += kThreads) {
    const float4 v = reinterpret_cast<const float4*>(prepared)[i];
    *reinterpret_cast<float4*>(act_lds + L::offset(4 * i)) = v;
  }
  if (tid < (1 << BITS)) cb[tid] = codebook[tid];
  __syncthreads();
  float act[NJ][32];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const float* src = act_lds + L::offset(32 * chunk_of(j));
#pragma unroll
    for (int k = 0; k < 32; k += 4) {
      const float4 v = *reinterpret_cast<const float4*>(src + k);
      act[j][k] = v.x;
      act[j][k + 1] = v.y;
      act[j][k + 2] = v.z;
      act[j][k + 3] = v.w;
    }
  }

  for (int s0 = (int)blockIdx.x * U; s0 < n_steps; s0 += stride) {
    uint32_t d[U][NJ][BITS];
    uint16_t nb[U][NJ];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = min((s0 + u) * SLOTS + slot, rows - 1);  // in bounds; dropped if clamped
      const uint32_t* pc = reinterpret_cast<const uint32_t*>(lane_base + (int64_t)i * row_bytes);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int off = CONTIG ? BITS * j : BITS * LPR * j;
#pragma unroll
        for (int t = 0; t < BITS; ++t) d[u][j][t] = pc[off + t];
      }
      const uint16_t* nr = norm_base + (int64_t)i * n_groups;
      if (one_norm) {
        const uint16_t n0 = nr[gidx[0]];
#pragma unroll
        for (int j = 0; j < NJ; ++j) nb[u][j] = n0;
      } else {
#pragma unroll
        for (int j = 0; j < NJ; ++j) nb[u][j] = nr[gidx[j]];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float acc = 0.0f;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        uint32_t a[32];
        chunk_addresses<BITS>(d[u][j], a);
        float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
        for (int k = 0; k < 32; k += 2) {
          p0 += lds_at(cb, a[k]) * act[j][k];
          p1 += lds_at(cb, a[k + 1]) * act[j][k + 1];
        }
        acc += f16_to_f32(nb[u][j]) * (p0 + p1);
      }
      acc = group_sum<LPR>(acc);
      const int i = (s0 + u) * SLOTS + slot;
      if (q == LPR - 1 && i < rows) y[i] = acc;
    }
  }
}

// -------------------------------------------------- fast matvec, NB vectors
// Same lane layout; NB activation vectors share each decoded weight.  Rows
// wider than one wavefront (LPR > 64) are split over LPR/64 wavefronts whose
// partial sums meet in LDS.
template <int BITS, int NJ, int LPR, int NB, int U>
__global__ __launch_bounds__(kThreads) void cq_matvec_nb(
    const uint8_t* __restrict__ packed, const uint16_t* __restrict__ norms,
    const float* __restrict__ codebook, const float* __restrict__ prepared, float* __restrict__ y,
    int64_t input_padded, int64_t row_bytes, int log2_group, int64_t row_begin, int64_t row_count,
    int64_t y_stride, int nb) {
  constexpr int SLOTS = LPR <= kThreads ? kThreads / LPR : 1;  // rows per step
  constexpr int WPS = LPR > kWave ? LPR / kWave : 1;            // wavefronts per row
  constexpr int RED = LPR > kWave ? kWavesPerBlock * U * NB : 1;
  typedef ActLayout<NJ, LPR, false> L;
  extern __shared__ float act_lds[];  // one padded activation row at a time
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
  for (int j = 0; j < NJ; ++j) gidx[j] = (int)((32 * (int64_t)(q + LPR * j)) >> log2_group);
  // Activations reach registers through LDS: coalesced float4 loads of one
  // vector, then 16-byte reads of each lane's chunks from the padded layout.
  // Vectors past nb reuse the last one; their sums are never stored.
  const int n4 = (int)(input_padded >> 2);
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const float4* src = reinterpret_cast<const float4*>(prepared + (int64_t)(b < nb ? b : nb - 1) * input_padded);
    for (int i = tid; i < n4; i += kThreads)
      *reinterpret_cast<float4*>(act_lds + L::offset(4 * i)) = src[i];
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const float* a = act_lds + L::offset(32 * (q + LPR * j));
#pragma unroll
      for (int k = 0; k < 32; k += 4) {
        const float4 v = *reinterpret_cast<const float4*>(a + k);
        act[b][j][k] = v.x;
        act[b][j][k + 1] = v.y;
        act[b][j][k + 2] = v.z;
        act[b][j][k + 3] = v.w;
      }
    }
    __syncthreads();
  }

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
        for (int t = 0; t < BITS; ++t) d[u][j][t] = pc[t];
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
        uint32_t a[32];
        chunk_addresses<BITS>(d[u][j], a);
        float part[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) part[b] = 0.0f;
#pragma unroll
        for (int k = 0; k < 32; ++k) {
          const float w = lds_at(cb, a[k]);
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
            if (b < nb) y[b * y_stride + i] = acc[b];
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
        if (b < nb && i < row_count) y[b * y_stride + i] = v;
      }
      __syncthreads();
    }
  }
}

// ------------------------------------------------ matrix-core matvec, B >= 2
// Several activation vectors share each decoded weight; the contraction runs
// on the matrix cores (v_mfma_f32_16x16x32_bf16: a 16-row x 32-column tile of
// weights times 32 columns x 16 vectors).  fp32 operands are carried exactly
// enough as bf16 pairs: x = hi + lo with hi = bf16(x), lo = bf16(x - hi), so
// |x - hi - lo| <= 2^-18 |x|; three products (hi*hi, hi*lo, lo*hi) per tile
// accumulate in fp32 (the dropped lo*lo term is below 2^-18 of each product).
// The codebook table in LDS holds each entry's (hi | lo << 16), so one LDS read
// per weight feeds both weight operands.
//
// A workgroup has one wavefront per 256-column span of the padded row (groups
// are >= 256, so a span has one norm per row).  Lane l owns tile row l % 16
// (and vector slot l % 16 of the B operand) and the 64-column quarter l / 16 of
// its span; K-block kb of the span takes, from quarter g, columns
// 64g + 8kb .. 64g + 8kb + 7.  Each wavefront keeps its span's activations as
// B operands in registers for the whole kernel and walks 16-row tiles; per
// tile the span partials (times their norms) meet in LDS and are summed in
// span order.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {  // finite x
  uint32_t u = __float_as_uint(x);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
// (hi, lo) bf16 split of x, packed as hi | lo << 16
__device__ __forceinline__ uint32_t bf16_split(float x) {
  const uint32_t hi = bf16_rne_bits(x);
  const float rest = x - __uint_as_float(hi << 16);
  return hi | (bf16_rne_bits(rest) << 16);
}

template <int BITS>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(4, 4)))
void cq_matvec_mfma(const uint8_t* __restrict__ packed, const uint16_t* __restrict__ norms,
                    const float* __restrict__ codebook, const float* __restrict__ prepared,
                    float* __restrict__ y, int64_t input_padded, int64_t row_bytes,
                    int log2_group, int64_t row_begin, int64_t row_count, int64_t y_stride,
                    int nb) {
  constexpr int kSpanBytes = 32 * BITS;  // 256 columns of BITS-bit indices
  __shared__ uint32_t cbs[32];
  __shared__ float red[16][16][17];      // [span][tile row][vector], padded
  const int tid = threadIdx.x;
  const int span = tid >> 6;             // wavefront = span
  const int n_spans = blockDim.x >> 6;
  const int l = tid & 63;
  const int r16 = l & 15;                // tile row (A, D) and vector slot (B)
  const int qg = l >> 4;                 // 64-column quarter of the span
  const int rows = (int)row_count;
  const int n_tiles = (rows + 15) >> 4;
  const int n_groups = (int)(input_padded >> log2_group);
  const int group = (256 * span) >> log2_group;  // the span's group (groups >= 256)

  // The first tile's weights and norms load before the operand set-up, so
  // their latency overlaps it; afterwards each tile's loads are issued before
  // the previous tile is decoded (ping-pong buffers, unconditional loads of
  // clamped rows).
  const uint8_t* lane_base = packed + row_begin * row_bytes + kSpanBytes * span + 8 * BITS * qg;
  typedef uint32_t Words[2 * BITS];  // this lane's 64 indices
  auto load_tile = [&](Words& d, float (&nrm)[4], int t) {
    const int r = min(16 * t + r16, rows - 1);  // in bounds; dropped if clamped
    const uint32_t* pc = reinterpret_cast<const uint32_t*>(lane_base + (int64_t)r * row_bytes);
#pragma unroll
    for (int i = 0; i < 2 * BITS; ++i) d[i] = pc[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = min(16 * t + 4 * qg + i, rows - 1);
      nrm[i] = f16_to_f32(norms[(row_begin + rr) * n_groups + group]);
    }
  };
  auto tile = [&](const Words& d, const float (&nrm)[4], const u32x4_t (&bhi)[8],
                  const u32x4_t (&blo)[8], int t) {
    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      uint32_t v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int k = 8 * kb + e;  // index position in the lane's 64
        const int bit = BITS * k, w = bit >> 5, sh = bit & 31;
        uint32_t idx;
        if (sh + BITS <= 32) idx = (d[w] >> sh) & ((1u << BITS) - 1u);
        else idx = __builtin_amdgcn_alignbit(d[w + 1], d[w], sh) & ((1u << BITS) - 1u);
        v[e] = cbs[idx];
      }
      u32x4_t ahi, alo;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ahi[j] = __builtin_amdgcn_perm(v[2 * j + 1], v[2 * j], 0x05040100u);
        alo[j] = __builtin_amdgcn_perm(v[2 * j + 1], v[2 * j], 0x07060302u);
      }
      const bf16x8_t a_hi = __builtin_bit_cast(bf16x8_t, ahi);
      const bf16x8_t a_lo = __builtin_bit_cast(bf16x8_t, alo);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_hi, __builtin_bit_cast(bf16x8_t, bhi[kb]), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_hi, __builtin_bit_cast(bf16x8_t, blo[kb]), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_lo, __builtin_bit_cast(bf16x8_t, bhi[kb]), acc, 0, 0, 0);
    }
    // acc[i] = tile row 4*qg + i, vector r16
#pragma unroll
    for (int i = 0; i < 4; ++i) red[span][4 * qg + i][r16] = acc[i] * nrm[i];
    __syncthreads();
    // 256 outputs per tile; blocks of fewer than 4 spans have fewer threads
    for (int o = tid; o < 256; o += blockDim.x) {
      const int row = o >> 4, vec = o & 15;
      float sum = 0.0f;
      for (int sp = 0; sp < n_spans; ++sp) sum += red[sp][row][vec];
      const int i = 16 * t + row;
      if (vec < nb && i < rows) y[vec * y_stride + i] = sum;
    }
    __syncthreads();
  };

  int t = blockIdx.x;  // < n_tiles: the grid has at most n_tiles blocks
  Words da, db;
  float na[4], nbn[4];
  load_tile(da, na, t);
  if (tid < (1 << BITS)) cbs[tid] = bf16_split(codebook[tid]);
  // B operands: vector r16's columns 256*span + 64*qg + 8*kb + e.  The loads
  // sit in one block under the lane's own condition, so slots past nb fetch
  // nothing and the 64 loads of a live lane are all in flight at once.
  u32x4_t bhi[8], blo[8];
  {
    float xv[64];
    if (r16 < nb) {
      const float* src = prepared + (int64_t)r16 * input_padded + 256 * span + 64 * qg;
#pragma unroll
      for (int k = 0; k < 64; ++k) xv[k] = src[k];
    } else {
#pragma unroll
      for (int k = 0; k < 64; ++k) xv[k] = 0.0f;
    }
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      uint32_t h[8], o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t sp = bf16_split(xv[8 * kb + e]);
        h[e] = sp & 0xffffu;
        o[e] = sp >> 16;
      }
#pragma unroll
      for (int dd = 0; dd < 4; ++dd) {
        bhi[kb][dd] = h[2 * dd] | (h[2 * dd + 1] << 16);
        blo[kb][dd] = o[2 * dd] | (o[2 * dd + 1] << 16);
      }
    }
  }
  __syncthreads();
  const int stride = (int)gridDim.x;
  while (true) {
    load_tile(db, nbn, t + stride);
    __builtin_amdgcn_sched_barrier(0);
    tile(da, na, bhi, blo, t);
    t += stride;
    if (t >= n_tiles) break;
    load_tile(da, na, t + stride);
    __builtin_amdgcn_sched_barrier(0);
    tile(db, nbn, bhi, blo, t);
    t += stride;
    if (t >= n_tiles) break;
  }
}

namespace {

constexpr int kMaxGrid = 4096;
constexpr int kB1BlocksPerCu = 4;
constexpr int kNbBlocksPerCu = 2;

struct FastShape {
  int lpr, nj;
};

// The fast kernels' lane layout for a row of n_chunk 32-column chunks, or
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

template <int BITS, int NJ, int LPR>
int launch_b1(const bqd_cq_matrix* m, const float* prepared, float* y, int64_t row_begin,
              int64_t row_count, hipStream_t s) {
  constexpr int U = 2;
  constexpr int SLOTS = kThreads / LPR;
  const int64_t n_steps = (row_count + SLOTS - 1) / SLOTS;
  const int per_cu = NJ > 2 ? 2 : kB1BlocksPerCu;  // the kernel's occupancy
  const int64_t grid = std::min<int64_t>((n_steps + U - 1) / U, (int64_t)cu_count() * per_cu);
  constexpr bool CONTIG = false;  // measured faster: each load instruction reads 64 consecutive chunks
  const size_t lds = sizeof(float) * ActLayout<NJ, LPR, CONTIG>::floats(m->input_padded);
  hipLaunchKernelGGL((cq_matvec_b1<BITS, NJ, LPR, U, CONTIG>), dim3((unsigned)grid), dim3(kThreads), lds, s,
                     m->packed, m->norms, m->codebook, prepared, y, m->input_padded, m->row_bytes,
                     ilog2(m->group), row_begin, row_count);
  return launch_status();
}

template <int BITS, int LPR>
int launch_nb(const bqd_cq_matrix* m, const float* prepared, float* y, int64_t y_stride, int nb,
              int64_t row_begin, int64_t row_count, hipStream_t s) {
  constexpr int U = 2;
  constexpr int SLOTS = LPR <= kThreads ? kThreads / LPR : 1;
  const int64_t n_steps = (row_count + SLOTS - 1) / SLOTS;
  // persistent: every workgroup loads all its activations once, so the
  // grid is kept to what the CUs hold at once (2 per CU at 128+ VGPRs)
  const int64_t grid = std::min<int64_t>((n_steps + U - 1) / U, (int64_t)cu_count() * kNbBlocksPerCu);
  const size_t lds = sizeof(float) * ActLayout<1, LPR, false>::floats(m->input_padded);
  hipLaunchKernelGGL((cq_matvec_nb<BITS, 1, LPR, 4, U>), dim3((unsigned)grid), dim3(kThreads), lds,
                     s, m->packed, m->norms, m->codebook, prepared, y, m->input_padded,
                     m->row_bytes, ilog2(m->group), row_begin, row_count, y_stride, nb);
  return launch_status();
}

template <int BITS>
int dispatch_b1(const bqd_cq_matrix* m, FastShape f, const float* prepared, float* y,
                int64_t row_begin, int64_t row_count, hipStream_t s) {
  switch (f.lpr * 16 + f.nj) {
    case 8 * 16 + 1: return launch_b1<BITS, 1, 8>(m, prepared, y, row_begin, row_count, s);
    case 16 * 16 + 1: return launch_b1<BITS, 1, 16>(m, prepared, y, row_begin, row_count, s);
    case 32 * 16 + 1: return launch_b1<BITS, 1, 32>(m, prepared, y, row_begin, row_count, s);
    case 64 * 16 + 1: return launch_b1<BITS, 1, 64>(m, prepared, y, row_begin, row_count, s);
    case 64 * 16 + 2: return launch_b1<BITS, 2, 64>(m, prepared, y, row_begin, row_count, s);
    case 64 * 16 + 4: return launch_b1<BITS, 4, 64>(m, prepared, y, row_begin, row_count, s);
  }
  return BQD_EINVAL;  // unreachable: fast_shape() only returns instantiated layouts
}

template <int BITS>
int dispatch_nb(const bqd_cq_matrix* m, FastShape f, const float* prepared, float* y,
                int64_t y_stride, int nb, int64_t row_begin, int64_t row_count, hipStream_t s) {
  switch (f.lpr) {
    case 8: return launch_nb<BITS, 8>(m, prepared, y, y_stride, nb, row_begin, row_count, s);
    case 16: return launch_nb<BITS, 16>(m, prepared, y, y_stride, nb, row_begin, row_count, s);
    case 32: return launch_nb<BITS, 32>(m, prepared, y, y_stride, nb, row_begin, row_count, s);
    case 64: return launch_nb<BITS, 64>(m, prepared, y, y_stride, nb, row_begin, row_count, s);
    case 128: return launch_nb<BITS, 128>(m, prepared, y, y_stride, nb, row_begin, row_count, s);
    case 256: return launch_nb<BITS, 256>(m, prepared, y, y_stride, nb, row_begin, row_count, s);
  }
  return BQD_EINVAL;
}

int run_b1(const bqd_cq_matrix* m, FastShape f, const float* prepared, float* y,
           int64_t row_begin, int64_t row_count, hipStream_t s) {
  switch (m->bits) {
    case 2: return dispatch_b1<2>(m, f, prepared, y, row_begin, row_count, s);
    case 3: return dispatch_b1<3>(m, f, prepared, y, row_begin, row_count, s);
    case 4: return dispatch_b1<4>(m, f, prepared, y, row_begin, row_count, s);
    case 5: return dispatch_b1<5>(m, f, prepared, y, row_begin, row_count, s);
  }
  return BQD_EINVAL;
}

int run_nb(const bqd_cq_matrix* m, FastShape f, const float* prepared, float* y, int64_t y_stride,
           int nb, int64_t row_begin, int64_t row_count, hipStream_t s) {
  switch (m->bits) {
    case 2: return dispatch_nb<2>(m, f, prepared, y, y_stride, nb, row_begin, row_count, s);
    case 3: return dispatch_nb<3>(m, f, prepared, y, y_stride, nb, row_begin, row_count, s);
    case 4: return dispatch_nb<4>(m, f, prepared, y, y_stride, nb, row_begin, row_count, s);
    case 5: return dispatch_nb<5>(m, f, prepared, y, y_stride, nb, row_begin, row_count, s);
  }
  return BQD_EINVAL;
}

// The matrix-core kernel's conditions: groups of >= 256, whole 256-column
// spans, at most 16 spans (one 1024-thread workgroup per row tile), dword
// rows.
bool mfma_ok(const bqd_cq_matrix* m) {
  return m->group >= 256 && m->input_padded % 256 == 0 && m->input_padded <= 4096 &&
         m->row_bytes % 4 == 0 && is_aligned(m->packed, 4);
}

template <int BITS>
int launch_mfma_b(const bqd_cq_matrix* m, const float* prepared, float* y, int64_t y_stride,
                  int nb, int64_t row_begin, int64_t row_count, hipStream_t s) {
  const int n_spans = (int)(m->input_padded / 256);
  const int64_t n_tiles = (row_count + 15) / 16;
  const int per_cu = 16 / n_spans;  // 16 wavefronts per CU at 4 per SIMD
  const int64_t grid = std::min<int64_t>(n_tiles, (int64_t)cu_count() * per_cu);
  hipLaunchKernelGGL((cq_matvec_mfma<BITS>), dim3((unsigned)grid), dim3(64 * n_spans), 0, s,
                     m->packed, m->norms, m->codebook, prepared, y, m->input_padded,
                     m->row_bytes, ilog2(m->group), row_begin, row_count, y_stride, nb);
  return launch_status();
}

int run_mfma(const bqd_cq_matrix* m, const float* prepared, float* y, int64_t y_stride, int nb,
             int64_t row_begin, int64_t row_count, hipStream_t s) {
  switch (m->bits) {
    case 2: return launch_mfma_b<2>(m, prepared, y, y_stride, nb, row_begin, row_count, s);
    case 3: return launch_mfma_b<3>(m, prepared, y, y_stride, nb, row_begin, row_count, s);
    case 4: return launch_mfma_b<4>(m, prepared, y, y_stride, nb, row_begin, row_count, s);
    case 5: return launch_mfma_b<5>(m, prepared, y, y_stride, nb, row_begin, row_count, s);
  }
  return BQD_EINVAL;
}

int launch_generic(const bqd_cq_matrix* m, const float* prepared, float* y, int64_t batch,
                   int64_t row_begin, int64_t row_count, hipStream_t s) {
  const int64_t grid = std::min<int64_t>((row_count + kWavesPerBlock - 1) / kWavesPerBlock, kMaxGrid);
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
  const FastShape f1 = fast_shape(n_chunk, 1);
  const FastShape f4 = fast_shape(n_chunk, 4);
  if (batch == 1 && f1.lpr) return run_b1(m, f1, prepared, y, row_begin, row_count, s);
  if (batch >= 2 && mfma_ok(m)) {
    // up to sixteen vectors per launch on the matrix cores
    for (int64_t b = 0; b < batch; b += 16) {
      const int nb = (int)std::min<int64_t>(16, batch - b);
      const int rc = run_mfma(m, prepared + b * m->input_padded, y + b * row_count, row_count, nb,
                              row_begin, row_count, s);
      if (rc) return rc;
    }
    return BQD_OK;
  }
  if (f4.lpr) {
    // up to four vectors share each decoded weight per launch
    for (int64_t b = 0; b < batch; b += 4) {
      const int nb = (int)std::min<int64_t>(4, batch - b);
      const int rc = run_nb(m, f4, prepared + b * m->input_padded, y + b * row_count, row_count,
                            nb, row_begin, row_count, s);
      if (rc) return rc;
    }
    return BQD_OK;
  }
  if (f1.lpr) {
    for (int64_t b = 0; b < batch; ++b) {
      const int rc = run_b1(m, f1, prepared + b * m->input_padded, y + b * row_count, row_begin,
                            row_count, s);
      if (rc) return rc;
    }
    return BQD_OK;
  }
  return launch_generic(m, prepared, y, batch, row_begin, row_count, s);
}

// ------------------------------------------------------------- unpack probe
// idx[c] for one row through the same decode the matvec uses for this
// matrix: the chunk address decode from dwords on the fast layout (address /
// 4 is the index), the byte decode otherwise.
template <int BITS>
__global__ void cq_unpack_chunks(const uint8_t* __restrict__ prow, uint8_t* __restrict__ idx,
                                 int64_t n_chunk) {
  const int64_t ch = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (ch >= n_chunk) return;
  const uint32_t* pc = reinterpret_cast<const uint32_t*>(prow) + BITS * ch;
  uint32_t d[BITS];
#pragma unroll
  for (int t = 0; t < BITS; ++t) d[t] = pc[t];
  uint32_t a[32];
  chunk_addresses<BITS>(d, a);
#pragma unroll
  for (int k = 0; k < 32; ++k) idx[32 * ch + k] = (uint8_t)(a[k] >> 2);
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

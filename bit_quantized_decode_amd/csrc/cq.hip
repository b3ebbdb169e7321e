// CQ (codebook-quantized) kernels for gfx950: activation prepare, packed-row
// matvec and dense row gather.
//
// Method: "Inference engine, part 2: kernels and token step" — §1 (the
// unnormalized Walsh–Hadamard butterfly), §2 (prepare: zero-pad, transform
// each group, multiply by 1/sqrt(group)), §3 (dot packed rows directly: per
// row and group, the fp16 norm times the sum of codebook[index] * prepared),
// "Row gather" (each group's codebook values scaled by the group norm, the
// normalized transform, the columns below the unpadded width) and §6 (a row
// range of a matrix).  The record layout is that of "Inference engine, part 1:
// loader and tokenizer", §4.
#include <algorithm>
#include <atomic>
#include <cmath>

#include "cq_device.h"
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
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// 1/sqrt(group) is applied as the page does: the scale is an fp64 value, the
// product is formed in fp64 and rounded once to fp32.  For groups that are
// powers of four the scale is a power of two: the fp64 product is then exact
// and its rounding equals the fp32 product, which is what runs.
__device__ __forceinline__ float scale_store(float v, double scale) {
  const float sf = (float)scale;
  if ((double)sf == scale && (__float_as_uint(sf) & 0x007fffffu) == 0) return v * sf;
  return (float)((double)v * scale);
}

// Elements per lane of the wavefront transform: a wavefront spans one group
// (64 * E = group) for groups of 64 and more, else 64 / group whole groups.
inline int lane_elems(int64_t group) { return group >= 64 ? (int)(group / 64) : 1; }

// ------------------------------------------------------------------ prepare
// One wavefront per (vector, span of 64*E padded columns); the grid is capped
// (kMaxStrideGrid) and the wavefronts loop over the work.
template <int E>
__global__ __launch_bounds__(kThreads) void cq_prepare_kernel(
    const float* __restrict__ x, float* __restrict__ p, int64_t input, int64_t input_padded,
    int log2_group, int64_t spans, int64_t n_waves, double scale) {
  const int lane = threadIdx.x & (kWave - 1);
  for (int64_t wv = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave; wv < n_waves;
       wv += (int64_t)gridDim.x * kWavesPerBlock) {  // wavefront-uniform
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
}

template <int E>
int launch_prepare_e(const bqd_cq_matrix* m, const float* x, float* prepared, int64_t batch,
                     hipStream_t s) {
  const int64_t spans = (m->input_padded + 64 * E - 1) / (64 * E);
  const int64_t n_waves = spans * batch;
  const int64_t grid = std::min<int64_t>((n_waves + kWavesPerBlock - 1) / kWavesPerBlock,
                                         kMaxStrideGrid);
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
// Generic form: any bit width and group, one index decode per element; the
// grid is capped (kMaxStrideGrid) and the wavefronts loop over the work.
template <int E>
__global__ __launch_bounds__(kThreads) void cq_gather_generic(
    const uint8_t* __restrict__ packed, const uint16_t* __restrict__ norms,
    const float* __restrict__ codebook, const int32_t* __restrict__ rows, float* __restrict__ out,
    int64_t output, int64_t input, int64_t input_padded, int64_t row_bytes, int bits,
    int log2_group, int64_t spans, int64_t n_waves, double scale) {
  __shared__ float cb[32];
  if (threadIdx.x < (1 << bits)) cb[threadIdx.x] = codebook[threadIdx.x];
  __syncthreads();
  const int lane = threadIdx.x & (kWave - 1);
  for (int64_t wv = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave; wv < n_waves;
       wv += (int64_t)gridDim.x * kWavesPerBlock) {  // wavefront-uniform
    const int64_t i = wv / spans;
    const int64_t c0 = (wv % spans) * (64 * E) + lane * E;
    const int64_t r = rows[i];
    float* o = out + i * input;
    if (r < 0 || r >= output) {  // an id outside the table: a NaN row
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (c0 + e < input) o[c0 + e] = __uint_as_float(0x7fc00000u);
      continue;
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
}

// Groups of 8 and more: lane l owns E = 8 or 16 consecutive columns, which lie
// in one group (one norm) and in E * BITS / 8 whole bytes of the row.  Work
// items are (id, span of 64 E columns); persistent wavefronts take items
// wv, wv + n_waves, ... (at most 64 each).  Lane j loads the id of the
// wavefront's j-th item up front; then the row bytes and norms of up to
// kGatherAhead items are requested together, and the items are decoded,
// transformed and stored one after another, so one item's stores drain while
// the next is computed.  LOG2G > 0 fixes the group at compile time (the
// transform's stage choices fold away); 0 takes log2_group.  WORDS: the lane's
// bytes are whole dwords at dword addresses (rows of a multiple of 4 bytes,
// packed 4-byte aligned, E * BITS / 8 a multiple of 4).  Rows whose visible
// columns fill the lane are stored as float4s when the output rows are
// 16-byte aligned; every output store is nontemporal.
constexpr int kGatherAhead = 8;
typedef float f32x4_nt __attribute__((ext_vector_type(4)));

template <int BITS, int E, bool WORDS>
struct GatherLoad {
  static constexpr int kBytes = E * BITS / 8;
  static constexpr int kRegs = WORDS ? kBytes / 4 : kBytes;  // dwords, or one byte each
  uint32_t reg[kRegs];
  uint32_t norm_bits;
  __device__ __forceinline__ uint32_t byte(int k) const {
    if constexpr (WORDS) return (reg[k >> 2] >> (8 * (k & 3))) & 0xffu;
    else return reg[k];
  }
};

template <int BITS, int E, bool WORDS>
__device__ __forceinline__ void gather_request(GatherLoad<BITS, E, WORDS>& g, const uint8_t* prow,
                                               const uint16_t* nrow, int cl, int log2_group) {
  const uint8_t* pb = prow + (int64_t)cl * BITS / 8;
  if constexpr (WORDS) {
    const uint32_t* pw = reinterpret_cast<const uint32_t*>(pb);
#pragma unroll
    for (int k = 0; k < GatherLoad<BITS, E, WORDS>::kRegs; ++k) g.reg[k] = pw[k];
  } else {
#pragma unroll
    for (int k = 0; k < GatherLoad<BITS, E, WORDS>::kRegs; ++k) g.reg[k] = pb[k];
  }
  g.norm_bits = nrow[cl >> log2_group];
}

template <int BITS, int E, int LOG2G, bool WORDS>
__global__ __launch_bounds__(kThreads) void cq_gather_kernel(
    const uint8_t* __restrict__ packed, const uint16_t* __restrict__ norms,
    const float* __restrict__ codebook, const int32_t* __restrict__ rows, float* __restrict__ out,
    int64_t output, int64_t input, int64_t input_padded, int64_t row_bytes, int log2_group_rt,
    int64_t spans, int64_t items, int64_t n_waves, double scale, bool vec_store) {
  const int log2_group = LOG2G > 0 ? LOG2G : log2_group_rt;
  __shared__ float cb[32];
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wv = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
  // lane j: the id of this wavefront's j-th item (requested with the codebook);
  // item = id index * spans + span, and one span per id is the common case
  const int64_t my_item = wv + lane * n_waves;
  const int32_t my_id = my_item < items ? rows[spans == 1 ? my_item : my_item / spans] : 0;
  if (threadIdx.x < (1 << BITS)) cb[threadIdx.x] = codebook[threadIdx.x];
  __syncthreads();
  if (wv >= items) return;  // whole wavefront, after the barrier
  const int n_mine = (int)((items - wv + n_waves - 1) / n_waves);  // <= 64
  const int64_t nrow_stride = input_padded >> log2_group;
  // columns fit in 32 bits (input_padded < 2^28)
  const int in = (int)input, in_pad = (int)input_padded;
  for (int base = 0; base < n_mine; base += kGatherAhead) {
    // request this round's items: row bytes and norm of the lane's columns
    // (an id outside the table, or columns past the stored row, load row 0 /
    // column 0 and use nothing)
    GatherLoad<BITS, E, WORDS> g[kGatherAhead];
#pragma unroll
    for (int q = 0; q < kGatherAhead; ++q) {
      if (base + q < n_mine) {
        const int64_t it = wv + (int64_t)(base + q) * n_waves;
        const int64_t r = __builtin_amdgcn_readlane(my_id, base + q);
        const int64_t rs = r >= 0 && r < output ? r : 0;
        const int c0 = (spans == 1 ? 0 : (int)(it % spans)) * (64 * E) + lane * E;
        gather_request<BITS, E, WORDS>(g[q], packed + rs * row_bytes, norms + rs * nrow_stride,
                                       c0 < in_pad ? c0 : 0, log2_group);
      }
    }
#pragma unroll
    for (int q = 0; q < kGatherAhead; ++q) {
      if (base + q >= n_mine) break;
      const int64_t it = wv + (int64_t)(base + q) * n_waves;
      const int64_t r = __builtin_amdgcn_readlane(my_id, base + q);
      const int c0 = (spans == 1 ? 0 : (int)(it % spans)) * (64 * E) + lane * E;
      float* o = out + (spans == 1 ? it : it / spans) * input + c0;
      if (r < 0 || r >= output) {  // an id outside the table: a NaN row
#pragma unroll
        for (int e = 0; e < E; ++e)
          if (c0 + e < in) o[e] = __uint_as_float(0x7fc00000u);
        continue;
      }
      // input_padded is a multiple of the group, so a lane's E columns are all
      // inside the stored row or all past it
      const bool live = c0 < in_pad;
      const float nrm = f16_to_f32((uint16_t)g[q].norm_bits);
      float v[E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int bit = BITS * e, k = bit >> 3, sh = bit & 7;
        uint32_t w = g[q].byte(k);
        if (sh + BITS > 8) w |= g[q].byte(k + 1) << 8;
        const float c = cb[(w >> sh) & ((1u << BITS) - 1u)] * nrm;
        v[e] = live ? c : 0.0f;
      }
      wave_fwht<E>(v, lane, log2_group);
      // nontemporal stores: the rows stream out to memory as they are made
      // instead of waiting in the L2 for the kernel's end
      if (vec_store && c0 + E <= in) {
#pragma unroll
        for (int e = 0; e < E; e += 4) {
          const f32x4_nt q = {scale_store(v[e], scale), scale_store(v[e + 1], scale),
                              scale_store(v[e + 2], scale), scale_store(v[e + 3], scale)};
          __builtin_nontemporal_store(q, reinterpret_cast<f32x4_nt*>(o + e));
        }
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e)
          if (c0 + e < in) __builtin_nontemporal_store(scale_store(v[e], scale), o + e);
      }
    }
  }
}

template <int E>
int launch_gather_generic(const bqd_cq_matrix* m, const int32_t* rows, int64_t n, float* out,
                          hipStream_t s) {
  // spans past the last visible column store nothing and are not launched
  const int64_t spans = (m->input + 64 * E - 1) / (64 * E);
  const int64_t n_waves = spans * n;
  const int64_t grid = std::min<int64_t>((n_waves + kWavesPerBlock - 1) / kWavesPerBlock,
                                         kMaxStrideGrid);
  hipLaunchKernelGGL((cq_gather_generic<E>), dim3((unsigned)grid), dim3(kThreads), 0, s,
                     m->packed, m->norms, m->codebook, rows, out, m->output, m->input,
                     m->input_padded, m->row_bytes, (int)m->bits, ilog2(m->group), spans,
                     n_waves, 1.0 / std::sqrt((double)m->group));
  return launch_status();
}

// Persistent wavefronts per CU for the gather: enough items each to overlap
// one item's loads with the previous item's arithmetic and stores.
constexpr int kGatherWavesPerCu = 16;

template <int BITS, int E, int LOG2G, bool WORDS>
int launch_gather_kernel(const bqd_cq_matrix* m, const int32_t* rows, int64_t items,
                         int64_t spans, float* out, hipStream_t s) {
  // at most 64 items per wavefront (one id per lane)
  int64_t n_waves = std::max<int64_t>((int64_t)cu_count() * kGatherWavesPerCu, (items + 63) / 64);
  n_waves = std::min(n_waves, items);
  const int64_t grid = (n_waves + kWavesPerBlock - 1) / kWavesPerBlock;
  const bool vec_store = m->input % 4 == 0 && is_aligned(out, 16);
  hipLaunchKernelGGL((cq_gather_kernel<BITS, E, LOG2G, WORDS>), dim3((unsigned)grid),
                     dim3(kThreads), 0, s, m->packed, m->norms, m->codebook, rows, out,
                     m->output, m->input, m->input_padded, m->row_bytes, ilog2(m->group),
                     spans, items, n_waves, 1.0 / std::sqrt((double)m->group), vec_store);
  return launch_status();
}

template <int BITS, int E>
int launch_gather_fast(const bqd_cq_matrix* m, const int32_t* rows, int64_t n, float* out,
                       hipStream_t s) {
  // spans past the last visible column store nothing and are not launched
  const int64_t spans = (m->input + 64 * E - 1) / (64 * E);
  const int64_t items = spans * n;
  constexpr bool kWholeWords = (E * BITS / 8) % 4 == 0;
  const bool words = kWholeWords && m->row_bytes % 4 == 0 && is_aligned(m->packed, 4);
  if (words && E == 8 && m->group == 128)
    return launch_gather_kernel<BITS, E, 7, kWholeWords>(m, rows, items, spans, out, s);
  if (words && E == 8 && m->group == 256)
    return launch_gather_kernel<BITS, E, 8, kWholeWords>(m, rows, items, spans, out, s);
  if (words) return launch_gather_kernel<BITS, E, 0, kWholeWords>(m, rows, items, spans, out, s);
  return launch_gather_kernel<BITS, E, 0, false>(m, rows, items, spans, out, s);
}

template <int E>
int launch_gather_bits(const bqd_cq_matrix* m, const int32_t* rows, int64_t n, float* out,
                       hipStream_t s) {
  switch (m->bits) {
    case 2: return launch_gather_fast<2, E>(m, rows, n, out, s);
    case 3: return launch_gather_fast<3, E>(m, rows, n, out, s);
    case 4: return launch_gather_fast<4, E>(m, rows, n, out, s);
    case 5: return launch_gather_fast<5, E>(m, rows, n, out, s);
  }
  return BQD_EINVAL;
}

int launch_cq_gather(const bqd_cq_matrix* m, const int32_t* rows, int64_t n, float* out,
                     hipStream_t s) {
  if (m->input == 0) return BQD_OK;
  // groups of 8..512 on 8 columns per lane, 1024 on 16
  if (m->group >= 8 && m->group <= 512) return launch_gather_bits<8>(m, rows, n, out, s);
  if (m->group == 1024) return launch_gather_bits<16>(m, rows, n, out, s);
  switch (lane_elems(m->group)) {
    case 1: return launch_gather_generic<1>(m, rows, n, out, s);
  }
  return BQD_EINVAL;  // unreachable: group <= 1024 is validated
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
// row and lane q owns the NJ chunks q + LPR*j, so each load instruction of a
// wavefront reads 64 consecutive chunks (measured faster than each lane
// owning NJ adjacent chunks, which would share one group norm).  Every lane
// keeps the prepared activations of its chunks in registers for the whole
// kernel (the same columns for every row).  They are staged once per
// workgroup through LDS: coalesced global loads, then 16-byte LDS reads from
// a layout padded by 4 floats per chunk so that the 16 lanes of a read phase
// hit distinct banks.  The codebook is
// looked up in LDS (2^BITS distinct words in distinct banks: conflict free),
// each chunk partial is multiplied by its group norm, and the LPR lanes of a
// row reduce with DPP.  The codebook lookups are the LDS's limit and their
// latency is hidden by occupancy: the kernel is held to 128 VGPRs (4
// wavefronts per SIMD; 2 for rows of 8192 columns, whose activations alone
// take 128) and the grid is persistent, each workgroup walking steps of
// SLOTS*U rows.
// LDS layout of the staged activations: each 32-column chunk padded to 36 floats.
struct ActLayout {
  static constexpr int kStride = 32 + 4;  // padded LDS stride of a chunk
  // LDS float offset of float f of the padded row
  __device__ static int offset(int f) { return (f >> 5) * kStride + (f & 31); }
  static int64_t floats(int64_t input_padded) { return input_padded / 32 * kStride; }
};

template <int BITS, int NJ, int LPR, int U>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(NJ > 2 ? 2 : 4, NJ > 2 ? 2 : 4)))
void cq_matvec_b1(const uint8_t* __restrict__ packed, const uint16_t* __restrict__ norms,
                  const float* __restrict__ codebook, const float* __restrict__ prepared,
                  float* __restrict__ y, int64_t input_padded, int64_t row_bytes, int log2_group,
                  int64_t row_begin, int64_t row_count) {
  typedef ActLayout L;
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
  auto chunk_of = [&](int j) { return q + LPR * j; };
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
        const int off = BITS * LPR * j;
#pragma unroll
        for (int t = 0; t < BITS; ++t) d[u][j][t] = stream_load(pc + off + t);
      }
      const uint16_t* nr = norm_base + (int64_t)i * n_groups;
#pragma unroll
      for (int j = 0; j < NJ; ++j) nb[u][j] = nr[gidx[j]];
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

// ------------------------------------------------------ 4-bit pair tables
// A packed 4-bit byte holds two indices; an LDS table indexed by the byte
// returns both codebook values as one 8-byte read.  Each table row holds 32
// copies of its entry and lane l reads copy l % 32, so no two lanes of a
// half-wavefront meet in one LDS bank; the byte-to-address step is one byte
// permute.  Per pair of weights: one permute, one LDS read, two FMAs.
constexpr int kPairRowBytes = 32 * 8;                  // 32 copies of (float, float)
constexpr int kPairTableFloats = 256 * kPairRowBytes / 4;

// ------------------------------------------- batch-1 matvec, a ring of rows
// 4-bit rows of input_padded = 128 * S * BPL columns (512 ... 8192).  A
// 1024-thread workgroup owns RPB = (16 / S) * 8 rows.  Wavefront w covers
// column slice w % S of rows (w / S) * 8 ... + 7: lane l owns the BPL
// consecutive packed bytes (2 * BPL columns, inside one group) at l * BPL of
// the slice, so every load instruction reads 64 * BPL contiguous bytes of one
// row, and the lane keeps only its own 2 * BPL activations in registers.
//  - Each wavefront keeps a ring of DR rows in flight and requests row k + DR
//    before it decodes row k, so the weight stream and the decode overlap
//    from the first row to the last (requesting every row up front stalls:
//    a CU holds only so many outstanding loads, and the decode of rows that
//    arrive late then piles up at the end).
//  - Decode through the 4-bit pair table above: a byte permute forms the
//    table address, one 8-byte LDS read returns the codebook values of both
//    nibbles, two FMAs; the lane's partial times the fp16 norm of its group.
//  - The eight row partials of a lane are reduced across the wavefront by a
//    transposed reduction (two lane-swap steps and one DPP step leave lane l
//    with row (l / 8) % 8 of the wavefront, three DPP adds finish it), and
//    the S slice partials of each row meet in LDS, summed in slice order.
// E > 0 fuses the prepare ([P1] §2) into the kernel: `act` is then the raw
// input (input floats), every workgroup zero-pads it and transforms its
// groups in registers exactly as cq_prepare does (E elements per lane,
// groups of 2^log2_group, the same butterflies and fp64 scale), and
// workgroup 0 also stores the prepared vector to `prepared_out` when it is
// not null.  E == 0: `act` is the prepared vector.
constexpr int kRingThreads = 1024;
constexpr int kRingRows = 8;  // rows per wavefront

template <int BPL> struct RingLoad;
template <> struct RingLoad<4> { typedef uint32_t T; };
template <> struct RingLoad<8> { typedef uint32_t T __attribute__((ext_vector_type(2))); };
template <> struct RingLoad<16> { typedef uint32_t T __attribute__((ext_vector_type(4))); };

template <int BPL>
__device__ __forceinline__ uint32_t ring_word(const typename RingLoad<BPL>::T& v, int t) {
  if constexpr (BPL == 4) return v; else return v[t];
}

// One launch can cover several matrices of the same shape class that read
// one activation ([P1] §6: one prepared vector for phiPre, phiPost and
// phiResidual, each a row range of its matrix): workgroups [end[k-1], end[k])
// belong to matrix k.
// The arguments are one kernel-argument block: the shared fields, then one
// entry per matrix, contiguous, so a single-matrix launch reads its
// arguments in one scalar round trip from two cache lines, and a
// several-matrix launch reads every entry in one round trip too.
constexpr int kRingMaxMats = 4;
struct RingMat {
  const uint8_t* packed;     // first row of the range
  const uint16_t* norms;     // its norms
  const float* codebook;
  float* y;                  // [rows]
  int64_t row_bytes;
  int32_t rows;
  int32_t block_end;         // one past this matrix's last workgroup
};
struct RingArgs {
  const float* act;          // prepared vector, or the raw input (fused prepare)
  float* prepared_out;       // fused prepare: workgroup 0 stores the prepared vector
  int32_t log2_group;
  int32_t input;             // unpadded width (fused prepare)
  int32_t x_vec;             // fused prepare: unpadded, 16-byte aligned input
  int32_t pad;
  double scale;              // 1 / sqrt(group)
  RingMat m[kRingMaxMats];
};

template <int BPL, int S, int E, bool MULTI>
__global__ __launch_bounds__(kRingThreads) void cq_matvec_ring(const RingArgs args) {
  constexpr int C = 128 * S * BPL;   // input_padded
  constexpr int CPL = 2 * BPL;       // columns per lane
  constexpr int AST = CPL + 4;       // padded floats per lane chunk in LDS
  constexpr int RS = 16 / S;         // row subsets
  constexpr int RPB = RS * kRingRows;
  constexpr int DR = BPL == 16 ? 2 : 3;
  typedef typename RingLoad<BPL>::T V;
  __shared__ __align__(16) float tab[kPairTableFloats];
  __shared__ __align__(16) float act_s[64 * S * AST];
  __shared__ float part[S][RPB];
  // this workgroup's matrix: entry 0 for a single matrix; otherwise every
  // entry is read in the same round trip (the values are made opaque so the
  // selection cannot turn into a second, dependent load)
  const float* __restrict__ act = args.act;
  float* __restrict__ prepared_out = args.prepared_out;
  RingMat mat = args.m[0];
  int block0 = 0;
  int log2_group = args.log2_group;
  if constexpr (MULTI) {
    RingMat mk[kRingMaxMats];
#pragma unroll
    for (int k = 1; k < kRingMaxMats; ++k) mk[k] = args.m[k];
    asm volatile("" : "+s"(mat.packed), "+s"(mat.norms), "+s"(mat.codebook), "+s"(mat.y),
                 "+s"(mat.row_bytes), "+s"(mat.rows), "+s"(mat.block_end), "+s"(log2_group));
    int prev_end = mat.block_end;
#pragma unroll
    for (int k = 1; k < kRingMaxMats; ++k) {
      asm volatile("" : "+s"(mk[k].packed), "+s"(mk[k].norms), "+s"(mk[k].codebook), "+s"(mk[k].y),
                   "+s"(mk[k].row_bytes), "+s"(mk[k].rows), "+s"(prev_end));
      if ((int)blockIdx.x >= prev_end) {
        mat = mk[k];
        block0 = prev_end;
      }
      prev_end = mk[k].block_end;
    }
  }
  const uint8_t* __restrict__ packed = mat.packed;
  const uint16_t* __restrict__ norms = mat.norms;
  const float* __restrict__ codebook = mat.codebook;
  float* __restrict__ y = mat.y;
  const int64_t row_bytes = mat.row_bytes;
  const int rows = mat.rows;
  const int input = args.input, x_vec = args.x_vec;
  const double scale = args.scale;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sl = wave % S, rs = wave / S;
  const int wg0 = ((int)blockIdx.x - block0) * RPB;
  const int row0 = wg0 + rs * kRingRows;
  // loads in the order they are needed: codebook (table), activations,
  // norms, then the first DR rows of weights
  const float cb_lo = codebook[(tid >> 4) & 15];
  float cb_hi[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) cb_hi[p] = codebook[(tid >> 8) + 4 * p];
  constexpr int XP = (C / 4 + kRingThreads - 1) / kRingThreads;  // float4 per thread (E == 0)
  constexpr int SPANS = E > 0 ? C / (64 * E) : 1;                // transform spans (E > 0)
  constexpr int SPW = (SPANS + 15) / 16;                         // spans per wavefront
  float4 xv[E == 0 ? XP : 1];
  float xr[E > 0 ? SPW : 1][E > 0 ? E : 1];
  if constexpr (E == 0) {
#pragma unroll
    for (int p = 0; p < XP; ++p) {
      const int i = tid + kRingThreads * p;
      if (i < C / 4) xv[p] = reinterpret_cast<const float4*>(act)[i];
    }
  } else {
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      const int c0 = (wave + 16 * j) * (64 * E) + lane * E;
      if (E == 4 && x_vec && (SPANS % 16 == 0 || wave + 16 * j < SPANS)) {
        // an unpadded, 16-byte aligned input: one float4 per lane and span
        const float4 v = reinterpret_cast<const float4*>(act)[c0 / 4];
        xr[j][0] = v.x; xr[j][1] = v.y; xr[j][2] = v.z; xr[j][3] = v.w;
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e)
          xr[j][e] = (c0 + e < input && wave + 16 * j < SPANS) ? act[c0 + e] : 0.0f;
      }
    }
  }
  const int g = ((sl * 64 + lane) * CPL) >> log2_group;
  const int n_groups = C >> log2_group;
  uint16_t nb[kRingRows];
#pragma unroll
  for (int k = 0; k < kRingRows; ++k)
    nb[k] = norms[(int64_t)min(row0 + k, rows - 1) * n_groups + g];
  V d[kRingRows];
  const uint8_t* base = packed + sl * 64 * BPL + lane * BPL;
  auto issue = [&](int k) {
    d[k] = stream_load(
        reinterpret_cast<const V*>(base + (int64_t)min(row0 + k, rows - 1) * row_bytes));
  };
#pragma unroll
  for (int k = 0; k < DR; ++k) issue(k);
  __builtin_amdgcn_sched_barrier(0);
  // Table: 16-byte slot t = tid + 1024 p holds row b = t / 16, copies
  // 2 (t % 16) and 2 (t % 16) + 1, each (codebook[b % 16], codebook[b / 16]).
#pragma unroll
  for (int p = 0; p < 4; ++p)
    *reinterpret_cast<float4*>(tab + 4 * (tid + kRingThreads * p)) =
        make_float4(cb_lo, cb_hi[p], cb_lo, cb_hi[p]);
  if constexpr (E == 0) {
#pragma unroll
    for (int p = 0; p < XP; ++p) {
      const int i = tid + kRingThreads * p;
      if (i < C / 4) {
        const int f = 4 * i;
        *reinterpret_cast<float4*>(act_s + (f / CPL) * AST + (f % CPL)) = xv[p];
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      if (SPANS % 16 == 0 || wave + 16 * j < SPANS) {  // wavefront-uniform
        // E >= 2 means group = 64 E: the stages are known at compile time
        wave_fwht<E>(xr[j], lane, E >= 2 ? 6 + ilog2_c(E) : log2_group);
        const int c0 = (wave + 16 * j) * (64 * E) + lane * E;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float v = scale_store(xr[j][e], scale);
          const int c = c0 + e;
          act_s[(c / CPL) * AST + (c % CPL)] = v;
          if (prepared_out != nullptr && blockIdx.x == 0) prepared_out[c] = v;
        }
      }
    }
  }
  __syncthreads();
  float a[CPL];
#pragma unroll
  for (int k = 0; k < CPL; k += 4) {
    const float4 v = *reinterpret_cast<const float4*>(act_s + (sl * 64 + lane) * AST + k);
    a[k] = v.x; a[k + 1] = v.y; a[k + 2] = v.z; a[k + 3] = v.w;
  }
  const uint32_t lane_off = 8u * (uint32_t)(lane & 31);
  const char* tb = reinterpret_cast<const char*>(tab);
  float acc[kRingRows];
#pragma unroll
  for (int k = 0; k < kRingRows; ++k) {
    if (k + DR < kRingRows) issue(k + DR);
    __builtin_amdgcn_sched_barrier(0);
    float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
    for (int t = 0; t < BPL / 4; ++t)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        // byte b of the dword: columns 8 t + 2 b (low nibble) and + 1
        const uint32_t adr = __builtin_amdgcn_perm(ring_word<BPL>(d[k], t), lane_off,
                                                   0x0c0c0400u | ((4u + b) << 8));
        const float2 c = *reinterpret_cast<const float2*>(tb + adr);
        p0 += c.x * a[8 * t + 2 * b];
        p1 += c.y * a[8 * t + 2 * b + 1];
      }
    acc[k] = (p0 + p1) * f16_to_f32(nb[k]);
    __builtin_amdgcn_sched_barrier(0);
  }
  // transposed reduction of the eight rows
#pragma unroll
  for (int k = 0; k < 4; ++k) acc[k] = swap_add32(acc[k], acc[k + 4]);
#pragma unroll
  for (int k = 0; k < 2; ++k) acc[k] = swap_add16(acc[k], acc[k + 2]);
  float v;
  {
    const bool up = (lane & 8) != 0;
    const float keep = up ? acc[1] : acc[0];
    const float send = up ? acc[0] : acc[1];
    v = keep + lane_xor<8>(send);
  }
  v += lane_xor<4>(v);
  v += lane_xor<2>(v);
  v += lane_xor<1>(v);
  if ((lane & 7) == 0) part[sl][rs * kRingRows + (lane >> 3)] = v;
  __syncthreads();
  if (tid < RPB) {
    float t = 0.0f;
#pragma unroll
    for (int j = 0; j < S; ++j) t += part[j][tid];
    const int r = wg0 + tid;
    if (r < rows) y[r] = t;
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
  typedef ActLayout L;
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
    const float4* src =
        reinterpret_cast<const float4*>(prepared + (int64_t)(b < nb ? b : nb - 1) * input_padded);
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
        for (int t = 0; t < BITS; ++t) d[u][j][t] = stream_load(pc + t);
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
// weights times a 32 x 16 operand).  fp32 values are carried as bf16 pairs,
// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi) (both rounded to
// nearest even), so |x - hi - lo| <= 2^-18 |x|.  The 16 operand columns hold
// the high halves of up to eight vectors and then their low halves, so two
// products per block (weight high halves, weight low halves) give hi*hi,
// hi*lo, lo*hi and lo*lo at once; column v and column v + 8 are added at the
// end.
//
// Columns come in 256-wide spans (groups are >= 256, so a span has one norm
// per row) and each wavefront owns one span for the whole kernel.  Lane l
// owns tile row l % 16 and, with q = l / 16, the 64 columns 32 q + 0..31 and
// 128 + 32 q + 0..31 of the span: its operand positions in K-block j (0..7)
// are the eight columns 8 j .. 8 j + 7 of that list, so a K-block's weight
// operand is one dword of packed 4-bit indices per lane, and each weight load
// instruction reads 64 consecutive bytes of 16 rows.  The span's activation
// operands stay in registers: lane l holds vector l % 8, high halves for
// l % 16 < 8 and low halves otherwise; lanes l and l ^ 8 split half of the
// values each and swap the halves they do not keep.  The activations reach
// the lanes through LDS: the workgroup loads them with whole-line reads and
// each lane then reads its own 32 values.
//
// 4-bit weights decode two indices at a time: tables indexed by a packed
// byte give the (high, low) bf16 halves of both codebook values as one dword
// each, already in operand order.  Each table row holds 32 copies of an
// entry, lane l reading copy l % 32, so no two lanes of a half-wavefront meet
// in one LDS bank; the byte-to-address step is a single byte permute.  Other
// widths read a per-index table of (hi | lo << 16) and pair the halves with
// byte permutes.
//
// A wavefront takes T tiles of 16 rows per row block, issuing all their
// weight loads at once; the workgroup's wavefronts are its spans times rg row
// groups.  The span partials (times their norms) of each row meet in LDS once
// per row block and are summed in span order.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMfmaMaxSpans = 16;  // 4096 columns: a workgroup has <= 16 wavefronts
constexpr int kMfmaTiles = 4;      // 16-row tiles per wavefront and row block
constexpr int kRedStride = 9;      // floats per row of span partials (8 vectors + pad)
constexpr int kPairCopies = 32;    // lane copies per 4-bit pair-table row
// Table row b (256 bytes): copies of the high-half pair of byte b in its first
// 128 bytes; the low-half pair of byte b sits kPairLoOffset bytes further (the
// second half of row b + 4), a distance no paired LDS read can encode, so the
// two reads of one byte keep separate destination registers.
constexpr int kPairLoOffset = 4 * 256 + 128;
constexpr int kPairTableBytes = (256 + 4) * 256;
// LDS of the kernel, in phases: the staged activations (8 vectors x 4096
// floats) first; then the tables, the span partials and the row block's norms.
constexpr int kMaxBlockRows = 16 * kMfmaTiles * kMfmaMaxSpans;
constexpr int kRedBytes = kMaxBlockRows * kRedStride * 4;
constexpr int kMfmaLdsBytes = 8 * 4096 * 4;
static_assert(kPairTableBytes + kRedBytes + 2 * kMaxBlockRows <= kMfmaLdsBytes, "LDS phases");

// bf16 of a and b (round to nearest even), a in the low half
__device__ __forceinline__ uint32_t bf16_pair(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
// (hi, lo) splits of a and b: *hp = hi(a) | hi(b) << 16, *lp likewise for lo
__device__ __forceinline__ void bf16_split_pair(float a, float b, uint32_t* hp, uint32_t* lp) {
  const uint32_t h = bf16_pair(a, b);
  *hp = h;
  *lp = bf16_pair(a - __uint_as_float(h << 16), b - __uint_as_float(h & 0xffff0000u));
}

// Position of 16-byte chunk cc of staged vector v: rotated by v + 8 (bit 5
// of cc) within its group of 16 chunks, so that the 16 lanes of a row of a
// wavefront (vectors 0..7, both halves) read 16 different bank groups.
__device__ __forceinline__ int stage_pos(int v, int cc, int chunks_per_vector) {
  return v * chunks_per_vector + (cc & ~15) + ((cc + v + 8 * ((cc >> 5) & 1)) & 15);
}

template <int BITS, int T>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(4, 4)))
void cq_matvec_mfma(const uint8_t* __restrict__ packed, const uint16_t* __restrict__ norms,
                    const float* __restrict__ codebook, const float* __restrict__ prepared,
                    float* __restrict__ y, int input_padded, int64_t row_bytes, int log2_group,
                    int rows, int64_t y_stride, int nb, int rg_n) {
  static_assert(T == kMfmaTiles, "LDS sized for kMfmaTiles");
  constexpr bool kPairs = BITS == 4;
  constexpr int kHalfBytes = 4 * BITS;  // one lane's 32 indices of a half span
  __shared__ __align__(16) uint8_t smem[kMfmaLdsBytes];
  u32x4_t* stage = reinterpret_cast<u32x4_t*>(smem);
  uint32_t* lut = reinterpret_cast<uint32_t*>(smem);  // pair tables, or 32 entries
  float* red = reinterpret_cast<float*>(smem + kPairTableBytes);  // [span][row][vector]
  uint16_t* nrm_lds = reinterpret_cast<uint16_t*>(smem + kPairTableBytes + kRedBytes);

  const int tid = threadIdx.x;
  const int wave = tid >> 6, l = tid & 63, r16 = l & 15, q = l >> 4;
  const int n_spans = input_padded >> 8;
  const int span = wave % n_spans, rg = wave / n_spans;
  const int block_rows = 16 * T * rg_n;
  const int n_tiles = (rows + 15) >> 4;
  const int n_groups = input_padded >> log2_group;
  const int g = (256 * span) >> log2_group;
  // Round `it` gives local tile T r + i (row group r, tile i) of the
  // workgroup global tile ((it T + i) rg_n + r) grid + blockIdx: in a round
  // the whole grid reads one contiguous run of tiles, tile by tile, so the
  // weight stream moves through memory as a front rather than as one
  // scattered request per workgroup.
  const int grid = (int)gridDim.x;
  auto tile_of = [&](int it, int lt) {
    return ((it * T + lt % T) * rg_n + lt / T) * grid + (int)blockIdx.x;
  };
  // the round's norms, [local row][group]: groups >= 256 give
  // block_rows * n_groups <= 64 T rg_n * n_spans <= blockDim entries
  const int block_norms = block_rows * n_groups;
  const int tile_norms = 16 * n_groups;
  const uint8_t* lane_bytes = packed + 32 * BITS * span + kHalfBytes * q;

  // Loads, in the order they are consumed: codebook, the activations, the row
  // block's norms, then the weights of its first two tiles; each wait then
  // covers only what it needs.  Later tiles load two tiles ahead of the one
  // being decoded: a wavefront blocked on issuing loads into a full memory
  // pipeline stalls only itself, not the set-up that the workgroup shares.
  const float cbv = codebook[kPairs ? (l & 15) : min(tid, (1 << BITS) - 1)];
  // Activation chunk k of this thread: 16-byte chunk cc of vector v, with
  // 2 input_padded / 4 chunks over blockDim >= input_padded / 4 threads.
  const int cpv = input_padded >> 2;  // chunks per vector
  float4 xs[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int c = tid + k * (int)blockDim.x;
    const int v = c / cpv;
    if (c < 8 * cpv && v < nb)
      xs[k] = reinterpret_cast<const float4*>(prepared)[(int64_t)v * cpv + (c - v * cpv)];
  }
  int it = 0;  // tile_of(0, 0) < n_tiles: the grid has at most n_tiles workgroups
  auto load_norm = [&](int it) {  // entry tid of the round's norms (tid < block_norms)
    const int t = min(tid, block_norms - 1);
    const int64_t e = min((int64_t)tile_of(it, t / tile_norms) * tile_norms + t % tile_norms,
                          (int64_t)rows * n_groups - 1);
    return norms[e];
  };
  uint16_t nv = load_norm(it);
  __builtin_amdgcn_sched_barrier(0);
  uint32_t d[T][2 * BITS];
  // Tile i of this wavefront's row group in round it into d[i]: an
  // unconditional load of a clamped row, whose result is dropped if clamped.
  auto load_tile = [&](int it, int i) {
    const int r = min(16 * tile_of(it, T * rg + i) + r16, rows - 1);
    const uint8_t* p = lane_bytes + (int64_t)r * row_bytes;
    const uint32_t* p0 = reinterpret_cast<const uint32_t*>(p);
    const uint32_t* p1 = reinterpret_cast<const uint32_t*>(p + 16 * BITS);
#pragma unroll
    for (int w = 0; w < BITS; ++w) d[i][w] = stream_load(p0 + w);
#pragma unroll
    for (int w = 0; w < BITS; ++w) d[i][BITS + w] = stream_load(p1 + w);
  };
  load_tile(it, 0);
  load_tile(it, 1);
  __builtin_amdgcn_sched_barrier(0);

  // Stage the activations, then read this lane's 32 values: vector r16 % 8,
  // columns 128 part + 32 q + 0..31 of the span, part = r16 / 8.
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int c = tid + k * (int)blockDim.x;
    const int v = c / cpv;
    if (c < 8 * cpv && v < nb)
      stage[stage_pos(v, c - v * cpv, cpv)] = __builtin_bit_cast(u32x4_t, xs[k]);
  }
  __syncthreads();
  const int part = r16 >> 3;
  float xv[32];
  {
    const int v = r16 & 7;
    const int cc0 = 64 * span + 32 * part + 8 * q;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32x4_t t = stage[stage_pos(v, cc0 + i, cpv)];
#pragma unroll
      for (int e = 0; e < 4; ++e) xv[4 * i + e] = __uint_as_float(t[e]);
    }
  }
  // Activation operands of the span, K-block j: lanes of part 0 (DPP banks 0
  // and 1 of each row) keep the high halves of values 0..31 and receive those
  // of 32..63 from the lane 8 above; lanes of part 1 keep the low halves of
  // 32..63 and receive those of 0..31.  A DPP move that writes only the
  // receiving part places each value without selects.  Vectors from nb on
  // hold stale LDS data; their columns are never stored.
  u32x4_t bx[8];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    uint32_t hp, lp;
    bf16_split_pair(xv[2 * i], xv[2 * i + 1], &hp, &lp);
    bx[i >> 2][i & 3] = __builtin_amdgcn_update_dpp(hp, lp, kRowRor8, 0xf, 0xc, false);
    bx[4 + (i >> 2)][i & 3] = __builtin_amdgcn_update_dpp(lp, hp, kRowRor8, 0xf, 0x3, false);
  }
  __syncthreads();  // the staged activations are read; the tables overwrite them

  // Codebook tables.
  if constexpr (kPairs) {
    uint32_t hs, ls;  // lane l % 16: halves of codebook[l % 16]
    bf16_split_pair(cbv, cbv, &hs, &ls);
    hs &= 0xffffu;
    ls &= 0xffffu;
    // slot t writes copies 4 (t % 8) .. + 3 of rows 16 h + 4 (t / 256) + 0..3,
    // h = (t / 16) % 16, in the high-half table for even t / 8 and the low-half
    // one for odd: the 16 lanes of one store pass cover a high row and a low
    // row, which sit in opposite halves of the banks.
    for (int t = tid; t < 1024; t += (int)blockDim.x) {
      const int c4 = 4 * (t & 7), lo_tab = (t >> 3) & 1, h = (t >> 4) & 15, e0 = 4 * (t >> 8);
      // odd column: index h
      const uint32_t hh = (uint32_t)__shfl((int)hs, h), lh = (uint32_t)__shfl((int)ls, h);
      const uint32_t hi16 = (lo_tab ? lh : hh) << 16;
#pragma unroll
      for (int e = 0; e < 4; ++e) {  // even column: index e0 + e (wave-uniform)
        const int b = 16 * h + e0 + e;
        const uint32_t he = (uint32_t)__builtin_amdgcn_readlane((int)hs, e0 + e);
        const uint32_t le = (uint32_t)__builtin_amdgcn_readlane((int)ls, e0 + e);
        const uint32_t val = (lo_tab ? le : he) | hi16;
        const u32x4_t v4 = {val, val, val, val};
        *reinterpret_cast<u32x4_t*>(&lut[lo_tab ? (b + 4) * 64 + 32 + c4 : b * 64 + c4]) = v4;
      }
    }
  } else {
    if (tid < (1 << BITS)) {
      uint32_t h, lo;
      bf16_split_pair(cbv, cbv, &h, &lo);
      lut[tid] = (h & 0xffffu) | (lo << 16);
    }
  }

  const uint32_t lane_off = 4u * (uint32_t)(l & (kPairCopies - 1));  // this lane's copy
  while (true) {
    if (tid < block_norms) nrm_lds[tid] = nv;
    __syncthreads();  // tables and norms written; the previous partials read
    const bool more = tile_of(it + 1, 0) < n_tiles;
#pragma unroll
    for (int i = 0; i < T; ++i) {
      // two tiles ahead: this round's, then the next round's first two
      if (i + 2 < T) {
        load_tile(it, i + 2);
      } else if (more) {
        if (i + 2 == T) nv = load_norm(it + 1);
        load_tile(it + 1, i + 2 - T);
      }
      __builtin_amdgcn_sched_barrier(0);
      f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        u32x4_t ahi, alo;
        if constexpr (kPairs) {
          const uint32_t w = d[i][j];  // indices of the lane's columns 8 j .. 8 j + 7
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            // row (byte p of w) of the tables, copy lane % 32
            const uint32_t a = __builtin_amdgcn_perm(w, lane_off, 0x0c0c0400u | ((4u + p) << 8));
            ahi[p] = *reinterpret_cast<const uint32_t*>(smem + a);
            alo[p] = *reinterpret_cast<const uint32_t*>(smem + a + kPairLoOffset);
          }
        } else {
          uint32_t v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int k = 8 * j + e;  // index position in the lane's 64
            const int bit = BITS * k, w = bit >> 5, sh = bit & 31;
            uint32_t idx;
            if (sh + BITS <= 32) idx = (d[i][w] >> sh) & ((1u << BITS) - 1u);
            else idx = __builtin_amdgcn_alignbit(d[i][w + 1], d[i][w], sh) & ((1u << BITS) - 1u);
            v[e] = lut[idx];
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            ahi[e] = __builtin_amdgcn_perm(v[2 * e + 1], v[2 * e], 0x05040100u);
            alo[e] = __builtin_amdgcn_perm(v[2 * e + 1], v[2 * e], 0x07060302u);
          }
        }
        const bf16x8_t bo = __builtin_bit_cast(bf16x8_t, bx[j]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ahi), bo, acc,
                                                      0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, alo), bo, acc,
                                                      0, 0, 0);
      }
      // acc[k]: row 16 T rg + 16 i + 4 q + k of the block, operand column r16;
      // times its norm, then column v (high halves) + column v + 8 (low halves)
      const int row = 16 * T * rg + 16 * i + 4 * q;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float s = acc[k] * f16_to_f32(nrm_lds[(row + k) * n_groups + g]);
        const float v = s + dpp<kRowRor8, 0xf, false>(0.0f, s);
        if (r16 < 8) red[(span * block_rows + row + k) * kRedStride + r16] = v;
      }
    }
    __syncthreads();
    for (int o = tid; o < block_rows * nb; o += (int)blockDim.x) {
      const int v = o / block_rows, row = o - v * block_rows;
      float sum = 0.0f;
      for (int s = 0; s < n_spans; ++s) sum += red[(s * block_rows + row) * kRedStride + v];
      const int r = 16 * tile_of(it, row >> 4) + (row & 15);
      if (r < rows) y[v * y_stride + r] = sum;
    }
    if (!more) break;
    ++it;
  }
}

// 4-bit rows on the matrix cores with each weight's two bf16 halves side by
// side in K: a 32-deep K block holds 16 weights as (hi, lo) pairs, and the
// matching operand rows hold each activation column twice, so one product
// sums (hi + lo) * x over 16 weights.  The pair table then returns, for a
// packed byte, both weights' (hi, lo) halves as one 8-byte read landing in
// two consecutive operand registers: two reads, two byte permutes and one
// product per 16 weights of a row (the split-table layout above needs eight
// 4-byte reads and two products per 32).  The activation operands go from
// memory straight to registers: eight whole-line loads per lane (each load
// instruction reads one 128-byte line per vector), rearranged with lane swaps,
// so the only workgroup barrier before the first product is the table's.  A
// CU reads all activations of its rows (8 x 4096 floats = 128 KiB) besides
// its ~128 KiB of weights; both go through the same per-CU memory path, and
// scattered 16-byte activation reads (32 lines per load instruction) cost
// ~3 us more than the line-wise ones.
//
// Lanes and columns: lane l = (r16, q) owns tile row r16 and, in the span's
// 128 bytes, the 16-byte chunks 16 q and 64 + 16 q (each weight load reads
// 64 consecutive bytes of 16 rows).  K block t (0..15) takes bytes 2t, 2t + 1
// of the first chunk (t < 8) or of the second: columns c(q, t) + 0..3 with
// c = 32 q + 4 t (t < 8) or 128 + 32 q + 4 (t - 8).  The operand lane
// (r16, q) holds, for vector r16 % 8, the high (r16 < 8) or low bf16 half of
// x at those four columns, each duplicated into both halves of a register.
constexpr int kPair4RowBytes = 32 * 8;                       // 32 copies of two packed halves
constexpr int kPair4TableBytes = 256 * kPair4RowBytes;       // 64 KiB
constexpr int kMfma4LdsBytes = kPair4TableBytes + kRedBytes + 2 * kMaxBlockRows;
constexpr int kMfma4Tiles = 4;  // 16-row tiles per wavefront and round
constexpr int kMfma4Ahead = 1;  // tiles requested ahead of the one decoded

template <int T, int AHEAD>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(4, 4)))
void cq_matvec_mfma4(const uint8_t* __restrict__ packed, const uint16_t* __restrict__ norms,
                     const float* __restrict__ codebook, const float* __restrict__ prepared,
                     float* __restrict__ y, int input_padded, int64_t row_bytes, int log2_group,
                     int rows, int64_t y_stride, int nb, int rg_n) {
  static_assert(T <= kMfmaTiles && AHEAD <= T, "LDS sized for kMfmaTiles");
  __shared__ __align__(16) uint8_t smem[kMfma4LdsBytes];
  float* red = reinterpret_cast<float*>(smem + kPair4TableBytes);  // [span][row][vector]
  uint16_t* nrm_lds = reinterpret_cast<uint16_t*>(smem + kPair4TableBytes + kRedBytes);

  const int tid = threadIdx.x;
  const int wave = tid >> 6, l = tid & 63, r16 = l & 15, q = l >> 4;
  const int n_spans = input_padded >> 8;
  const int span = wave % n_spans, rg = wave / n_spans;
  const int block_rows = 16 * T * rg_n;
  const int n_tiles = (rows + 15) >> 4;
  const int n_groups = input_padded >> log2_group;
  const int g = (256 * span) >> log2_group;
  const int grid = (int)gridDim.x;
  // round `it`: local tile T r + i is global tile ((it T + i) rg_n + r) grid + blockIdx
  auto tile_of = [&](int it, int lt) {
    return ((it * T + lt % T) * rg_n + lt / T) * grid + (int)blockIdx.x;
  };
  const int block_norms = block_rows * n_groups;
  const int tile_norms = 16 * n_groups;
  const uint8_t* lane_bytes = packed + 128 * span + 16 * q;

  // Loads in the order they are needed: the codebook (table), the activation
  // operands, the round's norms, then the first AHEAD tiles' weights.
  constexpr int kSlots = kPair4TableBytes / 16;  // 16-byte table slots
  const int nthreads = (int)blockDim.x;
  const float cbv = codebook[l & 15];  // lane l: codebook[l % 16]
  const int v = r16 & 7, part = r16 >> 3;
  // Activations in whole lines: load i gives lane (q, part, v) the float4 of
  // vector v at span column 32 i + 8 q + 4 part (4-column chunk 8 i + 2 q + part).
  float4 xa[8];
  {
    const float* xv =
        prepared + (int64_t)(v < nb ? v : 0) * input_padded + 256 * span + 8 * q + 4 * part;
#pragma unroll
    for (int i = 0; i < 8; ++i) xa[i] = *reinterpret_cast<const float4*>(xv + 32 * i);
  }
  int it = 0;  // tile_of(0, 0) < n_tiles: the grid has at most n_tiles workgroups
  auto load_norm = [&](int it) {
    const int t = min(tid, block_norms - 1);
    const int64_t e = min((int64_t)tile_of(it, t / tile_norms) * tile_norms + t % tile_norms,
                          (int64_t)rows * n_groups - 1);
    return norms[e];
  };
  uint16_t nv = load_norm(it);
  __builtin_amdgcn_sched_barrier(0);
  u32x4_t d[T][2];
  auto load_tile = [&](int it, int i) {
    const int r = min(16 * tile_of(it, T * rg + i) + r16, rows - 1);
    const uint8_t* p = lane_bytes + (int64_t)r * row_bytes;
    d[i][0] = stream_load(reinterpret_cast<const u32x4_nt*>(p));
    d[i][1] = stream_load(reinterpret_cast<const u32x4_nt*>(p + 64));
  };
#pragma unroll
  for (int i = 0; i < AHEAD; ++i) load_tile(it, i);
  __builtin_amdgcn_sched_barrier(0);

  // The table: slot t (16 bytes) is copies 2 (t % 16), + 1 of row b = t / 16,
  // each (pack(codebook[b % 16]), pack(codebook[b / 16])) with pack(w) =
  // bf16(w) | bf16(w - bf16(w)) << 16.  A wavefront's 64 slots share t / 256.
  for (int t = tid; t < kSlots; t += nthreads) {
    const float ca = __shfl(cbv, (t >> 4) & 15);
    const float cb = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cbv), t >> 8));
    uint32_t hp, lp;
    bf16_split_pair(ca, cb, &hp, &lp);  // hp = hi(ca) | hi(cb) << 16, lp likewise
    const uint32_t pa = (hp & 0xffffu) | (lp << 16);
    const uint32_t pb = (hp >> 16) | (lp & 0xffff0000u);
    const u32x4_t e = {pa, pb, pa, pb};
    *reinterpret_cast<u32x4_t*>(smem + 16 * t) = e;
  }
  // Activation operands, packed: K block t holds the chosen bf16 half of x
  // at the span's 4-column chunk 8 q + (t % 8) + 32 (t / 8) as two pairs; each
  // product's operand register j then duplicates the half of column j with
  // one byte permute.  From the whole-line loads: split every float4 into
  // (hi, lo) pairs, then for h = 0, 1 transpose loads 4 h + j (j = 0..3)
  // against the 16-lane rows q with the two lane swaps, which leaves in slot j
  // of row q the chunk 8 (4 h + q) + 2 j + part; the chunk of the other parity
  // comes from lane l ^ 8 (same q and v), which sends the half this lane takes.
  uint32_t bxp[16][2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t sl[4][4];  // [slot j][hi pair 0, hi pair 1, lo pair 0, lo pair 1]
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 f = xa[4 * h + j];
      bf16_split_pair(f.x, f.y, &sl[j][0], &sl[j][2]);
      bf16_split_pair(f.z, f.w, &sl[j][1], &sl[j][3]);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {  // rows 2, 3 of slot j trade with rows 0, 1 of slot j + 2
        const auto r = __builtin_amdgcn_permlane32_swap(sl[j][e], sl[j + 2][e], false, false);
        sl[j][e] = r[0];
        sl[j + 2][e] = r[1];
      }
#pragma unroll
      for (int j = 0; j < 4; j += 2) {  // rows 1, 3 of slot j trade with rows 0, 2 of slot j + 1
        const auto r = __builtin_amdgcn_permlane16_swap(sl[j][e], sl[j + 1][e], false, false);
        sl[j][e] = r[0];
        sl[j + 1][e] = r[1];
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const uint32_t own = part ? sl[j][2 + e] : sl[j][e];
        const uint32_t give = part ? sl[j][e] : sl[j][2 + e];
        const uint32_t got = __float_as_uint(lane_xor<8>(__uint_as_float(give)));
        bxp[8 * h + 2 * j][e] = part ? got : own;      // chunk parity 0
        bxp[8 * h + 2 * j + 1][e] = part ? own : got;  // chunk parity 1
      }
    }
  }

  const uint32_t lane_off = 8u * (uint32_t)(l & 31);  // this lane's table copy
  while (true) {
    if (tid < block_norms) nrm_lds[tid] = nv;
    __syncthreads();  // table and norms written; the previous partials read
    const bool more = tile_of(it + 1, 0) < n_tiles;
#pragma unroll
    for (int i = 0; i < T; ++i) {
      // AHEAD tiles ahead: this round's, then the next round's first ones
      if (i + AHEAD < T) {
        load_tile(it, i + AHEAD);
      } else if (more) {
        if (i + AHEAD == T) nv = load_norm(it + 1);
        load_tile(it + 1, i + AHEAD - T);
      }
      __builtin_amdgcn_sched_barrier(0);
      // keep the packed operands packed (32 registers, not 64): their
      // duplicates are made per product
#pragma unroll
      for (int t = 0; t < 16; ++t) asm volatile("" : "+v"(bxp[t][0]), "+v"(bxp[t][1]));
      f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const uint32_t w = d[i][t >> 3][(t >> 1) & 3];  // dword holding bytes 2t, 2t + 1
        const uint32_t b0 = 2u * (t & 1);                // byte position of 2t in it
        const uint32_t a0 = __builtin_amdgcn_perm(w, lane_off, 0x0c0c0400u | ((4u + b0) << 8));
        const uint32_t a1 = __builtin_amdgcn_perm(w, lane_off, 0x0c0c0400u | ((5u + b0) << 8));
        const f32x2_t e0 = *reinterpret_cast<const f32x2_t*>(smem + a0);
        const f32x2_t e1 = *reinterpret_cast<const f32x2_t*>(smem + a1);
        const u32x4_t a = {__float_as_uint(e0[0]), __float_as_uint(e0[1]), __float_as_uint(e1[0]),
                           __float_as_uint(e1[1])};
        const u32x4_t bx = {__builtin_amdgcn_perm(bxp[t][0], bxp[t][0], 0x01000100u),
                            __builtin_amdgcn_perm(bxp[t][0], bxp[t][0], 0x03020302u),
                            __builtin_amdgcn_perm(bxp[t][1], bxp[t][1], 0x01000100u),
                            __builtin_amdgcn_perm(bxp[t][1], bxp[t][1], 0x03020302u)};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                      __builtin_bit_cast(bf16x8_t, bx), acc,
                                                      0, 0, 0);
      }
      // acc[k]: row 16 T rg + 16 i + 4 q + k of the block, operand column r16;
      // times its norm, then column v (high halves) + column v + 8 (low halves)
      const int row = 16 * T * rg + 16 * i + 4 * q;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float s = acc[k] * f16_to_f32(nrm_lds[(row + k) * n_groups + g]);
        const float vv = s + dpp<kRowRor8, 0xf, false>(0.0f, s);
        if (r16 < 8) red[(span * block_rows + row + k) * kRedStride + r16] = vv;
      }
    }
    __syncthreads();
    for (int o = tid; o < block_rows * nb; o += (int)blockDim.x) {
      const int vec = o / block_rows, row = o - vec * block_rows;
      float sum = 0.0f;
#pragma unroll
      for (int s2 = 0; s2 < kMfmaMaxSpans; ++s2)
        if (s2 < n_spans) sum += red[(s2 * block_rows + row) * kRedStride + vec];
      const int r = 16 * tile_of(it, row >> 4) + (row & 15);
      if (r < rows) y[vec * y_stride + r] = sum;
    }
    if (!more) break;
    ++it;
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
  const size_t lds = sizeof(float) * ActLayout::floats(m->input_padded);
  hipLaunchKernelGGL((cq_matvec_b1<BITS, NJ, LPR, U>), dim3((unsigned)grid),
                     dim3(kThreads), lds, s, m->packed, m->norms, m->codebook, prepared, y,
                     m->input_padded, m->row_bytes, ilog2(m->group), row_begin, row_count);
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
  const int64_t grid =
      std::min<int64_t>((n_steps + U - 1) / U, (int64_t)cu_count() * kNbBlocksPerCu);
  const size_t lds = sizeof(float) * ActLayout::floats(m->input_padded);
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


// The ring kernel's shapes: 4-bit, input_padded in {512, ..., 8192}, groups
// that hold a lane's columns, 16-byte aligned rows.  Returns (BPL, S) or
// (0, 0) when the shape is not covered.
struct RingShape { int bpl, s; };
RingShape ring_shape(const bqd_cq_matrix* m) {
  if (m->bits != 4 || m->row_bytes % 16 || !is_aligned(m->packed, 16)) return {0, 0};
  RingShape r{0, 0};
  switch (m->input_padded) {
    case 512: r = {4, 1}; break;
    case 1024: r = {8, 1}; break;
    case 2048: r = {16, 1}; break;
    case 4096: r = {16, 2}; break;
    case 8192: r = {16, 4}; break;
    default: return {0, 0};
  }
  if (m->group < 2 * r.bpl) return {0, 0};
  return r;
}

// Workgroups of one ring launch: times 1024 threads, below the 2^32
// work-items one dispatch holds (reached only by 512- and 1024-column rows
// past 137 and 275 GB of weights).
constexpr int64_t kRingMaxBlocks = ((int64_t)1 << 32) / kRingThreads - 1;

// The ring kernel over up to kRingMaxMats row ranges of matrices that share
// the ring shape r, input width and group (ms[0] gives those).  Ranges that
// would need more than kRingMaxBlocks workgroups run one matrix at a time in
// row chunks (prepared_out is stored by the first launch).
template <int BPL, int S, int E>
int launch_ring_t(const bqd_cq_matrix* const* ms, const int64_t* row_begin,
                  const int64_t* row_count, float* const* ys, int n, const float* act,
                  float* prepared_out, hipStream_t s) {
  constexpr int RPB = (16 / S) * kRingRows;
  int64_t total = 0;
  for (int k = 0; k < n; ++k) total += (row_count[k] + RPB - 1) / RPB;
  if (total > kRingMaxBlocks) {
    constexpr int64_t chunk = kRingMaxBlocks * RPB;
    for (int k = 0; k < n; ++k) {
      for (int64_t r0 = 0; r0 < row_count[k]; r0 += chunk) {
        const int64_t rb = row_begin[k] + r0, rc = std::min(chunk, row_count[k] - r0);
        float* yk = ys[k] + r0;
        const int rc2 = launch_ring_t<BPL, S, E>(&ms[k], &rb, &rc, &yk, 1, act, prepared_out, s);
        if (rc2) return rc2;
        prepared_out = nullptr;
      }
    }
    return BQD_OK;
  }
  const bqd_cq_matrix* m0 = ms[0];
  RingArgs a{};
  int64_t blocks = 0;
  for (int k = 0; k < kRingMaxMats; ++k) a.m[k].block_end = INT32_MAX;
  for (int k = 0; k < n; ++k) {
    const bqd_cq_matrix* m = ms[k];
    blocks += (row_count[k] + RPB - 1) / RPB;
    a.m[k] = RingMat{m->packed + row_begin[k] * m->row_bytes,
                     m->norms + row_begin[k] * (m->input_padded / m->group), m->codebook, ys[k],
                     m->row_bytes, (int32_t)row_count[k], (int32_t)blocks};
  }
  a.act = act;
  a.prepared_out = prepared_out;
  a.log2_group = ilog2(m0->group);
  a.input = (int32_t)m0->input;
  a.x_vec = E > 0 && m0->input == m0->input_padded && is_aligned(act, 16);
  a.scale = 1.0 / std::sqrt((double)m0->group);
  if (n == 1)
    hipLaunchKernelGGL((cq_matvec_ring<BPL, S, E, false>), dim3((unsigned)blocks),
                       dim3(kRingThreads), 0, s, a);
  else
    hipLaunchKernelGGL((cq_matvec_ring<BPL, S, E, true>), dim3((unsigned)blocks),
                       dim3(kRingThreads), 0, s, a);
  return launch_status();
}

// E: 0 for a prepared activation, else the transform's elements per lane.
template <int E>
int launch_ring(const bqd_cq_matrix* const* ms, const int64_t* row_begin, const int64_t* row_count,
                float* const* ys, int n, RingShape r, const float* act, float* prepared_out,
                hipStream_t s) {
#define RING_ARGS ms, row_begin, row_count, ys, n, act, prepared_out, s
  if (r.bpl == 4) return launch_ring_t<4, 1, E>(RING_ARGS);
  if (r.bpl == 8) return launch_ring_t<8, 1, E>(RING_ARGS);
  switch (r.s) {
    case 1: return launch_ring_t<16, 1, E>(RING_ARGS);
    case 2: return launch_ring_t<16, 2, E>(RING_ARGS);
    case 4: return launch_ring_t<16, 4, E>(RING_ARGS);
  }
#undef RING_ARGS
  return BQD_EINVAL;  // unreachable: ring_shape() only returns instantiated shapes
}

template <int E>
int launch_ring1(const bqd_cq_matrix* m, RingShape r, const float* act, float* prepared_out,
                 float* y, int64_t row_begin, int64_t row_count, hipStream_t s) {
  return launch_ring<E>(&m, &row_begin, &row_count, &y, 1, r, act, prepared_out, s);
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
// spans, at most 16 spans (one wavefront each), dword rows, and activations
// that load as float4.
bool mfma_ok(const bqd_cq_matrix* m, const float* prepared) {
  return m->group >= 256 && m->input_padded % 256 == 0 &&
         m->input_padded <= 256 * kMfmaMaxSpans && m->row_bytes % 4 == 0 &&
         is_aligned(m->packed, 4) && is_aligned(prepared, 16);
}

template <int BITS>
int launch_mfma_b(const bqd_cq_matrix* m, const float* prepared, float* y, int64_t y_stride,
                  int nb, int64_t row_begin, int64_t row_count, hipStream_t s) {
  constexpr int T = kMfmaTiles;
  const int n_spans = (int)(m->input_padded / 256);
  // row groups per workgroup: enough to spread the rows over every CU, at
  // most 16 wavefronts
  const int64_t tiles = (row_count + 16 * T - 1) / (16 * T);
  const int64_t rg_need = (tiles + cu_count() - 1) / cu_count();
  const int rg = (int)std::max<int64_t>(1, std::min<int64_t>(rg_need, kMfmaMaxSpans / n_spans));
  const int64_t block_rows = 16 * T * rg;
  // every workgroup has a first tile: grid <= n_tiles
  const int64_t blocks = (row_count + block_rows - 1) / block_rows;
  const int64_t grid =
      std::min<int64_t>(std::min<int64_t>(blocks, cu_count()), (row_count + 15) / 16);
  hipLaunchKernelGGL((cq_matvec_mfma<BITS, T>), dim3((unsigned)grid),
                     dim3((unsigned)(64 * n_spans * rg)), 0, s,
                     m->packed + row_begin * m->row_bytes,
                     m->norms + row_begin * (m->input_padded / m->group), m->codebook, prepared, y,
                     (int)m->input_padded, m->row_bytes, ilog2(m->group), (int)row_count, y_stride,
                     nb, rg);
  return launch_status();
}

// 4-bit rows that load as 16-byte chunks take the paired-halves kernel.
int launch_mfma4(const bqd_cq_matrix* m, const float* prepared, float* y, int64_t y_stride, int nb,
                 int64_t row_begin, int64_t row_count, hipStream_t s) {
  constexpr int T = kMfma4Tiles, AHEAD = kMfma4Ahead;
  const int n_spans = (int)(m->input_padded / 256);
  const int64_t tiles = (row_count + 16 * T - 1) / (16 * T);
  const int64_t rg_need = (tiles + cu_count() - 1) / cu_count();
  const int rg = (int)std::max<int64_t>(1, std::min<int64_t>(rg_need, kMfmaMaxSpans / n_spans));
  const int64_t block_rows = 16 * T * rg;
  const int64_t blocks = (row_count + block_rows - 1) / block_rows;
  const int64_t grid =
      std::min<int64_t>(std::min<int64_t>(blocks, cu_count()), (row_count + 15) / 16);
  hipLaunchKernelGGL((cq_matvec_mfma4<T, AHEAD>), dim3((unsigned)grid),
                     dim3((unsigned)(64 * n_spans * rg)), 0, s,
                     m->packed + row_begin * m->row_bytes,
                     m->norms + row_begin * (m->input_padded / m->group), m->codebook, prepared, y,
                     (int)m->input_padded, m->row_bytes, ilog2(m->group), (int)row_count, y_stride,
                     nb, rg);
  return launch_status();
}

int run_mfma(const bqd_cq_matrix* m, const float* prepared, float* y, int64_t y_stride, int nb,
             int64_t row_begin, int64_t row_count, hipStream_t s) {
  switch (m->bits) {
    case 2: return launch_mfma_b<2>(m, prepared, y, y_stride, nb, row_begin, row_count, s);
    case 3: return launch_mfma_b<3>(m, prepared, y, y_stride, nb, row_begin, row_count, s);
    case 4:
      if (m->row_bytes % 16 == 0 && is_aligned(m->packed, 16))
        return launch_mfma4(m, prepared, y, y_stride, nb, row_begin, row_count, s);
      return launch_mfma_b<4>(m, prepared, y, y_stride, nb, row_begin, row_count, s);
    case 5: return launch_mfma_b<5>(m, prepared, y, y_stride, nb, row_begin, row_count, s);
  }
  return BQD_EINVAL;
}

int launch_generic(const bqd_cq_matrix* m, const float* prepared, float* y, int64_t batch,
                   int64_t row_begin, int64_t row_count, hipStream_t s) {
  const int64_t grid =
      std::min<int64_t>((row_count + kWavesPerBlock - 1) / kWavesPerBlock, kMaxGrid);
  hipLaunchKernelGGL(cq_matvec_generic, dim3((unsigned)grid), dim3(kThreads), 0, s, m->packed,
                     m->norms, m->codebook, prepared, y, m->input_padded, m->row_bytes,
                     (int)m->bits, ilog2(m->group), row_begin, row_count, batch);
  return launch_status();
}

}  // namespace

int launch_cq_matvec(const bqd_cq_matrix* m, const float* prepared, float* y, int64_t batch,
                     int64_t row_begin, int64_t row_count, hipStream_t s) {
  if (batch == 1) {
    const RingShape r = ring_shape(m);
    if (r.bpl && is_aligned(prepared, 16))
      return launch_ring1<0>(m, r, prepared, nullptr, y, row_begin, row_count, s);
  }
  if (!fast_ok(m)) return launch_generic(m, prepared, y, batch, row_begin, row_count, s);
  const int64_t n_chunk = m->input_padded / 32;
  const FastShape f1 = fast_shape(n_chunk, 1);
  const FastShape f4 = fast_shape(n_chunk, 4);
  if (batch == 1 && f1.lpr) return run_b1(m, f1, prepared, y, row_begin, row_count, s);
  if (batch >= 2 && mfma_ok(m, prepared)) {
    // up to eight vectors per launch on the matrix cores
    for (int64_t b = 0; b < batch; b += 8) {
      const int nb = (int)std::min<int64_t>(8, batch - b);
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

// [P1] §2 then §3 in one call: `prepared` receives the prepared vectors and y
// the matvec, exactly as cq_prepare followed by cq_matvec.  A single 4-bit
// vector on a ring shape with groups of at most 256 takes one launch (the
// prepare runs inside every workgroup of the matvec, workgroup 0 stores it);
// everything else takes the two launches.
int launch_cq_prepare_matvec(const bqd_cq_matrix* m, const float* x, float* prepared, float* y,
                             int64_t batch, int64_t row_begin, int64_t row_count, hipStream_t s) {
  if (batch == 1 && row_count > 0 && is_aligned(prepared, 16)) {
    const RingShape r = ring_shape(m);
    if (r.bpl) {
      switch (lane_elems(m->group)) {
        case 1: return launch_ring1<1>(m, r, x, prepared, y, row_begin, row_count, s);
        case 2: return launch_ring1<2>(m, r, x, prepared, y, row_begin, row_count, s);
        case 4: return launch_ring1<4>(m, r, x, prepared, y, row_begin, row_count, s);
      }
    }
  }
  const int rc = launch_cq_prepare(m, x, prepared, batch, s);
  if (rc || row_count == 0) return rc;
  return launch_cq_matvec(m, prepared, y, batch, row_begin, row_count, s);
}

// [P1] §6: several matrices, each a row range, on one activation.  Matrices
// on a common ring shape share launches (up to kRingMaxMats each); with
// `x` the first launch also prepares the activation in every workgroup and
// stores it, later ones read it back.  Anything else: the prepare (with x),
// then one cq_matvec per matrix.  Arguments arrive validated: one vector,
// equal input_padded and group (and input with x).
int launch_cq_matvec_multi(const bqd_cq_matrix* ms, int64_t n, const int64_t* row_begin,
                           const int64_t* row_count, bool with_x, const float* x,
                           float* prepared, float* const* ys, hipStream_t s) {
  const bqd_cq_matrix* sel[64];
  int64_t rb[64], rc[64];
  float* yy[64];
  int k_n = 0;
  for (int64_t k = 0; k < n; ++k) {
    if (row_count[k] == 0) continue;
    sel[k_n] = &ms[k];
    rb[k_n] = row_begin[k];
    rc[k_n] = row_count[k];
    yy[k_n] = ys[k];
    ++k_n;
  }
  RingShape r = k_n ? ring_shape(sel[0]) : RingShape{0, 0};
  for (int k = 1; k < k_n && r.bpl; ++k) {
    const RingShape rk = ring_shape(sel[k]);
    if (rk.bpl != r.bpl || rk.s != r.s) r = {0, 0};
  }
  const int e = lane_elems(ms[0].group);
  if (r.bpl && is_aligned(prepared, 16) && (!with_x || e <= 4)) {
    for (int k0 = 0; k0 < k_n; k0 += kRingMaxMats) {
      const int nk = std::min(kRingMaxMats, k_n - k0);
      int rc2 = BQD_EINVAL;
      if (with_x && k0 == 0) {
        switch (e) {
          case 1: rc2 = launch_ring<1>(sel, rb, rc, yy, nk, r, x, prepared, s); break;
          case 2: rc2 = launch_ring<2>(sel, rb, rc, yy, nk, r, x, prepared, s); break;
          case 4: rc2 = launch_ring<4>(sel, rb, rc, yy, nk, r, x, prepared, s); break;
        }
      } else {
        rc2 = launch_ring<0>(sel + k0, rb + k0, rc + k0, yy + k0, nk, r, prepared, nullptr, s);
      }
      if (rc2) return rc2;
    }
    if (k_n) return BQD_OK;
  }
  if (with_x) {
    const int rc2 = launch_cq_prepare(&ms[0], x, prepared, 1, s);
    if (rc2) return rc2;
  }
  for (int k = 0; k < k_n; ++k) {
    const int rc2 = launch_cq_matvec(sel[k], prepared, yy[k], 1, rb[k], rc[k], s);
    if (rc2) return rc2;
  }
  return BQD_OK;
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

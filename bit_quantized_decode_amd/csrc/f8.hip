// FP8 E4M3 matvec with E8M0 block scales for gfx950, plus the decode probes.
//
// Method: "attention + tokenizer + sampling: the path to real text (milestone
// 6)" — Step 1 (E4M3 decode with e = 0 subnormal and the 448 clamp; E8M0
// block scales where element (r, c) of an R x C weight takes the scale
// [r*SR/R][c*SC/C] of an SR x SC grid) and Step 4 (the vector path applies
// when each vector of columns stays inside one scale block).
#include <algorithm>

#include "device.h"
#include "launch.h"
#include "logit_key.h"
#include "validate.h"

namespace bqd {

constexpr int kF8Threads = 256;

// ----------------------------------------------------------- generic matvec
// Any shape and alignment: one wavefront per row, lanes stride over columns,
// the scale index of every element by integer floor division.
__global__ __launch_bounds__(kF8Threads) void f8_matvec_generic(
    const uint8_t* __restrict__ w, const uint8_t* __restrict__ scale, const float* __restrict__ x,
    float* __restrict__ y, int64_t R, int64_t C, int64_t SR, int64_t SC, int64_t batch) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  for (int64_t r = (int64_t)blockIdx.x * (kF8Threads / kWave) + wave; r < R;
       r += (int64_t)gridDim.x * (kF8Threads / kWave)) {
    const uint8_t* wr = w + r * C;
    const uint8_t* sr = scale + ((r * SR) / R) * SC;
    for (int64_t b = 0; b < batch; ++b) {
      const float* xb = x + b * C;
      float acc = 0.0f;
      for (int64_t c = lane; c < C; c += kWave) {
        const float s = e8m0_to_f32(sr[(c * SC) / C]);
        acc += (e4m3_to_f32(wr[c]) * s) * xb[c];
      }
      acc = group_sum<kWave>(acc);
      if (lane == kWave - 1) y[b * R + r] = acc;
    }
  }
}

// The largest key (logit_key.h) over a workgroup of THREADS threads: every
// lane ends with it.
template <int THREADS = kF8Threads>
__device__ __forceinline__ uint64_t block_max_key(uint64_t k) {
  __shared__ uint64_t wave_best[THREADS / kWave];
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) k = max(k, (uint64_t)__shfl_xor((unsigned long long)k, d));
  if ((threadIdx.x & (kWave - 1)) == 0) wave_best[threadIdx.x / kWave] = k;
  __syncthreads();
  uint64_t m = wave_best[0];
#pragma unroll
  for (int i = 1; i < THREADS / kWave; ++i) m = max(m, wave_best[i]);
  return m;
}

// -------------------------------------------------------------- fast matvec
// Rows of C = 16 * n_chunk bytes with 16-byte aligned rows and scale blocks
// that are a whole number of 16-column chunks wide.  LPR lanes share a row;
// lane q owns chunks q + LPR*j, so each load instruction of a wavefront reads
// 1 KiB of contiguous bytes.  The activation of a lane's columns stays in
// registers; each chunk's partial dot is multiplied by its power-of-two block
// scale (exact), then the row reduces across lanes with DPP.  Where NJ <= 4
// the kernel keeps to 128 registers (4 wavefronts per SIMD): the extra
// wavefronts hide more load latency (~3% on the 246272 x 4096 head).
//
// The scale row of weight row r is floor(r SR / R).  Where SR divides R
// (EXACT: R / SR rows per block) it is r / (R / SR), formed as
// (r * magic) >> shift with the launcher's magic = ceil(2^shift / (R / SR)),
// shift = 31 + ceil(log2(R / SR)), exact for every r < 2^31 (Granlund and
// Montgomery, "Division by invariant integers using multiplication", 1994,
// Theorem 4.2); a 64-bit division per row otherwise (~80 instructions, a
// large share of the loop's work on the head).
//
// SHARE: an iteration's U rows of a lane, (s0 + u) SLOTS + slot with s0 a
// multiple of U, lie in one aligned block of U SLOTS rows; where R / SR is a
// multiple of U SLOTS that block is inside one scale block, so the row's
// block scales are read once per iteration instead of once per row (a fifth
// fewer vector memory reads on the head, ~1.5% faster).
//
// The workgroup stages x in LDS once (float4 loads where x is 16-byte
// aligned, x_vec) and each wavefront takes its lanes' activations from there:
// one copy of x per workgroup from L2 instead of one per wavefront (~1%).
//
// ARGMAX fuses the argmax of y: each lane keeps the largest key (logit_key.h)
// of the rows it stores; each wavefront reads the largest of its storing
// lanes' into LDS and takes a ticket from an LDS counter, and the wavefront with the
// last ticket stores the workgroup's largest to its slot, slots[blockIdx]
// (plain stores).  No wavefront waits for another: a workgroup barrier there
// held three wavefronts at every workgroup's end, and an atomic per
// workgroup into one device word held every workgroup until it completed
// (~20 us over the head); a slot per wavefront made the last step read 4x
// the slots.
template <int NJ, int LPR, int U, bool EXACT, bool SHARE, bool ARGMAX>
__global__ __launch_bounds__(kF8Threads) __attribute__((amdgpu_waves_per_eu(NJ <= 4 ? 4 : 1)))
void f8_matvec_fast(
    const uint8_t* __restrict__ w, const uint8_t* __restrict__ scale, const float* __restrict__ x,
    float* __restrict__ y, int R, int64_t C, int64_t SR, int64_t SC, int64_t cols_per_block,
    uint32_t blk_magic, int blk_shift, int x_vec, uint64_t* __restrict__ slots) {
  constexpr int SLOTS = kF8Threads / LPR;
  constexpr int CX = 16 * LPR * NJ;  // = C
  __shared__ __align__(16) float xs[CX];
  const int tid = threadIdx.x;
  const int slot = tid / LPR;
  const int q = tid % LPR;
  __shared__ uint64_t wave_best[kF8Threads / kWave];
  __shared__ uint32_t tickets;
  if constexpr (ARGMAX)
    if (tid == 0) tickets = 0;  // ordered before any ticket by the staging barrier below
  if (x_vec) {
    for (int i = tid; i < CX / 4; i += kF8Threads)
      reinterpret_cast<float4*>(xs)[i] = reinterpret_cast<const float4*>(x)[i];
  } else {
    for (int i = tid; i < CX; i += kF8Threads) xs[i] = x[i];
  }
  __syncthreads();
  float act[NJ][16];
  int scol[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int c = 16 * (q + LPR * j);
    scol[j] = (int)(c / cols_per_block);
#pragma unroll
    for (int k = 0; k < 16; k += 4) {
      const float4 v = *reinterpret_cast<const float4*>(xs + c + k);
      act[j][k] = v.x;
      act[j][k + 1] = v.y;
      act[j][k + 2] = v.z;
      act[j][k + 3] = v.w;
    }
  }
  // rows < 2^30: 32-bit row arithmetic
  const int n_steps = (R + SLOTS - 1) / SLOTS;
  uint64_t best = 0;  // ARGMAX: the largest key of this lane's rows (0: none)
  for (int s0 = (int)blockIdx.x * U; s0 < n_steps; s0 += (int)gridDim.x * U) {
    uint4 d[U][NJ];
    uint32_t sb[U][NJ];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int r = (s0 + u) * SLOTS + slot;
      r = r < R ? r : R - 1;  // in-bounds load; the result is dropped
      const uint4* wr = reinterpret_cast<const uint4*>(w + (int64_t)r * C);
      const int64_t sr = EXACT ? (int64_t)(((uint64_t)(uint32_t)r * blk_magic) >> blk_shift)
                               : ((int64_t)r * SR) / R;
      const uint8_t* srow = scale + sr * SC;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const u32x4_nt t = stream_load(reinterpret_cast<const u32x4_nt*>(wr + q + LPR * j));
        d[u][j] = make_uint4(t.x, t.y, t.z, t.w);
        sb[u][j] = (SHARE && u > 0) ? sb[0][j] : srow[scol[j]];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float acc = 0.0f;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        float v[16];
        e4m3x4_to_f32(d[u][j].x, v + 0);
        e4m3x4_to_f32(d[u][j].y, v + 4);
        e4m3x4_to_f32(d[u][j].z, v + 8);
        e4m3x4_to_f32(d[u][j].w, v + 12);
        float part = 0.0f;
#pragma unroll
        for (int k = 0; k < 16; ++k) part += v[k] * act[j][k];
        acc += part * e8m0_to_f32(sb[u][j]);
      }
      acc = group_sum<LPR>(acc);
      const int r = (s0 + u) * SLOTS + slot;
      if (q == LPR - 1 && r < R) {
        y[r] = acc;
        if constexpr (ARGMAX) best = max(best, cand_key(acc, (uint32_t)r));
      }
    }
  }
  if constexpr (ARGMAX) {
    // only lanes q == LPR - 1 store rows: the wavefront's largest key is read
    // from those lanes directly (no exchange network at every workgroup's end)
    const uint32_t lo = (uint32_t)best, hi = (uint32_t)(best >> 32);
    uint64_t wbest = 0;
#pragma unroll
    for (int ln = LPR - 1; ln < kWave; ln += LPR)
      wbest = max(wbest, ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(hi, ln) << 32) |
                             (uint32_t)__builtin_amdgcn_readlane(lo, ln));
    if ((tid & (kWave - 1)) == 0) {
      wave_best[tid / kWave] = wbest;
      __threadfence_block();  // the value before the ticket
      if (atomicAdd(&tickets, 1u) == kF8Threads / kWave - 1) {
        __threadfence_block();  // every other wavefront's value after its ticket
        uint64_t m = wave_best[0];
#pragma unroll
        for (int i = 1; i < kF8Threads / kWave; ++i) m = max(m, wave_best[i]);
        slots[blockIdx.x] = m;
      }
    }
  }
}

namespace {

// Measured on the 246272 x 4096 head: 8192 workgroups of 256 threads stream at
// 98% of a plain read kernel's rate; fewer leave HBM queues short.
constexpr int kMaxGrid = 8192;
// the fused argmax's slots per vector: one per workgroup of the widest launch
constexpr int64_t kSlotsPerVector = kMaxGrid;

// The streaming kernel's grid for R rows at LPR lanes per row.
int64_t fast_grid(int64_t R, int lpr) {
  constexpr int U = 2;
  const int64_t slots = kF8Threads / lpr;
  const int64_t n_steps = (R + slots - 1) / slots;
  return std::min<int64_t>((n_steps + U - 1) / U, kMaxGrid);
}

template <int NJ, int LPR, bool ARGMAX>
int launch_f8_fast_a(const uint8_t* w, int64_t R, int64_t C, const uint8_t* scale, int64_t SR,
                     int64_t SC, const float* x, float* y, uint64_t* slots, hipStream_t s) {
  constexpr int U = 2;
  constexpr int SLOTS = kF8Threads / LPR;
  const int64_t grid = fast_grid(R, LPR);
  const int x_vec = is_aligned(x, 16) ? 1 : 0;
  if (R % SR == 0) {
    // rows per scale block d: magic = ceil(2^(31 + l) / d), 2^l >= d > 2^(l - 1)
    const uint64_t d = (uint64_t)(R / SR);
    int l = 0;
    while ((uint64_t(1) << l) < d) ++l;
    const uint64_t magic = ((uint64_t(1) << (31 + l)) + d - 1) / d;  // < 2^32
    if (d % (U * SLOTS) == 0)
      hipLaunchKernelGGL((f8_matvec_fast<NJ, LPR, U, true, true, ARGMAX>), dim3((unsigned)grid),
                         dim3(kF8Threads), 0, s, w, scale, x, y, (int)R, C, SR, SC, C / SC,
                         (uint32_t)magic, 31 + l, x_vec, slots);
    else
      hipLaunchKernelGGL((f8_matvec_fast<NJ, LPR, U, true, false, ARGMAX>), dim3((unsigned)grid),
                         dim3(kF8Threads), 0, s, w, scale, x, y, (int)R, C, SR, SC, C / SC,
                         (uint32_t)magic, 31 + l, x_vec, slots);
  } else {
    hipLaunchKernelGGL((f8_matvec_fast<NJ, LPR, U, false, false, ARGMAX>), dim3((unsigned)grid),
                       dim3(kF8Threads), 0, s, w, scale, x, y, (int)R, C, SR, SC, C / SC, 0u, 0,
                       x_vec, slots);
  }
  return launch_status();
}

template <int NJ, int LPR>
int launch_f8_fast(const uint8_t* w, int64_t R, int64_t C, const uint8_t* scale, int64_t SR,
                   int64_t SC, const float* x, float* y, uint64_t* slots, hipStream_t s) {
  if (slots != nullptr)
    return launch_f8_fast_a<NJ, LPR, true>(w, R, C, scale, SR, SC, x, y, slots, s);
  return launch_f8_fast_a<NJ, LPR, false>(w, R, C, scale, SR, SC, x, y, nullptr, s);
}

int launch_f8_generic(const uint8_t* w, int64_t R, int64_t C, const uint8_t* scale, int64_t SR,
                      int64_t SC, const float* x, float* y, int64_t batch, hipStream_t s) {
  const int64_t waves = kF8Threads / kWave;
  const int64_t grid = std::min<int64_t>((R + waves - 1) / waves, kMaxGrid);
  hipLaunchKernelGGL(f8_matvec_generic, dim3((unsigned)grid), dim3(kF8Threads), 0, s, w, scale, x,
                     y, R, C, SR, SC, batch);
  return launch_status();
}

// The slots of y's argmax where the generic kernel computed y: workgroup g
// takes rows [g chunk, (g + 1) chunk) of every vector.
__global__ __launch_bounds__(kF8Threads) void argmax_slots_from_y(
    const float* __restrict__ y, int64_t R, int64_t batch, int64_t chunk,
    uint64_t* __restrict__ slots) {
  const int64_t r0 = (int64_t)blockIdx.x * chunk, r1 = min(r0 + chunk, R);
  for (int64_t b = 0; b < batch; ++b) {  // workgroup-uniform
    uint64_t k = 0;
    for (int64_t r = r0 + threadIdx.x; r < r1; r += kF8Threads)
      k = max(k, cand_key(y[b * R + r], (uint32_t)r));
    const uint64_t m = block_max_key(k);
    if (threadIdx.x == 0) slots[b * kSlotsPerVector + blockIdx.x] = m;
    __syncthreads();  // block_max_key's LDS is reused by the next vector
  }
}

// The fused argmax's last step: workgroup b takes the largest of vector b's
// n_slots (<= kSlotsPerVector) slot keys, each thread's loads all issued at
// once; token[b] is the row in its low word.
constexpr int kFinishThreads = 1024;
constexpr int kFinishLoads = (int)(kSlotsPerVector / kFinishThreads);
static_assert(kSlotsPerVector == (int64_t)kFinishLoads * kFinishThreads, "whole loads per thread");
__global__ __launch_bounds__(kFinishThreads) void argmax_finish(
    const uint64_t* __restrict__ slots, int64_t n_slots, int32_t* __restrict__ token) {
  const uint64_t* sb = slots + (int64_t)blockIdx.x * kSlotsPerVector;
  uint64_t v[kFinishLoads];
#pragma unroll
  for (int j = 0; j < kFinishLoads; ++j) {  // unconditional loads (a clamped index), then the select
    const int64_t i = j * kFinishThreads + (int64_t)threadIdx.x;
    v[j] = sb[min(i, n_slots - 1)];
    v[j] = i < n_slots ? v[j] : 0;
  }
  uint64_t k = 0;
#pragma unroll
  for (int j = 0; j < kFinishLoads; ++j) k = max(k, v[j]);
  const uint64_t m = block_max_key<kFinishThreads>(k);
  if (threadIdx.x == 0) token[blockIdx.x] = (int32_t)(0xffffffffu - (uint32_t)m);
}

// Lane layout for rows of n_chunk 16-byte chunks, or {0, 0}.
struct F8Shape {
  int lpr, nj;
};

F8Shape f8_shape(int64_t n_chunk) {
  if (n_chunk >= 8 && n_chunk <= 64 && (n_chunk & (n_chunk - 1)) == 0) return {(int)n_chunk, 1};
  if (n_chunk == 128) return {64, 2};
  if (n_chunk == 256) return {64, 4};
  if (n_chunk == 512) return {64, 8};
  return {0, 0};
}

F8Shape f8_fast_shape(const uint8_t* w, int64_t C, int64_t SC, const float* x) {
  const bool fast = C % 16 == 0 && is_aligned(w, 16) && is_aligned(x, 4) && C % SC == 0 &&
                    (C / SC) % 16 == 0;
  return fast ? f8_shape(C / 16) : F8Shape{0, 0};
}

// y; with slots (kMaxGrid per vector), the streaming kernel also leaves each
// workgroup's largest key in them.
int run_f8(const uint8_t* w, int64_t R, int64_t C, const uint8_t* scale, int64_t SR, int64_t SC,
           const float* x, float* y, int64_t batch, F8Shape f, uint64_t* slots, hipStream_t s) {
  if (f.lpr == 0) return launch_f8_generic(w, R, C, scale, SR, SC, x, y, batch, s);
  // One weight pass per activation vector (the workloads here are batch 1).
  for (int64_t b = 0; b < batch; ++b) {
    const float* xb = x + b * C;
    float* yb = y + b * R;
    uint64_t* sb = slots ? slots + b * kSlotsPerVector : nullptr;
    int rc = BQD_EINVAL;
    switch (f.lpr * 16 + f.nj) {
      case 8 * 16 + 1: rc = launch_f8_fast<1, 8>(w, R, C, scale, SR, SC, xb, yb, sb, s); break;
      case 16 * 16 + 1: rc = launch_f8_fast<1, 16>(w, R, C, scale, SR, SC, xb, yb, sb, s); break;
      case 32 * 16 + 1: rc = launch_f8_fast<1, 32>(w, R, C, scale, SR, SC, xb, yb, sb, s); break;
      case 64 * 16 + 1: rc = launch_f8_fast<1, 64>(w, R, C, scale, SR, SC, xb, yb, sb, s); break;
      case 64 * 16 + 2: rc = launch_f8_fast<2, 64>(w, R, C, scale, SR, SC, xb, yb, sb, s); break;
      case 64 * 16 + 4: rc = launch_f8_fast<4, 64>(w, R, C, scale, SR, SC, xb, yb, sb, s); break;
      case 64 * 16 + 8: rc = launch_f8_fast<8, 64>(w, R, C, scale, SR, SC, xb, yb, sb, s); break;
    }
    if (rc) return rc;
  }
  return BQD_OK;
}

}  // namespace

static_assert(kSlotsPerVector == kF8ArgmaxSlots, "one workspace slot per workgroup");

int launch_f8_matvec(const uint8_t* w, int64_t R, int64_t C, const uint8_t* scale, int64_t SR,
                     int64_t SC, const float* x, float* y, int64_t batch, hipStream_t s) {
  return run_f8(w, R, C, scale, SR, SC, x, y, batch, f8_fast_shape(w, C, SC, x), nullptr, s);
}

int launch_f8_matvec_argmax(const uint8_t* w, int64_t R, int64_t C, const uint8_t* scale,
                            int64_t SR, int64_t SC, const float* x, float* y, int64_t batch,
                            void* workspace, int32_t* token, hipStream_t s) {
  uint64_t* slots = static_cast<uint64_t*>(workspace);
  const F8Shape f = f8_fast_shape(w, C, SC, x);
  int rc = run_f8(w, R, C, scale, SR, SC, x, y, batch, f, f.lpr ? slots : nullptr, s);
  if (rc) return rc;
  int64_t n_slots;
  if (f.lpr) {
    n_slots = fast_grid(R, f.lpr);
  } else {
    n_slots = std::min<int64_t>(kMaxGrid, (R + kF8Threads - 1) / kF8Threads);
    const int64_t chunk = (R + n_slots - 1) / n_slots;
    hipLaunchKernelGGL(argmax_slots_from_y, dim3((unsigned)n_slots), dim3(kF8Threads), 0, s, y,
                       R, batch, chunk, slots);
    if ((rc = launch_status())) return rc;
  }
  hipLaunchKernelGGL(argmax_finish, dim3((unsigned)batch), dim3(kFinishThreads), 0, s, slots,
                     n_slots, token);
  return launch_status();
}

// The head's pass with its slots, then top-k / temperature sampling from
// them (one workgroup per vector reads only the rows of the k groups that can
// hold a top-k logit).  The group of each slot is described to the sampler:
// the streaming kernel's workgroup w stores rows w L + t (grid L) + i for
// i < L = U (threads / LPR); the generic path's slot g covers rows
// [g chunk, (g + 1) chunk).
int launch_f8_matvec_sample(const uint8_t* w, int64_t R, int64_t C, const uint8_t* scale,
                            int64_t SR, int64_t SC, const float* x, float* y, int64_t batch,
                            int64_t k, float temperature, uint32_t* state, void* workspace,
                            int32_t* token, int32_t* topk_ids, float* topk_logits,
                            hipStream_t s) {
  uint64_t* slots = static_cast<uint64_t*>(workspace);
  const F8Shape f = f8_fast_shape(w, C, SC, x);
  int rc = run_f8(w, R, C, scale, SR, SC, x, y, batch, f, f.lpr ? slots : nullptr, s);
  if (rc) return rc;
  SlotRowsHost h{};
  h.R = R;
  if (f.lpr) {
    constexpr int64_t U = 2;
    const int64_t per_step = kF8Threads / f.lpr;
    const int64_t n_steps = (R + per_step - 1) / per_step;
    const int64_t grid = fast_grid(R, f.lpr);
    const int64_t L = U * per_step;  // a power of two
    const int64_t runs = (n_steps + grid * U - 1) / (grid * U);
    h.n_slots = h.G = grid;
    h.gstride = L;
    h.log2_L = ilog2(L);
    h.l_valid = L;
    h.S = grid * L;
    h.rows_pg = L * runs;
    h.log2_pg = ceil_log2(h.rows_pg);
  } else {
    const int64_t n_slots = std::min<int64_t>(kMaxGrid, (R + kF8Threads - 1) / kF8Threads);
    const int64_t chunk = (R + n_slots - 1) / n_slots;
    hipLaunchKernelGGL(argmax_slots_from_y, dim3((unsigned)n_slots), dim3(kF8Threads), 0, s, y,
                       R, batch, chunk, slots);
    if ((rc = launch_status())) return rc;
    h.n_slots = h.G = n_slots;
    h.gstride = chunk;
    h.log2_pg = h.log2_L = ceil_log2(chunk);
    h.l_valid = chunk;
    h.S = 0;
    h.rows_pg = chunk;
  }
  return launch_slots_sample(y, slots, h, batch, k, temperature, state, token, topk_ids,
                             topk_logits, s);
}

// ------------------------------------------------------------ decode probes
// Each thread decodes four consecutive codes with the matvec's own routine.
__global__ void f8_decode_probe(const uint8_t* __restrict__ codes, int64_t n,
                                float* __restrict__ out) {
  const int64_t i0 = 4 * ((int64_t)blockIdx.x * blockDim.x + threadIdx.x);
  if (i0 >= n) return;
  uint32_t word = 0;
  for (int k = 0; k < 4; ++k)
    if (i0 + k < n) word |= (uint32_t)codes[i0 + k] << (8 * k);
  float v[4];
  e4m3x4_to_f32(word, v);
  for (int k = 0; k < 4; ++k)
    if (i0 + k < n) out[i0 + k] = v[k];
}

__global__ void e8m0_decode_probe(const uint8_t* __restrict__ codes, int64_t n,
                                  float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = e8m0_to_f32(codes[i]);
}

__global__ void f16_decode_probe(const uint16_t* __restrict__ codes, int64_t n,
                                 float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = f16_to_f32(codes[i]);
}

int launch_f8_decode(const uint8_t* codes, int64_t n, float* out, hipStream_t s) {
  const int64_t threads = (n + 3) / 4;
  hipLaunchKernelGGL(f8_decode_probe, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                     codes, n, out);
  return launch_status();
}

int launch_e8m0_decode(const uint8_t* codes, int64_t n, float* out, hipStream_t s) {
  hipLaunchKernelGGL(e8m0_decode_probe, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, codes,
                     n, out);
  return launch_status();
}

int launch_f16_decode(const uint16_t* codes, int64_t n, float* out, hipStream_t s) {
  hipLaunchKernelGGL(f16_decode_probe, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, codes,
                     n, out);
  return launch_status();
}

}  // namespace bqd

// Top-k and temperature sampling over a logits vector for gfx950.
//
// Method: "attention + tokenizer + sampling: the path to real text (milestone
// 6)" — work item 3 (logits = head x state; top-k / temperature sampling) and
// "Step 3 done" (a deterministic sampler: softmax + xorshift, same seed, same
// token).
//
// Order of candidates: a larger value first; equal values (+0 = -0) by the
// lower index; NaNs after every number.  Every logit becomes one 64-bit key
// whose unsigned order is exactly that order, with no two keys equal:
//   high 32 bits: the float's bits mapped to an unsigned order (NaN lowest),
//   low 32 bits:  0xffffffff - index.
// Sorting keys then orders candidates with no tie handling.  Padding slots
// get small distinct keys (below every real key, whose low half is at least
// 2^32 - 2^20); they are never selected, since k <= n real logits compete.
//
// Two launches.  Blocks of 1024 R logits (R = 1, 2 or 4: the smallest that
// leaves at most 256 blocks, so that the work spreads over many CUs): each
// wavefront sorts R runs of 64 keys across its lanes (a bitonic network on
// lane exchanges, no barriers), merges them into its top 64, and the
// wavefronts' lists merge in LDS down to the block's top 64, of which the
// first k go to the caller's workspace.
//
// One block then selects the first k of the blocks' lists.  Pruning: with H
// the k-th largest of the lists' first keys, at least k keys are >= H, so
// every one of the first k overall is >= H, and in each (descending) list the
// keys >= H are a prefix.  The block reads the first 8 keys of every list,
// keeps those >= H (typically a few per list), sorts and merges them; where a
// list may hold more than 8 such keys, or more than 1024 survive, or there are
// fewer than k lists, it merges every list in full instead.  Either way it
// draws the token in fp64.  Keys carry the index, so the logits are re-read
// for the k values (copied bit for bit).
#include <math.h>

#include "cq_device.h"
#include "launch.h"
#include "validate.h"

namespace bqd {

constexpr int kSampleThreads = 1024;
constexpr int kMaxCandidates = 16384; // second-stage capacity (16 per thread)
constexpr int kPeek = 8;              // keys read per list by the pruned selection
constexpr int kMaxK = 64;

// Unsigned key of a logit: the order of values, NaN below everything, -0 = +0.
__device__ __forceinline__ uint32_t value_key(float v) {
  if (v != v) return 0u;
  uint32_t b = __float_as_uint(v);
  if ((b << 1) == 0u) b = 0u;  // -0 -> +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ uint64_t cand_key(float v, uint32_t index) {
  return ((uint64_t)value_key(v) << 32) | (uint64_t)(0xffffffffu - index);
}

// A 64-bit key of lane (lane ^ D): both halves through the transform's lane
// exchange (DPP within 16-lane rows, ds_bpermute beyond), which moves bits
// unchanged.
template <int D>
__device__ __forceinline__ uint64_t key_xor(uint64_t v) {
  const uint32_t lo = __float_as_uint(lane_xor<D>(__uint_as_float((uint32_t)v)));
  const uint32_t hi = __float_as_uint(lane_xor<D>(__uint_as_float((uint32_t)(v >> 32))));
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t key_from_lane(uint64_t v, int src) {
  const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)v, src, 64);
  const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(v >> 32), src, 64);
  return ((uint64_t)hi << 32) | lo;
}

// One compare-exchange stage across lanes l and l ^ D on R independent keys
// per lane: the lane keeps the larger key if (lower lane) == descending, else
// the smaller (keys are distinct).
template <int D, int R>
__device__ __forceinline__ void cx(uint64_t (&v)[R], bool desc) {
  const bool take_max = ((threadIdx.x & D) == 0) == desc;
  uint64_t o[R];
#pragma unroll
  for (int r = 0; r < R; ++r) o[r] = key_xor<D>(v[r]);
#pragma unroll
  for (int r = 0; r < R; ++r) v[r] = ((v[r] > o[r]) == take_max) ? v[r] : o[r];
}

// Sort R sets of 64 keys of the wavefront (one key per lane and set)
// descending: lane l ends with the l-th largest of each set.
template <int R>
__device__ __forceinline__ void wave_sort_desc(uint64_t (&v)[R]) {
  const int l = threadIdx.x & 63;
#define BQD_SORT_STAGE(SIZE, D) cx<D, R>(v, (SIZE) == 64 || (l & (SIZE)) == 0)
  BQD_SORT_STAGE(2, 1);
  BQD_SORT_STAGE(4, 2); BQD_SORT_STAGE(4, 1);
  BQD_SORT_STAGE(8, 4); BQD_SORT_STAGE(8, 2); BQD_SORT_STAGE(8, 1);
  BQD_SORT_STAGE(16, 8); BQD_SORT_STAGE(16, 4); BQD_SORT_STAGE(16, 2); BQD_SORT_STAGE(16, 1);
  BQD_SORT_STAGE(32, 16); BQD_SORT_STAGE(32, 8); BQD_SORT_STAGE(32, 4); BQD_SORT_STAGE(32, 2);
  BQD_SORT_STAGE(32, 1);
  BQD_SORT_STAGE(64, 32); BQD_SORT_STAGE(64, 16); BQD_SORT_STAGE(64, 8); BQD_SORT_STAGE(64, 4);
  BQD_SORT_STAGE(64, 2); BQD_SORT_STAGE(64, 1);
#undef BQD_SORT_STAGE
}

// The 64 largest of two descending lists, descending: a holds A[l], b_rev
// holds B[63 - l].  max(A[l], B[63 - l]) is a bitonic sequence holding the 64
// largest; a bitonic merge sorts it.
__device__ __forceinline__ uint64_t wave_merge_desc(uint64_t a, uint64_t b_rev) {
  uint64_t v[1] = {a > b_rev ? a : b_rev};
  cx<32, 1>(v, true);
  cx<16, 1>(v, true);
  cx<8, 1>(v, true);
  cx<4, 1>(v, true);
  cx<2, 1>(v, true);
  cx<1, 1>(v, true);
  return v[0];
}

// In-place tree merge of `n_lists` descending lists of 64 keys in LDS (list i
// at lists[64 i ..]) down to list 0.  Every thread of the workgroup calls it.
__device__ void block_merge_lists(uint64_t* lists, int n_lists) {
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
  constexpr int kWaves = kSampleThreads / 64;
  while (n_lists > 1) {
    const int pairs = n_lists >> 1;
    uint64_t merged[(kMaxCandidates / 64 / 2 + kWaves - 1) / kWaves];
    int m = 0;
    __syncthreads();
    for (int pi = wave; pi < pairs; pi += kWaves, ++m)
      merged[m] = wave_merge_desc(lists[64 * (2 * pi) + l], lists[64 * (2 * pi + 1) + 63 - l]);
    __syncthreads();
    m = 0;
    for (int pi = wave; pi < pairs; pi += kWaves, ++m) lists[64 * pi + l] = merged[m];
    if ((n_lists & 1) && wave == 0) lists[64 * pairs + l] = lists[64 * (n_lists - 1) + l];
    n_lists = pairs + (n_lists & 1);
  }
  __syncthreads();
}

// The 64 largest of R sorted runs of the wavefront (R = 1, 2 or 4),
// descending: lane l holds the l-th largest.
template <int R>
__device__ __forceinline__ uint64_t wave_top_of_runs(const uint64_t (&run)[R]) {
  const int l = threadIdx.x & 63;
  if constexpr (R == 1) return run[0];
  if constexpr (R == 2) return wave_merge_desc(run[0], key_from_lane(run[1], 63 - l));
  const uint64_t m01 = wave_merge_desc(run[0], key_from_lane(run[1], 63 - l));
  const uint64_t m23 = wave_merge_desc(run[2], key_from_lane(run[3], 63 - l));
  return wave_merge_desc(m01, key_from_lane(m23, 63 - l));
}

// Stage 1: block b keeps the first k keys of logits [C b, C b + C), C = 1024 R,
// in workspace slots [k b, k b + k).
template <int R>
__global__ __launch_bounds__(kSampleThreads) void topk_chunk_kernel(
    const float* __restrict__ logits, int64_t n, int k, uint64_t* __restrict__ ws) {
  static_assert(R == 1 || R == 2 || R == 4, "runs per wavefront");
  constexpr int kChunk = kSampleThreads * R;
  __shared__ uint64_t lists[kSampleThreads];  // one list of 64 per wavefront
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
  uint64_t run[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {  // run r: chunk elements 64 R wave + 64 r + lane
    const int t = 64 * R * wave + 64 * r + l;
    const int64_t i = (int64_t)blockIdx.x * kChunk + t;
    run[r] = i < n ? cand_key(logits[i], (uint32_t)i) : (uint64_t)(i - n);  // padding < kChunk
  }
  wave_sort_desc<R>(run);
  lists[64 * wave + l] = wave_top_of_runs<R>(run);
  block_merge_lists(lists, kSampleThreads / 64);
  if ((int)threadIdx.x < k) ws[(int64_t)blockIdx.x * k + threadIdx.x] = lists[threadIdx.x];
}

// Stage 2: the blocks' lists (k keys each, padded to 64) merged, the first k
// kept, then the draw.
__global__ __launch_bounds__(kSampleThreads) void topk_final_kernel(
    const float* __restrict__ logits, const uint64_t* __restrict__ ws, int n_lists, int k,
    float temperature, uint32_t* __restrict__ state, int32_t* __restrict__ token,
    int32_t* __restrict__ topk_ids, float* __restrict__ topk_vals) {
  __shared__ uint64_t lists[kMaxCandidates];
  __shared__ float sel_v[kMaxK];
  __shared__ int32_t sel_i[kMaxK];
  __shared__ double weight[kMaxK];
  __shared__ uint64_t thr;
  __shared__ int n_keep, full_merge;
  const int t = threadIdx.x, wave = t >> 6, l = t & 63;
  // The first kPeek keys of list t (all requested together).  A list holds k
  // keys; its padding keys (a short chunk's) are below every real key.
  const bool has = t < n_lists;
  uint64_t pk[kPeek];
#pragma unroll
  for (int q = 0; q < kPeek; ++q) pk[q] = (has && q < k) ? ws[(int64_t)t * k + q] : 0;
  lists[t] = has ? pk[0] : 0;  // the lists' first keys (n_lists <= 256)
  __syncthreads();
  if (wave == 0) {  // H = the k-th largest first key
    uint64_t h[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) h[r] = lists[64 * r + l];
    wave_sort_desc<4>(h);
    const uint64_t top = wave_top_of_runs<4>(h);
    if (l == k - 1) thr = top;
  }
  __syncthreads();
  const uint64_t H = n_lists >= k ? thr : 0;
  int c = 0;  // keys >= H among the first kPeek of list t: a prefix
#pragma unroll
  for (int q = 0; q < kPeek; ++q) c += (has && q < k && pk[q] >= H) ? 1 : 0;
  // exclusive prefix of the counts over the lists (wavefront 0 on 4 per lane)
  __syncthreads();
  lists[t] = (uint64_t)c;
  __syncthreads();
  if (wave == 0) {
    const int c0 = (int)lists[4 * l], c1 = (int)lists[4 * l + 1], c2 = (int)lists[4 * l + 2],
              c3 = (int)lists[4 * l + 3];
    const int s = c0 + c1 + c2 + c3;
    int incl = s;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d, 64);
      if (l >= d) incl += o;
    }
    const int excl = incl - s;
    lists[4 * l] = (uint64_t)excl;
    lists[4 * l + 1] = (uint64_t)(excl + c0);
    lists[4 * l + 2] = (uint64_t)(excl + c0 + c1);
    lists[4 * l + 3] = (uint64_t)(excl + c0 + c1 + c2);
    if (l == 63) n_keep = incl;
    if (l == 0) full_merge = n_lists < k;
  }
  __syncthreads();
  if (c == kPeek && kPeek < k) full_merge = 1;  // list t may hold more keys >= H
  const int off = (int)lists[t];
  __syncthreads();
  if (!full_merge && n_keep <= kSampleThreads) {
    // the survivors in slots [0, n_keep), distinct small keys after them;
    // each wavefront sorts its 64 slots, then the 16 lists merge
    const int kept = n_keep;
    if (t >= kept) lists[t] = (uint64_t)t;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kPeek; ++q)
      if (q < c) lists[off + q] = pk[q];
    __syncthreads();
    uint64_t v[1] = {lists[t]};
    wave_sort_desc<1>(v);
    lists[t] = v[0];
    block_merge_lists(lists, kSampleThreads / 64);
  } else {
    for (int c2 = t; c2 < 64 * n_lists; c2 += kSampleThreads) {
      const int b = c2 >> 6, j = c2 & 63;
      const uint64_t v = j < k ? ws[(int64_t)b * k + j] : 0;
      // padding (a short chunk's, or past k): distinct keys below every real
      // key, decreasing along the list so that each list stays sorted
      lists[c2] = v < (uint64_t)kMaxCandidates ? (uint64_t)(kMaxCandidates - 1 - c2) : v;
    }
    block_merge_lists(lists, n_lists);
  }
  if (t < k) {
    const int32_t i = (int32_t)(0xffffffffu - (uint32_t)lists[t]);
    sel_i[t] = i;
    sel_v[t] = logits[i];
    topk_ids[t] = i;
    topk_vals[t] = sel_v[t];
  }
  __syncthreads();
  const float top = sel_v[0];
  const bool draw = temperature > 0.0f && k > 1 && isfinite(top);
  if (draw && t < k) {  // the softmax weights in fp64, one per lane
    const float v = sel_v[t];
    weight[t] = (v != v) ? 0.0 : exp(((double)v - (double)top) / (double)temperature);
  }
  __syncthreads();
  if (t == 0) {
    // one xorshift step (13, 17, 5), u = state / 2^32, then the inverse of the
    // cumulative softmax: sums in list order, in fp64
    uint32_t s = *state;
    s ^= s << 13;
    s ^= s >> 17;
    s ^= s << 5;
    *state = s;
    int32_t tok = sel_i[0];
    if (draw) {
      double S = 0.0;
      for (int j = 0; j < k; ++j) S += weight[j];
      const double target = ((double)s / 4294967296.0) * S;
      double run = 0.0;
      tok = sel_i[k - 1];
      for (int j = 0; j < k; ++j) {
        run += weight[j];
        if (target < run) {
          tok = sel_i[j];
          break;
        }
      }
    }
    *token = tok;
  }
}

int launch_logits_sample(const float* logits, int64_t n, int64_t k, float temperature,
                         uint32_t* state, void* workspace, int32_t* token, int32_t* topk_ids,
                         float* topk_logits, hipStream_t s) {
  const int64_t chunk = sample_chunk(n);
  const int64_t chunks = (n + chunk - 1) / chunk;
  uint64_t* ws = reinterpret_cast<uint64_t*>(workspace);
  if (chunk == 1024)
    hipLaunchKernelGGL(topk_chunk_kernel<1>, dim3((unsigned)chunks), dim3(kSampleThreads), 0, s,
                       logits, n, (int)k, ws);
  else if (chunk == 2048)
    hipLaunchKernelGGL(topk_chunk_kernel<2>, dim3((unsigned)chunks), dim3(kSampleThreads), 0, s,
                       logits, n, (int)k, ws);
  else
    hipLaunchKernelGGL(topk_chunk_kernel<4>, dim3((unsigned)chunks), dim3(kSampleThreads), 0, s,
                       logits, n, (int)k, ws);
  int rc = launch_status();
  if (rc) return rc;
  hipLaunchKernelGGL(topk_final_kernel, dim3(1), dim3(kSampleThreads), 0, s, logits, ws,
                     (int)chunks, (int)k, temperature, state, token, topk_ids, topk_logits);
  return launch_status();
}

}  // namespace bqd

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
// Two launches.  First, blocks of 1024 R logits (R = 1, 2 or 4: the smallest
// that leaves at most 256 blocks, so that the work spreads over many CUs):
// each wavefront sorts R runs of 64 keys across its lanes (a bitonic network
// on lane exchanges, no barriers), merges them into its top 64, and the
// wavefronts' lists merge in LDS down to the block's top 64, of which the
// first k go to the caller's workspace.  (One launch, with the last block to
// finish selecting, measured slower here: the device-scope release every
// block needs before counting itself done cost ~4 us across 241 blocks, more
// than the kernel boundary.)
//
// Then one block selects the first k of the blocks' lists.  Pruning: with H
// the k-th largest of the lists' first keys, at least k keys are >= H, so
// every one of the first k overall is >= H, and in each (descending) list the
// keys >= H are a prefix.  The block reads the first 8 keys of every list and
// keeps those >= H (typically a few per list).  H itself and, for up to 256
// survivors, their order come from counting: with distinct keys, a key's rank
// is the number of larger ones, each count split over the block's 16
// wavefronts, with no sorting network.  More survivors are sorted and merged;
// where a list may hold more than 8 such keys, or more than 1024 survive, or
// there are fewer than k lists, every list is merged in full instead.  The
// token is drawn in fp64 by one wavefront (one weight per lane, the sums over
// LDS broadcasts).  The k values are rebuilt from the keys (the order map is
// invertible except for the sign of zero and NaN payloads; those few are
// re-read from the logits), so they are copied bit for bit.
//
// The same selection and draw also run fused onto a matvec that leaves one
// slot per workgroup (the largest key of the rows it stored): one launch then
// reads only the rows of the workgroups whose slots can hold a top-k logit
// (slots_sample_kernel below), with the same results.
#include <math.h>

#include <mutex>

#include "cq_device.h"
#include "launch.h"
#include "logit_key.h"
#include "validate.h"

namespace bqd {

constexpr int kSampleThreads = 1024;
constexpr int kMaxCandidates = 16384; // second-stage capacity (16 per thread)
constexpr int kPeek = 8;              // keys read per list by the pruned selection
constexpr int kMaxK = 64;
constexpr int kRankMax = 256;         // survivors ranked by counting (more: sorted)
constexpr int kTopSlot = kSampleThreads;  // LDS slot of the counted top k

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

// Stage 1: the block's top 64 keys of logits [C b, C b + C), C = 1024 R,
// descending in lists[0 .. 64); every thread of the workgroup calls it.
template <int R>
__device__ __forceinline__ void block_top64(const float* __restrict__ logits, int64_t n,
                                            uint64_t* lists) {
  static_assert(R == 1 || R == 2 || R == 4, "runs per wavefront");
  constexpr int kChunk = kSampleThreads * R;
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
}

// The logit a key was made from, bit for bit: the inverse of value_key, or
// a re-read where the key does not determine the bits (zeros, NaNs).
__device__ __forceinline__ float key_logit(uint64_t key, const float* __restrict__ logits) {
  const uint32_t vk = (uint32_t)(key >> 32);
  if (vk == 0u || vk == 0x80000000u) return logits[0xffffffffu - (uint32_t)key];
  return __uint_as_float((vk & 0x80000000u) ? (vk & 0x7fffffffu) : ~vk);
}

// The number of keys among keys[b0, b1) larger than `mine` (b0, b1 even;
// keys 16-byte aligned in LDS, read two at a time, eight reads in flight;
// every lane of a wavefront reads the same address).
__device__ __forceinline__ int count_above(const uint64_t* keys, int b0, int b1, uint64_t mine) {
  const ulonglong2* p = reinterpret_cast<const ulonglong2*>(keys);
  int above = 0, u = b0 / 2;
  const int end = b1 / 2;
  for (; u + 8 <= end; u += 8) {
    ulonglong2 r[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = p[u + j];
#pragma unroll
    for (int j = 0; j < 8; ++j) above += (r[j].x > mine ? 1 : 0) + (r[j].y > mine ? 1 : 0);
  }
  for (; u < end; ++u) {
    const ulonglong2 two = p[u];
    above += (two.x > mine ? 1 : 0) + (two.y > mine ? 1 : 0);
  }
  return above;
}

// Ranks of keys[0, m) (m <= 256, keys distinct, a zero key at keys[m] when m
// is odd) counted by all 1024 threads: thread t counts, for key t % 256, the
// larger keys in quarter t / 256 of the range.  Returns, in thread i < m, the
// rank of keys[i] (the number of larger keys).  Every thread calls it.
__device__ __forceinline__ int block_rank(const uint64_t* keys, int m, int (*part)[256]) {
  const int t = threadIdx.x, i = t & 255, q = t >> 8;
  const int even = (m + 1) & ~1, span = ((m + 7) / 8) * 2;
  const int b0 = q * span, b1 = min(b0 + span, even);
  part[q][i] = (i < m && b0 < b1) ? count_above(keys, b0, b1, keys[i]) : 0;
  __syncthreads();
  return t < m ? part[0][t] + part[1][t] + part[2][t] + part[3][t] : 0;
}

// The draw, by one wavefront alone: lane t holds `key`, candidate t of the
// first k keys (descending; any value on lanes t >= k); the draw stays in
// registers.  Writes the k ids and values, the token and the advanced
// generator state.
__device__ void draw_from_key(uint64_t key, int k, float temperature, uint32_t state_in,
                              const float* __restrict__ logits, uint32_t* __restrict__ state,
                              int32_t* __restrict__ token, int32_t* __restrict__ topk_ids,
                              float* __restrict__ topk_vals) {
  const int t = threadIdx.x & 63;
  key = t < k ? key : 0;
  const int32_t id = (int32_t)(0xffffffffu - (uint32_t)key);
  const float v = t < k ? key_logit(key, logits) : 0.0f;
  if (t < k) {
    topk_ids[t] = id;
    topk_vals[t] = v;
  }
  const float top0 = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(v)));
  const bool draw = temperature > 0.0f && k > 1 && isfinite(top0);
  // one xorshift step (13, 17, 5), u = state / 2^32
  uint32_t s = __builtin_amdgcn_readfirstlane(state_in);
  s ^= s << 13;
  s ^= s >> 17;
  s ^= s << 5;
  int32_t tok = __builtin_amdgcn_readfirstlane(id);
  if (draw) {
    // the softmax weights in fp64, one per lane (NaN values and lanes past k
    // weigh 0); every sum below is formed as one fp64 add on the previous one
    const double w = (t < k && v == v) ? exp(((double)v - (double)top0) / (double)temperature)
                                       : 0.0;
    // S: the weights added in list order, every lane the same chain, reading
    // them back from LDS as broadcasts (the same wavefront's writes, in
    // order), eight requested ahead
    __shared__ double wsh[64];
    wsh[t] = w;
    __builtin_amdgcn_wave_barrier();
    double S = 0.0;
    int j = 0;
    for (; j + 8 <= k; j += 8) {
      double wj[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) wj[q] = wsh[j + q];
#pragma unroll
      for (int q = 0; q < 8; ++q) S += wj[q];
    }
    for (; j < k; ++j) S += wsh[j];  // lanes past k weigh 0: the sum is unchanged
    // the token: the first candidate whose running sum (the same additions
    // again) exceeds u * S, else the last one
    const double target = ((double)s / 4294967296.0) * S;
    double run = 0.0;
    int pick = k - 1;
    for (j = 0; j < k; ++j) {
      run += wsh[j];
      if (__builtin_amdgcn_readfirstlane(run > target ? 1 : 0)) {
        pick = j;
        break;
      }
    }
    tok = __builtin_amdgcn_readlane(id, pick);
  }
  if (t == 0) {
    *state = s;
    *token = tok;
  }
}

// draw_from_key with the keys in LDS: top[0 .. k), descending.
__device__ __forceinline__ void draw_from_top(const uint64_t* top, int k, float temperature,
                                              uint32_t state_in, const float* __restrict__ logits,
                                              uint32_t* __restrict__ state,
                                              int32_t* __restrict__ token,
                                              int32_t* __restrict__ topk_ids,
                                              float* __restrict__ topk_vals) {
  const int t = threadIdx.x & 63;
  draw_from_key(t < k ? top[t] : 0, k, temperature, state_in, logits, state, token, topk_ids,
                topk_vals);
}

// Stage 2 (one block): the blocks' lists (k keys each, padded to 64) merged,
// the first k kept, then the draw.  `lists` is the workgroup's LDS buffer of
// kMaxCandidates keys.
__device__ void select_and_draw(const float* __restrict__ logits, const uint64_t* ws,
                                int n_lists, int k, float temperature,
                                uint32_t* __restrict__ state, int32_t* __restrict__ token,
                                int32_t* __restrict__ topk_ids, float* __restrict__ topk_vals,
                                uint64_t* lists) {
  __shared__ uint64_t thr;
  __shared__ int n_keep, full_merge;
  __shared__ int part[4][256];
  const int t = threadIdx.x, wave = t >> 6, l = t & 63;
  // the generator state, requested first so that its latency overlaps the
  // selection
  const uint32_t state_in = wave == 0 ? *state : 0u;
  // The first kPeek keys of list t (all requested together).  A list holds k
  // keys; its padding keys (a short chunk's) are below every real key.
  const bool has = t < n_lists;
  uint64_t pk[kPeek];
#pragma unroll
  for (int q = 0; q < kPeek; ++q) pk[q] = (has && q < k) ? ws[(int64_t)t * k + q] : 0;
  lists[t] = has ? pk[0] : 0;  // the lists' first keys (n_lists <= 256), zeros after
  __syncthreads();
  // H = the k-th largest first key: the one with exactly k - 1 larger (keys
  // are distinct)
  if (n_lists >= k) {
    const int rank = block_rank(lists, n_lists, part);
    if (has && rank == k - 1) thr = pk[0];
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
  int top_at = 0;  // where the first k keys end up in LDS
  if (!full_merge && n_keep <= kRankMax) {
    // the survivors in slots [0, n_keep) (a zero key after an odd count); each
    // one's rank is the number of larger survivors, and ranks below k are the
    // first k in order
    const int kept = n_keep;
#pragma unroll
    for (int q = 0; q < kPeek; ++q)
      if (q < c) lists[off + q] = pk[q];
    if (t == kept) lists[t] = 0;
    __syncthreads();
    const int rank = block_rank(lists, kept, part);
    if (t < kept && rank < k) lists[kTopSlot + rank] = lists[t];
    __syncthreads();
    top_at = kTopSlot;
  } else if (!full_merge && n_keep <= kSampleThreads) {
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
  if (wave != 0) return;
  draw_from_top(lists + top_at, k, temperature, state_in, logits, state, token, topk_ids,
                topk_vals);
}

// Stage 1: block b keeps the first k keys of its logits in workspace slots
// [k b, k b + k).
template <int R>
__global__ __launch_bounds__(kSampleThreads) void topk_chunk_kernel(
    const float* __restrict__ logits, int64_t n, int k, uint64_t* __restrict__ ws) {
  __shared__ uint64_t lists[kSampleThreads];  // one list of 64 per wavefront
  block_top64<R>(logits, n, lists);
  if ((int)threadIdx.x < k) ws[(int64_t)blockIdx.x * k + threadIdx.x] = lists[threadIdx.x];
}

// Stage 2: one block selects from the n_lists lists and draws.
__global__ __launch_bounds__(kSampleThreads) void topk_select_kernel(
    const float* __restrict__ logits, const uint64_t* __restrict__ ws, int n_lists, int k,
    float temperature, uint32_t* __restrict__ state, int32_t* __restrict__ token,
    int32_t* __restrict__ topk_ids, float* __restrict__ topk_vals) {
  __shared__ uint64_t lists[kMaxCandidates];
  select_and_draw(logits, ws, n_lists, k, temperature, state, token, topk_ids, topk_vals, lists);
}

// ---------------------------------------------------------------------------
// Sampling fused onto a matvec that leaves, per vector, one slot per
// workgroup holding the largest key of the rows that workgroup stored (the
// F8 head's pass; f8.hip).  Workgroup (group) g owns the rows
//   g gstride + t S + i   for t >= 0 and i < L with i < l_valid, below R,
// rows_pg of them at most, and a row r belongs to group (r / gstride) % G.
//
// Why the slots suffice: a logit >= X lies in a group whose slot key is >= X.
// Let H be the k-th largest of 256 maxima of 32 slots each: those k maxima
// are k distinct logits >= H, so the k-th largest logit is >= H, and each of
// the k best logits lies in a group whose slot key is >= H.  One workgroup
// reads only those groups' rows (about k groups of rows_pg rows on the
// head's logits; 32 k groups at most) instead of the whole vector.  Where
// their rows would not fit its LDS, it narrows them first to the k groups of
// the k largest slot keys, T the k-th of them.
struct SlotRows {
  int64_t R;        // rows of a vector
  int n_slots;      // groups (slots) per vector, <= kSlotCapacity
  int G;            // the group of row r is (r / gstride) % G
  int gstride;      // first row of group g: g gstride
  int log2_L;       // rows of a run: L = 2^log2_L, the first l_valid of them real
  int l_valid;
  int64_t S;        // run t starts at g gstride + t S
  int log2_pg;      // 2^log2_pg >= the positions of a group's rows (runs of L)
  int rows_pg;      // positions of a group that are rows: [0, rows_pg)
};
constexpr int kSlotCapacity = 8192;
constexpr int kSlotLoads = kSlotCapacity / kSampleThreads;
// Slots that pass the first bound: 32 k at most (H real: the keys >= H lie in
// the k sets of 32 whose maxima are >= H), or every real slot where fewer
// than k of the 256 sets hold one (then fewer than 256 slots are real).
constexpr int kMaxPass = 32 * kMaxK;

// The first min(k, m) of m distinct keys keys[0 .. m) (m <= kMaxCandidates),
// descending, in LDS; returns where they start.  Up to 256 keys are ranked by
// counting, more are sorted in lists of 64 and merged.  Every thread calls it
// after the keys are written (it begins with a barrier).
__device__ int block_first_k(uint64_t* keys, int m, int k, int (*part)[256]) {
  const int t = threadIdx.x, wave = t >> 6, l = t & 63;
  if (m <= kRankMax) {
    if (t == m && (m & 1)) keys[m] = 0;  // the counting reads keys in pairs
    __syncthreads();
    const int rank = block_rank(keys, m, part);
    if (t < m && rank < k) keys[kTopSlot + rank] = keys[t];
    __syncthreads();
    return kTopSlot;
  }
  const int n_lists = (m + 63) / 64;
  for (int i = m + t; i < 64 * n_lists; i += kSampleThreads) keys[i] = (uint64_t)i;  // below all
  __syncthreads();
  for (int li = wave; li < n_lists; li += kSampleThreads / 64) {
    uint64_t v[1] = {keys[64 * li + l]};
    wave_sort_desc<1>(v);
    keys[64 * li + l] = v[0];
  }
  block_merge_lists(keys, n_lists);
  return 0;
}

// Appends the keys whose pass flag is set to out[] (and idx[] to out_idx[]
// at the same places, if given), at offsets taken from an LDS counter once
// per wavefront (the wavefront's count from ballots, each
// lane's place from the lanes below it): the order of the packed keys
// depends on scheduling, the set does not.
template <int N>
__device__ __forceinline__ void wave_pack(const bool (&pass)[N], const uint64_t (&key)[N],
                                          int* counter, uint64_t* out,
                                          const int* idx = nullptr, int* out_idx = nullptr) {
  uint64_t mask[N];
  int n = 0;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    mask[j] = __ballot(pass[j]);
    n += __popcll(mask[j]);
  }
  if (n == 0) return;  // uniform
  int base = 0;
  if ((threadIdx.x & 63) == 0) base = atomicAdd(counter, n);
  base = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const uint32_t lo = (uint32_t)mask[j], hi = (uint32_t)(mask[j] >> 32);
    const int below = __builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, 0));
    if (pass[j]) {
      out[base + below] = key[j];
      if (idx) out_idx[base + below] = idx[j];
    }
    base += __popcll(mask[j]);
  }
}

// The first k of up to 128 distinct keys keys[0 .. m), ranked by one
// wavefront: a key's rank is the number of larger keys (each lane counts for
// keys l and l + 64, reading every key as a broadcast); the first k go to
// out[rank] and lane l returns out[l] (0 past min(k, m)).  out must not
// overlap keys[0 .. m).
__device__ __forceinline__ uint64_t wave_rank_small(const uint64_t* keys, int m, int k,
                                                    uint64_t* out) {
  const int l = threadIdx.x & 63;
  const uint64_t a = l < m ? keys[l] : 0, b = l + 64 < m ? keys[l + 64] : 0;
  int ra = 0, rb = 0;
  const ulonglong2* p = reinterpret_cast<const ulonglong2*>(keys);
  int u = 0;
  for (; 2 * u + 8 <= m; u += 4) {
    ulonglong2 r[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = p[u + q];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ra += (r[q].x > a) + (r[q].y > a);
      rb += (r[q].x > b) + (r[q].y > b);
    }
  }
  for (int j = 2 * u; j < m; ++j) {
    const uint64_t kj = keys[j];
    ra += kj > a;
    rb += kj > b;
  }
  if (l < m && ra < k) out[ra] = a;
  if (l + 64 < m && rb < k) out[rb] = b;
  __builtin_amdgcn_wave_barrier();
  return l < min(k, m) ? out[l] : 0;
}

// One workgroup per vector b: the k best logits of logits[b][0 .. R) and the
// draw, from the vector's slots (slot keys are >= 2^31; a smaller one marks
// a group with no rows).  Phases: the slots and H (counting over the 256
// maxima); the slots >= H packed by an LDS counter (their order there is
// immaterial: what follows depends only on the keys); the candidates (the
// rows of those groups with keys >= H, or >= T), packed the same way; their
// first k (one wavefront where at most 128 passed, else the workgroup); the
// draw.
__global__ __launch_bounds__(kSampleThreads) void slots_sample_kernel(
    const float* __restrict__ logits, const uint64_t* __restrict__ slots, SlotRows g, int k,
    float temperature, uint32_t* __restrict__ state, int32_t* __restrict__ token,
    int32_t* __restrict__ topk_ids, float* __restrict__ topk_vals) {
  __shared__ __align__(16) uint64_t lists[kMaxCandidates];
  __shared__ int part[4][256];
  __shared__ int grp[kMaxPass];
  __shared__ uint64_t bound, thr;
  __shared__ int n_pass, n_cand;
  const int t = threadIdx.x, wave = t >> 6;
  const int64_t b = blockIdx.x;
  logits += b * g.R;
  slots += b * kSlotCapacity;
  state += b;
  token += b;
  topk_ids += b * k;
  topk_vals += b * k;
  const uint32_t state_in = wave == 0 ? *state : 0u;  // requested first
  constexpr uint64_t kReal = uint64_t(1) << 31;
  if (t == 0) n_pass = n_cand = 0;  // ordered before their atomics by the barriers below

  // the slots, all of a thread's loads issued at once (clamped index, then
  // the select), and each thread's largest real one (t where it has none:
  // distinct, below every real key)
  uint64_t sk[kSlotLoads];
#pragma unroll
  for (int j = 0; j < kSlotLoads; ++j) {
    const int i = j * kSampleThreads + t;
    sk[j] = slots[min(i, g.n_slots - 1)];
    sk[j] = (i < g.n_slots && sk[j] >= kReal) ? sk[j] : 0;
  }
  uint64_t mx = 0;
#pragma unroll
  for (int j = 0; j < kSlotLoads; ++j) mx = max(mx, sk[j]);
  mx = mx ? mx : (uint64_t)t;
  // maxima of 4 threads (32 slots each): 256 distinct keys; H = the k-th
  // largest, found by counting (a key's rank is the number of larger ones)
  mx = max(mx, key_xor<1>(mx));
  mx = max(mx, key_xor<2>(mx));
  if ((t & 3) == 0) lists[t >> 2] = mx;
  __syncthreads();
  if (block_rank(lists, 256, part) == k - 1 && t < 256) bound = lists[t];
  __syncthreads();
  const uint64_t H = bound;
  // the real slots with keys >= H: keys packed into lists[0 .. m), their
  // slot (group) numbers at the same places in grp
  {
    bool pass[kSlotLoads];
    int idx[kSlotLoads];
#pragma unroll
    for (int j = 0; j < kSlotLoads; ++j) {
      pass[j] = sk[j] >= kReal && sk[j] >= H;
      idx[j] = j * kSampleThreads + t;
    }
    wave_pack<kSlotLoads>(pass, sk, &n_pass, lists, idx, grp);
  }
  __syncthreads();
  const int m = n_pass;
  // The groups to read and the threshold.  Where their rows fit, every group
  // that passed, with H: each of the k best logits is >= T >= H and lies in
  // a group whose slot key is >= T.  Otherwise T and the k groups of the k
  // largest slot keys (every group that passed where fewer than k: then
  // they are all the groups with rows, and T = 0 admits every row).
  int n_grp = m;
  if ((m << g.log2_pg) <= kMaxCandidates) {
    if (t == 0) thr = H;
  } else {
    n_grp = min(m, k);
    const int top_at = block_first_k(lists, m, k, part);
    if (t < n_grp) {
      const uint64_t key = lists[top_at + t];
      grp[t] = (int)(0xffffffffu - (uint32_t)key) / g.gstride % g.G;
      if (t == k - 1) thr = key;
    }
    if (t == 0 && m < k) thr = 0;
  }
  __syncthreads();
  const uint64_t T = thr;
  // candidates: the rows of those groups with keys >= T, every load issued
  // before the first compare; positions past the groups' rows are skipped
  // (at most kMaxCandidates positions, 16 per thread)
  const int total = n_grp << g.log2_pg;
  constexpr int kPosLoads = kMaxCandidates / kSampleThreads;
  float v[kPosLoads];
  int rw[kPosLoads];  // the row, or -1 (rows < 2^20)
#pragma unroll
  for (int j = 0; j < kPosLoads; ++j) {
    rw[j] = -1;
    v[j] = 0.0f;
    if (j * kSampleThreads < total) {  // uniform
      const int p = j * kSampleThreads + t;
      const int gi = p >> g.log2_pg, within = p & ((1 << g.log2_pg) - 1);
      const int run = within >> g.log2_L, i = within & ((1 << g.log2_L) - 1);
      const int64_t row = (int64_t)grp[min(gi, kMaxPass - 1)] * g.gstride + run * g.S + i;
      const bool ok = p < total && within < g.rows_pg && i < g.l_valid && row < g.R;
      rw[j] = ok ? (int)row : -1;
      v[j] = logits[ok ? row : 0];
    }
  }
  {
    uint64_t ck[kPosLoads];
    bool pass[kPosLoads];
#pragma unroll
    for (int j = 0; j < kPosLoads; ++j) {
      ck[j] = rw[j] >= 0 ? cand_key(v[j], (uint32_t)rw[j]) : 0;
      pass[j] = rw[j] >= 0 && ck[j] >= T;
    }
    wave_pack<kPosLoads>(pass, ck, &n_cand, lists);
  }
  __syncthreads();
  const int nc = n_cand;
  if (nc <= 128) {
    if (wave != 0) return;
    const uint64_t key = wave_rank_small(lists, nc, k, lists + kTopSlot);
    draw_from_key(key, k, temperature, state_in, logits, state, token, topk_ids, topk_vals);
    return;
  }
  const int at = block_first_k(lists, nc, k, part);
  if (wave != 0) return;
  draw_from_top(lists + at, k, temperature, state_in, logits, state, token, topk_ids, topk_vals);
}

int launch_slots_sample(const float* logits, const uint64_t* slots, const SlotRowsHost& h,
                        int64_t batch, int64_t k, float temperature, uint32_t* state,
                        int32_t* token, int32_t* topk_ids, float* topk_logits, hipStream_t s) {
  if (h.n_slots < 1 || h.n_slots > kSlotCapacity || h.rows_pg < 1 ||
      (int64_t(1) << h.log2_pg) * kMaxK > kMaxCandidates || h.rows_pg > (1 << h.log2_pg) ||
      h.log2_L > h.log2_pg || h.l_valid > (1 << h.log2_L) || h.G < 1 || h.gstride < 1 ||
      k < 1 || k > kMaxK || batch < 1)
    return BQD_EINVAL;  // a layout the kernel cannot take (never for validated calls)
  SlotRows g;
  g.R = h.R;
  g.n_slots = (int)h.n_slots;
  g.G = (int)h.G;
  g.gstride = (int)h.gstride;
  g.log2_L = h.log2_L;
  g.l_valid = (int)h.l_valid;
  g.S = h.S;
  g.log2_pg = h.log2_pg;
  g.rows_pg = (int)h.rows_pg;
  hipLaunchKernelGGL(slots_sample_kernel, dim3((unsigned)batch), dim3(kSampleThreads), 0, s,
                     logits, slots, g, (int)k, temperature, state, token, topk_ids, topk_logits);
  return launch_status();
}

int launch_logits_sample(const float* logits, int64_t n, int64_t k, float temperature,
                         uint32_t* state, void* workspace, int32_t* token, int32_t* topk_ids,
                         float* topk_logits, hipStream_t s) {
  const int64_t chunk = sample_chunk(n);
  const int64_t chunks = (n + chunk - 1) / chunk;
  uint64_t* ws = reinterpret_cast<uint64_t*>(workspace);
  const dim3 grid((unsigned)chunks), block(kSampleThreads);
  if (chunk == 1024)
    hipLaunchKernelGGL(topk_chunk_kernel<1>, grid, block, 0, s, logits, n, (int)k, ws);
  else if (chunk == 2048)
    hipLaunchKernelGGL(topk_chunk_kernel<2>, grid, block, 0, s, logits, n, (int)k, ws);
  else
    hipLaunchKernelGGL(topk_chunk_kernel<4>, grid, block, 0, s, logits, n, (int)k, ws);
  int rc = launch_status();
  if (rc) return rc;
  hipLaunchKernelGGL(topk_select_kernel, dim3(1), block, 0, s, logits, ws, (int)chunks, (int)k,
                     temperature, state, token, topk_ids, topk_logits);
  return launch_status();
}

// ---------------------------------------------------------------------------
// Allocation-free variant.  Its workspace is this file-scope device array,
// sized for the largest call (n = 2^20 logits: 256 blocks of lists of k = 64
// keys): 128 KiB.  Each GPU holds its own copy for the life of the process.
// Nothing in it needs clearing: every first-stage block writes its list
// before the second stage, a later launch on the stream, reads it.  Calls on
// one GPU share the array: calls that overlap in time race.
constexpr int64_t kScratchBytes = (int64_t)256 * kMaxSampleK * (int64_t)sizeof(uint64_t);
static_assert(kMaxSampleLogits / 4096 <= 256, "the largest call has at most 256 blocks");
static __device__ __align__(256) uint64_t scratch[kScratchBytes / sizeof(uint64_t)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void* scratch_ptr[kMaxDevices] = {};
}  // namespace

int64_t sample_scratch_bytes() { return kScratchBytes; }

// The device address of `scratch` on the device that runs stream s (the
// current device for the null stream), looked up once per device with that
// device current (the host-side name of the array is not a device address;
// each GPU holds its own copy).
int sample_scratch(hipStream_t s, void** out) {
  int cur = -1, dev = -1;
  if (hipGetDevice(&cur) != hipSuccess) return BQD_EHIP;
  if (s == nullptr || s == hipStreamPerThread) {
    dev = cur;
  } else if (hipStreamGetDevice(s, &dev) != hipSuccess) {
    return BQD_EHIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return BQD_EHIP;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_ptr[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return BQD_EHIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return BQD_EHIP;
    if (e != hipSuccess || !p) return BQD_EHIP;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return BQD_OK;
}

}  // namespace bqd

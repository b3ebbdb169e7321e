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
// token is drawn in fp64 in one wavefront's registers.  The k values are
// rebuilt from the keys (the order map is invertible except for the sign of
// zero and NaN payloads; those few are re-read from the logits), so they are
// copied bit for bit.
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
  // Wavefront 0: lane t holds candidate t (t < k); the draw stays in registers.
  const uint64_t key = t < k ? lists[top_at + t] : 0;
  const int32_t id = (int32_t)(0xffffffffu - (uint32_t)key);
  const float v = t < k ? key_logit(key, logits) : 0.0f;
  if (t < k) {
    topk_ids[t] = id;
    topk_vals[t] = v;
  }
  const float top = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(v)));
  const bool draw = temperature > 0.0f && k > 1 && isfinite(top);
  // one xorshift step (13, 17, 5), u = state / 2^32
  uint32_t s = __builtin_amdgcn_readfirstlane(state_in);
  s ^= s << 13;
  s ^= s >> 17;
  s ^= s << 5;
  int32_t tok = __builtin_amdgcn_readfirstlane(id);
  if (draw) {
    // the softmax weights in fp64, one per lane (NaN values and lanes past k
    // weigh 0), then the running sums in list order: lane j receives
    // w_0 + ... + w_j, each sum formed as one fp64 add on the previous one
    const double w = (t < k && v == v) ? exp(((double)v - (double)top) / (double)temperature)
                                       : 0.0;
    const uint64_t wb = __builtin_bit_cast(uint64_t, w);
    const uint32_t wlo = (uint32_t)wb, whi = (uint32_t)(wb >> 32);
    double run = 0.0, mine = 0.0;
#pragma unroll
    for (int j = 0; j < 64; ++j) {
      const uint64_t bj = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(whi, j) << 32) |
                          (uint32_t)__builtin_amdgcn_readlane(wlo, j);
      run += __builtin_bit_cast(double, bj);
      if (t == j) mine = run;
    }
    // S = run (the zeros past k leave it unchanged); the token is the first
    // candidate whose running sum exceeds u * S, else the last one
    const double target = ((double)s / 4294967296.0) * run;
    const uint64_t over = __ballot(t < k && target < mine);
    const int pick = over ? __ffsll((unsigned long long)over) - 1 : k - 1;
    tok = __builtin_amdgcn_readlane(id, pick);
  }
  if (t == 0) {
    *state = s;
    *token = tok;
  }
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

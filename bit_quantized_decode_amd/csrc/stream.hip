// A plain read of a device buffer: the achievable-HBM reference that the
// decode kernels' bandwidth is read against.  No method arithmetic; the XOR
// of the words read keeps the loads live and lets a test check every byte
// was read.
//
// Layout: a wavefront step reads 4 KiB contiguous as four nontemporal
// 16-byte loads per lane (each load instruction 1 KiB contiguous); the
// 2048 workgroups of 256 threads loop over the steps, which read 6.6-7.05
// TB/s on a 1 GB buffer on MI355X (more, shorter-lived workgroups read
// 6.0-6.5).  Chunks after the last whole step are read one per thread.
#include <algorithm>

#include "device.h"
#include "launch.h"

namespace bqd {

constexpr int kReadThreads = 256;
constexpr int kReadLoads = 4;  // 16-byte loads in flight per lane
static_assert(BQD_READ_STREAM_WORDS % kReadThreads == 0, "zero-fill loop");

__global__ __launch_bounds__(kReadThreads) void read_stream_kernel(const u32x4_nt* __restrict__ p,
                                                                   int64_t n16,
                                                                   uint32_t* __restrict__ out) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t gtid = (int64_t)blockIdx.x * kReadThreads + threadIdx.x;
  const int64_t n_threads = (int64_t)gridDim.x * kReadThreads;
  const int64_t wave = gtid / kWave, n_waves = n_threads / kWave;
  constexpr int64_t kStep = (int64_t)kWave * kReadLoads;  // chunks per wavefront step
  const int64_t n_steps = n16 / kStep;
  uint32_t acc = 0;
  for (int64_t st = wave; st < n_steps; st += n_waves) {
    const u32x4_nt* q = p + st * kStep + lane;
    u32x4_nt v[kReadLoads];
#pragma unroll
    for (int u = 0; u < kReadLoads; ++u) v[u] = stream_load(q + kWave * u);
#pragma unroll
    for (int u = 0; u < kReadLoads; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (int64_t c = n_steps * kStep + gtid; c < n16; c += n_threads) {
    const u32x4_nt v = stream_load(p + c);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) acc ^= (uint32_t)__shfl_xor((int)acc, d);
  __shared__ uint32_t part[kReadThreads / kWave];
  if (lane == 0) part[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int w = 0; w < kReadThreads / kWave; ++w) r ^= part[w];
    out[blockIdx.x] = r;
  }
  if (blockIdx.x == 0) {
    for (int k = (int)gridDim.x + (int)threadIdx.x; k < BQD_READ_STREAM_WORDS; k += kReadThreads)
      out[k] = 0;
  }
}

int launch_read_stream(const void* buf, int64_t bytes, uint32_t* out, hipStream_t s) {
  const int64_t n16 = bytes / 16;
  const int64_t per_block = (int64_t)kReadThreads * kReadLoads;
  const int64_t blocks = (n16 + per_block - 1) / per_block;
  const int64_t grid = std::max<int64_t>(1, std::min<int64_t>(BQD_READ_STREAM_WORDS, blocks));
  hipLaunchKernelGGL(read_stream_kernel, dim3((unsigned)grid), dim3(kReadThreads), 0, s,
                     static_cast<const u32x4_nt*>(buf), n16, out);
  return launch_status();
}

}  // namespace bqd

// Hadamard MLP for gfx950 ("Inference engine, part 2: kernels and token
// step", §8), from the normalized block input on:
//   z = pad(n, H); z *= d1; normalized FWHT; z = silu(d2 * z);
//   normalized FWHT; z *= d3; out = resid + z[0 .. hidden) (- u).
// Arithmetic as the page's: arrays are Float32Array (every store rounds to
// fp32), products, silu and the 1/sqrt(H) scale are JavaScript numbers (fp64)
// rounded once when stored.  silu(t) = t / (1 + exp(-t)).
#include <algorithm>
#include <cmath>

#include "cq_device.h"
#include "launch.h"

namespace bqd {

namespace {

// (float)((double)v * scale), with the fp32 product when the scale is a
// power of two (then both round the same exact value).
__device__ __forceinline__ float scaled(float v, double scale, bool pow2) {
  return pow2 ? v * (float)scale : (float)((double)v * scale);
}

// Unnormalized transform of the whole H-element vector held E per thread
// (element i = thread * E + e): strides up to 64 E - 1 inside each
// wavefront (registers and lane exchanges), larger strides through LDS, in
// ascending order, with the page's butterflies (a + b, a - b) in fp32.
template <int E>
__device__ void block_fwht(float (&v)[E], int log2_h, float* lds) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  constexpr int span_log2 = 6 + ilog2_c(E);
  wave_fwht<E>(v, lane, log2_h < span_log2 ? log2_h : span_log2);
  for (int sl = span_log2; sl < log2_h; ++sl) {
    const int s = 1 << sl;
#pragma unroll
    for (int e = 0; e < E; ++e) lds[tid * E + e] = v[e];
    __syncthreads();
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = tid * E + e;
      const float o = lds[i ^ s];
      v[e] = (i & s) ? o - v[e] : v[e] + o;  // upper: a - b with a the lower element
    }
    __syncthreads();
  }
}

}  // namespace

// One workgroup per vector; the grid is capped (kMaxStrideGrid) and each
// workgroup loops over the batch.
template <int E>
__global__ __launch_bounds__(1024) void hadamard_mlp_kernel(
    const float* __restrict__ n, int hidden, int log2_h, const float* __restrict__ d1,
    const float* __restrict__ d2, const float* __restrict__ d3, const float* __restrict__ resid,
    const float* __restrict__ u, float* __restrict__ out, double scale, int pow2, int64_t batch) {
  extern __shared__ float lds[];
  const int H = 1 << log2_h;
  const int tid = threadIdx.x;
  for (int64_t b = blockIdx.x; b < batch; b += gridDim.x) {  // workgroup-uniform
    const float* nb = n + b * hidden;
    float v[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = tid * E + e;
      // pad, then z *= d1 (the fp32 product is the rounded fp64 product)
      v[e] = (i < hidden ? nb[i] : 0.0f) * (i < H ? d1[i] : 0.0f);
    }
    block_fwht<E>(v, log2_h, lds);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = tid * E + e;
      const float z = scaled(v[e], scale, pow2);
      const double t = (double)(i < H ? d2[i] : 0.0f) * (double)z;
      v[e] = (float)(t / (1.0 + exp(-t)));
    }
    block_fwht<E>(v, log2_h, lds);
    const float* rb = resid + b * hidden;
    const float* ub = u ? u + b * hidden : nullptr;
    float* ob = out + b * hidden;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = tid * E + e;
      if (i < hidden) {
        const float z = scaled(v[e], scale, pow2) * d3[i];
        const float block = rb[i] + z;
        ob[i] = ub ? block - ub[i] : block;
      }
    }
  }
}

namespace {

template <int E>
int launch_mlp_e(const float* n, int64_t hidden, int64_t H, const float* d1, const float* d2,
                 const float* d3, const float* resid, const float* u, float* out, int64_t batch,
                 hipStream_t s) {
  const int log2_h = ilog2(H);
  const int64_t threads = H > 64 * E ? H / E : 64;  // at least one full wavefront
  const size_t lds = H > 64 * E ? (size_t)H * sizeof(float) : 0;
  const double scale = 1.0 / std::sqrt((double)H);
  const int pow2 = (log2_h % 2) == 0;
  const int64_t grid = std::min<int64_t>(batch, kMaxStrideGrid);
  hipLaunchKernelGGL((hadamard_mlp_kernel<E>), dim3((unsigned)grid), dim3((unsigned)threads), lds,
                     s, n, (int)hidden, log2_h, d1, d2, d3, resid, u, out, scale, pow2, batch);
  return launch_status();
}

}  // namespace

int launch_hadamard_mlp(const float* n, int64_t hidden, int64_t H, const float* d1,
                        const float* d2, const float* d3, const float* resid, const float* u,
                        float* out, int64_t batch, hipStream_t s) {
  // One element per thread up to 1024 (the fp64 silu of each element is the
  // longest chain, so the widest workgroup finishes first), then H / 1024.
  switch (H <= 1024 ? 1 : (int)(H / 1024)) {
    case 1: return launch_mlp_e<1>(n, hidden, H, d1, d2, d3, resid, u, out, batch, s);
    case 2: return launch_mlp_e<2>(n, hidden, H, d1, d2, d3, resid, u, out, batch, s);
    case 4: return launch_mlp_e<4>(n, hidden, H, d1, d2, d3, resid, u, out, batch, s);
    case 8: return launch_mlp_e<8>(n, hidden, H, d1, d2, d3, resid, u, out, batch, s);
    case 16: return launch_mlp_e<16>(n, hidden, H, d1, d2, d3, resid, u, out, batch, s);
  }
  return BQD_EINVAL;  // unreachable: H <= 16384 is validated
}

}  // namespace bqd

// Int8 weight paths for gfx950: the I8 matvec with E8M0 group scales, and the
// int8 key cache (per-vector quantization and the scaled key dot).
//
// Methods:
//  - "attention + tokenizer + sampling: the path to real text (milestone 6)",
//    Step 4: the I8 matvec widens int8 weights and applies one E8M0 scale per
//    group of 16 consecutive columns of a row (here any group of G columns;
//    the fast path takes G a multiple of 16).
//  - "Inference engine, part 2: kernels and token step", §7: storeInt8 (the
//    largest magnitude, floored at 1e-12, over 127 is the vector's scale;
//    every element over the scale, rounded half to even, is its code), and
//    the key dot, which multiplies the cached integers by the row's scale.
#include <algorithm>

#include "device.h"
#include "launch.h"

namespace bqd {

constexpr int kI8Threads = 256;

// Sixteen int8 weights (a 16-byte chunk) dotted with sixteen activations.
// Each byte converts with one sign-extending byte select (exact).
__device__ __forceinline__ float i8_chunk_dot(const uint4& d, const float (&a)[16]) {
  const uint32_t w[4] = {d.x, d.y, d.z, d.w};
  float p = 0.0f;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int b = 0; b < 4; ++b) p += (float)(int8_t)(w[t] >> (8 * b)) * a[4 * t + b];
  return p;
}

// ----------------------------------------------------------- generic matvec
// Any shape and alignment: one wavefront per row, lanes stride over columns.
// ROWSCALE: one fp32 scale per row (the key dot); else E8M0 per G columns.
template <bool ROWSCALE>
__global__ __launch_bounds__(kI8Threads) void i8_matvec_generic(
    const int8_t* __restrict__ w, const uint8_t* __restrict__ gscale,
    const float* __restrict__ rscale, const float* __restrict__ x, float* __restrict__ y,
    int64_t R, int64_t C, int64_t G, int64_t batch) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int64_t ns = ROWSCALE ? 0 : (C + G - 1) / G;
  for (int64_t r = (int64_t)blockIdx.x * (kI8Threads / kWave) + wave; r < R;
       r += (int64_t)gridDim.x * (kI8Threads / kWave)) {
    const int8_t* wr = w + r * C;
    for (int64_t b = 0; b < batch; ++b) {
      const float* xb = x + b * C;
      float acc = 0.0f;
      for (int64_t c = lane; c < C; c += kWave) {
        const float s = ROWSCALE ? 1.0f : e8m0_to_f32(gscale[r * ns + c / G]);
        acc += ((float)wr[c] * s) * xb[c];
      }
      acc = group_sum<kWave>(acc);
      if (ROWSCALE) acc *= rscale[r];
      if (lane == kWave - 1) y[b * R + r] = acc;
    }
  }
}

// -------------------------------------------------------------- fast matvec
// Rows of C = 16 * n_chunk bytes, 16-byte aligned; LPR lanes share a row and
// lane q owns chunks q + LPR*j, so each load instruction of a wavefront reads
// LPR * 16 contiguous bytes.  Each 16-column chunk lies inside one scale
// group (G a multiple of 16): its partial dot is multiplied by the group's
// power-of-two scale (exact).  The row then reduces across lanes with DPP
// and, for ROWSCALE, is multiplied by the row's fp32 scale.
// Where NJ <= 4 (and no row scale, which would spill) the kernel keeps to
// 128 registers, 4 wavefronts per SIMD, as the F8 kernel does.
template <int NJ, int LPR, int U, bool ROWSCALE>
__global__ __launch_bounds__(kI8Threads)
__attribute__((amdgpu_waves_per_eu(NJ <= 4 && !ROWSCALE ? 4 : 1))) void i8_matvec_fast(
    const int8_t* __restrict__ w, const uint8_t* __restrict__ gscale,
    const float* __restrict__ rscale, const float* __restrict__ x, float* __restrict__ y,
    int64_t R, int64_t C, int64_t G, int x_vec) {
  constexpr int SLOTS = kI8Threads / LPR;
  constexpr int CX = 16 * LPR * NJ;  // = C
  __shared__ __align__(16) float xs[CX];
  const int tid = threadIdx.x;
  const int slot = tid / LPR;
  const int q = tid % LPR;
  const int64_t ns = ROWSCALE ? 0 : (C + G - 1) / G;
  // x staged in LDS once per workgroup (float4 loads where it is 16-byte
  // aligned), then each lane's activations read from there
  if (x_vec) {
    for (int i = tid; i < CX / 4; i += kI8Threads)
      reinterpret_cast<float4*>(xs)[i] = reinterpret_cast<const float4*>(x)[i];
  } else {
    for (int i = tid; i < CX; i += kI8Threads) xs[i] = x[i];
  }
  __syncthreads();
  float act[NJ][16];
  int64_t scol[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int c = 16 * (q + LPR * j);
    scol[j] = ROWSCALE ? 0 : c / G;
#pragma unroll
    for (int k = 0; k < 16; k += 4) {
      const float4 v = *reinterpret_cast<const float4*>(xs + c + k);
      act[j][k] = v.x;
      act[j][k + 1] = v.y;
      act[j][k + 2] = v.z;
      act[j][k + 3] = v.w;
    }
  }
  const int64_t n_steps = (R + SLOTS - 1) / SLOTS;
  for (int64_t s0 = (int64_t)blockIdx.x * U; s0 < n_steps; s0 += (int64_t)gridDim.x * U) {
    uint4 d[U][NJ];
    uint32_t sb[U][NJ];
    float rs[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int64_t r = (s0 + u) * SLOTS + slot;
      r = r < R ? r : R - 1;  // in-bounds load; the result is dropped
      const uint4* wr = reinterpret_cast<const uint4*>(w + r * C);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const u32x4_nt t = stream_load(reinterpret_cast<const u32x4_nt*>(wr + q + LPR * j));
        d[u][j] = make_uint4(t.x, t.y, t.z, t.w);
        if (!ROWSCALE) sb[u][j] = gscale[r * ns + scol[j]];
      }
      rs[u] = ROWSCALE ? rscale[r] : 1.0f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float acc = 0.0f;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const float part = i8_chunk_dot(d[u][j], act[j]);
        acc += ROWSCALE ? part : part * e8m0_to_f32(sb[u][j]);
      }
      acc = group_sum<LPR>(acc);
      if (ROWSCALE) acc *= rs[u];
      const int64_t r = (s0 + u) * SLOTS + slot;
      if (q == LPR - 1 && r < R) y[r] = acc;
    }
  }
}

namespace {

constexpr int kI8MaxGrid = 8192;

template <int NJ, int LPR, bool ROWSCALE>
int launch_i8_fast(const int8_t* w, int64_t R, int64_t C, const uint8_t* gscale, int64_t G,
                   const float* rscale, const float* x, float* y, hipStream_t s) {
  constexpr int U = 2;
  constexpr int SLOTS = kI8Threads / LPR;
  const int64_t n_steps = (R + SLOTS - 1) / SLOTS;
  const int64_t grid = std::min<int64_t>((n_steps + U - 1) / U, kI8MaxGrid);
  hipLaunchKernelGGL((i8_matvec_fast<NJ, LPR, U, ROWSCALE>), dim3((unsigned)grid),
                     dim3(kI8Threads), 0, s, w, gscale, rscale, x, y, R, C, G,
                     is_aligned(x, 16) ? 1 : 0);
  return launch_status();
}

// Lane layout for rows of n_chunk 16-byte chunks (as the F8 head's), or 0.
int i8_layout(int64_t n_chunk) {
  if (n_chunk >= 1 && n_chunk <= 64 && (n_chunk & (n_chunk - 1)) == 0)
    return (int)(n_chunk * 16 + 1);
  if (n_chunk == 128) return 64 * 16 + 2;
  if (n_chunk == 256) return 64 * 16 + 4;
  if (n_chunk == 512) return 64 * 16 + 8;
  return 0;
}

template <bool ROWSCALE>
int launch_i8(const int8_t* w, int64_t R, int64_t C, const uint8_t* gscale, int64_t G,
              const float* rscale, const float* x, float* y, int64_t batch, hipStream_t s) {
  const bool fast = C % 16 == 0 && is_aligned(w, 16) && (ROWSCALE || G % 16 == 0);
  const int lay = fast ? i8_layout(C / 16) : 0;
  if (lay == 0) {
    const int64_t waves = kI8Threads / kWave;
    const int64_t grid = std::min<int64_t>((R + waves - 1) / waves, kI8MaxGrid);
    hipLaunchKernelGGL(i8_matvec_generic<ROWSCALE>, dim3((unsigned)grid), dim3(kI8Threads), 0, s,
                       w, gscale, rscale, x, y, R, C, G, batch);
    return launch_status();
  }
  for (int64_t b = 0; b < batch; ++b) {
    const float* xb = x + b * C;
    float* yb = y + b * R;
    int rc = BQD_EINVAL;
    switch (lay) {
#define I8_CASE(LPR, NJ)                                                                          \
  case LPR * 16 + NJ:                                                                             \
    rc = launch_i8_fast<NJ, LPR, ROWSCALE>(w, R, C, gscale, G, rscale, xb, yb, s);                \
    break;
      I8_CASE(1, 1) I8_CASE(2, 1) I8_CASE(4, 1) I8_CASE(8, 1) I8_CASE(16, 1) I8_CASE(32, 1)
      I8_CASE(64, 1) I8_CASE(64, 2) I8_CASE(64, 4) I8_CASE(64, 8)
#undef I8_CASE
    }
    if (rc) return rc;
  }
  return BQD_OK;
}

}  // namespace

int launch_i8_matvec(const int8_t* w, int64_t R, int64_t C, const uint8_t* scale, int64_t G,
                     const float* x, float* y, int64_t batch, hipStream_t s) {
  return launch_i8<false>(w, R, C, scale, G, nullptr, x, y, batch, s);
}

int launch_kv_int8_dot(const int8_t* K, const float* scales, int64_t R, int64_t d, const float* x,
                       float* y, int64_t batch, hipStream_t s) {
  return launch_i8<true>(K, R, d, nullptr, 1, scales, x, y, batch, s);
}

// ------------------------------------------------------ storeInt8, per vector
// One wavefront per vector of d floats.  The largest magnitude is exact in
// fp32 (a NaN anywhere makes it NaN, as JavaScript's Math.max does); the
// scale max(1e-12, maximum) / 127 and every quotient are formed in fp64 and
// the quotient rounds half to even, so the codes are the page's bit for bit.
// A NaN quotient stores 0 (the Int8Array conversion); finite quotients lie
// in [-127, 127].
__global__ __launch_bounds__(kI8Threads) void kv_quantize_int8_kernel(
    const float* __restrict__ v, int64_t n_vec, int64_t d, int8_t* __restrict__ q,
    float* __restrict__ scales) {
  // one wavefront per vector, the grid capped and looping over the vectors
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t stride = (int64_t)gridDim.x * (kI8Threads / kWave);
  for (int64_t i = (int64_t)blockIdx.x * (kI8Threads / kWave) + threadIdx.x / kWave; i < n_vec;
       i += stride) {  // wavefront-uniform
    const float* vi = v + i * d;
    float m = 0.0f;
    int nan = 0;
    for (int64_t j = lane; j < d; j += kWave) {
      const float a = fabsf(vi[j]);
      nan |= a != a;
      m = fmaxf(m, a);
    }
    // wavefront max: every lane ends with the maximum (DPP within rows, then
    // the row maxima through the lane swaps)
    m = fmaxf(m, dpp<kQuadXor1, 0xf, false>(0.0f, m));
    m = fmaxf(m, dpp<kQuadXor2, 0xf, false>(0.0f, m));
    m = fmaxf(m, dpp<kRowHalfMirror, 0xf, false>(0.0f, m));
    m = fmaxf(m, dpp<kRowMirror, 0xf, false>(0.0f, m));
    {
      const uint32_t u = __float_as_uint(m);
      const auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
      m = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
      const uint32_t u2 = __float_as_uint(m);
      const auto r32 = __builtin_amdgcn_permlane32_swap(u2, u2, false, false);
      m = fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
    }
    const bool any_nan = __any(nan);
    double maximum = fmax(1e-12, (double)m);
    if (any_nan) maximum = __longlong_as_double(0x7ff8000000000000ll);
    const double scale = maximum / 127.0;
    if (lane == 0) scales[i] = (float)scale;
    int8_t* qi = q + i * d;
    for (int64_t j = lane; j < d; j += kWave) {
      const double t = rint((double)vi[j] / scale);
      qi[j] = (t == t && t >= -128.0 && t <= 127.0) ? (int8_t)(int)t : (int8_t)0;
    }
  }
}

int launch_kv_quantize_int8(const float* v, int64_t n_vec, int64_t d, int8_t* q, float* scales,
                            hipStream_t s) {
  const int64_t waves = kI8Threads / kWave;
  const int64_t grid = std::min<int64_t>((n_vec + waves - 1) / waves, kMaxStrideGrid);
  hipLaunchKernelGGL(kv_quantize_int8_kernel, dim3((unsigned)grid), dim3(kI8Threads), 0, s, v,
                     n_vec, d, q, scales);
  return launch_status();
}

}  // namespace bqd

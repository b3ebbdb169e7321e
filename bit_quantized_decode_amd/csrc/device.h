// Device-side building blocks shared by the gfx950 kernels: value decoders,
// DPP lane exchanges and wavefront reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace bqd {

constexpr int kWave = 64;

// A load of streamed weight data, marked nontemporal: every weight byte is
// read once per launch, and on gfx950 such loads keep the HBM stream at a
// measurably higher rate than ordinary loads (6.6 vs 5.9 TB/s on the 1 GB F8
// head).
template <typename T>
__device__ __forceinline__ T stream_load(const T* p) {
  return __builtin_nontemporal_load(p);
}
typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));

// fp16 bit pattern -> fp32 (hardware conversion; exact for every non-NaN
// code, subnormals included).  Norms are fp16 per (row, group) in the CQ
// record ("Inference engine, part 1", §3 and §4).
__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return __half2float(__ushort_as_half(h));
}

// E8M0 block scale -> 2^(e-127) as an fp32 bit pattern; e = 0 is the fp32
// subnormal 2^-127, e = 255 is NaN ("attention + tokenizer + sampling",
// Step 1: E8M0 block scales).
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
  uint32_t bits = e ? (e << 23) : 0x00400000u;
  bits = (e == 255u) ? 0x7fc00000u : bits;
  return __uint_as_float(bits);
}

// E4M3 with the clamp of "attention + tokenizer + sampling" Step 1: the only
// codes whose value the clamp changes are 0x7F / 0xFF (480 -> 448), which the
// OCP E4M3FN hardware conversion reads as NaN.  Rewriting those bytes to
// 0x7E / 0xFE (exactly +-448) before conversion gives the clamped decode for
// all 256 codes.  SWAR on four bytes: a byte b has (b & 0x7F) + 1 >= 0x80 iff
// its low seven bits are all ones; subtracting 1 from such a byte never
// borrows because it is odd.
__device__ __forceinline__ uint32_t e4m3_clamp_bytes(uint32_t w) {
  uint32_t t = (w & 0x7f7f7f7fu) + 0x01010101u;
  return w - ((t & 0x80808080u) >> 7);
}

typedef float float2_v __attribute__((ext_vector_type(2)));

// Four E4M3 codes (little-endian bytes of w) -> four fp32 values.
__device__ __forceinline__ void e4m3x4_to_f32(uint32_t w, float out[4]) {
  uint32_t c = e4m3_clamp_bytes(w);
  float2_v lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)c, false);
  float2_v hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)c, true);
  out[0] = lo[0];
  out[1] = lo[1];
  out[2] = hi[0];
  out[3] = hi[1];
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) {
  float v[4];
  e4m3x4_to_f32(byte & 0xffu, v);
  return v[0];
}

// ---------------------------------------------------------------------------
// DPP lane exchanges (gfx9 encodings).  `old` is returned in rows that the
// row mask disables.
template <int CTRL, int ROW_MASK, bool BOUND_CTRL>
__device__ __forceinline__ float dpp(float old, float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v),
                                                    CTRL, ROW_MASK, 0xf, BOUND_CTRL));
}
constexpr int kQuadXor1 = 0xb1;        // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4e;        // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;  // lane i <-> 7-i within 8 lanes
constexpr int kRowMirror = 0x140;      // lane i <-> 15-i within 16 lanes
constexpr int kRowBcast15 = 0x142;     // lane 15 of a row -> the next row
constexpr int kRowBcast31 = 0x143;     // lane 31 -> rows 2 and 3
// row_ror:n rotates a 16-lane row right: lane i receives lane (i - n) mod 16
constexpr int kRowRor4 = 0x124;        // lane i <- lane (i - 4) % 16 = (i + 12) % 16
constexpr int kRowRor8 = 0x128;        // lane i <- lane (i + 8) % 16
constexpr int kRowRor12 = 0x12c;       // lane i <- lane (i + 4) % 16

// Transposed (multi-row) reductions.  Each lane holds partial sums of several
// rows; one exchange step halves the rows a lane holds and doubles the lanes
// each sum covers, so a wavefront reduces n rows in about n exchanges instead
// of 6n.  The gfx950 lane-swap instructions do the two cross-row steps in one
// instruction each:
//  swap_add32(a, b): lanes 0-31 receive a(l) + a(l + 32), lanes 32-63 receive
//    b(l - 32) + b(l) (v_permlane32_swap: the upper half of a trades places
//    with the lower half of b);
//  swap_add16(a, b): in 16-lane rows 0 and 2, a(l) + a(l + 16); in rows 1 and
//    3, b(l - 16) + b(l) (v_permlane16_swap: odd rows of a with even rows of b).
__device__ __forceinline__ float swap_add32(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap_add16(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum over aligned groups of N lanes (N a power of two, <= 64).  After the
// call the group's last lane (lane % N == N - 1) holds the group total; the
// summation order is fixed, so results are reproducible.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2) v += dpp<kQuadXor1, 0xf, true>(0.0f, v);
  if constexpr (N >= 4) v += dpp<kQuadXor2, 0xf, true>(0.0f, v);
  if constexpr (N >= 8) v += dpp<kRowHalfMirror, 0xf, true>(0.0f, v);
  if constexpr (N >= 16) v += dpp<kRowMirror, 0xf, true>(0.0f, v);
  if constexpr (N >= 32) v += dpp<kRowBcast15, 0xa, false>(0.0f, v);
  if constexpr (N >= 64) v += dpp<kRowBcast31, 0xc, false>(0.0f, v);
  return v;
}

}  // namespace bqd

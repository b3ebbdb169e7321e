// Device-side building blocks of the gfx950 kernels: value decoders and
// wavefront reductions.  Used by the matvec, gather and probe kernels only.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace bqd {

constexpr int kWave = 64;

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
// Codebook index decode.  A 32-column chunk of a row occupies exactly BITS
// dwords (4*BITS bytes) of the little-endian bit stream; index k sits at bit
// BITS*k.  Indices that straddle two dwords are funnel-shifted out.
template <int BITS>
__device__ __forceinline__ uint32_t chunk_index(const uint32_t (&d)[BITS], int k) {
  const int bit = BITS * k;
  const int w = bit >> 5;
  const int sh = bit & 31;
  uint32_t v;
  if (sh + BITS <= 32) {
    v = d[w] >> sh;
  } else {
    v = __builtin_amdgcn_alignbit(d[w + 1], d[w], sh);
  }
  return v & ((1u << BITS) - 1u);
}

// Byte addresses (index * 4) of the 32 indices of a chunk, for an fp32 table
// in LDS.  2- and 4-bit fields never straddle a byte: one shift and one mask
// per dword and field position leave four addresses in the four bytes of a
// register, and each is then one byte extract (1.5 VALU ops per index for
// 4-bit, 1.25 for 2-bit; SDWA byte selects issue at a lower rate on gfx950).
// 3- and 5-bit fields are funnel-shifted out of the dwords (two ops each).
__device__ __forceinline__ void byte_addresses(uint32_t packed4, uint32_t* a) {
  a[0] = packed4 & 0xffu;
  a[1] = __builtin_amdgcn_ubfe(packed4, 8, 8);
  a[2] = __builtin_amdgcn_ubfe(packed4, 16, 8);
  a[3] = packed4 >> 24;
}

template <int BITS>
__device__ __forceinline__ void chunk_addresses(const uint32_t (&d)[BITS], uint32_t (&a)[32]) {
  if constexpr (BITS == 4) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t lo[4], hi[4];
      byte_addresses((d[w] << 2) & 0x3c3c3c3cu, lo);  // even columns (low nibbles)
      byte_addresses((d[w] >> 2) & 0x3c3c3c3cu, hi);  // odd columns (high nibbles)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        a[8 * w + 2 * m] = lo[m];
        a[8 * w + 2 * m + 1] = hi[m];
      }
    }
  } else if constexpr (BITS == 2) {
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      uint32_t c[4][4];
      byte_addresses((d[w] << 2) & 0x0c0c0c0cu, c[0]);  // crumb 0 of each byte
      byte_addresses(d[w] & 0x0c0c0c0cu, c[1]);         // crumb 1
      byte_addresses((d[w] >> 2) & 0x0c0c0c0cu, c[2]);  // crumb 2
      byte_addresses((d[w] >> 4) & 0x0c0c0c0cu, c[3]);  // crumb 3
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int k = 0; k < 4; ++k) a[16 * w + 4 * m + k] = c[k][m];
    }
  } else {
#pragma unroll
    for (int k = 0; k < 32; ++k) a[k] = chunk_index<BITS>(d, k) << 2;
  }
}

// An fp32 table entry at a byte address in LDS.
__device__ __forceinline__ float lds_at(const float* table, uint32_t byte_addr) {
  return *reinterpret_cast<const float*>(reinterpret_cast<const char*>(table) + byte_addr);
}

// Generic single-index decode from a byte row of any alignment: the index
// spans at most two bytes for BITS <= 5.  The second byte is read only when
// the index reaches into it, so no read passes the row's last needed byte.
__device__ __forceinline__ uint32_t byte_index(const uint8_t* row, int bits, int64_t col) {
  const int64_t t = (int64_t)bits * col;
  const int64_t byte = t >> 3;
  const int sh = (int)(t & 7);
  uint32_t v = row[byte];
  if (sh + bits > 8) v |= (uint32_t)row[byte + 1] << 8;
  return (v >> sh) & ((1u << bits) - 1u);
}

// ---------------------------------------------------------------------------
// Unnormalized Walsh–Hadamard transform of the groups held by one wavefront
// ("Inference engine, part 2", §1).  Lane l holds E consecutive elements
// (l*E .. l*E+E-1) of a 64*E span; groups of 2^log2_group elements are aligned
// inside the span.  Strides ascend 1, 2, 4, ...: strides below E pair elements
// inside a lane, larger ones pair lane l with lane l ^ (stride / E).  Every
// pair (a at the lower index, b at the upper) becomes (a + b, a - b) in fp32,
// the scalar loop's exact operations and order, so results are bit-identical.
template <int E>
__device__ __forceinline__ void wave_fwht(float (&v)[E], int lane, int log2_group) {
  const int g = 1 << log2_group;
#pragma unroll
  for (int s = 1; s < E; s <<= 1) {
    if (s < g) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if ((e & s) == 0) {
          const float a = v[e], b = v[e + s];
          v[e] = a + b;
          v[e + s] = a - b;
        }
      }
    }
  }
  for (int d = 1; E * d < g; d <<= 1) {
    const bool upper = (lane & d) != 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float o = __shfl_xor(v[e], d, kWave);
      v[e] = upper ? o - v[e] : v[e] + o;
    }
  }
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

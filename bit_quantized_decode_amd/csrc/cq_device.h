// Device-side helpers of the CQ kernels (prepare, matvec, gather): codebook
// index decode and the wavefront Walsh–Hadamard transform.
#pragma once
#include "device.h"

namespace bqd {

// log2 of a power of two, at compile time.
constexpr int ilog2_c(int v) { return v <= 1 ? 0 : 1 + ilog2_c(v / 2); }

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
// The values of lanes l and l ^ D (D = 16 or 32), lower lane first: one
// gfx950 lane-swap instruction on two copies of v hands every lane both
// members of its pair (v_permlane16_swap trades 16-lane rows 1 and 3 of its
// first operand for rows 0 and 2 of its second; v_permlane32_swap trades
// the upper half of the first for the lower half of the second), with no
// LDS round trip.  .x is the value of the lane whose bit D is clear.
template <int D>
__device__ __forceinline__ float2 lane_pair(float v) {
  static_assert(D == 16 || D == 32, "lane swaps cross 16-lane rows or wavefront halves");
  const uint32_t u = __float_as_uint(v);
  if constexpr (D == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
}

// Value of lane (lane ^ D) of the wavefront.  D < 16 stays inside a 16-lane
// DPP row: xor 1 and 2 are quad permutes, xor 8 is a rotation by 8, and xor 4
// reads lane i + 4 (a right rotation by 12) in lanes with bit 2 clear and lane
// i - 4 (a right rotation by 4, written to DPP banks 1 and 3 only) in the
// others.  D = 16 and 32 take the lane swaps of lane_pair.
template <int D>
__device__ __forceinline__ float lane_xor(float v) {
  if constexpr (D == 1) {
    return dpp<kQuadXor1, 0xf, false>(0.0f, v);
  } else if constexpr (D == 2) {
    return dpp<kQuadXor2, 0xf, false>(0.0f, v);
  } else if constexpr (D == 4) {
    const float up = dpp<kRowRor12, 0xf, false>(0.0f, v);  // lane i + 4
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(up), __float_as_int(v),
                                                      kRowRor4, 0xf, 0xa, false));
  } else if constexpr (D == 8) {
    return dpp<kRowRor8, 0xf, false>(0.0f, v);
  } else {
    const float2 p = lane_pair<D>(v);
    return (__lane_id() & D) ? p.x : p.y;
  }
}

// One butterfly stage across lanes l and l ^ D: the lower lane keeps a + b,
// the upper one a - b, where a is the lower lane's value.  Both are one fused
// multiply-add with a per-lane sign: fma(x, +-1, y) forms x * (+-1) exactly
// and rounds the sum once, so it is the fp32 a + b (lower lane: x = a, y = b)
// or a - b (upper lane: x = b, y = a) bit for bit, signed zeros and
// infinities included.
template <int E, int D>
__device__ __forceinline__ void lane_stage(float (&v)[E], int lane) {
  const float sign = (lane & D) ? -1.0f : 1.0f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if constexpr (D >= 16) {
      const float2 p = lane_pair<D>(v[e]);  // (a, b): the lower and the upper element
      v[e] = __builtin_fmaf(p.y, sign, p.x);
    } else {
      const float o = lane_xor<D>(v[e]);
      v[e] = __builtin_fmaf(v[e], sign, o);
    }
  }
}

// ---------------------------------------------------------------------------
// Unnormalized Walsh–Hadamard transform of the groups held by one wavefront
// ("Inference engine, part 2", §1).  Lane l holds E consecutive elements
// (l*E .. l*E+E-1) of a 64*E span; groups of 2^log2_group elements are aligned
// inside the span.  Strides ascend 1, 2, 4, ...: strides below E pair elements
// inside a lane, larger ones pair lane l with lane l ^ (stride / E).  Every
// pair (a at the lower index, b at the upper) becomes (a + b, a - b) in fp32,
// the scalar loop's exact operations and order, so results are bit-identical.
// Callers are wavefront-uniform (every lane active), as the DPP exchanges need.
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
  if (E * 1 < g) lane_stage<E, 1>(v, lane);
  if (E * 2 < g) lane_stage<E, 2>(v, lane);
  if (E * 4 < g) lane_stage<E, 4>(v, lane);
  if (E * 8 < g) lane_stage<E, 8>(v, lane);
  if (E * 16 < g) lane_stage<E, 16>(v, lane);
  if (E * 32 < g) lane_stage<E, 32>(v, lane);
}

}  // namespace bqd

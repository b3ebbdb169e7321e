// The candidate order of sampling ("attention + tokenizer + sampling",
// work item 3 and "Step 3 done"): larger values first, equal values by the
// lower index, NaNs after every number, -0 equal to +0.  Every logit becomes
// one 64-bit key whose unsigned order is exactly that order, no two equal:
//   high 32 bits: the float's bits mapped to an unsigned order (NaN lowest),
//   low 32 bits:  0xffffffff - index (the lower index is the larger key).
#pragma once
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace bqd {

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

}  // namespace bqd

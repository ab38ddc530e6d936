// OCP FP8 E4M3 encoding with power-of-two block scales (gfx950), shared by the weight
// quantizer and the FP8 MFMA layer's activation quantizers.  Block scale 2^k: k the smallest
// integer with the block's max |v| <= 448 * 2^k; each v / 2^k (exact) rounds to the nearest
// E4M3 value, ties to the even code (LongCat-Flash article, itouyu.top, section
// "System-level optimisation", quantization paragraph: fine-grained block quantization as
// in DeepSeek-V3).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lcm {

// Nearest E4M3 code of v (finite, |v| <= 448), ties to even; sign bit from v.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 31) << 7;
  const float a = fabsf(v);
  uint32_t q;
  if (a < 0.015625f) {                         // below 2^-6: subnormal steps of 2^-9
    q = static_cast<uint32_t>(rintf(a * 512.f));  // 0..8 (8 is the smallest normal)
  } else {
    const int e = ilogbf(a);                   // -6..8
    const float m = ldexpf(a, -e);             // [1, 2), exact
    q = static_cast<uint32_t>((e + 7) << 3) + static_cast<uint32_t>(rintf((m - 1.f) * 8.f));
  }
  return q | sign;
}

// Smallest k with amax <= 448 * 2^k (0 for amax == 0); 448 = 1.75 * 2^8.
__device__ __forceinline__ int block_exp(float amax) {
  if (amax == 0.f) return 0;
  const int e = ilogbf(amax);
  return ldexpf(amax, -e) <= 1.75f ? e - 8 : e - 7;
}

}  // namespace lcm

// Softmax and biased top-K of one token in one wavefront (gfx950 / CDNA4), shared by the
// router's top-K kernel and the fused top-K + permutation kernel of few-token layers.
// (LongCat-Flash article, itouyu.top, section "Zero-computation experts": softmax router
// over the whole N+Z pool; the expert bias is added for the choice only.)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Wavefront reductions of the ROCm device library (ockl): DPP steps in a fixed order, the
// result in every active lane.
extern "C" __device__ __attribute__((const)) float __ockl_wfred_max_f32(float);
extern "C" __device__ __attribute__((const)) float __ockl_wfred_add_f32(float);
extern "C" __device__ __attribute__((const)) int __ockl_wfred_min_i32(int);

namespace lcm {

// row: the token's E fp32 logits; EPL experts per lane (expert e lives in lane e % 64,
// slot e / 64).  fp32 max, exp, sum and IEEE division give p; s = p + b; K rounds each take
// the largest s left, the lowest expert index among equal s.  Writes idx_out[0..K) and
// gate_out[0..K) (the unbiased p of each pick), in pick order.
template <int EPL>
__device__ __forceinline__ void router_topk_token(const float* __restrict__ row,
                                                  const float* __restrict__ bias, int E, int K,
                                                  int lane, int32_t* __restrict__ idx_out,
                                                  float* __restrict__ gate_out) {
  // All loads first, unconditionally (slots past E read expert E-1 and are masked below),
  // so they are in flight together: loads under per-slot branches each waited on their own,
  // and a token's chain then took one memory latency per slot.
  float v[EPL], b[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + 64 * j;
    const int ec = e < E ? e : E - 1;
    v[j] = row[ec];
    b[j] = bias[ec];
  }
  // keeps the bias loads here: left alone, the compiler sinks them to their use after the
  // softmax, a second memory round trip on each token's chain
#pragma unroll
  for (int j = 0; j < EPL; ++j) asm volatile("" : "+v"(v[j]), "+v"(b[j]));
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + 64 * j;
    v[j] = e < E ? v[j] : -INFINITY;
    m = fmaxf(m, v[j]);
  }
  // wavefront reductions (DPP, fixed order; every lane gets the same result)
  m = __ockl_wfred_max_f32(m);
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + 64 * j;
    v[j] = e < E ? expf(v[j] - m) : 0.f;
    sum += v[j];
  }
  sum = __ockl_wfred_add_f32(sum);
  float s[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + 64 * j;
    v[j] = v[j] / sum;  // p, IEEE division
    s[j] = e < E ? v[j] + b[j] : -INFINITY;
  }
  // K rounds: the largest s left wins, the lowest expert index among equal s.  Each round
  // takes the lane's best remaining slot (ascending slots keep the lower index), the
  // wavefront maximum of those, then the lowest expert index holding that maximum.
  // Branch-free: slots past E and taken slots hold -inf, so "the first remaining slot, then
  // any strictly larger one" is s > bv from bv = -inf (equal s keep the lower slot).
  for (int k = 0; k < K; ++k) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const bool better = s[j] > bv;
      bv = better ? s[j] : bv;
      be = better ? lane + 64 * j : be;
    }
    const float wm = __ockl_wfred_max_f32(bv);
    const int we = __ockl_wfred_min_i32(bv == wm ? be : 0x7fffffff);
    const bool mine = (we & 63) == lane;
    const int jw = we >> 6;
    float p = 0.f;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const bool hit = mine && j == jw;
      p = hit ? v[j] : p;
      s[j] = hit ? -INFINITY : s[j];  // taken
    }
    if (mine) {
      idx_out[k] = we;
      gate_out[k] = p;
    }
  }
}

}  // namespace lcm

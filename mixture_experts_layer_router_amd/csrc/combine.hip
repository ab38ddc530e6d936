// Fused combine: y_t = sum over the token's FFN picks, in pick order, of g * E_i(x_t),
// plus (sum of the gates of its zero-computation picks, in pick order) * x_t
// (LongCat-Flash article, itouyu.top, section "Zero-computation experts": the identity
// expert returns its input, so all of a token's zero picks together add their gates times
// x_t).  fp32 accumulation, one rounding to the output dtype.  One workgroup per token;
// 16-byte vector loads along d; x_t is read once, after the FFN rows.
#include "common.h"

namespace lcm {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 8 bf16 -> fp32.  STREAM: non-temporal load, for the FFN output rows, which are read
// exactly once here (whole rows, whole lines); x rows may be read again by later picks.
template <bool STREAM>
__device__ __forceinline__ void load8(const bf16_t* p, float* v) {
  const u32x4* q4 = reinterpret_cast<const u32x4*>(p);
  const u32x4 q = STREAM ? __builtin_nontemporal_load(q4) : *q4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(q[i] << 16);
    v[2 * i + 1] = __uint_as_float(q[i] & 0xFFFF0000u);
  }
}

__global__ __launch_bounds__(256) void combine_bf16_kernel(const bf16_t* __restrict__ x,
                                                           const bf16_t* __restrict__ ybuf,
                                                           const int32_t* __restrict__ slot_row,
                                                           const float* __restrict__ gate,
                                                           bf16_t* __restrict__ y, int d, int K) {
  const int t = blockIdx.x;
  const bf16_t* xt = x + size_t(t) * d;
  for (int c = threadIdx.x * 8; c < d; c += 256 * 8) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float gz = 0.f;  // sum of the zero picks' gates
    // Picks in groups of 4: the 4 row loads go out together, unconditionally (a zero pick
    // reads FFN output row 0 and ignores it), then the terms are added in pick order.  With
    // the loads under per-pick branches each waited on its own, and a layer of few tokens,
    // which has nothing else to overlap, took one memory latency per pick.
    int k = 0;
    for (; k + 4 <= K; k += 4) {
      float g[4], v[4][8];
      int r[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        g[i] = gate[size_t(t) * K + k + i];
        r[i] = slot_row[size_t(t) * K + k + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) load8<true>(ybuf + size_t(r[i] >= 0 ? r[i] : 0) * d + c, v[i]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (r[i] >= 0) {
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] = fmaf(g[i], v[i][e], acc[e]);
        } else {
          gz += g[i];
        }
      }
    }
    for (; k < K; ++k) {
      const float g = gate[size_t(t) * K + k];
      const int r = slot_row[size_t(t) * K + k];
      if (r >= 0) {
        float v[8];
        load8<true>(ybuf + size_t(r) * d + c, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(g, v[i], acc[i]);
      } else {
        gz += g;
      }
    }
    if (gz != 0.f) {
      float v[8];
      load8<false>(xt + c, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(gz, v[i], acc[i]);
    }
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = f2bf(acc[2 * i]) | (uint32_t(f2bf(acc[2 * i + 1])) << 16);
    *reinterpret_cast<uint4*>(y + size_t(t) * d + c) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

__global__ __launch_bounds__(256) void combine_f32_kernel(const float* __restrict__ x,
                                                          const float* __restrict__ ybuf,
                                                          const int32_t* __restrict__ slot_row,
                                                          const float* __restrict__ gate,
                                                          float* __restrict__ y, int d, int K) {
  const int t = blockIdx.x;
  const float* xt = x + size_t(t) * d;
  for (int c = threadIdx.x * 4; c < d; c += 256 * 4) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float gz = 0.f;  // sum of the zero picks' gates
    for (int k = 0; k < K; ++k) {
      const float g = gate[size_t(t) * K + k];
      const int r = slot_row[size_t(t) * K + k];
      if (r < 0) {
        gz += g;
        continue;
      }
      const float4 v = *reinterpret_cast<const float4*>(ybuf + size_t(r) * d + c);
      acc.x = fmaf(g, v.x, acc.x);
      acc.y = fmaf(g, v.y, acc.y);
      acc.z = fmaf(g, v.z, acc.z);
      acc.w = fmaf(g, v.w, acc.w);
    }
    if (gz != 0.f) {
      const float4 v = *reinterpret_cast<const float4*>(xt + c);
      acc.x = fmaf(gz, v.x, acc.x);
      acc.y = fmaf(gz, v.y, acc.y);
      acc.z = fmaf(gz, v.z, acc.z);
      acc.w = fmaf(gz, v.w, acc.w);
    }
    *reinterpret_cast<float4*>(y + size_t(t) * d + c) = acc;
  }
}

hipError_t launch_combine(const lc_moe_shape& s, const void* x, const void* ybuf,
                          const int32_t* slot_row, const float* gate, void* y, hipStream_t st) {
  if (s.dtype == LC_MOE_BF16) {
    hipLaunchKernelGGL(combine_bf16_kernel, dim3(s.T), dim3(256), 0, st,
                       static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(ybuf), slot_row,
                       gate, static_cast<bf16_t*>(y), s.d, s.K);
  } else {
    hipLaunchKernelGGL(combine_f32_kernel, dim3(s.T), dim3(256), 0, st,
                       static_cast<const float*>(x), static_cast<const float*>(ybuf), slot_row,
                       gate, static_cast<float*>(y), s.d, s.K);
  }
  return hipGetLastError();
}

}  // namespace lcm

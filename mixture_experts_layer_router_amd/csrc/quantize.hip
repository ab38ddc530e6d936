// Block-FP8 expert weights (LongCat-Flash article, itouyu.top, section "System-level
// optimisation", quantization paragraph: fine-grained block quantization as in
// DeepSeek-V3).  Every expert matrix is cut into blocks of 128 rows x 128 reduction
// columns; a block gets the scale 2^k, k the smallest integer with max|w| <= 448 * 2^k,
// and each w / 2^k (exact) is rounded to the nearest OCP E4M3 value, ties to the even
// code.  The codes are written straight into the packed pair-row layout the FFN kernel
// streams (see Fp8Plan), the scales as fp32 powers of two.
#include "common.h"
#include "fp8.h"

namespace lcm {

// One workgroup per 128x128 block of one matrix: blockIdx = (column block, row block,
// expert * nmat + matrix).  MAT_GU: matrices 0 (gate) and 1 (up) of [N][I][d]; else
// W_down [N][d][I].  Thread t handles the 8-column groups t, t+256, ... of the block
// (row = idx / 16, group = idx % 16): one 16-byte load, one 8-byte store of codes.
template <bool MAT_GU>
__global__ __launch_bounds__(256) void quantize_kernel(const bf16_t* __restrict__ w0,
                                                       const bf16_t* __restrict__ w1,
                                                       unsigned char* __restrict__ codes,
                                                       float* __restrict__ scales, int R, int C,
                                                       int rows_per_tile, int ntiles) {
  const int cb = blockIdx.x, rb = blockIdx.y;
  const int mat = MAT_GU ? int(blockIdx.z & 1) : 0;
  const int e = MAT_GU ? int(blockIdx.z >> 1) : int(blockIdx.z);
  const bf16_t* w = (mat == 0 ? w0 : w1) + size_t(e) * R * C;
  const int tid = threadIdx.x;
  uint4 v[8];
  float amax = 0.f;
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int idx = tid + 256 * it, r = rb * 128 + (idx >> 4), c = cb * 128 + (idx & 15) * 8;
    v[it] = (r < R && c < C) ? *reinterpret_cast<const uint4*>(w + size_t(r) * C + c) : make_uint4(0, 0, 0, 0);
    const uint32_t u[4] = {v[it].x, v[it].y, v[it].z, v[it].w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      amax = fmaxf(amax, fabsf(bf2f(bf16_t(u[q] & 0xFFFF))));
      amax = fmaxf(amax, fabsf(bf2f(bf16_t(u[q] >> 16))));
    }
  }
  __shared__ float wmax[4];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  if ((tid & 63) == 0) wmax[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const int k = block_exp(amax);
  const int nrb = (R + 127) / 128, ncb = (C + 127) / 128;
  if (tid == 0) scales[(size_t(MAT_GU ? e * 2 + mat : e) * nrb + rb) * ncb + cb] = ldexpf(1.f, k);
  const int nk = C / 32;
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int idx = tid + 256 * it, r = rb * 128 + (idx >> 4), c = cb * 128 + (idx & 15) * 8;
    if (r >= R || c >= C) continue;
    const uint32_t u[4] = {v[it].x, v[it].y, v[it].z, v[it].w};
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t c0 = e4m3_code(ldexpf(bf2f(bf16_t(u[q] & 0xFFFF)), -k));
      const uint32_t c1 = e4m3_code(ldexpf(bf2f(bf16_t(u[q] >> 16)), -k));
      const uint32_t pair = c0 | (c1 << 8);
      if (q < 2) lo |= pair << (16 * q);
      else hi |= pair << (16 * (q - 2));
    }
    const int nt = r / rows_per_tile, rt = r % rows_per_tile;  // row of the n-tile
    // pair-row and half: gate/up pair row rt of both matrices; W_down pairs rows rt and
    // rt + 32 of each 64-row group
    const int p = MAT_GU ? rt : (rt >> 6) * 32 + (rt & 31);
    const int half = MAT_GU ? mat : (rt >> 5) & 1;
    const int kt = c >> 5, grp = (c >> 3) & 3;
    const size_t off = ((size_t(e) * ntiles + nt) * nk + kt) * 8192 + size_t(p) * 64 +
                       ((grp ^ swz4(p)) << 4) + half * 8;
    *reinterpret_cast<uint2*>(codes + off) = make_uint2(lo, hi);
  }
}

__global__ void zero_bytes_kernel(uint4* __restrict__ p, size_t n16) {
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += size_t(gridDim.x) * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

hipError_t launch_quantize_weights(const lc_moe_shape& s, const void* w_gate, const void* w_up,
                                   const void* w_down, void* out, hipStream_t st) {
  const Fp8Plan p = plan_fp8(s);
  unsigned char* base = static_cast<unsigned char*>(out);
  // tile rows past I (gate/up) or d (down) stay zero
  const size_t zbytes = p.scales_gu;  // both code regions
  hipLaunchKernelGGL(zero_bytes_kernel, dim3(2048), dim3(256), 0, st, reinterpret_cast<uint4*>(base),
                     zbytes / 16);
  hipLaunchKernelGGL(quantize_kernel<true>, dim3((s.d + 127) / 128, (s.I + 127) / 128, 2 * s.N),
                     dim3(256), 0, st, static_cast<const bf16_t*>(w_gate),
                     static_cast<const bf16_t*>(w_up), base + p.codes_gu,
                     reinterpret_cast<float*>(base + p.scales_gu), s.I, s.d, 128, p.nt_gu);
  hipLaunchKernelGGL(quantize_kernel<false>, dim3((s.I + 127) / 128, (s.d + 127) / 128, s.N),
                     dim3(256), 0, st, static_cast<const bf16_t*>(w_down),
                     static_cast<const bf16_t*>(w_down), base + p.codes_d,
                     reinterpret_cast<float*>(base + p.scales_d), s.d, s.I, 256, p.nt_d);
  return hipGetLastError();
}

}  // namespace lcm

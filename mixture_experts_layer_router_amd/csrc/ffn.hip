// Grouped SwiGLU FFN over the FFN picks only; zero-computation picks never reach these
// kernels (LongCat-Flash article, itouyu.top, section "Zero-computation experts": the
// identity experts cost no compute).
//
//   gate/up:  H[r] = silu(W_gate,e x_t) * (W_up,e x_t)    for row r of expert e, t = perm_token[r]
//   down:     Y[r] = W_down,e H[r]
//
// Work unit = (M-tile of one expert, n-tile of output columns).  The M-tile list is built
// on the device by the scan kernel, so the host never learns the per-expert row counts;
// the grid is sized for the worst case and surplus workgroups exit at once.
//
// XCD-aware mapping: MI355X dispatches workgroup w to XCD w % 8.  Work units are ordered
// expert by expert, n-tile-major inside an expert (the M-tiles that share one weight tile
// are adjacent), and each XCD takes one contiguous eighth of that order, so the tiles
// that share weights or activations run together on one XCD and meet in its L2.
#include "common.h"

namespace lcm {

// Map a workgroup to (M-tile j, n-tile).  Returns false for surplus workgroups.
__device__ __forceinline__ bool unit_of_block(const MTile* __restrict__ mtiles,
                                              const int32_t* __restrict__ offsets,
                                              int n_mtiles, int n_ntiles, int bm, int& j,
                                              int& ntile) {
  const int U = n_mtiles * n_ntiles;
  const int per = (U + 7) >> 3;
  const int w = blockIdx.x;
  const int slot = w >> 3;
  if (slot >= per) return false;
  const int u = (w & 7) * per + slot;
  if (u >= U) return false;
  const MTile tb = mtiles[u / n_ntiles];
  const int mt = (offsets[tb.expert + 1] - offsets[tb.expert] + bm - 1) / bm;
  const int ul = u - tb.first_tile * n_ntiles;
  ntile = ul / mt;
  j = tb.first_tile + (ul - ntile * mt);
  return true;
}

// ---------------------------------------------------------------------------------------
// bf16 MFMA kernel.  Tile: 128 rows x 256 weight rows, K step 64, 256 threads (2x2 waves;
// each wave 64 rows x 4 blocks of 32 weight rows; v_mfma_f32_32x32x16_bf16).
//   MODE 0 (gate/up): weight rows 0..127 = gate rows n0..n0+127, 128..255 = up rows
//                     n0..n0+127; A rows gathered from x through perm_token; epilogue
//                     silu(g)*u -> H (128 columns per tile).
//   MODE 1 (down):    weight rows = W_down rows n0..n0+255; A rows = H rows; epilogue
//                     -> Y (256 columns per tile).
// Single LDS buffer with register prefetch of the next K step.
// ---------------------------------------------------------------------------------------
namespace fk {
constexpr int BM = kBmBf16, BR = 256, BK = 64, LD = BK + 8;  // LDS row: 144 bytes
}

template <int MODE>
__global__ __launch_bounds__(256, 2) void ffn_bf16_kernel(
    const bf16_t* __restrict__ a_src, const int32_t* __restrict__ perm_token,
    const bf16_t* __restrict__ w0, const bf16_t* __restrict__ w1, bf16_t* __restrict__ out,
    const MTile* __restrict__ mtiles, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ n_mtiles_ptr, int kdim, int ncols, int n_ntiles) {
  using namespace fk;
  __shared__ __attribute__((aligned(16))) bf16_t As[BM * LD];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[BR * LD];

  int j, ntile;
  if (!unit_of_block(mtiles, offsets, *n_mtiles_ptr, n_ntiles, BM, j, ntile)) return;
  const MTile tile = mtiles[j];
  const int e = tile.expert, row0 = tile.row0, rows = tile.rows;
  const int n0 = ntile * (MODE == 0 ? 128 : 256);
  const int tid = threadIdx.x;

  // register-prefetch assignment: A 128 rows x 8 chunks -> 4/thread; B 256 x 8 -> 8/thread
  const bf16_t* a_ptr[4];
  const bf16_t* b_ptr[8];
  const int kc = (tid & 7) * 8;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid >> 3) + i * 32;
    const bf16_t* p = nullptr;
    if (r < rows) {
      const int grow = row0 + r;
      p = MODE == 0 ? a_src + size_t(perm_token[grow]) * kdim : a_src + size_t(grow) * kdim;
    }
    a_ptr[i] = p;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = (tid >> 3) + i * 32;
    const bf16_t* p = nullptr;
    if (MODE == 0) {
      const int c = n0 + (r & 127);
      if (c < ncols) p = (r < 128 ? w0 : w1) + (size_t(e) * ncols + c) * kdim;
    } else {
      const int c = n0 + r;
      if (c < ncols) p = w0 + (size_t(e) * ncols + c) * kdim;
    }
    b_ptr[i] = p;
  }
  uint4 ra[4], rb[8];
  auto load = [&](int k0) {
    const int k = k0 + kc;
    const bool kin = k < kdim;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      ra[i] = (a_ptr[i] && kin) ? *reinterpret_cast<const uint4*>(a_ptr[i] + k) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      rb[i] = (b_ptr[i] && kin) ? *reinterpret_cast<const uint4*>(b_ptr[i] + k) : make_uint4(0, 0, 0, 0);
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4*>(&As[((tid >> 3) + i * 32) * LD + kc]) = ra[i];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<uint4*>(&Bs[((tid >> 3) + i * 32) * LD + kc]) = rb[i];
  };

  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lk = (lane >> 5) * 8;
  // weight-row base of the wave's 4 blocks
  int brow[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
    brow[nb] = MODE == 0 ? (nb >> 1) * 128 + wn * 64 + (nb & 1) * 32 : wn * 128 + nb * 32;
  const bool mv0 = wm * 64 < rows, mv1 = wm * 64 + 32 < rows;

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][nb][r] = 0.f;

  const int nk = (kdim + BK - 1) / BK;
  load(0);
  for (int kt = 0; kt < nk; ++kt) {
    __syncthreads();
    store();
    __syncthreads();
    if (kt + 1 < nk) load((kt + 1) * BK);
    if (mv0) {
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        const int kk = ks * 16 + lk;
        bf16x8 a0 = *reinterpret_cast<const bf16x8*>(&As[(wm * 64 + lr) * LD + kk]);
        bf16x8 a1 = *reinterpret_cast<const bf16x8*>(&As[(wm * 64 + 32 + lr) * LD + kk]);
        bf16x8 b[4];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          b[nb] = *reinterpret_cast<const bf16x8*>(&Bs[(brow[nb] + lr) * LD + kk]);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[0][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b[nb], acc[0][nb], 0, 0, 0);
        if (mv1) {
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
            acc[1][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b[nb], acc[1][nb], 0, 0, 0);
        }
      }
    }
  }

  // epilogue; 32x32 D layout: column lane & 31, rows 8*(r/4) + 4*(lane/32) + r%4
  if (MODE == 0) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int col = n0 + wn * 64 + nb * 32 + lr;
        if (col >= ncols) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (row < rows) {
            const float g = acc[i][nb][r], u = acc[i][nb + 2][r];
            const float h = g / (1.f + expf(-g)) * u;
            out[size_t(row0 + row) * ncols + col] = f2bf(h);
          }
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int col = n0 + wn * 128 + nb * 32 + lr;
        if (col >= ncols) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (row < rows) out[size_t(row0 + row) * ncols + col] = f2bf(acc[i][nb][r]);
        }
      }
  }
}

// ---------------------------------------------------------------------------------------
// fp32 kernel (FMA): tile 64 rows x 64 output columns, K step 16, 4x4 outputs per thread.
// MODE 0 keeps gate and up accumulators for the same columns.
// ---------------------------------------------------------------------------------------
template <int MODE>
__global__ __launch_bounds__(256) void ffn_f32_kernel(
    const float* __restrict__ a_src, const int32_t* __restrict__ perm_token,
    const float* __restrict__ w0, const float* __restrict__ w1, float* __restrict__ out,
    const MTile* __restrict__ mtiles, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ n_mtiles_ptr, int kdim, int ncols, int n_ntiles) {
  constexpr int BM = kBmF32;
  __shared__ float As[BM][17];
  __shared__ float Gs[64][17];
  __shared__ float Us[64][17];
  int j, ntile;
  if (!unit_of_block(mtiles, offsets, *n_mtiles_ptr, n_ntiles, BM, j, ntile)) return;
  const MTile tile = mtiles[j];
  const int e = tile.expert, row0 = tile.row0, rows = tile.rows;
  const int n0 = ntile * 64;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  float ag[4][4] = {}, au[4][4] = {};
  for (int k0 = 0; k0 < kdim; k0 += 16) {
    for (int c = tid; c < 64 * 16; c += 256) {
      const int r = c >> 4, k = c & 15, kk = k0 + k;
      float av = 0.f;
      if (r < rows && kk < kdim) {
        const int grow = row0 + r;
        const size_t arow = MODE == 0 ? size_t(perm_token[grow]) : size_t(grow);
        av = a_src[arow * kdim + kk];
      }
      As[r][k] = av;
      const int col = n0 + r;
      const bool ok = col < ncols && kk < kdim;
      Gs[r][k] = ok ? w0[(size_t(e) * ncols + col) * kdim + kk] : 0.f;
      if (MODE == 0) Us[r][k] = ok ? w1[(size_t(e) * ncols + col) * kdim + kk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          ag[i][jj] = fmaf(As[ty * 4 + i][k], Gs[tx * 4 + jj][k], ag[i][jj]);
          if (MODE == 0) au[i][jj] = fmaf(As[ty * 4 + i][k], Us[tx * 4 + jj][k], au[i][jj]);
        }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int row = ty * 4 + i, col = n0 + tx * 4 + jj;
      if (row < rows && col < ncols) {
        float v = ag[i][jj];
        if (MODE == 0) v = v / (1.f + expf(-v)) * au[i][jj];
        out[size_t(row0 + row) * ncols + col] = v;
      }
    }
}

hipError_t launch_ffn_gate_up(const lc_moe_shape& s, const void* x, const int32_t* perm_token,
                              const void* w_gate, const void* w_up, void* hbuf,
                              const MTile* mtiles, const int32_t* offsets,
                              const int32_t* n_mtiles, int mt_max, hipStream_t st) {
  if (s.dtype == LC_MOE_BF16) {
    const int nn = (s.I + 127) / 128;
    const size_t units = size_t(mt_max) * nn;
    const unsigned grid = static_cast<unsigned>((units + 7) / 8 * 8);
    hipLaunchKernelGGL(ffn_bf16_kernel<0>, dim3(grid), dim3(256), 0, st,
                       static_cast<const bf16_t*>(x), perm_token, static_cast<const bf16_t*>(w_gate),
                       static_cast<const bf16_t*>(w_up), static_cast<bf16_t*>(hbuf), mtiles, offsets,
                       n_mtiles, s.d, s.I, nn);
  } else {
    const int nn = (s.I + 63) / 64;
    const size_t units = size_t(mt_max) * nn;
    const unsigned grid = static_cast<unsigned>((units + 7) / 8 * 8);
    hipLaunchKernelGGL(ffn_f32_kernel<0>, dim3(grid), dim3(256), 0, st,
                       static_cast<const float*>(x), perm_token, static_cast<const float*>(w_gate),
                       static_cast<const float*>(w_up), static_cast<float*>(hbuf), mtiles, offsets,
                       n_mtiles, s.d, s.I, nn);
  }
  return hipGetLastError();
}

hipError_t launch_ffn_down(const lc_moe_shape& s, const void* hbuf, const void* w_down,
                           void* ybuf, const MTile* mtiles, const int32_t* offsets,
                           const int32_t* n_mtiles, int mt_max, hipStream_t st) {
  if (s.dtype == LC_MOE_BF16) {
    const int nn = (s.d + 255) / 256;
    const size_t units = size_t(mt_max) * nn;
    const unsigned grid = static_cast<unsigned>((units + 7) / 8 * 8);
    hipLaunchKernelGGL(ffn_bf16_kernel<1>, dim3(grid), dim3(256), 0, st,
                       static_cast<const bf16_t*>(hbuf), nullptr, static_cast<const bf16_t*>(w_down),
                       nullptr, static_cast<bf16_t*>(ybuf), mtiles, offsets, n_mtiles, s.I, s.d, nn);
  } else {
    const int nn = (s.d + 63) / 64;
    const size_t units = size_t(mt_max) * nn;
    const unsigned grid = static_cast<unsigned>((units + 7) / 8 * 8);
    hipLaunchKernelGGL(ffn_f32_kernel<1>, dim3(grid), dim3(256), 0, st,
                       static_cast<const float*>(hbuf), nullptr, static_cast<const float*>(w_down),
                       nullptr, static_cast<float*>(ybuf), mtiles, offsets, n_mtiles, s.I, s.d, nn);
  }
  return hipGetLastError();
}

}  // namespace lcm

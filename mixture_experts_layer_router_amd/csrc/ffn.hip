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
#include <type_traits>

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
// Pipelined bf16 MFMA kernel (used when d and I are multiples of 32).
// Tile: 256 rows x 256 weight rows, K step 32, 4-stage LDS ring (4 x 32 KB) filled by
// direct global->LDS loads (global_load_lds_dwordx4), so up to three K steps are in
// flight while one is multiplied.  256 threads = 2x2 waves; each wave owns 4x4 blocks of
// 32x32 (v_mfma_f32_32x32x16_bf16, 256 fp32 accumulators per lane).  Wave row wm takes
// the 32-row blocks 2*mb + wm, so a partly filled tile splits its blocks evenly.
// LDS rows are 64 bytes (four 16-byte chunks); chunk c of row r sits in slot c ^ swz(r),
// which spreads the 32 rows of one MFMA operand read over all banks.
// ---------------------------------------------------------------------------------------
#ifndef LCM_PIPE_BK
#define LCM_PIPE_BK 32
#endif

// XOR swizzle of the 16-byte chunk slot for LDS rows of CPR chunks (CPR = 4: 64-byte rows,
// CPR = 8: 128-byte rows).  Conflict-free for the 32-row MFMA operand reads whether the
// LDS serves 8 or 16 lanes of a ds_read_b128 per cycle.
template <int CPR>
__device__ __forceinline__ int swz(int r) {
  if (CPR == 4) return (((r >> 1) & 1) << 1) ^ ((r >> 2) & 1) ^ (((r >> 3) & 1) << 1);
  return (r & 7) ^ ((r >> 3) & 1);
}

#ifdef LCM_PROFILE
__device__ unsigned long long lcm_prof[2][4096][6];
extern "C" hipError_t lc_moe_debug_prof(void* host, size_t bytes) {
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(lcm_prof), bytes, 0, hipMemcpyDeviceToHost);
}
#endif

typedef __attribute__((address_space(3))) void lds_void;

// One wave-wide direct global->LDS load: lane l copies 16 bytes from g to lds + 16*l.
__device__ __forceinline__ void dma16(const void* g, unsigned char* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 16, 0, 0);
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
#define LCM_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt((((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14)))

__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Pipelined bf16 MFMA kernel (used when d and I are multiples of 32).
// Tile: 256 rows x 256 weight rows, K step 32, 4-stage LDS ring (4 x 32 KB) filled by
// direct global->LDS loads (global_load_lds_dwordx4): up to three K steps in flight.
// 256 threads = 2x2 waves; wave (wm, wn) owns 4x4 blocks of 32x32 (v_mfma_f32_32x32x16_bf16,
// 256 fp32 accumulators per lane): M blocks 2*mb + wm (a partly filled tile splits its
// blocks evenly), N blocks = weight rows brow[nb].
// Software pipeline: a K step has two substeps of 16.  The operand fragments of the next
// substep are read from LDS while the MFMAs of the current one run; the barrier that
// publishes the next stage sits between the two substeps, so every LDS read hides behind
// 16 MFMAs.  The 8 loads of the stage three steps ahead are spread over the first
// substep's MFMAs (one per two MFMAs) instead of bursting.
// LDS row = 64 bytes = 4 chunks of 16 bytes; chunk c of row r sits in slot c ^ swz(r).
template <int MODE, int BK, int NST>
__global__ __launch_bounds__(256, 1) void ffn_bf16_pipe_kernel(
    const bf16_t* __restrict__ a_src, const int32_t* __restrict__ perm_token,
    const bf16_t* __restrict__ w0, const bf16_t* __restrict__ w1, bf16_t* __restrict__ out,
    const MTile* __restrict__ mtiles, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ n_mtiles_ptr, int kdim, int ncols, int n_ntiles) {
  static_assert(BK == 32 && NST == 4, "stage body written for two 16-wide substeps");
  constexpr int BM = kBmPipe;
  constexpr int CPR = BK / 8;             // 16-byte chunks per LDS row
  constexpr int RB = BK * 2;              // bytes per LDS row
  constexpr int RPI = 64 / CPR;           // rows filled by one wave-wide DMA instruction
  constexpr int IPW = 256 / (4 * RPI);    // DMA instructions per wave per operand per stage
  constexpr int A_BYTES = BM * RB;
  constexpr int STAGE = A_BYTES + 256 * RB;
  constexpr int VM_STAGE = 2 * IPW;       // loads per wave per stage
  __shared__ __attribute__((aligned(1024))) unsigned char smem[NST * STAGE];

  int j, ntile;
  if (!unit_of_block(mtiles, offsets, *n_mtiles_ptr, n_ntiles, BM, j, ntile)) return;
  const MTile tile = mtiles[j];
  const int e = tile.expert, row0 = tile.row0, rows = tile.rows;
  const int n0 = ntile * (MODE == 0 ? 128 : 256);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // DMA sources: wave w fills rows (IPW*w + i)*RPI .. +RPI of the A and B tiles;
  // lane l writes LDS row l/CPR, slot l%CPR, i.e. global chunk (l%CPR) ^ swz(row).
  const bf16_t* src[2 * IPW];
  const int lrow = lane / CPR, lslot = lane % CPR;
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int r = (wave * IPW + i) * RPI + lrow;
    const int chunk = (lslot ^ swz<CPR>(r)) * 8;
    const int ar = r < rows ? r : 0;  // rows past the tile read a valid row; never stored
    const size_t src_row = MODE == 0 ? size_t(perm_token[row0 + ar]) : size_t(row0 + ar);
    src[i] = a_src + src_row * kdim + chunk;
    int c;
    const bf16_t* mat;
    if (MODE == 0) {
      c = n0 + (r & 127);
      mat = r < 128 ? w0 : w1;
    } else {
      c = n0 + r;
      mat = w0;
    }
    const int brow = c < ncols ? c : n0;
    src[IPW + i] = mat + (size_t(e) * ncols + brow) * kdim + chunk;
  }
  const int nk = kdim / BK;
#ifdef LCM_NO_KROT
  const int krot = 0;
#else
  // Each work unit starts its K loop at its own offset: rows of one tile share their low
  // address bits (row strides are multiples of 4 KB), so tiles running side by side are
  // spread over the L2 channels.
  const int krot = (j * 7 + ntile * 3) % nk;
#endif
  auto kphys = [&](int kt) { const int k = kt + krot; return (k >= nk ? k - nk : k) * BK; };
  auto issue_one = [&](int i, unsigned char* st, int k0) {
    dma16(src[i] + k0, st + (i < IPW ? 0 : A_BYTES) + (wave * IPW + (i % IPW)) * 1024);
  };

  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, sw = swz<CPR>(l32), khalf = lane >> 5;
  int brow[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
    brow[nb] = MODE == 0 ? (nb >> 1) * 128 + wn * 64 + (nb & 1) * 32 : wn * 128 + nb * 32;
  bool bv[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) bv[mb] = (mb * 2 + wm) * 32 < rows;

  f32x16 acc[4][4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.f;

  for (int s = 0; s < NST - 1 && s < nk; ++s) {
#pragma unroll
    for (int i = 0; i < 2 * IPW; ++i) issue_one(i, smem + s * STAGE, kphys(s));
  }
  // wait until stage kt landed, with `ahead` later stages allowed in flight
  auto wait_stage = [&](int ahead) {
    if (ahead >= 2) LCM_WAIT_VMCNT(2 * VM_STAGE);
    else if (ahead == 1) LCM_WAIT_VMCNT(VM_STAGE);
    else LCM_WAIT_VMCNT(0);
  };

  auto run = [&](auto full) {
    constexpr bool FULL = decltype(full)::value;
    auto read = [&](const unsigned char* st, int ks, bf16x8 (&fa)[4], bf16x8 (&fb)[4]) {
      const int slot = ((ks * 2 + khalf) ^ sw) * 16;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        fb[nb] = *reinterpret_cast<const bf16x8*>(st + A_BYTES + (brow[nb] + l32) * RB + slot);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        if (FULL || bv[mb])
          fa[mb] = *reinterpret_cast<const bf16x8*>(st + ((mb * 2 + wm) * 32 + l32) * RB + slot);
    };
    // 16 MFMAs of one substep.  DMA: the wave's 8 loads of the stage NST-1 ahead go between
    // them; `after_first` runs after the first MFMA pair (used to start the next substep's
    // LDS reads once this substep's operands are known to be in registers).
    auto mfmas = [&](const bf16x8 (&fa)[4], const bf16x8 (&fb)[4], auto dma, unsigned char* nst,
                     int k0n, auto after_first) {
      constexpr bool DMA = decltype(dma)::value;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if (DMA) issue_one(mb * 2 + h, nst, k0n);
          __builtin_amdgcn_sched_barrier(0);
          if (FULL || bv[mb]) {
#pragma unroll
            for (int nb = h * 2; nb < h * 2 + 2; ++nb)
              acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mb], fb[nb], acc[mb][nb], 0, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
          if (mb == 0 && h == 0) after_first();
        }
      }
    };
#ifdef LCM_PROFILE
    unsigned long long pt[6] = {0, 0, 0, 0, 0, 0};
    const unsigned long long tstart = __builtin_amdgcn_s_memtime();
#endif
    bf16x8 a0[4], b0[4], a1[4], b1[4];
    wait_stage(nk - 1 < NST - 2 ? nk - 1 : NST - 2);
    block_barrier();
    read(smem, 0, a0, b0);
    auto step = [&](int kt, auto more_tag, auto last_tag) {
      constexpr bool MORE = decltype(more_tag)::value;
      constexpr bool LAST = decltype(last_tag)::value;
      const unsigned char* st = smem + (kt % NST) * STAGE;
      mfmas(a0, b0, more_tag, smem + ((kt + NST - 1) % NST) * STAGE, kphys(kt + NST - 1),
            [&] { read(st, 1, a1, b1); });
      if (!LAST) {
#ifdef LCM_PROFILE
        unsigned long long t0 = __builtin_amdgcn_s_memtime();
#endif
        // stage kt+1 must have landed; stages after it may stay in flight
        const int issued_after = (MORE ? kt + NST - 1 : nk - 1) - (kt + 1);
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's reads of stage kt done
        wait_stage(issued_after);
#ifdef LCM_PROFILE
        unsigned long long t1 = __builtin_amdgcn_s_memtime();
        pt[0] += t1 - t0;
#endif
        block_barrier();
#ifdef LCM_PROFILE
        pt[1] += __builtin_amdgcn_s_memtime() - t1;
#endif
        read(smem + ((kt + 1) % NST) * STAGE, 0, a0, b0);
      }
      mfmas(a1, b1, std::false_type{}, nullptr, 0, [] {});
    };
    // main steps load the stage NST-1 ahead; the last NST-1 steps have nothing left to load;
    // the final step has no next stage to publish
    const int nmain = nk - (NST - 1) > 0 ? nk - (NST - 1) : 0;
    for (int kt = 0; kt < nmain; ++kt) step(kt, std::true_type{}, std::false_type{});
    for (int kt = nmain; kt < nk - 1; ++kt) step(kt, std::false_type{}, std::false_type{});
    step(nk - 1, std::false_type{}, std::true_type{});
#ifdef LCM_PROFILE
    unsigned long long tend = __builtin_amdgcn_s_memtime();
    pt[4] = tend - tstart;
    pt[3] = pt[4] - pt[0] - pt[1];
    pt[5] = FULL ? 1 : 0;
    if (lane == 0 && blockIdx.x < 4096 * 8 && (blockIdx.x & 7) == 0 && wave == 0)
      for (int q = 0; q < 6; ++q) lcm_prof[MODE][blockIdx.x >> 3][q] = pt[q];
#endif
  };
  if (bv[3]) run(std::true_type{});
  else run(std::false_type{});

  // epilogue; 32x32 D layout: column lane & 31, rows 8*(r/4) + 4*(lane/32) + r%4
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    if (!bv[mb]) continue;
    if (MODE == 0) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int col = n0 + wn * 64 + nb * 32 + l32;
        if (col >= ncols) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = (mb * 2 + wm) * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3);
          if (row < rows) {
            const float g = acc[mb][nb][r], u = acc[mb][nb + 2][r];
            out[size_t(row0 + row) * ncols + col] = f2bf(g / (1.f + expf(-g)) * u);
          }
        }
      }
    } else {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int col = n0 + wn * 128 + nb * 32 + l32;
        if (col >= ncols) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = (mb * 2 + wm) * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3);
          if (row < rows) out[size_t(row0 + row) * ncols + col] = f2bf(acc[mb][nb][r]);
        }
      }
    }
  }
}

constexpr int kPipeBK = LCM_PIPE_BK;
constexpr int kPipeNST = (160 * 1024) / (2 * 256 * LCM_PIPE_BK * 2) < 4 ? (160 * 1024) / (2 * 256 * LCM_PIPE_BK * 2) : 4;

template __global__ void ffn_bf16_pipe_kernel<0, kPipeBK, kPipeNST>(
    const bf16_t* __restrict__, const int32_t* __restrict__, const bf16_t* __restrict__,
    const bf16_t* __restrict__, bf16_t* __restrict__, const MTile* __restrict__,
    const int32_t* __restrict__, const int32_t* __restrict__, int, int, int);
template __global__ void ffn_bf16_pipe_kernel<1, kPipeBK, kPipeNST>(
    const bf16_t* __restrict__, const int32_t* __restrict__, const bf16_t* __restrict__,
    const bf16_t* __restrict__, bf16_t* __restrict__, const MTile* __restrict__,
    const int32_t* __restrict__, const int32_t* __restrict__, int, int, int);

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
  if (s.dtype == LC_MOE_BF16 && ffn_pipelined(s)) {
    const int nn = (s.I + 127) / 128;
    const size_t units = size_t(mt_max) * nn;
    const unsigned grid = static_cast<unsigned>((units + 7) / 8 * 8);
    ffn_bf16_pipe_kernel<0, kPipeBK, kPipeNST><<<dim3(grid), dim3(256), 0, st>>>(
        static_cast<const bf16_t*>(x), perm_token, static_cast<const bf16_t*>(w_gate),
        static_cast<const bf16_t*>(w_up), static_cast<bf16_t*>(hbuf), mtiles, offsets, n_mtiles, s.d,
        s.I, nn);
  } else if (s.dtype == LC_MOE_BF16) {
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
  if (s.dtype == LC_MOE_BF16 && ffn_pipelined(s)) {
    const int nn = (s.d + 255) / 256;
    const size_t units = size_t(mt_max) * nn;
    const unsigned grid = static_cast<unsigned>((units + 7) / 8 * 8);
    ffn_bf16_pipe_kernel<1, kPipeBK, kPipeNST><<<dim3(grid), dim3(256), 0, st>>>(
        static_cast<const bf16_t*>(hbuf), nullptr, static_cast<const bf16_t*>(w_down), nullptr,
        static_cast<bf16_t*>(ybuf), mtiles, offsets, n_mtiles, s.I, s.d, nn);
  } else if (s.dtype == LC_MOE_BF16) {
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

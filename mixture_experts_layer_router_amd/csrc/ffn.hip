// Grouped SwiGLU FFN over the FFN picks only; zero-computation picks never reach these
// kernels (LongCat-Flash article, itouyu.top, section "Zero-computation experts": the
// identity experts cost no compute).
//
//   gate/up:  H[r] = silu(W_gate,e x_t) * (W_up,e x_t)    for row r of expert e, t = perm_token[r]
//   down:     Y[r] = W_down,e H[r]
// MODE 0 is gate/up, MODE 1 down; MODE 2 is gate/up with the backward epilogue of the FFN's
// gradient (G and U recomputed; g*H, dG and dU written from dH and the row's gate).
//
// Work unit = (M-tile of one expert, n-tile of output columns).  The M-tile list is built
// on the device by the scan kernel, so the host never learns the per-expert row counts;
// the grid is sized for the worst case and surplus workgroups exit at once.
//
// XCD-aware mapping: MI355X dispatches workgroup w to XCD w % 8.  Work units are ordered
// expert by expert, n-tile-major inside an expert (the M-tiles that share one weight tile
// are adjacent), and each XCD takes one contiguous eighth of that order, so the tiles
// that share weights or activations run together on one XCD and meet in its L2.
//
// Kernels, by layer:
//   ffn_bf16_pipe_kernel<MODE, FP8, false>  bf16, d and I multiples of 32, more than 256
//                                           tokens: 320-row tiles, one workgroup per CU
//   ffn_bf16_pipe_kernel<MODE, FP8, true>   the same for at most 256 tokens on packed or
//                                           block-FP8 weights: 64-row tiles, two per CU
//   ffn_bf16_line_kernel<MODE>              at most 256 tokens on row-major weights with K
//                                           a multiple of 64: whole-line stages
//   ffn_bf16_kernel<MODE>                   other bf16 shapes (multiples of 8)
//   ffn_f32_kernel<MODE>                    fp32 layers
#include <type_traits>

#include "common.h"
#include "lds_dma.h"

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
            out[size_t(row0 + row) * ncols + col] = f2bf(swiglu_fast(g, u));
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
//
// Tile: 320 rows x 256 weight rows, K step 32.  An expert with up to 320 rows is a single
// tile, so its weights stream from HBM once (one M-tile per expert covers the prefill
// layer, whose per-expert row counts cluster near T*K*(1-zero share)/N = 256).
// 512 threads = 8 waves, two per SIMD.  Wave w owns the 32-row blocks 2*mb + (w >> 2)
// (mb < 5) against two 32-column weight blocks chosen by w & 3: 5 x 2 blocks of 32x32
// (v_mfma_f32_32x32x16_bf16), 160 fp32 accumulators per lane, which leaves room for two
// full sets of operand fragments.  The waves sharing a SIMD (w, w + 4) take alternate row
// blocks of the same columns, so a partly filled tile keeps every SIMD equally busy.
//   MODE 0 (gate/up): weight rows 0..127 = gate rows n0..n0+127, 128..255 = up rows
//                     n0..n0+127; a wave's two column blocks are the gate and up rows of
//                     the same 32 outputs; activations gathered through perm_token;
//                     epilogue silu(g)*u -> H (128 columns per tile).
//   MODE 1 (down):    weight rows = W_down rows n0..n0+255; activations = H rows;
//                     epilogue -> Y (256 columns per tile).
// Operands reach LDS by direct global->LDS loads (global_load_lds_dwordx4) through a
// 160 KB ring whose stage holds the tile's activation rows (rounded up to 32) and the 256
// weight rows, so few-row tiles get more stages; activation row groups past the tile's
// rows are not loaded.  Layers of few tokens run the few-row form (SMALL): 64-row tiles,
// one row block per wave, half the ring, two workgroups per CU.
// LDS row = 64 bytes = 4 chunks of 16 bytes; chunk c of row r sits in slot c ^ swz(r).
// Software pipeline: a K step has two substeps of 16 (one MFMA deep).  While one substep
// multiplies, the wave reads all its fragments of the next substep into the other
// register set.  Between the substeps of step kt each wave waits for its own LDS reads and
// for its share of stage kt+1, then meets the others at a barrier; past it no wave reads
// stage kt again, so the second substep refills stage kt's slot with stage kt+NST, NST
// steps ahead of its use.
// ---------------------------------------------------------------------------------------

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// 8 E4M3 codes -> 8 bf16 values code * scale (scale a power of two: exact).
__device__ __forceinline__ bf16x8 dequant8(uint2 q, float scale) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.x, scale, false);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.x, scale, true);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.y, scale, false);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.y, scale, true);
  bf16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// FP8 = false: weights bf16, row-major (w0, w1) or, with bpacked, packed by
// lc_moe_pack_weights (w0: this matrix pair's region; stage kt of a unit is one 16 KB block
// holding exactly the LDS image of the stage's 256 weight rows).  FP8 = true: weights are
// the packed block-FP8 codes (qcodes: this matrix pair's region, one 8 KB tile block per stage) with
// fp32 power-of-two scales (qscales; nrb_rows row blocks x nkb column blocks per matrix);
// each weight fragment is converted to bf16 (v_cvt_scalef32_pk_bf16_fp8, exact) one
// substep before its MFMAs, so the MFMAs see exactly the dequantized weights.
// SMALL: the few-row form for layers whose experts get few rows (decode): M-tiles of 64
// rows (one row block per wave) and an 80 KB ring, so two workgroups share a CU and one's
// per-step chain of barrier, LDS reads, conversion and MFMAs runs while the other waits.
template <int MODE, bool FP8, bool SMALL>
__global__ __launch_bounds__(512, SMALL ? 2 : 1) void ffn_bf16_pipe_kernel(
    const bf16_t* __restrict__ a_src, const int32_t* __restrict__ perm_token,
    const bf16_t* __restrict__ w0, const bf16_t* __restrict__ w1,
    const unsigned char* __restrict__ qcodes, const float* __restrict__ qscales, int nrb_rows,
    int nkb, bf16_t* __restrict__ out, const MTile* __restrict__ mtiles,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ n_mtiles_ptr, int kdim,
    int ncols, int n_ntiles, int bpacked, GuGrad gg) {
  constexpr int BM = SMALL ? kBmSmall : kBmPipe;  // 64 / 320
  constexpr bool GATE_UP = MODE != 1;               // MODE 0 forward, MODE 2 backward recompute
  constexpr int BK = 32;                  // K step
  constexpr int LDS_BYTES = (SMALL ? 80 : 160) * 1024;  // the ring
  constexpr int MAX_NST = 16;             // ring stages at most
  constexpr int MB = BM / 64;             // row blocks per wave (5; few-row form 1)
  constexpr int RB = BK * 2;              // bytes per LDS activation row (64)
  constexpr int RPI = 16;                 // rows filled by one wave-wide load
  constexpr int NIA = BM / RPI;           // activation loads per stage (20; 4)
  constexpr int NIB = FP8 ? 8 : 256 / RPI;  // weight loads per stage (8 of 32 FP8 rows, 16)
  constexpr int IA = (NIA + 7) / 8;       // activation load slots per wave (3; 1)
  constexpr int IB = NIB / 8;             // weight loads per wave (1, 2)
  constexpr int B_BYTES = FP8 ? 256 * 32 : 256 * RB;  // 8 KB / 16 KB
  __shared__ __attribute__((aligned(1024))) unsigned char smem[LDS_BYTES];

  int j, ntile;
  if (!unit_of_block(mtiles, offsets, *n_mtiles_ptr, n_ntiles, BM, j, ntile)) return;
  const MTile tile = mtiles[j];
  const int e = tile.expert, row0 = tile.row0, rows = tile.rows;
  const int n0 = ntile * (GATE_UP ? 128 : 256);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;

  // Load sources.  Activation load q (LDS rows 16q..16q+15) and weight load q belong to
  // wave q % 8.  Lane l fills LDS row 16q + l/4, slot l%4, with global chunk
  // (l%4) ^ swz4(row).  Activation loads whose 16 rows all lie past the tile's rows are
  // skipped; they are a suffix of the wave's list, so the wave issues its first na.
  const bf16_t* srcA[IA];
  const bf16_t* srcB[IB];
  const int lrow = lane >> 2, lslot = lane & 3;
  int na = 0;
#pragma unroll
  for (int i = 0; i < IA; ++i) {
    const int q = wave + 8 * i;
    const int r = q * RPI + lrow;
    na += (q < NIA && q * RPI < rows) ? 1 : 0;
    const int ar = r < rows ? r : 0;  // rows past the tile read a valid row; never stored
    const size_t src_row = GATE_UP ? size_t(perm_token[row0 + ar]) : size_t(row0 + ar);
    srcA[i] = a_src + src_row * kdim + (lslot ^ swz4(r)) * 8;
  }
  // FP8: weight load q is the 1 KB piece q of the stage's 8 KB tile block, copied as is.
  // (addressed through a bf16_t pointer like the other weight loads, so the compiler's
  // alias view of these loads matches theirs and it adds no waits of its own)
  const bf16_t* srcQ = nullptr;
  if (FP8) {
    srcQ = reinterpret_cast<const bf16_t*>(qcodes + (size_t(e) * n_ntiles + ntile) * (kdim / BK) * size_t(8192) +
                                           wave * 1024 + lane * 16);
  } else if (bpacked) {
    // packed bf16: weight load q is the 1 KB piece q of the stage's 16 KB block (the block
    // of K step k starts k * 8192 elements, i.e. kphys * 256, into the unit's blocks)
#pragma unroll
    for (int i = 0; i < IB; ++i)
      srcB[i] = w0 + (size_t(e) * n_ntiles + ntile) * (kdim / BK) * size_t(8192) + (wave + 8 * i) * 512 +
                lane * 8;
  } else {
#pragma unroll
    for (int i = 0; i < IB; ++i) {
      const int r = (wave + 8 * i) * RPI + lrow;  // weight row of the tile, 0..255
      int c;
      const bf16_t* mat;
      if (GATE_UP) {
        c = n0 + (r & 127);
        mat = r < 128 ? w0 : w1;
      } else {
        c = n0 + r;
        mat = w0;
      }
      const int brow = c < ncols ? c : n0;  // columns past the matrix repeat a valid row
      srcB[i] = mat + (size_t(e) * ncols + brow) * kdim + (lslot ^ swz4(r)) * 8;
    }
  }
  const int per_stage = na + IB;  // this wave's loads per stage (vmcnt increments)
  const int nk = kdim / BK;
  // Each work unit starts its K loop at its own offset: rows of one tile share their low
  // address bits (row strides are multiples of 4 KB), so tiles running side by side are
  // spread over the memory channels.
  const int krot = (j * 7 + ntile * 3) % nk;
  auto kphys = [&](int kt) { const int k = kt + krot; return (k >= nk ? k - nk : k) * BK; };
  // Ring geometry from the tile's rows: a stage holds the activation rows the MFMAs read
  // (rows rounded up to 32) and the 256 weight rows, and the ring has as many stages as
  // fit in its 160 KB (few-row form: 80 KB), up to 16 (bf16 weights: 4 at 320 rows, 5 at
  // 256, 4 at up to 64 rows in 80 KB; FP8 weights: 5 at 320 rows, 8 at up to 32 rows in
  // 80 KB).  Loads run that many stages ahead, so few-row tiles keep more weight bytes in
  // flight.
  const int a_bytes = __builtin_amdgcn_readfirstlane(((rows + 31) & ~31) * RB);
  const int stage_bytes = a_bytes + B_BYTES;
  const int nst = LDS_BYTES / stage_bytes < MAX_NST ? LDS_BYTES / stage_bytes : MAX_NST;
  // this wave's load number i (0..IA+IB-1) of stage kt, into ring slot `slot`
  auto issue_one = [&](int i, int kt, int slot) {
    unsigned char* st = smem + slot * stage_bytes;
    if (i < IA) {
      if (i < na) dma16(srcA[i] + kphys(kt), st + (wave + 8 * i) * 1024);
    } else if (FP8) {  // the packed layouts are read once in whole lines: streaming loads
      dma16_stream(srcQ + size_t(kphys(kt)) * 128, st + a_bytes + wave * 1024);  // 8 KB per stage
    } else if (bpacked) {
      dma16_stream(srcB[i - IA] + size_t(kphys(kt)) * 256, st + a_bytes + (wave + 8 * (i - IA)) * 1024);
    } else {
      dma16(srcB[i - IA] + kphys(kt), st + a_bytes + (wave + 8 * (i - IA)) * 1024);
    }
  };
  // wait until this wave's loads of stage s landed, `newest` being the last stage issued
  auto wait_stage = [&](int s, int newest) { wait_vmcnt((newest - s) * per_stage); };

  const int l32 = lane & 31, sw = swz4(l32), khalf = lane >> 5;
  int boff[2];  // LDS byte offset of this lane's row in the wave's two weight blocks
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
    boff[nb] = a_bytes + (FP8 ? (wn * 32 + l32) * 64  // FP8: pair-row wn*32 + l32 holds both blocks
                              : ((GATE_UP ? nb * 128 + wn * 32 : wn * 64 + nb * 32) + l32) * RB);
  // FP8 scales of the wave's two weight blocks (the rows of one 32-row weight block lie in
  // one 128-row block): lane l holds the scale of column block l in vsc[nb][0] and of
  // column block 64 + l in vsc[nb][1] (nkb <= 128), loaded once before the loads start;
  // stage kt reads column block kphys(kt) / 128 from them with v_readlane.
  float vsc[2][2] = {{1.f, 1.f}, {1.f, 1.f}};
  if (FP8) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      // MODE 1: the 256-row n-tile spans two 128-row blocks; in the last n-tile of a
      // matrix whose rows end in its first half the second block does not exist (its rows
      // hold zero codes), so its lanes take the last block's scales instead.
      const int rb = MODE == 0 ? ntile : min(ntile * 2 + ((wn * 64 + nb * 32) >> 7), nrb_rows - 1);
      const int sbase = MODE == 0 ? ((e * 2 + nb) * nrb_rows + rb) * nkb : (e * nrb_rows + rb) * nkb;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kb = h * 64 + lane;
        vsc[nb][h] = qscales[sbase + (kb < nkb ? kb : nkb - 1)];  // lanes past nkb: unused
      }
    }
    LCM_WAIT_VMCNT(0);  // before the first direct load, so the vmcnt counts below hold
  }
  int nvb = 0;  // row blocks of this wave holding tile rows (a prefix in mb)
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) nvb += (mb * 2 + wm) * 32 < rows;

  f32x16 acc[MB][2];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.f;

  const int npro = nk < nst ? nk : nst;
  for (int s = 0; s < npro; ++s)
    for (int i = 0; i < IA + IB; ++i) issue_one(i, s, s);

  auto run = [&](auto nv_tag) {
    constexpr int NV = decltype(nv_tag)::value;  // row blocks holding tile rows
    // Weight fragments as read from LDS; FP8: b[0] holds the codes of both blocks (the 16
    // bytes of one read).  Every LDS operand read here has the bf16x8 type: the compiler's
    // type-based alias analysis then keeps the reads apart from the LDS writes of the direct
    // loads and it adds no waits of its own (the explicit vmcnt waits order them).  Reading
    // the FP8 bytes as an integer vector made it wait for every load in flight before each
    // read.
    using BFrag = bf16x8;
    auto rd = [&](int ring_slot, int ks, bf16x8 (&a)[MB], BFrag (&b)[2]) {
      const unsigned char* st = smem + ring_slot * stage_bytes;
      const int slot = ((ks * 2 + khalf) ^ sw) * 16;
#pragma unroll
      for (int mb = 0; mb < NV; ++mb)
        a[mb] = *reinterpret_cast<const bf16x8*>(st + ((mb * 2 + wm) * 32 + l32) * RB + slot);
      if constexpr (FP8) {
        // one 16-byte read: 8 codes of the block-0 row, then 8 codes of the block-1 row
        b[0] = *reinterpret_cast<const bf16x8*>(st + boff[0] + slot);
      } else {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) b[nb] = *reinterpret_cast<const bf16x8*>(st + boff[nb] + slot);
      }
    };
    // FP8 block scales of stage kt for the wave's two weight blocks
    auto scales_of = [&](int kt, float (&sc)[2]) {
      if constexpr (FP8) {
        const int kb = __builtin_amdgcn_readfirstlane(kphys(kt) >> 7);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const float v = kb < 64 ? vsc[nb][0] : vsc[nb][1];
          sc[nb] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), kb & 63));
        }
      }
    };
    // FP8: the two weight fragments of one substep as bf16 (codes times scales, exact).
    // Each substep's fragments are converted one substep ahead, right after the MFMAs of
    // the substep before were issued, so the conversions run beside those MFMAs instead of
    // holding up the MFMAs that need them.
    auto cvt = [&](const BFrag (&bq)[2], const float (&sc)[2], bf16x8 (&b)[2]) {
      if constexpr (FP8 && NV > 0) {  // waves without rows skip it
        const uint4 q = __builtin_bit_cast(uint4, bq[0]);
        b[0] = dequant8(make_uint2(q.x, q.y), sc[0]);
        b[1] = dequant8(make_uint2(q.z, q.w), sc[1]);
      }
    };
    // Keeps converted fragments where they are computed: without it the compiler sinks
    // the conversions to their first use, past the barrier, back onto the MFMAs' path.
    auto pin = [&](bf16x8 (&b)[2]) {
      if constexpr (FP8 && NV > 0) asm volatile("" : "+v"(b[0]), "+v"(b[1]));
    };
    // MFMAs of one substep on bf16 weight fragments b; with DMA, this wave's loads of stage
    // kt_load (into ring slot `slot`) go one per row block, the rest after the last block.
    auto mm = [&](const bf16x8 (&a)[MB], const bf16x8 (&b)[2], auto dma, int kt_load, int slot) {
      constexpr bool DMA = decltype(dma)::value;
#pragma unroll
      for (int mb = 0; mb < NV; ++mb) {
        if (DMA && mb < IA + IB) issue_one(mb, kt_load, slot);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mb], b[nb], acc[mb][nb], 0, 0, 0);
      }
      if (DMA)
        for (int i = NV; i < IA + IB; ++i) issue_one(i, kt_load, slot);
    };
    bf16x8 ca[MB], xa[MB];  // activation fragments of the current / next substep
    BFrag cb[2], xb[2];     // weight fragments of the current / next substep, as read
    bf16x8 cw[2], xw[2];    // FP8: the same converted to bf16
    float sc[2] = {1.f, 1.f}, scn[2] = {1.f, 1.f};  // FP8 scales of stages kt / kt+1
    scales_of(0, sc);
    wait_stage(0, npro - 1);
    block_barrier();
    rd(0, 0, ca, cb);
    cvt(cb, sc, cw);
    int sk = 0;  // ring slot of stage kt
    auto step = [&](int kt, auto more_tag, auto last_tag) {
      constexpr bool LAST = decltype(last_tag)::value;
      const int sk1 = sk + 1 == nst ? 0 : sk + 1;  // slot of stage kt+1
      if (!LAST) scales_of(kt + 1, scn);
      rd(sk, 1, xa, xb);
      if constexpr (FP8) {
        mm(ca, cw, std::false_type{}, 0, 0);
        __builtin_amdgcn_sched_barrier(0);  // conversions after the MFMAs, before the wait
        cvt(xb, sc, xw);
        pin(xw);
      } else {
        mm(ca, cb, std::false_type{}, 0, 0);
      }
      if (!LAST) {
        wait_lds_reads();  // this wave's reads of stage kt done
        const int newest = kt + nst - 1 < nk - 1 ? kt + nst - 1 : nk - 1;
        wait_stage(kt + 1, newest);
        block_barrier();  // stage kt+1 visible to all waves; nobody reads stage kt again
        rd(sk1, 0, ca, cb);
      }
      // stage kt+nst takes stage kt's slot
      if constexpr (FP8) {
        mm(xa, xw, more_tag, kt + nst, sk);
        __builtin_amdgcn_sched_barrier(0);
        if (!LAST) {
          cvt(cb, scn, cw);
          pin(cw);
        }
      } else {
        mm(xa, xb, more_tag, kt + nst, sk);
      }
      sk = sk1;
      if (!LAST) {
        sc[0] = scn[0];
        sc[1] = scn[1];
      }
    };
    const int nmain = nk - nst > 0 ? nk - nst : 0;
    for (int kt = 0; kt < nmain; ++kt) step(kt, std::true_type{}, std::false_type{});
    for (int kt = nmain; kt < nk - 1; ++kt) step(kt, std::false_type{}, std::false_type{});
    step(nk - 1, std::false_type{}, std::true_type{});
  };
  if constexpr (MB == 1) {
    if (nvb == 0) run(std::integral_constant<int, 0>{});
    else run(std::integral_constant<int, 1>{});
  } else {
    switch (nvb) {
      case 0: run(std::integral_constant<int, 0>{}); break;
      case 1: run(std::integral_constant<int, 1>{}); break;
      case 2: run(std::integral_constant<int, 2>{}); break;
      case 3: run(std::integral_constant<int, 3>{}); break;
      case 4: run(std::integral_constant<int, 4>{}); break;
      default: run(std::integral_constant<int, 5>{}); break;
    }
  }

  // epilogue; 32x32 D layout: column lane & 31, rows 8*(r/4) + 4*(lane/32) + r%4
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    if (mb >= nvb) continue;
    if (MODE == 0) {
      const int col = n0 + wn * 32 + l32;
      if (col >= ncols) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = (mb * 2 + wm) * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3);
        if (row < rows)
          out[size_t(row0 + row) * ncols + col] = f2bf(swiglu_fast(acc[mb][0][r], acc[mb][1][r]));
      }
    } else if (MODE == 2) {
      // backward of the SwiGLU (s = sigmoid(G), a = G s): g*H = g a U, dG = dH U (s + a (1 - s)),
      // dU = dH a, each rounded to bf16
      const int col = n0 + wn * 32 + l32;
      if (col >= ncols) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = (mb * 2 + wm) * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3);
        if (row >= rows) continue;
        const size_t o = size_t(row0 + row) * ncols + col;
        const float G = acc[mb][0][r], U = acc[mb][1][r];
        const float sg = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-G * 1.4426950408889634f));
        const float act = G * sg;
        const float dh = gg.dh[o], g = gg.g_row[row0 + row];
        out[o] = f2bf(g * (act * U));
        gg.dg[o] = f2bf(dh * U * (sg + act * (1.f - sg)));
        gg.du[o] = f2bf(dh * act);
      }
    } else {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int col = n0 + wn * 64 + nb * 32 + l32;
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

#define LCM_INST(M, Q, S)                                                                     \
  template __global__ void ffn_bf16_pipe_kernel<M, Q, S>(                                     \
      const bf16_t* __restrict__, const int32_t* __restrict__, const bf16_t* __restrict__,    \
      const bf16_t* __restrict__, const unsigned char* __restrict__, const float* __restrict__, \
      int, int, bf16_t* __restrict__, const MTile* __restrict__, const int32_t* __restrict__, \
      const int32_t* __restrict__, int, int, int, int, GuGrad);
LCM_INST(2, false, false)
LCM_INST(2, false, true)
LCM_INST(0, false, false)
LCM_INST(1, false, false)
LCM_INST(0, true, false)
LCM_INST(1, true, false)
LCM_INST(0, false, true)
LCM_INST(1, false, true)
LCM_INST(0, true, true)
LCM_INST(1, true, true)
#undef LCM_INST

// ---------------------------------------------------------------------------------------
// Whole-line kernel: the few-row form for row-major bf16 weights (layers of at most 256
// tokens, K a multiple of 64).  The 320-row and few-row forms above stage 32 K elements of
// 256 weight rows, i.e. half of each row's 128-byte line per stage, and the other half one
// stage later: the line has to stay in the L2 in between, and a decode layer streamed its
// weights at 72-75% of the HBM peak.  Here a stage holds 64 K elements of 128 weight rows
// -- whole lines, read once, so they take the streaming hint -- and the two halves of the
// tile's 256 weight rows alternate:
//   MODE 0: even stages gate rows n0..n0+127, odd stages up rows n0..n0+127;
//   MODE 1: even stages W_down rows n0..n0+127, odd stages n0+128..n0+255.
// A stage also holds the tile's activation rows for its 64 K elements (read from L2 by both
// stages of the pair).  LDS rows are 128 bytes = 8 chunks; chunk c of row r sits in slot
// c ^ swz8(r), which spreads the 16 rows a read phase touches over all 64 banks.
// 512 threads = 8 waves, two workgroups per CU: wave w owns the 32-row block w >> 2 of the
// 64-row tile against the 32 weight rows 32 * (w & 3) of each half; a stage is 4 substeps
// of 16.  Ring, waits and barriers as in the kernel above.
// ---------------------------------------------------------------------------------------
__host__ __device__ __forceinline__ int swz8(int r) { return (r >> 1) & 7; }

template <int MODE>
__global__ __launch_bounds__(512, 2) void ffn_bf16_line_kernel(
    const bf16_t* __restrict__ a_src, const int32_t* __restrict__ perm_token,
    const bf16_t* __restrict__ w0, const bf16_t* __restrict__ w1, bf16_t* __restrict__ out,
    const MTile* __restrict__ mtiles, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ n_mtiles_ptr, int kdim, int ncols, int n_ntiles) {
  constexpr int BM = kBmSmall;          // 64 rows
  constexpr int BK = 64;                // K elements per stage
  constexpr int RB = BK * 2;            // bytes per LDS row (128)
  constexpr int LDS_BYTES = 80 * 1024;  // the ring
  constexpr int MAX_NST = 16;
  constexpr int B_BYTES = 128 * RB;     // 16 KB: one half's 128 weight rows
  __shared__ __attribute__((aligned(1024))) unsigned char smem[LDS_BYTES];

  int j, ntile;
  if (!unit_of_block(mtiles, offsets, *n_mtiles_ptr, n_ntiles, BM, j, ntile)) return;
  const MTile tile = mtiles[j];
  const int e = tile.expert, row0 = tile.row0, rows = tile.rows;
  const int n0 = ntile * (MODE == 0 ? 128 : 256);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int lrow = lane >> 3, lslot = lane & 7;

  // Activation load of wave w: LDS rows 8w..8w+7 (lane l: row 8w + l/8, slot l%8, global
  // chunk (l%8) ^ swz8(row)); skipped when all 8 rows lie past the tile's rows.
  const int na = wave * 8 < rows ? 1 : 0;
  const int ra = wave * 8 + lrow;
  const int ar = ra < rows ? ra : 0;  // rows past the tile read a valid row; never stored
  const size_t a_row = MODE == 0 ? size_t(perm_token[row0 + ar]) : size_t(row0 + ar);
  const bf16_t* srcA = a_src + a_row * kdim + (lslot ^ swz8(ra)) * 8;
  // Weight load i of wave w in half h: rows 8(w + 8i)..+7 of the half's 128 rows.
  const bf16_t* srcB[2][2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = (wave + 8 * i) * 8 + lrow;  // 0..127
      const int c = MODE == 0 ? n0 + r : n0 + h * 128 + r;
      const bf16_t* mat = MODE == 0 ? (h ? w1 : w0) : w0;
      const int brow = c < ncols ? c : n0;  // rows past the matrix repeat a valid row
      srcB[h][i] = mat + (size_t(e) * ncols + brow) * kdim + (lslot ^ swz8(r)) * 8;
    }
  const int per_stage = na + 2;  // this wave's loads per stage
  const int nk = kdim / BK;      // K chunks
  const int total = 2 * nk;      // stages: two halves per K chunk
  // each work unit starts its K loop at its own chunk (spreads tiles over the channels)
  const int krot = (j * 7 + ntile * 3) % nk;
  auto kphys = [&](int kt) { const int k = (kt >> 1) + krot; return (k >= nk ? k - nk : k) * BK; };
  const int a_bytes = __builtin_amdgcn_readfirstlane(((rows + 31) & ~31) * RB);
  const int stage_bytes = a_bytes + B_BYTES;
  const int nst = LDS_BYTES / stage_bytes < MAX_NST ? LDS_BYTES / stage_bytes : MAX_NST;  // 4 (<= 32 rows), 3
  auto issue_one = [&](int i, int kt, int slot) {
    unsigned char* st = smem + slot * stage_bytes;
    if (i == 0) {
      if (na) dma16(srcA + kphys(kt), st + wave * 1024);
    } else {
      const bf16_t* g = (kt & 1) ? srcB[1][i - 1] : srcB[0][i - 1];
      dma16_stream(g + kphys(kt), st + a_bytes + (wave + 8 * (i - 1)) * 1024);
    }
  };
  auto wait_stage = [&](int s, int newest) { wait_vmcnt((newest - s) * per_stage); };

  const int l32 = lane & 31, khalf = lane >> 5;
  const int arow = wm * 32 + l32, brow_l = wn * 32 + l32;
  const int sa = swz8(arow), sb = swz8(brow_l);
  const bool active = wm * 32 < rows;  // this wave's row block holds tile rows

  f32x16 acc[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[h][r] = 0.f;

  const int npro = total < nst ? total : nst;
  for (int s2 = 0; s2 < npro; ++s2)
    for (int i = 0; i < 3; ++i) issue_one(i, s2, s2);

  auto run = [&](auto act_tag) {
    constexpr bool ACT = decltype(act_tag)::value;
    auto rd = [&](int ring_slot, int ks, bf16x8& a, bf16x8& b) {
      if constexpr (ACT) {
        const unsigned char* st = smem + ring_slot * stage_bytes;
        const int c = ks * 2 + khalf;
        a = *reinterpret_cast<const bf16x8*>(st + arow * RB + ((c ^ sa) << 4));
        b = *reinterpret_cast<const bf16x8*>(st + a_bytes + brow_l * RB + ((c ^ sb) << 4));
      }
    };
    // MFMA of one substep into the half's accumulator; with DMA, this wave's loads of
    // stage kt_load go out behind it
    auto mm = [&](auto h_tag, const bf16x8& a, const bf16x8& b, bool dma, int kt_load, int slot) {
      constexpr int H = decltype(h_tag)::value;
      if constexpr (ACT) acc[H] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[H], 0, 0, 0);
      if (dma)
        for (int i = 0; i < 3; ++i) issue_one(i, kt_load, slot);
    };
    bf16x8 ca, cb, xa, xb;
    wait_stage(0, npro - 1);
    block_barrier();
    rd(0, 0, ca, cb);
    int sk = 0;
    auto step = [&](int kt, auto h_tag, auto last_tag) {
      constexpr bool LAST = decltype(last_tag)::value;
      const int sk1 = sk + 1 == nst ? 0 : sk + 1;
      rd(sk, 1, xa, xb);
      mm(h_tag, ca, cb, false, 0, 0);
      rd(sk, 2, ca, cb);
      mm(h_tag, xa, xb, false, 0, 0);
      rd(sk, 3, xa, xb);
      mm(h_tag, ca, cb, false, 0, 0);
      if (!LAST) {
        wait_lds_reads();  // this wave's reads of stage kt done
        const int newest = kt + nst - 1 < total - 1 ? kt + nst - 1 : total - 1;
        wait_stage(kt + 1, newest);
        block_barrier();  // stage kt+1 visible to all waves; nobody reads stage kt again
        rd(sk1, 0, ca, cb);
      }
      mm(h_tag, xa, xb, kt + nst < total, kt + nst, sk);  // stage kt+nst takes stage kt's slot
      sk = sk1;
    };
    using H0 = std::integral_constant<int, 0>;
    using H1 = std::integral_constant<int, 1>;
    for (int kt = 0; kt < total - 2; kt += 2) {
      step(kt, H0{}, std::false_type{});
      step(kt + 1, H1{}, std::false_type{});
    }
    step(total - 2, H0{}, std::false_type{});
    step(total - 1, H1{}, std::true_type{});
  };
  if (active) run(std::true_type{});
  else run(std::false_type{});

  if (!active) return;
  // epilogue; 32x32 D layout: column lane & 31, rows 8*(r/4) + 4*(lane/32) + r%4
  if (MODE == 0) {
    const int col = n0 + wn * 32 + l32;
    if (col < ncols) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3);
        if (row < rows) out[size_t(row0 + row) * ncols + col] = f2bf(swiglu_fast(acc[0][r], acc[1][r]));
      }
    }
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int col = n0 + h * 128 + wn * 32 + l32;
      if (col >= ncols) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3);
        if (row < rows) out[size_t(row0 + row) * ncols + col] = f2bf(acc[h][r]);
      }
    }
  }
}

template __global__ void ffn_bf16_line_kernel<0>(const bf16_t* __restrict__, const int32_t* __restrict__,
                                                 const bf16_t* __restrict__, const bf16_t* __restrict__,
                                                 bf16_t* __restrict__, const MTile* __restrict__,
                                                 const int32_t* __restrict__, const int32_t* __restrict__, int,
                                                 int, int);
template __global__ void ffn_bf16_line_kernel<1>(const bf16_t* __restrict__, const int32_t* __restrict__,
                                                 const bf16_t* __restrict__, const bf16_t* __restrict__,
                                                 bf16_t* __restrict__, const MTile* __restrict__,
                                                 const int32_t* __restrict__, const int32_t* __restrict__, int,
                                                 int, int);

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

// The instantiation of the pipelined kernel for the layer: its few-row form for layers of
// few tokens, else the 320-row form (the M-tile list was built with the matching height).
using PipeKernel = void (*)(const bf16_t*, const int32_t*, const bf16_t*, const bf16_t*,
                            const unsigned char*, const float*, int, int, bf16_t*, const MTile*,
                            const int32_t*, const int32_t*, int, int, int, int, GuGrad);
template <int MODE, bool FP8>
PipeKernel pipe_kernel(const lc_moe_shape& s) {
  return ffn_small(s) ? ffn_bf16_pipe_kernel<MODE, FP8, true> : ffn_bf16_pipe_kernel<MODE, FP8, false>;
}

hipError_t launch_ffn_gate_up(const lc_moe_shape& s, const void* x, const int32_t* perm_token,
                              const void* w_gate, const void* w_up, const void* fp8,
                              const void* packed, void* hbuf, const MTile* mtiles,
                              const int32_t* offsets, const int32_t* n_mtiles, int mt_max,
                              hipStream_t st) {
  if (s.dtype == LC_MOE_BF16 && ffn_pipelined(s)) {
    const int nn = (s.I + 127) / 128;
    const size_t units = size_t(mt_max) * nn;
    const unsigned grid = static_cast<unsigned>((units + 7) / 8 * 8);
    const Fp8Plan q = plan_fp8(s);
    const unsigned char* qb = static_cast<const unsigned char*>(fp8);
    if (fp8)
      pipe_kernel<0, true>(s)<<<dim3(grid), dim3(512), 0, st>>>(
          static_cast<const bf16_t*>(x), perm_token, nullptr, nullptr, qb + q.codes_gu,
          reinterpret_cast<const float*>(qb + q.scales_gu), q.nrb_i, q.nrb_d,
          static_cast<bf16_t*>(hbuf), mtiles, offsets, n_mtiles, s.d, s.I, nn, 0, GuGrad{});
    else if (packed)
      pipe_kernel<0, false>(s)<<<dim3(grid), dim3(512), 0, st>>>(
          static_cast<const bf16_t*>(x), perm_token,
          reinterpret_cast<const bf16_t*>(static_cast<const unsigned char*>(packed) + plan_packed(s).gu),
          nullptr, nullptr, nullptr, 0, 0, static_cast<bf16_t*>(hbuf), mtiles, offsets, n_mtiles, s.d,
          s.I, nn, 1, GuGrad{});
    else if (ffn_small(s) && s.d % 64 == 0)
      ffn_bf16_line_kernel<0><<<dim3(grid), dim3(512), 0, st>>>(
          static_cast<const bf16_t*>(x), perm_token, static_cast<const bf16_t*>(w_gate),
          static_cast<const bf16_t*>(w_up), static_cast<bf16_t*>(hbuf), mtiles, offsets, n_mtiles, s.d,
          s.I, nn);
    else
      pipe_kernel<0, false>(s)<<<dim3(grid), dim3(512), 0, st>>>(
          static_cast<const bf16_t*>(x), perm_token, static_cast<const bf16_t*>(w_gate),
          static_cast<const bf16_t*>(w_up), nullptr, nullptr, 0, 0, static_cast<bf16_t*>(hbuf),
          mtiles, offsets, n_mtiles, s.d, s.I, nn, 0, GuGrad{});
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

hipError_t launch_ffn_gate_up_grad(const lc_moe_shape& s, const void* x, const int32_t* perm_token,
                                   const void* w_gate, const void* w_up, const GuGrad& gg, void* gh,
                                   const MTile* mtiles, const int32_t* offsets, const int32_t* n_mtiles,
                                   int mt_max, hipStream_t st) {
  const int nn = (s.I + 127) / 128;
  const size_t units = size_t(mt_max) * nn;
  const unsigned grid = static_cast<unsigned>((units + 7) / 8 * 8);
  pipe_kernel<2, false>(s)<<<dim3(grid), dim3(512), 0, st>>>(
      static_cast<const bf16_t*>(x), perm_token, static_cast<const bf16_t*>(w_gate),
      static_cast<const bf16_t*>(w_up), nullptr, nullptr, 0, 0, static_cast<bf16_t*>(gh), mtiles, offsets,
      n_mtiles, s.d, s.I, nn, 0, gg);
  return hipGetLastError();
}

hipError_t launch_ffn_down(const lc_moe_shape& s, const void* hbuf, const void* w_down,
                           const void* fp8, const void* packed, void* ybuf, const MTile* mtiles,
                           const int32_t* offsets, const int32_t* n_mtiles, int mt_max,
                           hipStream_t st) {
  if (s.dtype == LC_MOE_BF16 && ffn_pipelined(s)) {
    const int nn = (s.d + 255) / 256;
    const size_t units = size_t(mt_max) * nn;
    const unsigned grid = static_cast<unsigned>((units + 7) / 8 * 8);
    const Fp8Plan q = plan_fp8(s);
    const unsigned char* qb = static_cast<const unsigned char*>(fp8);
    if (fp8)
      pipe_kernel<1, true>(s)<<<dim3(grid), dim3(512), 0, st>>>(
          static_cast<const bf16_t*>(hbuf), nullptr, nullptr, nullptr, qb + q.codes_d,
          reinterpret_cast<const float*>(qb + q.scales_d), q.nrb_d, q.nrb_i,
          static_cast<bf16_t*>(ybuf), mtiles, offsets, n_mtiles, s.I, s.d, nn, 0, GuGrad{});
    else if (packed)
      pipe_kernel<1, false>(s)<<<dim3(grid), dim3(512), 0, st>>>(
          static_cast<const bf16_t*>(hbuf), nullptr,
          reinterpret_cast<const bf16_t*>(static_cast<const unsigned char*>(packed) + plan_packed(s).d),
          nullptr, nullptr, nullptr, 0, 0, static_cast<bf16_t*>(ybuf), mtiles, offsets, n_mtiles, s.I,
          s.d, nn, 1, GuGrad{});
    else if (ffn_small(s) && s.I % 64 == 0)
      ffn_bf16_line_kernel<1><<<dim3(grid), dim3(512), 0, st>>>(
          static_cast<const bf16_t*>(hbuf), nullptr, static_cast<const bf16_t*>(w_down), nullptr,
          static_cast<bf16_t*>(ybuf), mtiles, offsets, n_mtiles, s.I, s.d, nn);
    else
      pipe_kernel<1, false>(s)<<<dim3(grid), dim3(512), 0, st>>>(
          static_cast<const bf16_t*>(hbuf), nullptr, static_cast<const bf16_t*>(w_down), nullptr,
          nullptr, nullptr, 0, 0, static_cast<bf16_t*>(ybuf), mtiles, offsets, n_mtiles, s.I, s.d,
          nn, 0, GuGrad{});
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

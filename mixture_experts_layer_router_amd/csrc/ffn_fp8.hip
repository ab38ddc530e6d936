// The FP8 MFMA grouped FFN: block-FP8 weights and block-FP8 activations on gfx950's scaled
// FP8 MFMA (LongCat-Flash article, itouyu.top, section "System-level optimisation",
// quantization paragraph: fine-grained block quantization as in DeepSeek-V3; here weights
// in 128 x 128 blocks and activations in 1 x 128 blocks, power-of-two scales).
//
//   quantize_act_kernel          x [T][d] bf16 -> E4M3 codes + one E8M0 scale per 128 columns
//   ffn_fp8_mfma_kernel<0, S>    G = Q(x) Q(W_gate)^T, U = Q(x) Q(W_up)^T; H = silu(G) U is
//                                quantized in the epilogue, per row and 128-column n-tile
//   ffn_fp8_mfma_kernel<1, S>    Y = Q(H) Q(W_down)^T (bf16)
//
// v_mfma_scale_f32_32x32x64_f8f6f4 multiplies E4M3 codes and applies one E8M0 scale per row
// (A) or column (B) and 32-element K block, taking the scale of row m's K block kb from lane
// m + 32 kb.  The products are exact (the dequantized operands' products), but the sums are
// not fp32-exact: the instruction adds its 64 products and the accumulator with about 12
// bits below the largest addend, so a chained K loop carries errors up to about
// 2^-13 (|G| + rss of G's products), measured.  Every scale here covers 128 K elements, so
// lanes m and m + 32 pass the same scale and each lane may hold any 32 of its row's 64 K
// codes as long as A and B agree: lane l (half h = l / 32) holds K h*32 .. h*32 + 31 of the
// stage.
//
// A 64-element K stage of FP8 codes is 64 bytes per row, the same bytes as a 32-element
// bf16 stage, so the ring, the direct global->LDS loads, the waits and the XCD-aware unit
// order are those of the pipelined bf16 kernel (ffn.hip), with twice the MACs per stage:
//   activation rows: 64 bytes per row, 16-byte chunk c in slot c ^ swz4(row)
//   weight rows: the packed block-FP8 layout of lc_moe_quantize_weights, whose 8 KB blocks
//   of two consecutive 32-element K steps are adjacent (one contiguous 16 KB per stage)
// The activation scales of the tile's rows are copied to LDS when a unit starts; the weight
// scales of the wave's two column blocks sit in registers.
#include <type_traits>

#include "common.h"
#include "fp8.h"
#include "lanes.h"
#include "lds_dma.h"

namespace lcm {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// 16 lanes per 128-column block of one row, 8 columns (one 16-byte load) per lane; the
// blocks of a row are consecutive 16-lane groups, so a group never straddles two rows.  cols
// is a multiple of 64: in a last block of 64 columns the upper 8 lanes hold nothing.
__global__ __launch_bounds__(256) void quantize_act_kernel(const bf16_t* __restrict__ x,
                                                           unsigned char* __restrict__ codes,
                                                           unsigned char* __restrict__ scales,
                                                           int rows, int cols, int nkb) {
  const size_t t = size_t(blockIdx.x) * 256 + threadIdx.x;
  const size_t per_row = size_t(nkb) * 16;
  const bool live = t < size_t(rows) * per_row;  // whole 16-lane groups live or not
  const int r = live ? int(t / per_row) : 0;
  const int j = int(t - size_t(r) * per_row), cb = j >> 4;
  const int c = cb * 128 + (j & 15) * 8;
  const bool in = live && c < cols;
  float v[8];
  float amax = 0.f;
  if (in) {
    const uint4 u = *reinterpret_cast<const uint4*>(x + size_t(r) * cols + c);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = bf2f(bf16_t(w[q] & 0xFFFF));
      v[2 * q + 1] = bf2f(bf16_t(w[q] >> 16));
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) amax = fmaxf(amax, fabsf(v[q]));
  }
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));  // within the group
  const int k = block_exp(amax);
  if (in) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      lo |= e4m3_code(ldexpf(v[q], -k)) << (8 * q);
      hi |= e4m3_code(ldexpf(v[q + 4], -k)) << (8 * q);
    }
    *reinterpret_cast<uint2*>(codes + size_t(r) * cols + c) = make_uint2(lo, hi);
  }
  if (live && (j & 15) == 0) scales[size_t(r) * nkb + cb] = static_cast<unsigned char>(k + 127);
}

// Map a workgroup to (M-tile j, n-tile), as the pipelined bf16 kernel does.
__device__ __forceinline__ bool fp8_unit_of_block(const MTile* __restrict__ mtiles,
                                                  const int32_t* __restrict__ offsets, int n_mtiles,
                                                  int n_ntiles, int bm, int& j, int& ntile) {
  const int U = n_mtiles * n_ntiles;
  const int per = (U + 7) >> 3;
  const int slot = blockIdx.x >> 3;
  if (slot >= per) return false;
  const int u = (blockIdx.x & 7) * per + slot;
  if (u >= U) return false;
  const MTile tb = mtiles[u / n_ntiles];
  const int mt = (offsets[tb.expert + 1] - offsets[tb.expert] + bm - 1) / bm;
  const int ul = u - tb.first_tile * n_ntiles;
  ntile = ul / mt;
  j = tb.first_tile + (ul - ntile * mt);
  return true;
}

// MODE 0 (gate/up): activations = x codes of the tile's tokens (through perm_token) with
// their scales; weight rows 0..127 of the n-tile's pair rows = gate and up rows n0..n0+127;
// epilogue: H = silu(G) U quantized per row and n-tile (128 H columns) into hq / hs.
// MODE 1 (down): activations = H codes of the tile's rows; weight pair rows = W_down rows
// of the 256-row n-tile; epilogue: Y (bf16) into yout.
// 512 threads = 8 waves: wave w owns row blocks 2 mb + (w >> 2) and column blocks (w & 3)
// of both halves, as in the bf16 kernel; per stage one MFMA (K = 64) per block.
template <int MODE, bool SMALL>
__global__ __launch_bounds__(512, SMALL ? 2 : 1) void ffn_fp8_mfma_kernel(
    const unsigned char* __restrict__ a_codes, const unsigned char* __restrict__ a_scales,
    const int32_t* __restrict__ perm_token, const unsigned char* __restrict__ qcodes,
    const float* __restrict__ qscales, int nrb_rows, bf16_t* __restrict__ yout,
    unsigned char* __restrict__ hq, unsigned char* __restrict__ hs, const MTile* __restrict__ mtiles,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ n_mtiles_ptr, int kdim, int ncols,
    int n_ntiles) {
  constexpr int BM = SMALL ? kBmSmall : kBmPipe;  // 64 / 320
  constexpr int BK = 64;                          // K elements (= bytes) per stage
  constexpr int LDS_BYTES = (SMALL ? 80 : 160) * 1024;
  constexpr int MAX_NST = 16;
  constexpr int MB = BM / 64;                     // row blocks per wave (5; 1)
  constexpr int RB = 64;                          // bytes per LDS row
  constexpr int RPI = 16;                         // rows filled by one wave-wide load
  constexpr int NIA = BM / RPI;                   // activation loads per stage (20; 4)
  constexpr int IA = (NIA + 7) / 8;               // activation load slots per wave (3; 1)
  constexpr int IB = 2;                           // weight loads per wave (16 KB per stage)
  constexpr int B_BYTES = 16384;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[LDS_BYTES];

  int j, ntile;
  if (!fp8_unit_of_block(mtiles, offsets, *n_mtiles_ptr, n_ntiles, BM, j, ntile)) return;
  const MTile tile = mtiles[j];
  const int e = tile.expert, row0 = tile.row0, rows = tile.rows;
  const int n0 = ntile * (MODE == 0 ? 128 : 256);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int nkb = (kdim + 127) / 128;  // 128-element K blocks (scale columns)
  const int nk = kdim / BK;            // stages

  // ---- activation scales of the tile's rows -> LDS (rows past the tile: scale 1) -------
  // Every LDS read in the K loop uses a bf16 vector or bf16 type, like the direct loads' LDS
  // writes are seen by the compiler's type-based alias analysis; reads of other types made
  // it wait for every load in flight first.  So the scales are kept as 16-bit slots.
  // Layout [K block][row pair], the scale bytes of rows 2p and 2p+1 in one 16-bit slot: a row
  // block's slots sit at a fixed offset from the first's, and the table takes half the LDS of
  // one slot per row (four ring stages at d = 6144 instead of three).
  const int sc_bytes = (BM * nkb + 1023) & ~1023;
  __bf16* sc = reinterpret_cast<__bf16*>(smem + LDS_BYTES - sc_bytes);
  {
    // thread = (row pair p, group g of the K blocks kb = g, g + NG, ...): the pair's source
    // rows are looked up once and its scale bytes read in batches of independent loads, so
    // the copy waits for a few memory round trips rather than one per slot
    constexpr int NP = BM / 2, NG = 512 / NP, NB = 8;
    const int p = tid % NP, g = tid / NP, r = 2 * p;
    if (g < NG) {
      const bool v0 = r < rows, v1 = r + 1 < rows;
      const size_t s0 = !v0 ? 0 : MODE == 0 ? size_t(perm_token[row0 + r]) : size_t(row0 + r);
      const size_t s1 = !v1 ? 0 : MODE == 0 ? size_t(perm_token[row0 + r + 1]) : size_t(row0 + r + 1);
      const unsigned char* a0 = a_scales + s0 * nkb;
      const unsigned char* a1 = a_scales + s1 * nkb;
      for (int kb0 = g; kb0 < nkb; kb0 += NG * NB) {
        uint32_t b0[NB], b1[NB];
#pragma unroll
        for (int u = 0; u < NB; ++u) {
          const int kb = kb0 + u * NG;
          b0[u] = v0 && kb < nkb ? a0[kb] : 127u;
          b1[u] = v1 && kb < nkb ? a1[kb] : 127u;
        }
#pragma unroll
        for (int u = 0; u < NB; ++u) {
          const int kb = kb0 + u * NG;
          if (kb < nkb) sc[kb * NP + p] = __builtin_bit_cast(__bf16, uint16_t(b0[u] | (b1[u] << 8)));
        }
      }
    }
  }
  // ---- weight scales of the wave's two column blocks (E8M0 = the fp32 exponent field) --
  // lane l holds column block l in vsc[nb][0] and 64 + l in vsc[nb][1] (nkb <= 128)
  int vsc[2][2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int rb = MODE == 0 ? ntile : min(ntile * 2 + ((wn * 64 + nb * 32) >> 7), nrb_rows - 1);
    const int sbase = MODE == 0 ? ((e * 2 + nb) * nrb_rows + rb) * nkb : (e * nrb_rows + rb) * nkb;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int kb = h * 64 + lane;
      vsc[nb][h] = int((__float_as_uint(qscales[sbase + (kb < nkb ? kb : nkb - 1)]) >> 23) & 0xFF);
    }
  }
  __syncthreads();  // the scale copies are in LDS and no load is in flight (vmcnt counts below)

  // ---- load sources (as the bf16 pipelined kernel) -------------------------------------
  // byte offsets from a_codes (the activation matrix is under 2 GiB): one register each
  uint32_t srcA[IA];
  const int lrow = lane >> 2, lslot = lane & 3;
  int na = 0;
#pragma unroll
  for (int i = 0; i < IA; ++i) {
    const int q = wave + 8 * i;
    const int r = q * RPI + lrow;
    na += (q < NIA && q * RPI < rows) ? 1 : 0;
    const int ar = r < rows ? r : 0;  // rows past the tile read a valid row; never stored
    const uint32_t src_row = MODE == 0 ? uint32_t(perm_token[row0 + ar]) : uint32_t(row0 + ar);
    srcA[i] = src_row * uint32_t(kdim) + uint32_t((lslot ^ swz4(r)) * 16);
  }
  // weight stage kt: 16 contiguous KB = the packed blocks of 32-element K steps 2k, 2k+1;
  // wave-wide load i of wave w copies 1 KB piece w + 8 i
  const unsigned char* srcB = qcodes + (size_t(e) * n_ntiles + ntile) * (kdim / 32) * size_t(8192) + wave * 1024;
  const int per_stage = na + IB;
  const int krot = (j * 7 + ntile * 3) % nk;  // each unit starts at its own K stage
  auto kphys = [&](int kt) { const int k = kt + krot; return k >= nk ? k - nk : k; };
  const int a_bytes = __builtin_amdgcn_readfirstlane(((rows + 31) & ~31) * RB);
  const int stage_bytes = a_bytes + B_BYTES;
  const int ring = LDS_BYTES - sc_bytes;
  const int nst = ring / stage_bytes < MAX_NST ? ring / stage_bytes : MAX_NST;
  auto issue_one = [&](int i, int kt, int slot) {
    unsigned char* st = smem + slot * stage_bytes;
    if (i < IA) {
      if (i < na) dma16(a_codes + (srcA[i] + uint32_t(kphys(kt) * BK)), st + (wave + 8 * i) * 1024);
    } else {
      dma16_stream(srcB + size_t(kphys(kt)) * 16384 + (i - IA) * 8192 + lane * 16,
                   st + a_bytes + (wave + 8 * (i - IA)) * 1024);
    }
  };
  auto wait_stage = [&](int s, int newest) { wait_vmcnt((newest - s) * per_stage); };

  const int l32 = lane & 31, h = lane >> 5;
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
    constexpr int NV = decltype(nv_tag)::value;
    const int bp = wn * 32 + l32;  // this lane's weight pair row (both column blocks)
    i32x8 fa[2], fb[2];            // A fragments of two row blocks in turn; B of both blocks
    int sa[2], sb[2];
    // A fragment and scale of row block mb in stage slot `st`: K h*32 .. h*32+31 of the row.
    // swz4 reads row bits 1..3 only, the same in every row block: one lane offset serves all
    // row blocks, each 64 rows (4 KB) further on.
    const int a_lo = (wm * 32 + l32) * RB + (((2 * h) ^ swz4(l32)) << 4);
    const int a_hi = a_lo ^ 16;  // chunk 2h+1 sits in the slot next to chunk 2h's, xor 1
    auto rd_a = [&](const unsigned char* st, int mb, int kb, int buf) {
      const i32x4 lo = __builtin_bit_cast(i32x4, *reinterpret_cast<const bf16x8*>(st + a_lo + mb * 64 * RB));
      const i32x4 hi = __builtin_bit_cast(i32x4, *reinterpret_cast<const bf16x8*>(st + a_hi + mb * 64 * RB));
      fa[buf] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      sa[buf] = __builtin_bit_cast(uint16_t, sc[kb * (BM / 2) + ((wm * 32 + l32) >> 1) + mb * 32]);  // both rows' bytes
    };
    // B fragments (the lane's pair row, both halves) and their scales: one 16-byte read per
    // 8-element K group holds both halves' 8 bytes.  Lanes l and l + 16 read the same banks,
    // but a 16-byte read serves a quarter wave at a time, whose 16 lanes hit 16 distinct
    // 16-byte bank groups (row bits 0..1 and the swizzle of bits 2..3).
    auto rd_b = [&](const unsigned char* st, int kb) {
      const unsigned char* bb = st + a_bytes + h * 8192 + bp * 64;
      const int swb = swz4(bp);
      i32x4 p[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) p[g] = __builtin_bit_cast(i32x4, *reinterpret_cast<const bf16x8*>(bb + ((g ^ swb) << 4)));
      fb[0] = i32x8{p[0][0], p[0][1], p[1][0], p[1][1], p[2][0], p[2][1], p[3][0], p[3][1]};
      fb[1] = i32x8{p[0][2], p[0][3], p[1][2], p[1][3], p[2][2], p[2][3], p[3][2], p[3][3]};
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int v = kb < 64 ? vsc[nb][0] : vsc[nb][1];
        sb[nb] = __builtin_amdgcn_readlane(v, kb & 63);
      }
    };
    wait_stage(0, npro - 1);
    block_barrier();
    int sk = 0;
    for (int kt = 0; kt < nk; ++kt) {
      const int sk1 = sk + 1 == nst ? 0 : sk + 1;
      const unsigned char* st = smem + sk * stage_bytes;
      const int kb = __builtin_amdgcn_readfirstlane(kphys(kt) >> 1);  // 128-element block of this stage
      const bool last = kt + 1 == nk;
      const bool dma = kt + nst < nk;  // stage kt+nst takes stage kt's slot
      // every wave's reads of stage kt done, stage kt+1 landed: then the slot can be refilled
      auto stage_sync = [&]() {
        if (!last) {
          wait_lds_reads();
          const int newest = kt + nst - 1 < nk - 1 ? kt + nst - 1 : nk - 1;
          wait_stage(kt + 1, newest);
          block_barrier();
        }
      };
      if constexpr (NV == 0) {
        stage_sync();
        if (dma)
          for (int i = 0; i < IA + IB; ++i) issue_one(i, kt + nst, sk);
      } else {
        rd_a(st, 0, kb, 0);
        __builtin_amdgcn_sched_barrier(0);
        rd_b(st, kb);
        // Row block mb: wait for its operands (read one block earlier), issue the next block's
        // reads, then its two MFMAs.  The compiler's LDS waits cover every read in flight, so
        // a block's wait has to come before the next block's reads go out: the empty asm that
        // uses the operands places it there.  The asm after the MFMAs keeps them ahead of the
        // stage's barrier; without it they sink past the wait's branches, below the barrier,
        // and every read of a step is issued before any of its MFMAs.
#pragma unroll
        for (int mb = 0; mb < NV; ++mb) {
          const int cur = mb & 1;
          asm volatile("" ::"v"(fa[cur]), "v"(fb[0]), "v"(fb[1]), "v"(sa[cur]), "v"(sb[0]), "v"(sb[1]));
          __builtin_amdgcn_sched_barrier(0);
          if (mb + 1 < NV) rd_a(st, mb + 1, kb, cur ^ 1);  // next row block, beside these MFMAs
          else stage_sync();                                 // the stage's last reads are issued
          const int sa_row = (sa[cur] >> (8 * (l32 & 1))) & 0xFF;
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
            acc[mb][nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[cur], fb[nb], acc[mb][nb], 0, 0, 0,
                                                                          sa_row, 0, sb[nb]);
          asm volatile("" : "+v"(acc[mb][0]), "+v"(acc[mb][1]));
          // keep the scheduler from hoisting every row block's reads (registers for two only)
          __builtin_amdgcn_sched_barrier(0);
        }
        if (dma)
          for (int i = 0; i < IA + IB; ++i) issue_one(i, kt + nst, sk);
      }
      sk = sk1;
    }
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

  // ---- epilogue; 32x32 D layout: column lane & 31, rows 8*(r/4) + 4*(lane/32) + r%4 --------
  if constexpr (MODE == 1) {
    // one bf16 per lane and accumulator: a 4-lane transpose into 8-byte stores (as for H
    // below) made this kernel slower, its 32 K steps per unit being too few to carry the
    // transposes
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (mb >= nvb) continue;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int col = n0 + wn * 64 + nb * 32 + l32;
        if (col >= ncols) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = (mb * 2 + wm) * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (row < rows) yout[size_t(row0 + row) * ncols + col] = f2bf(acc[mb][nb][r]);
        }
      }
    }
  } else {
    // H = silu(G) U; its block of this row is the n-tile's 128 columns, spread over the 4
    // column waves (32 lanes each).  Row maxima over a wave's 32 columns: a butterfly over
    // lane bits 4..0 that halves the rows a lane carries at each step, so that lane l ends
    // with the maximum of accumulator index (l & 31) >> 1; then LDS and the 4 column waves.
    // The codes go out through a 4-lane transpose: each lane gets 4 adjacent columns of one
    // row (row 8 rq + 4 h + q4 of the row block for accumulators 4 rq .. 4 rq + 3) and stores
    // them as one 4-byte piece; column counts are multiples of 64, so a piece is in range or
    // out of it as a whole.
    const int q4 = lane & 3;
    const int col = n0 + wn * 32 + l32;
    const bool cin = col < ncols;
    __syncthreads();  // every wave is done with the ring
    float* pmax = reinterpret_cast<float*>(smem);  // [4 column waves][BM rows]
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (mb >= nvb) continue;
      float m[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float hv = cin ? swiglu_fast(acc[mb][0][r], acc[mb][1][r]) : 0.f;
        acc[mb][0][r] = hv;
        m[r] = fabsf(hv);
      }
#pragma unroll
      for (int step = 0, half = 8; step < 4; ++step, half >>= 1) {  // lane bits 4, 3, 2, 1
        const bool b = (l32 >> (4 - step)) & 1;
#pragma unroll
        for (int i = 0; i < half; ++i) {
          const float keep = b ? m[i + half] : m[i];
          const float send = b ? m[i] : m[i + half];
          m[i] = fmaxf(keep, __shfl_xor(send, 16 >> step));
        }
      }
      const float rmax = fmaxf(m[0], __shfl_xor(m[0], 1));
      const int ri = l32 >> 1;
      if ((l32 & 1) == 0) pmax[wn * BM + (mb * 2 + wm) * 32 + 8 * (ri >> 2) + 4 * h + (ri & 3)] = rmax;
    }
    __syncthreads();
    const int nkbh = (ncols + 127) / 128;
    const int colq = n0 + wn * 32 + (l32 & 28);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (mb >= nvb) continue;
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        float v[4], w[4];
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) v[t4] = acc[mb][0][rq * 4 + t4];
        quad_transpose(v, q4, w);
        const int row = (mb * 2 + wm) * 32 + 8 * rq + 4 * h + q4;
        if (row >= rows) continue;
        const float amax = fmaxf(fmaxf(pmax[row], pmax[BM + row]), fmaxf(pmax[2 * BM + row], pmax[3 * BM + row]));
        const int k = block_exp(amax);
        if (colq < ncols) {
          uint32_t c = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j) c |= e4m3_code(ldexpf(w[j], -k)) << (8 * j);
          *reinterpret_cast<uint32_t*>(hq + size_t(row0 + row) * ncols + colq) = c;
        }
        if (wn == 0 && l32 < 4) hs[size_t(row0 + row) * nkbh + ntile] = static_cast<unsigned char>(k + 127);
      }
    }
  }
}

#define LCM_INST(M, S)                                                                              \
  template __global__ void ffn_fp8_mfma_kernel<M, S>(                                              \
      const unsigned char* __restrict__, const unsigned char* __restrict__, const int32_t* __restrict__, \
      const unsigned char* __restrict__, const float* __restrict__, int, bf16_t* __restrict__,      \
      unsigned char* __restrict__, unsigned char* __restrict__, const MTile* __restrict__,          \
      const int32_t* __restrict__, const int32_t* __restrict__, int, int, int);
LCM_INST(0, false)
LCM_INST(1, false)
LCM_INST(0, true)
LCM_INST(1, true)
#undef LCM_INST

using Fp8MfmaKernel = void (*)(const unsigned char*, const unsigned char*, const int32_t*, const unsigned char*,
                               const float*, int, bf16_t*, unsigned char*, unsigned char*, const MTile*,
                               const int32_t*, const int32_t*, int, int, int);
template <int MODE>
Fp8MfmaKernel fp8_mfma_kernel(const lc_moe_shape& s) {
  return ffn_small(s) ? ffn_fp8_mfma_kernel<MODE, true> : ffn_fp8_mfma_kernel<MODE, false>;
}

hipError_t launch_quantize_act(const void* x, int rows, int cols, unsigned char* codes,
                               unsigned char* scales, hipStream_t st) {
  const int nkb = (cols + 127) / 128;
  const size_t threads = size_t(rows) * nkb * 16;
  hipLaunchKernelGGL(quantize_act_kernel, dim3(unsigned((threads + 255) / 256)), dim3(256), 0, st,
                     static_cast<const bf16_t*>(x), codes, scales, rows, cols, nkb);
  return hipGetLastError();
}

hipError_t launch_ffn_fp8_mfma(const lc_moe_shape& s, const WsPlan& p, void* ws, const void* fp8, int mode,
                               hipStream_t st) {
  char* w = static_cast<char*>(ws);
  const Fp8Plan q = plan_fp8(s);
  const unsigned char* qb = static_cast<const unsigned char*>(fp8);
  const int32_t* perm_token = reinterpret_cast<const int32_t*>(w + p.perm_token);
  const MTile* mtiles = reinterpret_cast<const MTile*>(w + p.mtiles);
  const int32_t* offsets = reinterpret_cast<const int32_t*>(w + p.offsets);
  const int32_t* n_mtiles = reinterpret_cast<const int32_t*>(w + p.n_mtiles);
  unsigned char* hq = reinterpret_cast<unsigned char*>(w + p.hbuf);
  unsigned char* hs = reinterpret_cast<unsigned char*>(w + p.hbuf + align256(size_t(s.T) * s.K * s.I));
  if (mode == 0) {
    const int nn = (s.I + 127) / 128;
    const unsigned grid = static_cast<unsigned>((size_t(p.mt_max) * nn + 7) / 8 * 8);
    fp8_mfma_kernel<0>(s)<<<dim3(grid), dim3(512), 0, st>>>(
        reinterpret_cast<const unsigned char*>(w + p.xq), reinterpret_cast<const unsigned char*>(w + p.xs),
        perm_token, qb + q.codes_gu, reinterpret_cast<const float*>(qb + q.scales_gu), q.nrb_i, nullptr, hq, hs,
        mtiles, offsets, n_mtiles, s.d, s.I, nn);
  } else {
    const int nn = (s.d + 255) / 256;
    const unsigned grid = static_cast<unsigned>((size_t(p.mt_max) * nn + 7) / 8 * 8);
    fp8_mfma_kernel<1>(s)<<<dim3(grid), dim3(512), 0, st>>>(
        hq, hs, nullptr, qb + q.codes_d, reinterpret_cast<const float*>(qb + q.scales_d), q.nrb_d,
        reinterpret_cast<bf16_t*>(w + p.ybuf), nullptr, nullptr, mtiles, offsets, n_mtiles, s.I, s.d, nn);
  }
  return hipGetLastError();
}

}  // namespace lcm

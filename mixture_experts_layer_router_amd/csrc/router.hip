// Softmax router R and biased top-K selection (LongCat-Flash article, itouyu.top,
// section "Zero-computation experts": softmax router over the whole N+Z expert pool;
// the expert bias only steers which K experts are chosen).
//
// Stage 1 (logits): L = x W_r^T with W_r fp32.
//   bf16 x: bf16 MFMA.  Each fp32 router weight is split exactly into three bf16 parts
//   w = hi + mid + lo (8 significant bits each; the remainders are exact in fp32), every
//   product of a bf16 x with a part is exact in fp32, and the MFMA sums them in fp32 --
//   an fp32 dot product at bf16-MFMA rate (3 MFMAs per fp32 product).  With few tokens
//   the reduction is split over workgroups and the partial sums are added in split
//   order by a reduction kernel (no atomics).
//   fp32 x: plain fp32 FMA, LDS-tiled.
// Stage 2 (top-K): one wavefront per token: max, exp, sum and divide in fp32, then K
//   rounds of a wavefront argmax over s = p + b (ties -> lower index) by shuffles.
#include <type_traits>

#include "common.h"
#include "lds_dma.h"
#include "topk.h"

namespace lcm {

// ---------------------------------------------------------------------------------------
// bf16 MFMA logits.  W_r is split once per call into three bf16 matrices (hi, mid, lo);
// the GEMM then reads bf16 operands only.  Tile: 128 tokens x 128 experts, K step 32,
// 256 threads (2x2 waves, 64x64 per wave, v_mfma_f32_32x32x16_bf16, three MFMAs per
// block and k step, one per part).  blockIdx.z picks a chunk of the reduction (split-K
// for layers with few tokens); each chunk's partial logits go to their own array.
// ---------------------------------------------------------------------------------------
namespace rl {
constexpr int BM = 128, BN = 128, BK = 32, LDA = BK + 8;  // LDS row: 80 bytes
}

__device__ __forceinline__ void split3(float w, bf16_t& hi, bf16_t& mid, bf16_t& lo) {
  hi = f2bf(w);
  float r1 = w - bf2f(hi);
  mid = f2bf(r1);
  float r2 = r1 - bf2f(mid);
  lo = f2bf(r2);
}

// wsplit = [hi | mid | lo], each [E][d] bf16: n = E*d fp32 weights, 4 per thread.
__global__ __launch_bounds__(256) void router_split_kernel(const float* __restrict__ wr,
                                                           bf16_t* __restrict__ wsplit, size_t n) {
  const size_t i = (size_t(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  const float4 w = *reinterpret_cast<const float4*>(wr + i);
  bf16_t h[4], m[4], l[4];
  split3(w.x, h[0], m[0], l[0]);
  split3(w.y, h[1], m[1], l[1]);
  split3(w.z, h[2], m[2], l[2]);
  split3(w.w, h[3], m[3], l[3]);
  *reinterpret_cast<uint2*>(wsplit + i) = make_uint2(h[0] | (uint32_t(h[1]) << 16), h[2] | (uint32_t(h[3]) << 16));
  *reinterpret_cast<uint2*>(wsplit + n + i) = make_uint2(m[0] | (uint32_t(m[1]) << 16), m[2] | (uint32_t(m[3]) << 16));
  *reinterpret_cast<uint2*>(wsplit + 2 * n + i) = make_uint2(l[0] | (uint32_t(l[1]) << 16), l[2] | (uint32_t(l[3]) << 16));
}

__global__ __launch_bounds__(256, 2) void router_logits_bf16_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ wsplit, float* __restrict__ out,
    int T, int d, int E, int chunk, int32_t* __restrict__ zero_word) {
  using namespace rl;
  if (zero_word && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0) *zero_word = 0;

  __shared__ __attribute__((aligned(16))) bf16_t As[BM * LDA];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[3][BN * LDA];

  const int tid = threadIdx.x;
  const int e0 = blockIdx.x * BN;
  const int t0 = blockIdx.y * BM;
  const int kbeg = blockIdx.z * chunk;
  const int kend = kbeg + chunk < d ? kbeg + chunk : d;
  float* logits = out + size_t(blockIdx.z) * T * E;
  const size_t part = size_t(E) * d;

  // global -> register prefetch: 128 rows x 4 chunks of 8 bf16 per operand -> 2 per thread
  const bf16_t* a_ptr[2];
  const bf16_t* b_ptr[2];
  int r_row[2], r_kc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + i * 256;
    r_row[i] = c >> 2;
    r_kc[i] = (c & 3) * 8;
    const int t = t0 + r_row[i], e = e0 + r_row[i];
    a_ptr[i] = t < T ? x + size_t(t) * d : nullptr;
    b_ptr[i] = e < E ? wsplit + size_t(e) * d : nullptr;
  }

  uint4 ra[2], rb[3][2];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int k = k0 + r_kc[i];
      const bool ka = k < kend;  // d is a multiple of 8, so a chunk of 8 is all in or all out
      ra[i] = (a_ptr[i] && ka) ? *reinterpret_cast<const uint4*>(a_ptr[i] + k) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int p = 0; p < 3; ++p)
        rb[p][i] = (b_ptr[i] && ka) ? *reinterpret_cast<const uint4*>(b_ptr[i] + p * part + k)
                                    : make_uint4(0, 0, 0, 0);
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int o = r_row[i] * LDA + r_kc[i];
      *reinterpret_cast<uint4*>(&As[o]) = ra[i];
#pragma unroll
      for (int p = 0; p < 3; ++p) *reinterpret_cast<uint4*>(&Bs[p][o]) = rb[p][i];
    }
  };

  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lk = (lane >> 5) * 8;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = (kend - kbeg + BK - 1) / BK;
  load(kbeg);
  for (int kt = 0; kt < nk; ++kt) {
    __syncthreads();
    store();
    __syncthreads();
    if (kt + 1 < nk) load(kbeg + (kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int kk = ks * 16 + lk;
      bf16x8 a[2], b[3][2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(&As[(wm * 64 + i * 32 + lr) * LDA + kk]);
#pragma unroll
      for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          b[p][j] = *reinterpret_cast<const bf16x8*>(&Bs[p][(wn * 64 + j * 32 + lr) * LDA + kk]);
#pragma unroll
      for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[p][j], acc[i][j], 0, 0, 0);
    }
  }

  // D layout of 32x32 MFMA: lane holds column (lane & 31), rows 8*(r/4) + 4*(lane/32) + r%4
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int e = e0 + wn * 64 + j * 32 + lr;
      if (e >= E) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = t0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (t < T) logits[size_t(t) * E + e] = acc[i][j][r];
      }
    }
}

// ---------------------------------------------------------------------------------------
// Pipelined bf16 MFMA logits (d a multiple of 32).  Tile: 256 tokens x 192 experts, K step
// 32.  The weight operand is the tile's 3 x 192 = 576 part rows (all hi rows, then all
// mid rows, then all lo rows).  512 threads = 8 waves; wave w owns token blocks
// 2*(w >> 1) + {0, 1} against expert blocks 3*(w & 1) + {0, 1, 2}: 2 x 3 blocks of 32x32,
// three MFMAs per block and 16-wide substep (hi, mid, lo: the same order of additions as
// the 128 x 128 kernel), 96 fp32 accumulators per lane.
// Operands reach LDS by direct global->LDS loads into a 3-stage ring (52 KB a stage, 64
// bytes per row, chunk c of row r in slot c ^ swz4(r)).  A K step has two substeps of 16;
// between them each wave waits for its own loads of stage kt+1 and meets the others at a
// barrier, past which no wave reads stage kt again, so the second substep refills that
// slot with stage kt+3.  Token row groups past T are not loaded and waves skip the MFMAs
// of token blocks past T.
// Work unit = (token tile, expert tile, K chunk), ordered token tile, expert tile, chunk;
// workgroup w runs on XCD w % 8 and each XCD takes one contiguous eighth of the units, so
// the expert tiles of one token tile run side by side on one XCD and share its
// activation rows in that XCD's L2.
// ---------------------------------------------------------------------------------------
namespace rp {
constexpr int BM = kRouterBm, BE = kRouterBe, NP = 3, BK = 32, RB = BK * 2;
constexpr int BROWS = NP * BE;             // 576 part rows
constexpr int STAGE = (BM + BROWS) * RB;   // 52 KB
constexpr int NST = 3;                     // ring stages
constexpr int NL = (BM + BROWS) / 16;      // wave-wide loads per stage (52)
constexpr int LPW = (NL + 7) / 8;          // load slots per wave (7)
}

// FSPLIT: for units whose K chunk fits the ring (at most NST steps: the split-K layers of
// few tokens), the part rows are not loaded from wsplit but made here from the fp32 router
// weight wr with the same split as router_split_kernel (so the same bits), and the split
// kernel is not run: the layer saves its launch and the 1.5x bytes of the parts.
template <bool FSPLIT>
__global__ __launch_bounds__(512, 1) void router_logits_pipe_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ wsplit, const float* __restrict__ wr,
    float* __restrict__ out, int T, int d, int E, int chunk, int n_et, int splits, int n_units,
    int32_t* __restrict__ zero_word) {
  using namespace rp;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[NST * STAGE];
  if (zero_word && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0) *zero_word = 0;

  const int per = (n_units + 7) >> 3;
  const int wslot = blockIdx.x >> 3;
  if (wslot >= per) return;
  const int u = (blockIdx.x & 7) * per + wslot;
  if (u >= n_units) return;
  const int sp = u % splits;
  const int et = (u / splits) % n_et;
  const int tt = u / (splits * n_et);
  const int t0 = tt * BM, e0 = et * BE;
  const int kbeg = sp * chunk;
  const int kend = kbeg + chunk < d ? kbeg + chunk : d;
  const int nk = (kend - kbeg) / BK;
  const int rows = T - t0 < BM ? T - t0 : BM;  // tokens of this tile
  float* logits = out + size_t(sp) * T * E;
  const size_t part = size_t(E) * d;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // Load q (0..51) belongs to wave q % 8 and fills stage rows 16q..16q+15 (rows 0..255:
  // tokens, 256..831: part rows); lane l fills row 16q + l/4, slot l%4, with global chunk
  // (l%4) ^ swz4(row).  Token loads whose 16 rows all lie past T are skipped.
  const bf16_t* src[LPW];
  int lmask = 0;  // bit i: this wave issues its load i
  const int lrow = lane >> 2, lslot = lane & 3;
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int q = wave + 8 * i;
    const int r = q * 16 + lrow;  // stage row
    const bf16_t* p = x;
    if (q < BM / 16) {
      if (q * 16 < rows) lmask |= 1 << i;
      const int t = r < rows ? t0 + r : t0;  // rows past T read a valid row; never stored
      p = x + size_t(t) * d;
    } else if (!FSPLIT && q < NL) {
      lmask |= 1 << i;
      const int br = r - BM, pp = br / BE, c = e0 + br % BE;
      p = wsplit + pp * part + size_t(c < E ? c : e0) * d;  // experts past E: a valid row
    }
    src[i] = p + kbeg + (lslot ^ swz4(r)) * 8;
  }
  const int nl = __builtin_popcount(lmask);  // this wave's loads per stage
  auto issue_one = [&](int i, int kt, int slot) {
    if ((lmask >> i) & 1) dma16(src[i] + kt * BK, smem + slot * STAGE + (wave + 8 * i) * 1024);
  };
  auto wait_stage = [&](int s, int newest) { wait_vmcnt((newest - s) * nl); };

  const int l32 = lane & 31, sw = swz4(l32), khalf = lane >> 5;
  int nvb = 0;  // token blocks of this wave holding tokens (a prefix)
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) nvb += (wm * 2 + mb) * 32 < rows;

  f32x16 acc[2][3];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 3; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.f;

  const int npro = nk < NST ? nk : NST;
  for (int s = 0; s < npro; ++s) {
#pragma unroll
    for (int i = 0; i < LPW; ++i) issue_one(i, s, s);
  }
  if constexpr (FSPLIT) {
    // nk <= NST: every stage of the chunk is in the ring.  Group g (0..1535) of a stage is
    // 4 weights of expert row g / 8, columns 4 * (g % 8); thread tid takes g = tid + 512 i.
    float4 wv[NST][3];
#pragma unroll
    for (int s = 0; s < NST; ++s)
#pragma unroll
      for (int gi = 0; gi < 3; ++gi) {
        const int g = tid + 512 * gi, er = g >> 3, c = e0 + er;
        const int kk = kbeg + (s < nk ? s : 0) * BK + (g & 7) * 4;
        wv[s][gi] = *reinterpret_cast<const float4*>(wr + size_t(c < E ? c : e0) * d + kk);
      }
#pragma unroll
    for (int s = 0; s < NST; ++s) {
      if (s >= nk) break;
#pragma unroll
      for (int gi = 0; gi < 3; ++gi) {
        const int g = tid + 512 * gi, er = g >> 3, cg = g & 7;
        bf16_t h[4], m[4], l[4];
        split3(wv[s][gi].x, h[0], m[0], l[0]);
        split3(wv[s][gi].y, h[1], m[1], l[1]);
        split3(wv[s][gi].z, h[2], m[2], l[2]);
        split3(wv[s][gi].w, h[3], m[3], l[3]);
        const uint2 pv[3] = {make_uint2(h[0] | (uint32_t(h[1]) << 16), h[2] | (uint32_t(h[3]) << 16)),
                             make_uint2(m[0] | (uint32_t(m[1]) << 16), m[2] | (uint32_t(m[3]) << 16)),
                             make_uint2(l[0] | (uint32_t(l[1]) << 16), l[2] | (uint32_t(l[3]) << 16))};
#pragma unroll
        for (int pp = 0; pp < 3; ++pp) {  // part row pp*BE + er: slot of 16-byte chunk cg/2, half cg%2
          const int r = BM + pp * BE + er;
          *reinterpret_cast<uint2*>(smem + s * STAGE + r * RB + (((cg >> 1) ^ swz4(r)) << 4) + (cg & 1) * 8) = pv[pp];
        }
      }
    }
    LCM_WAIT_VMCNT(0);  // this wave's token rows landed
    wait_lds_reads();   // and its part rows are written
    block_barrier();
  }

  auto run = [&](auto nv_tag) {
    constexpr int NV = decltype(nv_tag)::value;
    // fragments of one substep: a[mb] tokens, b[p][nb] part p of expert block nb
    auto rd = [&](int ring_slot, int ks, bf16x8 (&a)[2], bf16x8 (&b)[3][3]) {
      const unsigned char* st = smem + ring_slot * STAGE;
      const int cs = ((ks * 2 + khalf) ^ sw) * 16;
#pragma unroll
      for (int mb = 0; mb < NV; ++mb)
        a[mb] = *reinterpret_cast<const bf16x8*>(st + ((wm * 2 + mb) * 32 + l32) * RB + cs);
      if (NV > 0) {
#pragma unroll
        for (int p = 0; p < 3; ++p)
#pragma unroll
          for (int nb = 0; nb < 3; ++nb)
            b[p][nb] = *reinterpret_cast<const bf16x8*>(
                st + (BM + p * BE + (wn * 3 + nb) * 32 + l32) * RB + cs);
      }
    };
    // MFMAs of one substep; with DMA, this wave's loads of stage kt_load (ring slot `slot`)
    // go one per block, the rest after the last block.
    auto mm = [&](const bf16x8 (&a)[2], const bf16x8 (&b)[3][3], auto dma, int kt_load, int slot) {
      constexpr bool DMA = decltype(dma)::value;
#pragma unroll
      for (int mb = 0; mb < NV; ++mb)
#pragma unroll
        for (int nb = 0; nb < 3; ++nb) {
          if (DMA && mb * 3 + nb < LPW) issue_one(mb * 3 + nb, kt_load, slot);
#pragma unroll
          for (int p = 0; p < 3; ++p)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mb], b[p][nb], acc[mb][nb], 0, 0, 0);
        }
      if (DMA) {
#pragma unroll
        for (int i = NV * 3; i < LPW; ++i) issue_one(i, kt_load, slot);
      }
    };
    bf16x8 ca[2], xa[2], cb[3][3], xb[3][3];
    wait_stage(0, npro - 1);
    block_barrier();
    rd(0, 0, ca, cb);
    int sk = 0;  // ring slot of stage kt
    auto step = [&](int kt, auto more_tag, auto last_tag) {
      constexpr bool LAST = decltype(last_tag)::value;
      const int sk1 = sk + 1 == NST ? 0 : sk + 1;
      rd(sk, 1, xa, xb);
      mm(ca, cb, std::false_type{}, 0, 0);
      if (!LAST) {
        wait_lds_reads();  // this wave's reads of stage kt done
        const int newest = kt + NST - 1 < nk - 1 ? kt + NST - 1 : nk - 1;
        wait_stage(kt + 1, newest);
        block_barrier();  // stage kt+1 visible to all waves; nobody reads stage kt again
        rd(sk1, 0, ca, cb);
      }
      mm(xa, xb, more_tag, kt + NST, sk);  // stage kt+NST takes stage kt's slot
      sk = sk1;
    };
    const int nmain = nk - NST > 0 ? nk - NST : 0;
    for (int kt = 0; kt < nmain; ++kt) step(kt, std::true_type{}, std::false_type{});
    for (int kt = nmain; kt < nk - 1; ++kt) step(kt, std::false_type{}, std::false_type{});
    step(nk - 1, std::false_type{}, std::true_type{});
  };
  switch (nvb) {
    case 0: run(std::integral_constant<int, 0>{}); break;
    case 1: run(std::integral_constant<int, 1>{}); break;
    default: run(std::integral_constant<int, 2>{}); break;
  }

  // 32x32 D layout: column lane & 31, rows 8*(r/4) + 4*(lane/32) + r%4
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    if (mb >= nvb) continue;
#pragma unroll
    for (int nb = 0; nb < 3; ++nb) {
      const int e = e0 + (wn * 3 + nb) * 32 + l32;
      if (e >= E) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = (wm * 2 + mb) * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3);
        if (row < rows) logits[size_t(t0 + row) * E + e] = acc[mb][nb][r];
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// fp32 logits: 64 tokens x 64 experts per block, K step 16, 4x4 outputs per thread.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void router_logits_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ wr, float* __restrict__ logits,
    int T, int d, int E, int32_t* __restrict__ zero_word) {
  if (zero_word && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0) *zero_word = 0;
  __shared__ float Xs[64][17];
  __shared__ float Ws[64][17];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.y * 64, e0 = blockIdx.x * 64;
  const int ty = tid >> 4, tx = tid & 15;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < d; k0 += 16) {
    for (int c = tid; c < 64 * 16; c += 256) {
      int r = c >> 4, k = c & 15;
      int t = t0 + r, e = e0 + r, kk = k0 + k;
      Xs[r][k] = (t < T && kk < d) ? x[size_t(t) * d + kk] : 0.f;
      Ws[r][k] = (e < E && kk < d) ? wr[size_t(e) * d + kk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(Xs[ty * 4 + i][k], Ws[tx * 4 + j][k], acc[i][j]);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int t = t0 + ty * 4 + i, e = e0 + tx * 4 + j;
      if (t < T && e < E) logits[size_t(t) * E + e] = acc[i][j];
    }
}

// ---------------------------------------------------------------------------------------
// Softmax + biased top-K: one wavefront per token (router_topk_token in topk.h).
// ---------------------------------------------------------------------------------------
template <int EPL>
__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ logits,
                                                          const float* __restrict__ bias,
                                                          int32_t* __restrict__ idx,
                                                          float* __restrict__ gate, int T,
                                                          int E, int K) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  router_topk_token<EPL>(logits + size_t(t) * E, bias, E, K, threadIdx.x & 63, idx + size_t(t) * K,
                         gate + size_t(t) * K);
}

// logits = sum of the split partials, added in split order (n = T*E, 4 per thread).  The
// partials are loaded eight splits at a time before they are added, so each thread keeps
// eight loads in flight (a few-token layer has few threads and up to 64 splits).
__global__ __launch_bounds__(256) void router_reduce_kernel(const float* __restrict__ rpart,
                                                            float* __restrict__ logits,
                                                            int splits, size_t n) {
  const size_t i = (size_t(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (n % 4 == 0 && i + 3 < n) {  // every partial array starts 16-byte aligned
    float4 a = *reinterpret_cast<const float4*>(rpart + i);
    for (int s0 = 1; s0 < splits; s0 += 8) {
      float4 b[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (s0 + j < splits) b[j] = *reinterpret_cast<const float4*>(rpart + (s0 + j) * n + i);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (s0 + j < splits) {
          a.x += b[j].x;
          a.y += b[j].y;
          a.z += b[j].z;
          a.w += b[j].w;
        }
      }
    }
    *reinterpret_cast<float4*>(logits + i) = a;
  } else {
    for (size_t q = i; q < n && q < i + 4; ++q) {
      float a = rpart[q];
      for (int sp = 1; sp < splits; ++sp) a += rpart[sp * n + q];
      logits[q] = a;
    }
  }
}

hipError_t launch_router_logits(const lc_moe_shape& s, const void* x, const float* w_router,
                                bf16_t* wsplit, float* logits, float* rpart, hipStream_t st,
                                int32_t* zero_word) {
  const int E = s.N + s.Z;
  if (s.dtype == LC_MOE_BF16) {
    const size_t n = size_t(E) * s.d;  // a multiple of 8
    const RouterSplit rs = router_split(s);
    float* dst = rs.splits > 1 ? rpart : logits;
    // split-K chunks that fit the ring: the pipelined kernel splits the weight itself
    const bool fsplit = router_fused_split(s);
    static_assert(rp::NST * rp::BK == kRouterRingK, "ring depth of the pipelined router");
    if (!fsplit)
      hipLaunchKernelGGL(router_split_kernel, dim3(unsigned((n / 4 + 255) / 256)), dim3(256), 0, st,
                         w_router, wsplit, n);
    if (router_pipelined(s)) {
      const int n_et = (E + rp::BE - 1) / rp::BE;
      const int units = ((s.T + rp::BM - 1) / rp::BM) * n_et * rs.splits;
      const dim3 grid(unsigned((units + 7) / 8 * 8));
      if (fsplit)
        hipLaunchKernelGGL(router_logits_pipe_kernel<true>, grid, dim3(512), 0, st,
                           static_cast<const bf16_t*>(x), wsplit, w_router, dst, s.T, s.d, E, rs.chunk,
                           n_et, rs.splits, units, zero_word);
      else
        hipLaunchKernelGGL(router_logits_pipe_kernel<false>, grid, dim3(512), 0, st,
                           static_cast<const bf16_t*>(x), wsplit, w_router, dst, s.T, s.d, E, rs.chunk,
                           n_et, rs.splits, units, zero_word);
    } else {
      dim3 grid((E + rl::BN - 1) / rl::BN, (s.T + rl::BM - 1) / rl::BM, rs.splits);
      hipLaunchKernelGGL(router_logits_bf16_kernel, grid, dim3(256), 0, st,
                         static_cast<const bf16_t*>(x), wsplit, dst, s.T, s.d, E, rs.chunk, zero_word);
    }
    if (rs.splits > 1) {
      const size_t nl = size_t(s.T) * E;
      hipLaunchKernelGGL(router_reduce_kernel, dim3(unsigned((nl + 1023) / 1024)), dim3(256), 0, st,
                         rpart, logits, rs.splits, nl);
    }
  } else {
    dim3 grid((E + 63) / 64, (s.T + 63) / 64);
    hipLaunchKernelGGL(router_logits_f32_kernel, grid, dim3(256), 0, st,
                       static_cast<const float*>(x), w_router, logits, s.T, s.d, E, zero_word);
  }
  return hipGetLastError();
}

hipError_t launch_router_topk(const lc_moe_shape& s, const float* logits, const float* bias,
                              int32_t* idx, float* gate, hipStream_t st) {
  const int E = s.N + s.Z;
  const int epl = (E + 63) / 64;
  dim3 grid((s.T + 3) / 4), block(256);
#define LCM_TOPK(n)                                                                       \
  hipLaunchKernelGGL(router_topk_kernel<n>, grid, block, 0, st, logits, bias, idx, gate, \
                     s.T, E, s.K)
  if (epl <= 2) LCM_TOPK(2);
  else if (epl <= 4) LCM_TOPK(4);
  else if (epl <= 8) LCM_TOPK(8);
  else if (epl <= 16) LCM_TOPK(16);
  else if (epl <= 32) LCM_TOPK(32);
  else LCM_TOPK(64);
#undef LCM_TOPK
  return hipGetLastError();
}

}  // namespace lcm

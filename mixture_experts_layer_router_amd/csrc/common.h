// Internal definitions shared by the lc_moe HIP sources (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "lc_moe.h"

namespace lcm {

typedef uint16_t bf16_t;  // bf16 bit pattern in memory
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kMaxE = 4096;     // N + Z limit (router registers, histogram LDS)
constexpr int kMaxN = 2048;     // N limit (permutation bitmask LDS)
constexpr int kTokBlock = 256;  // tokens per permutation block

// M-tile height (rows of one expert) of the grouped FFN kernels.
constexpr int kBmBf16 = 128;  // ffn_bf16_kernel (any d, I multiple of 8)
constexpr int kBmPipe = 320;  // ffn_bf16_pipe_kernel (d and I multiples of 32)
constexpr int kBmSmall = 64;  // its few-row form, two workgroups per CU
constexpr int kSmallMaxT = 256;  // layers of at most this many tokens run the few-row form
constexpr int kBmF32 = 64;

// The pipelined bf16 FFN kernel needs whole 32-element K steps in both GEMMs.
inline bool ffn_pipelined(const lc_moe_shape& s) {
  return s.dtype == LC_MOE_BF16 && s.d % 32 == 0 && s.I % 32 == 0;
}
// Its few-row form runs for layers of few tokens (decode), whose experts get a few rows
// each: there the 320-row form's single workgroup per CU leaves the loads idle while it
// waits at its barriers, and two smaller workgroups per CU keep them busy.  An expert with
// more than 64 rows (at most T) gets several M-tiles; they read the same weight tiles side
// by side on one XCD, so the repeats come from its L2.
inline bool ffn_small(const lc_moe_shape& s) { return ffn_pipelined(s) && s.T <= kSmallMaxT; }

__device__ __forceinline__ float bf2f(bf16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16, round to nearest even (inputs are finite).
__device__ __forceinline__ bf16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

// silu(g) * u for the bf16 FFN epilogues: silu(g) = g / (1 + e^-g) evaluated with the
// hardware base-2 exponential and reciprocal (v_exp_f32, v_rcp_f32; each within a few
// ulp of fp32), far inside the bf16 rounding the result then takes.  Very negative g gives
// e^-g = inf and a zero reciprocal, so silu -> -0; very positive g gives e^-g = 0 -> g.
__device__ __forceinline__ float swiglu_fast(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
  return g * __builtin_amdgcn_rcpf(1.f + e) * u;
}

// One M-tile of the grouped FFN: rows row0..row0+rows-1 of expert `expert`;
// first_tile is the index of that expert's first M-tile.
struct MTile {
  int expert, row0, rows, first_tile;
};

// bf16 router GEMM tiles.  With d a multiple of 32 the pipelined kernel runs, on tiles of
// kRouterBm tokens x kRouterBe experts, one workgroup per CU; otherwise the 128 x 128
// kernel, two workgroups per CU.
constexpr int kRouterBm = 256, kRouterBe = 192;
inline bool router_pipelined(const lc_moe_shape& s) {
  return s.dtype == LC_MOE_BF16 && s.d % 32 == 0;
}

// Split-K of the bf16 router GEMM.  When the layer has few tokens (decode) there are too
// few tiles to fill 256 CUs, so the reduction over d is cut into `splits` chunks of
// `chunk` columns (a multiple of 32) whose partial logits are summed, in chunk order, by a
// reduction kernel.
struct RouterSplit {
  int splits, chunk;
};
inline RouterSplit router_split(const lc_moe_shape& s) {
  RouterSplit r{1, s.d};
  if (s.dtype != LC_MOE_BF16) return r;
  const int E = s.N + s.Z;
  const bool pipe = router_pipelined(s);
  const long long tiles = pipe ? (long long)((E + kRouterBe - 1) / kRouterBe) * ((s.T + kRouterBm - 1) / kRouterBm)
                               : (long long)((E + 127) / 128) * ((s.T + 127) / 128);
  const long long slots = pipe ? 256 : 512;  // workgroups the chip holds at once
  long long want = (slots + tiles - 1) / tiles;
  const int kmax = (s.d + 31) / 32;
  if (want > kmax) want = kmax;
  if (want <= 1) return r;
  r.chunk = ((s.d + int(want) - 1) / int(want) + 31) / 32 * 32;
  r.splits = (s.d + r.chunk - 1) / r.chunk;
  return r;
}

// The pipelined router's ring holds 3 stages of 32 K columns.  A split-K chunk of at most
// that many columns is loaded as fp32 and split into its bf16 parts inside the kernel, so
// the layer needs no separate split of the router weight (nor its workspace region).
constexpr int kRouterRingK = 3 * 32;
inline bool router_fused_split(const lc_moe_shape& s) {
  return router_pipelined(s) && router_split(s).chunk <= kRouterRingK;
}

// Byte offsets of the workspace regions (all 256-byte aligned).
struct WsPlan {
  size_t logits, wsplit, rpart, idx, gate, block_counts, block_base, load, offsets, mtiles,
      n_mtiles, done, perm_token, slot_row, hbuf, ybuf, xq, xs, total;
  int nblocks;  // token blocks of the permutation
  int bm;       // M-tile height for this dtype
  int mt_max;   // capacity of the M-tile list
};

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Shapes the FP8 MFMA layer takes: 64-element K stages, at most 128 scale blocks per row,
// and activation matrices (x codes [T][d], H codes [T*K][I]) addressed by 32-bit offsets.
inline bool fp8_mfma_ok(const lc_moe_shape& s) {
  return s.dtype == LC_MOE_BF16 && s.d % 64 == 0 && s.I % 64 == 0 && s.d <= 16384 && s.I <= 16384 &&
         size_t(s.T) * s.K * s.I < (size_t(1) << 31) && size_t(s.T) * s.d < (size_t(1) << 31);
}

inline WsPlan plan_workspace(const lc_moe_shape& s) {
  WsPlan p{};
  const size_t T = s.T, K = s.K, E = size_t(s.N) + s.Z, N = s.N;
  const size_t es = s.dtype == LC_MOE_BF16 ? 2 : 4;
  p.nblocks = int((T + kTokBlock - 1) / kTokBlock);
  p.bm = s.dtype == LC_MOE_BF16 ? (ffn_pipelined(s) ? (ffn_small(s) ? kBmSmall : kBmPipe) : kBmBf16) : kBmF32;
  const size_t tk = T * K;
  size_t mt = N + (tk + p.bm - 1) / p.bm;
  if (mt > tk) mt = tk;
  p.mt_max = int(mt);
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align256(o + bytes); return at; };
  p.logits = take(T * E * 4);
  const RouterSplit rs = router_split(s);
  // the fp32 router weight as three bf16 parts (bf16 layers whose router does not split it
  // in the kernel)
  p.wsplit = take(s.dtype == LC_MOE_BF16 && !router_fused_split(s) ? 3 * E * size_t(s.d) * 2 : 0);
  p.rpart = take(rs.splits > 1 ? size_t(rs.splits) * T * E * 4 : 0);
  p.idx = take(tk * 4);
  p.gate = take(tk * 4);
  p.block_counts = take(size_t(p.nblocks) * E * 4);
  p.block_base = take(size_t(p.nblocks) * N * 4);
  p.load = take(E * 4);
  p.offsets = take((N + 1) * 4);
  p.mtiles = take(mt * sizeof(MTile));
  p.n_mtiles = take(4);
  p.done = take(4);  // workgroups done with their top-K (fused top-K + permutation)
  p.perm_token = take(tk * 4);
  p.slot_row = take(tk * 4);
  p.hbuf = take(tk * size_t(s.I) * es);
  p.ybuf = take(tk * size_t(s.d) * es);
  // the FP8 MFMA layer's x codes and scales (its H codes and scales live in hbuf)
  p.xq = take(fp8_mfma_ok(s) ? T * size_t(s.d) : 0);
  p.xs = take(fp8_mfma_ok(s) ? T * size_t((s.d + 127) / 128) : 0);
  p.total = o;
  return p;
}

// Every kernel launch of a shape must fit the device's grid: at most 2^32 - 1 work-items
// along x and 65535 workgroups along y and z.  The launchers below size their grids by
// these same formulas; shapes whose largest launch would not fit are rejected up front.
inline bool grids_fit(const lc_moe_shape& s) {
  typedef unsigned long long u64;
  const u64 lim = 0xFFFFFFFFull;
  const u64 T = u64(s.T), K = u64(s.K), E = u64(s.N) + u64(s.Z), d = u64(s.d), I = u64(s.I);
  const bool bf = s.dtype == LC_MOE_BF16;
  bool f = true;
  f = f && T * K * 256 <= lim;          // gather_rows_kernel: one workgroup per pick
  f = f && T * 256 <= lim;              // combine: one workgroup per token
  f = f && (T + 3) / 4 * 256 <= lim;    // top-K: one wave per token
  const WsPlan p = plan_workspace(s);
  const u64 nn_gu = bf ? (I + 127) / 128 : (I + 63) / 64;
  const u64 nn_d = bf ? (d + 255) / 256 : (d + 63) / 64;
  const u64 units = u64(p.mt_max) * (nn_gu > nn_d ? nn_gu : nn_d);
  f = f && (units + 7) / 8 * 8 * 512 <= lim;  // grouped FFN: one workgroup per work unit
  if (bf) {
    const RouterSplit rs = router_split(s);
    f = f && (E * d / 4 + 255) / 256 * 256 <= lim;  // router weight split
    if (router_pipelined(s))
      f = f && ((T + kRouterBm - 1) / kRouterBm) * ((E + kRouterBe - 1) / kRouterBe) * u64(rs.splits) * 512 <= lim;
    else
      f = f && (T + 127) / 128 <= 65535 && u64(rs.splits) <= 65535;
    f = f && (T * E + 1023) / 1024 * 256 <= lim;  // split-K sum
  } else {
    f = f && (T + 63) / 64 <= 65535;
  }
  return f;
}

// Workspace of lc_moe_ffn_backward (bf16 layers, d and I multiples of 32): the permutation
// of the given picks (M-tiles of kBmBwd rows), each row's gate, and the row intermediates
// dH (fp32), g*H, dG, dU (bf16, [T*K][I]) and dX (bf16, [T*K][d]).
constexpr int kBmBwd = 256;
struct BwPlan {
  size_t block_counts, block_base, load, offsets, mtiles, n_mtiles, done, perm_token, slot_row, g_row,
      dh, gh, dg, du, dxp, pipe_mtiles, pipe_n_mtiles, xp, dyp, zero, total;
  int nblocks, mt_max;
  int pipe_bm, pipe_mt_max;  // the M-tile list of the pipelined gate/up kernel's recompute
};
inline BwPlan plan_backward(const lc_moe_shape& s) {
  BwPlan p{};
  const size_t T = s.T, K = s.K, E = size_t(s.N) + s.Z, N = s.N, tk = T * K;
  p.nblocks = int((T + kTokBlock - 1) / kTokBlock);
  size_t mt = N + (tk + kBmBwd - 1) / kBmBwd;
  if (mt > tk) mt = tk;
  p.mt_max = int(mt);
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align256(o + bytes); return at; };
  p.block_counts = take(size_t(p.nblocks) * E * 4);
  p.block_base = take(size_t(p.nblocks) * N * 4);
  p.load = take(E * 4);
  p.offsets = take((N + 1) * 4);
  p.mtiles = take(mt * sizeof(MTile));
  p.n_mtiles = take(4);
  p.done = take(4);
  p.perm_token = take(tk * 4);
  p.slot_row = take(tk * 4);
  p.g_row = take(tk * 4);
  p.dh = take(tk * size_t(s.I) * 4);
  p.gh = take(tk * size_t(s.I) * 2);
  p.dg = take(tk * size_t(s.I) * 2);
  p.du = take(tk * size_t(s.I) * 2);
  p.dxp = take(tk * size_t(s.d) * 2);
  // G and U are recomputed by the forward's pipelined gate/up kernel, on its own tile height
  p.pipe_bm = ffn_small(s) ? kBmSmall : kBmPipe;
  size_t mt2 = N + (tk + p.pipe_bm - 1) / p.pipe_bm;
  if (mt2 > tk) mt2 = tk;
  p.pipe_mt_max = int(mt2);
  p.pipe_mtiles = take(mt2 * sizeof(MTile));
  p.pipe_n_mtiles = take(4);
  // x and dy rows gathered in FFN-row order, and 16 zero bytes, for the weight gradients
  p.xp = take(tk * size_t(s.d) * 2);
  p.dyp = take(tk * size_t(s.d) * 2);
  p.zero = take(16);
  p.total = o;
  return p;
}

// XOR swizzle of the 16-byte chunk slot for 64-byte LDS rows: the 32 rows of one MFMA
// operand read spread over all banks.
__host__ __device__ __forceinline__ int swz4(int r) {
  return (((r >> 1) & 1) << 1) ^ ((r >> 2) & 1) ^ (((r >> 3) & 1) << 1);
}

// Block-FP8 expert weights (E4M3 codes, one power-of-two scale per 128x128 block), packed
// for the pipelined FFN kernel.  Regions (256-byte aligned, in this order):
//   codes_gu  [N][ceil(I/128)][d/32][128 pair-rows][64 B]  pair-row p of n-tile nt holds
//             W_gate row nt*128+p and W_up row nt*128+p (rows past I are zero)
//   codes_d   [N][ceil(d/256)][I/32][128 pair-rows][64 B]  pair-row p of n-tile nt holds
//             W_down rows nt*256 + (p/32)*64 + p%32 and that + 32 (rows past d: zero)
//   scales_gu [N][2][ceil(I/128)][ceil(d/128)] fp32     2^k of each gate (0) / up (1) block
//   scales_d  [N][ceil(d/128)][ceil(I/128)] fp32        2^k of each W_down block
// A pair-row is four 16-byte chunks; chunk g holds the codes of columns 8g..8g+7 (of the
// 32) of its first row, then of its second row, and sits in slot g ^ swz4(p).  A wave's
// two weight blocks thus come from one 16-byte LDS read per lane, and the 32 pair-rows of
// one read hit distinct banks.
struct Fp8Plan {
  size_t codes_gu, codes_d, scales_gu, scales_d, total;
  int nt_gu, nt_d, nrb_i, nrb_d;  // n-tiles of gate/up and down; 128-row blocks of I and d
};
inline Fp8Plan plan_fp8(const lc_moe_shape& s) {
  Fp8Plan p{};
  // the kernel keeps a row of up to 128 column-block scales in two registers per lane
  if (!ffn_pipelined(s) || s.d > 16384 || s.I > 16384) return p;
  const size_t N = s.N;
  p.nt_gu = (s.I + 127) / 128;
  p.nt_d = (s.d + 255) / 256;
  p.nrb_i = (s.I + 127) / 128;
  p.nrb_d = (s.d + 127) / 128;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align256(o + bytes); return at; };
  p.codes_gu = take(N * p.nt_gu * size_t(s.d / 32) * 8192);
  p.codes_d = take(N * p.nt_d * size_t(s.I / 32) * 8192);
  p.scales_gu = take(N * 2 * size_t(p.nrb_i) * p.nrb_d * 4);
  p.scales_d = take(N * size_t(p.nrb_d) * p.nrb_i * 4);
  p.total = o;
  return p;
}

// The FP8 MFMA layer (block-FP8 weights and activations): 64-element K stages in both GEMMs.

// bf16 expert weights packed for the pipelined FFN kernel (lc_moe_pack_weights).  Regions
// (256-byte aligned, in this order):
//   gu [N][ceil(I/128)][d/32][256 rows][64 B]  rows 0..127 of n-tile nt are W_gate rows
//      nt*128 + r, rows 128..255 the W_up rows nt*128 + r - 128 (rows past I are zero)
//   d  [N][ceil(d/256)][I/32][256 rows][64 B]  row r of n-tile nt is W_down row nt*256 + r
//      (rows past d are zero)
// A row holds the 32 columns of one K step as four 16-byte chunks, chunk c in slot
// c ^ swz4(r): each 16 KB block is exactly the LDS image of one stage's weight rows.
struct PackPlan {
  size_t gu, d, total;
};
inline PackPlan plan_packed(const lc_moe_shape& s) {
  PackPlan p{};
  if (!ffn_pipelined(s)) return p;
  const size_t N = s.N;
  p.gu = 0;
  p.d = align256(N * size_t((s.I + 127) / 128) * size_t(s.d / 32) * 16384);
  p.total = p.d + N * size_t((s.d + 255) / 256) * size_t(s.I / 32) * 16384;
  return p;
}

// ---- launchers (host functions defined in the .hip files) ------------------------------

// Router logits L[T][E] = x W_r^T (fp32 result).  bf16 layers: W_r is first split into
// three bf16 parts (wsplit, 3*E*d bf16); with more than one split (router_split) the
// GEMM writes `splits` partial logit arrays [splits][T][E] to rpart, which are then summed
// in split order into logits.
// When zero_word is not NULL, the kernel also sets *zero_word = 0 (the counter of the fused
// top-K + permutation kernel that follows it on the stream).
hipError_t launch_router_logits(const lc_moe_shape& s, const void* x, const float* w_router,
                                bf16_t* wsplit, float* logits, float* rpart, hipStream_t st,
                                int32_t* zero_word = nullptr);
// Softmax over E, biased top-K; writes idx [T][K] and gate [T][K].
hipError_t launch_router_topk(const lc_moe_shape& s, const float* logits, const float* bias,
                              int32_t* idx, float* gate, hipStream_t st);

// Per-block expert histogram (+ per-token FFN count when ffn_cnt != nullptr).
hipError_t launch_histogram(const lc_moe_shape& s, const int32_t* idx, int32_t* block_counts,
                            int32_t* ffn_cnt, int nblocks, hipStream_t st);
// Column sums -> load [E]; offsets [N+1]; per-(block, expert) row bases; M-tile list.
hipError_t launch_scan(const lc_moe_shape& s, const int32_t* block_counts, int nblocks,
                       int32_t* load, int32_t* offsets, int32_t* block_base, MTile* mtiles,
                       int32_t* n_mtiles, int bm, hipStream_t st);
// Histogram, scan and scatter in one workgroup, for layers of one token block (T <= 256).
hipError_t launch_permute_small(const lc_moe_shape& s, const int32_t* idx, int32_t* load,
                                int32_t* ffn_cnt, int32_t* offsets, MTile* mtiles,
                                int32_t* n_mtiles, int bm, int32_t* slot_row, int32_t* perm_token,
                                hipStream_t st);
// The forward of a layer of one token block: softmax + biased top-K (idx, gate), then, in
// the workgroup that finishes last, the permutation (load, offsets, M-tile list, slot_row,
// perm_token) -- one launch for router_topk + permute_small.  *done must be 0 on entry
// (launch_router_logits zeroes it).
hipError_t launch_topk_permute(const lc_moe_shape& s, const float* logits, const float* bias,
                               int32_t* idx, float* gate, int32_t* done, int32_t* load,
                               int32_t* offsets, MTile* mtiles, int32_t* n_mtiles, int bm,
                               int32_t* slot_row, int32_t* perm_token, hipStream_t st);
// Stable scatter: slot_row [T][K], perm_token [nnz].
hipError_t launch_scatter(const lc_moe_shape& s, const int32_t* idx, const int32_t* block_base,
                          int nblocks, int32_t* slot_row, int32_t* perm_token, hipStream_t st);
// x_perm[r] = x[perm_token[r]] for r < offsets[N].
hipError_t launch_gather_rows(const lc_moe_shape& s, const void* x, const int32_t* perm_token,
                              const int32_t* offsets, void* x_perm, hipStream_t st);
// Copy n int32 values on the device (kernel, capturable).
hipError_t launch_copy_i32(const int32_t* src, int32_t* dst, size_t n, hipStream_t st);
hipError_t launch_copy_f32(const float* src, float* dst, size_t n, hipStream_t st);

// Grouped SwiGLU FFN over the FFN picks.
// With fp8 != nullptr (packed block-FP8 weights, pipelined shapes only) the weights come
// from it and w_gate / w_up / w_down are not read.
// With packed != nullptr (lc_moe_pack_weights, pipelined shapes only) the bf16 weights
// come from it instead.
hipError_t launch_ffn_gate_up(const lc_moe_shape& s, const void* x, const int32_t* perm_token,
                              const void* w_gate, const void* w_up, const void* fp8,
                              const void* packed, void* hbuf, const MTile* mtiles,
                              const int32_t* offsets, const int32_t* n_mtiles, int mt_max,
                              hipStream_t st);
hipError_t launch_ffn_down(const lc_moe_shape& s, const void* hbuf, const void* w_down,
                           const void* fp8, const void* packed, void* ybuf, const MTile* mtiles,
                           const int32_t* offsets, const int32_t* n_mtiles, int mt_max,
                           hipStream_t st);
// bf16 expert weights -> the packed layout of plan_packed.
hipError_t launch_pack_weights(const lc_moe_shape& s, const void* w_gate, const void* w_up,
                               const void* w_down, void* packed, hipStream_t st);
// Quantize bf16 W_gate, W_up [N][I][d] and W_down [N][d][I] into the packed block-FP8
// form (plan_fp8) at `out`.
hipError_t launch_quantize_weights(const lc_moe_shape& s, const void* w_gate, const void* w_up,
                                   const void* w_down, void* out, hipStream_t st);

// y_t = (sum over the token's FFN picks, in pick order, of g * FFN row)
//       + (sum of its zero-computation picks' gates, in pick order) * x_t, fp32 accumulation.
hipError_t launch_combine(const lc_moe_shape& s, const void* x, const void* ybuf,
                          const int32_t* slot_row, const float* gate, void* y, hipStream_t st);

// Backward of the grouped SwiGLU FFN (bf16): from the permutation of the given picks
// (offsets, M-tile list with kBmBwd-row tiles, perm_token, slot_row) and the picks' gates,
// writes dx [T][d] and dW_gate, dW_up [N][I][d], dW_down [N][d][I] (bf16).
hipError_t launch_ffn_backward(const lc_moe_shape& s, const BwPlan& p, void* ws, const void* x,
                               const void* w_gate, const void* w_up, const void* w_down,
                               const int32_t* idx, const float* gate, const void* dy, void* dx,
                               void* dw_gate, void* dw_up, void* dw_down, hipStream_t st);

// Block-FP8 activations: rows x cols bf16 (cols a multiple of 64) -> E4M3 codes [rows][cols]
// and E8M0 scales [rows][ceil(cols/128)] (exponent k + 127 of each 1 x 128 block's 2^k).
hipError_t launch_quantize_act(const void* x, int rows, int cols, unsigned char* codes,
                               unsigned char* scales, hipStream_t st);
// The pipelined gate/up kernel's backward form (MODE 2): G and U recomputed for the rows of
// an M-tile list of the pipelined kernel's height; with dH (fp32 [rows][I]) and each FFN row's
// gate g it writes g*H into gh and dG, dU (bf16 [rows][I]).
struct GuGrad {
  const float* dh;
  const float* g_row;
  bf16_t* dg;
  bf16_t* du;
};
hipError_t launch_ffn_gate_up_grad(const lc_moe_shape& s, const void* x, const int32_t* perm_token,
                                   const void* w_gate, const void* w_up, const GuGrad& gg, void* gh,
                                   const MTile* mtiles, const int32_t* offsets, const int32_t* n_mtiles,
                                   int mt_max, hipStream_t st);
// An M-tile list of height bm over the FFN experts' rows given by offsets [N+1] (one
// workgroup; the same tiles the permutation's scan would list at that height).
hipError_t launch_mtile_list(const lc_moe_shape& s, const int32_t* offsets, int bm, MTile* mtiles,
                             int32_t* n_mtiles, hipStream_t st);

// The FP8 MFMA grouped FFN from the x codes and scales in the workspace (p.xq, p.xs) and the
// block-FP8 weights.  mode 0: gate/up, H quantized in the epilogue into p.hbuf (codes
// [T*K][I], then E8M0 scales [T*K][ceil(I/128)] at the next 256-byte boundary); mode 1:
// down, Y rows (bf16) into p.ybuf.
hipError_t launch_ffn_fp8_mfma(const lc_moe_shape& s, const WsPlan& p, void* ws, const void* fp8, int mode,
                               hipStream_t st);

// One PID update of the selection bias over the E = N+Z experts.
hipError_t launch_bias_update(int E, long long tk, float kp, float ki, float kd,
                              const int32_t* load, const float* target, float* bias,
                              float* integral, float* prev_err, hipStream_t st);

}  // namespace lcm

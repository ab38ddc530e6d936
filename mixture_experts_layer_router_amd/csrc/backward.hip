// Backward of the grouped SwiGLU FFN for fixed picks and gates: the gradients of
// L = sum_t <dy_t, y_t> with respect to x and every expert matrix.  The pages describe the
// layer's training (LongCat-Flash article, itouyu.top, section "Model scaling and
// multi-stage training") but give no backward pass; this is the plain gradient of the
// layer's sum (section "Zero-computation experts") with the routing held fixed.
//
// For the rows r of FFN expert e (pick (t, k) with gate g, x_r = x_t, dy_r = dy_t):
//   G = x_r W_gate^T, U = x_r W_up^T, s = sigmoid(G), a = G s, H = a U
//   dH_r   = g dy_r W_down                      (kind DH)
//   gH_r   = g H_r;  dG_r = dH_r U (s + a (1 - s));  dU_r = dH_r a     (G and U recomputed by
//            the forward's pipelined gate/up kernel with its backward epilogue, ffn.hip MODE 2)
//   dX_r   = dG_r W_gate + dU_r W_up            (kind DX)
//   dW_down_e = sum_r dy_r^T gH_r               (kind DWD, ffn_wgrad_kernel)
//   dW_gate_e = sum_r dG_r^T x_r, dW_up_e = sum_r dU_r^T x_r        (kind DWGU, ffn_wgrad_kernel)
//   dx_t = sum over the token's FFN picks, in pick order, of dX_r + (zero picks' gate sum) dy_t
//
// Every product is a bf16 grouped GEMM on v_mfma_f32_32x32x16_bf16 with fp32 accumulation,
// its operands staged in LDS as they lie in memory by direct global->LDS loads: an operand
// whose reduction index is contiguous (dy, dG, dU rows) as the forward stages its rows, one
// whose output index is contiguous (W_down, W_gate, W_up read along their rows; activation
// rows read along the tokens) in 512-byte rows read by gfx950's transposing LDS read.  So no
// weight or activation needs a transposed copy.  No atomics: every output element is
// written once, by one workgroup, so the results are deterministic.
#include "common.h"
#include "lanes.h"
#include "lds_dma.h"

namespace lcm {

namespace bw {
enum { DH = 0, DX = 2, DWD = 3, DWGU = 4 };  // (1: G/U, on the pipelined gate/up kernel)
}  // namespace bw

struct BwArgs {
  int d, I, N;
  const bf16_t* x;
  const bf16_t* dy;
  const bf16_t* wg;
  const bf16_t* wu;
  const bf16_t* wd;
  const int32_t* perm_token;
  const float* g_row;
  const int32_t* offsets;
  float* dh;
  bf16_t* gh;
  bf16_t* dg;
  bf16_t* du;
  bf16_t* dxp;
  bf16_t* dwg;
  bf16_t* dwu;
  bf16_t* dwd;
  const bf16_t* xp;     // x rows gathered in FFN-row order [rows][d] (weight gradients)
  const bf16_t* dyp;    // dy rows gathered the same way
  const bf16_t* zero;   // 16 zero bytes (the source of operand chunks past the data)
  int n_ntiles;  // N-tiles per M-tile (dH, dX)
};

// ---------------------------------------------------------------------------------------
// Weight gradients on a persistent direct-load ring: dW_down_e = dY_e^T gH_e and
// dW_gate_e, dW_up_e = dG_e^T X_e, dU_e^T X_e, the reductions running over the expert's rows.
// Both operands lie with the reduction index slowest ([row][column]), so a stage of 32 rows
// of each is staged as it lies (rows of 512 bytes = 256 columns of the tile) by direct
// global->LDS loads and read with the transposing LDS read.  Tile 256 x 256 (64 MACs per
// loaded byte), 512 threads = 8 waves of 64 rows x 128 columns, 4-stage ring of 32 KB
// stages.  A unit (expert, matrix, 256-row block, 256-column block) has as many stages as
// the expert has 32-row steps, often 8 to 10, so one workgroup per CU loops over its units
// and the ring runs on across unit boundaries: the next unit's first stages load while
// this one's last stages compute and its tile is stored.  Units of one expert run on one
// XCD (each XCD takes a contiguous eighth of the unit order), where their shared rows meet
// in its L2.  Rows past the expert's last and columns past the matrix load zeros.
// LDS: 16-byte chunk c of a stage row r of either operand sits in the 32-byte granule
// (c / 2) ^ 2 (r % 4); a transposing read's 16-lane groups then read the 4 rows of a group
// from 8 distinct granules (64 banks).
// ---------------------------------------------------------------------------------------
namespace wg {
constexpr int BM = 256, BN = 256, BK = 32, NST = 4;
constexpr int OPB = BK * BM * 2;   // bytes of one operand in one stage (16 KB)
constexpr int STAGE = 2 * OPB;     // A then B (32 KB)
constexpr int LDS = NST * STAGE;   // 128 KB
constexpr int LOADS = 4;           // direct loads per wave and stage (2 per operand)
}  // namespace wg

template <int KIND>
__global__ __launch_bounds__(512, 1) void ffn_wgrad_kernel(BwArgs a) {
  using namespace wg;
  static_assert(KIND == bw::DWD || KIND == bw::DWGU, "weight-gradient kinds only");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[LDS];
  const int Mdim = KIND == bw::DWD ? a.d : a.I;  // rows of the gradient matrix
  const int Ndim = KIND == bw::DWD ? a.I : a.d;  // its columns
  const int n_mt = (Mdim + BM - 1) / BM, n_nt = (Ndim + BN - 1) / BN;
  const int per_mat = n_mt * n_nt;
  const int per_exp = (KIND == bw::DWGU ? 2 : 1) * per_mat;
  const int U = a.N * per_exp;
  // this workgroup's units: XCD x = blockIdx.x % 8 owns units [x U / 8, (x + 1) U / 8); its
  // gridDim.x / 8 workgroups take every (gridDim.x / 8)-th of them
  const int xcd = blockIdx.x & 7, sl = blockIdx.x >> 3, nsl = gridDim.x >> 3;
  const int u_lo = int(int64_t(xcd) * U / 8), u_hi = int(int64_t(xcd + 1) * U / 8);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  struct Unit {
    int e, mat, m0, n0, row0, ktot, nk;
  };
  auto decode = [&](int u) {
    Unit t;
    t.e = __builtin_amdgcn_readfirstlane(u / per_exp);
    int r = u - t.e * per_exp;
    t.mat = r / per_mat;
    r -= t.mat * per_mat;
    t.m0 = (r / n_nt) * BM;
    t.n0 = (r % n_nt) * BN;
    // offsets[e], offsets[e+1] through one scalar load (waited for in the same block): a
    // vector load here would make the compiler wait for every direct load in flight, which
    // empties the ring at each unit boundary
    uint64_t oo;
    asm volatile("s_load_dwordx2 %0, %1, 0x0\n"
                 "s_waitcnt lgkmcnt(0)"
                 : "=s"(oo)
                 : "s"(a.offsets + t.e)
                 : "memory");
    t.row0 = int(uint32_t(oo));
    t.ktot = int(uint32_t(oo >> 32)) - t.row0;
    t.nk = (t.ktot + BK - 1) / BK;
    return t;
  };

  // ---- the load stream: stage (unit, kt) of this workgroup's units with rows --------------
  // Wave w's load i (i < 2) of an operand fills stage rows 2 (w + 8 i) and 2 (w + 8 i) + 1:
  // lane l writes row 2 (w + 8 i) + l / 32, 16-byte slot l % 32, with logical chunk
  // 2 ((slot / 2) ^ 2 (row % 4)) + slot % 2 of that row.
  int iu = u_lo + sl, ikt = 0, issued = 0;
  Unit iunit{};
  auto iskip = [&]() {
    for (; iu < u_hi; iu += nsl) {
      iunit = decode(iu);
      if (iunit.nk > 0) break;
    }
  };
  iskip();
  const int slot16 = lane & 31;
  auto issue = [&](int slot) {
    unsigned char* st = smem + slot * STAGE;
    const Unit& t = iunit;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int kr = 2 * (wave + 8 * i) + (lane >> 5);                       // stage row
      const int c = 2 * ((slot16 >> 1) ^ (2 * (kr & 3))) + (slot16 & 1);      // logical chunk
      const int k = ikt * BK + kr;                                          // expert row
      const size_t row = size_t(t.row0 + k);
      const bool kin = k < t.ktot;
      // A: (m, k) = the row's column m0 + m
      const int ma = t.m0 + c * 8;
      const bf16_t* srca;
      if constexpr (KIND == bw::DWD) srca = a.dyp + row * a.d + ma;
      else srca = (t.mat == 0 ? a.dg : a.du) + row * a.I + ma;
      dma16(kin && ma < Mdim ? srca : a.zero, st + (wave + 8 * i) * 1024);
      // B: (n, k) = the row's column n0 + n
      const int nb = t.n0 + c * 8;
      const bf16_t* srcb;
      if constexpr (KIND == bw::DWD) srcb = a.gh + row * a.I + nb;
      else srcb = a.xp + row * a.d + nb;
      dma16(kin && nb < Ndim ? srcb : a.zero, st + OPB + (wave + 8 * i) * 1024);
    }
    ++issued;
    if (++ikt == t.nk) {
      ikt = 0;
      iu += nsl;
      iskip();
    }
  };

  // ---- fragments: transposing reads (see ffn_backward_kernel) with the granule swizzle ----
  // A substep's 12 reads (2 per fragment: k rows +0..3 and +4..7) go out in one asm block
  // that waits for them itself.  Written with the builtin, each read got a wait for every
  // direct load in flight (the compiler cannot tell the stage it reads from the stages
  // still loading), which emptied the ring at every step; the explicit vmcnt waits and
  // the barrier already order the reads after their stage's loads.
  const int tr_j = (lane >> 2) & 3;                  // the row in its group of 4 (= row % 4)
  const int tr_row = 8 * (lane >> 5) + tr_j;         // + 4 h + substep
  const int tr_g = (lane >> 4) & 1;                  // + column granule base / 16
  const int tr_byte = 8 * (lane & 3);
  typedef __attribute__((address_space(3))) unsigned char lds_u8;
  auto lds_addr = [&](const unsigned char* op, int base, int ks) -> uint32_t {
    const int lg = (base >> 4) + tr_g;
    const unsigned char* p = op + (ks + tr_row) * 512 + ((lg ^ (2 * tr_j)) << 5) + tr_byte;
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(reinterpret_cast<const lds_u8*>(
        reinterpret_cast<uintptr_t>(p))));
  };
  auto frags = [&](const unsigned char* st, int ks, bf16x8 (&fa)[2], bf16x8 (&fb)[4]) {
    const uint32_t a0 = lds_addr(st, wm * 64, ks), a1 = lds_addr(st, wm * 64 + 32, ks);
    const uint32_t b0 = lds_addr(st + OPB, wn * 128, ks), b1 = lds_addr(st + OPB, wn * 128 + 32, ks);
    const uint32_t b2 = lds_addr(st + OPB, wn * 128 + 64, ks), b3 = lds_addr(st + OPB, wn * 128 + 96, ks);
    uint64_t r[12];
    asm volatile(
        "ds_read_b64_tr_b16 %0, %12\n"
        "ds_read_b64_tr_b16 %1, %12 offset:2048\n"
        "ds_read_b64_tr_b16 %2, %13\n"
        "ds_read_b64_tr_b16 %3, %13 offset:2048\n"
        "ds_read_b64_tr_b16 %4, %14\n"
        "ds_read_b64_tr_b16 %5, %14 offset:2048\n"
        "ds_read_b64_tr_b16 %6, %15\n"
        "ds_read_b64_tr_b16 %7, %15 offset:2048\n"
        "ds_read_b64_tr_b16 %8, %16\n"
        "ds_read_b64_tr_b16 %9, %16 offset:2048\n"
        "ds_read_b64_tr_b16 %10, %17\n"
        "ds_read_b64_tr_b16 %11, %17 offset:2048\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]),
          "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11])
        : "v"(a0), "v"(a1), "v"(b0), "v"(b1), "v"(b2), "v"(b3)
        : "memory");
    auto pack = [](uint64_t lo, uint64_t hi) {
      typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));
      return __builtin_bit_cast(bf16x8, u64x2{lo, hi});
    };
    fa[0] = pack(r[0], r[1]);
    fa[1] = pack(r[2], r[3]);
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[j] = pack(r[4 + 2 * j], r[5 + 2 * j]);
  };

  f32x16 acc[2][4];
  for (int s = 0; s < NST - 1 && iu < u_hi; ++s) issue(s);
  int g = 0;  // stages consumed
  for (int cu = u_lo + sl; cu < u_hi; cu += nsl) {
    const Unit t = decode(cu);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    for (int kt = 0; kt < t.nk; ++kt, ++g) {
      wait_vmcnt((issued - 1 - g) * LOADS);  // this wave's loads of stage g landed
      wait_lds_reads();
      block_barrier();  // every wave's loads of stage g visible; stage g-1 read by all
      if (iu < u_hi) issue(issued % NST);  // stage g+NST-1 into stage g-1's slot
      const unsigned char* st = smem + (g % NST) * STAGE;
#pragma unroll
      for (int ks = 0; ks < BK; ks += 16) {
        bf16x8 fa[2], fb[4];
        frags(st, ks, fa, fb);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
      }
    }
    // ---- the unit's tile (zeros for an expert without rows).  32x32 D layout: column
    // lane % 32, rows 8 (r / 4) + 4 (lane / 32) + r % 4.  Lanes 4q .. 4q+3 hold a 4 x 4
    // block (4 rows r % 4 = 0..3 of columns 4q .. 4q+3); a transpose among them gives each
    // lane one row of 4 columns, stored as 8 bytes.
    bf16_t* out;
    if constexpr (KIND == bw::DWD) out = a.dwd + (size_t(t.e) * a.d + t.m0) * a.I + t.n0;
    else out = (t.mat == 0 ? a.dwg : a.dwu) + (size_t(t.e) * a.I + t.m0) * a.d + t.n0;
    const int q4 = lane & 3;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          float v[4];
#pragma unroll
          for (int t4 = 0; t4 < 4; ++t4) v[t4] = acc[i][j][rq * 4 + t4];
          float w[4];
          quad_transpose(v, q4, w);
          const int m = wm * 64 + i * 32 + 8 * rq + 4 * (lane >> 5) + q4;
          const int n = wn * 128 + j * 32 + (lane & 28);
          if (m < Mdim - t.m0 && n < Ndim - t.n0) {
            const uint32_t lo = f2bf(w[0]) | (uint32_t(f2bf(w[1])) << 16);
            const uint32_t hi = f2bf(w[2]) | (uint32_t(f2bf(w[3])) << 16);
            *reinterpret_cast<uint2*>(out + size_t(m) * Ndim + n) = make_uint2(lo, hi);
          }
        }
  }
}

// ---------------------------------------------------------------------------------------
// dH = g dY W_down and dX = dG W_gate + dU W_up on a direct-load ring: work unit (256-row
// M-tile of an expert's rows, 256 output columns), K = d (dH) or 2 I (dX: dG against W_gate,
// then dU against W_up).  A (dY rows gathered in FFN-row order, or dG / dU rows) is
// K-contiguous: staged as the forward stages its activation rows (64-byte LDS rows, 16-byte
// chunk c of row r in slot c ^ swz4(r)) and read with 16-byte reads.  B (W_down, W_gate,
// W_up rows) is N-contiguous: staged as the weight-gradient kernel stages its operands
// (512-byte rows, 32-byte-granule swizzle) and read with transposing reads.  512 threads =
// 8 waves of 64 rows x 128 columns, 4-stage ring of 32 KB stages, one workgroup per CU,
// XCD-aware unit order as in the forward.  Rows past the tile read the tile's first row
// (never stored); columns past the matrix load zeros.
// ---------------------------------------------------------------------------------------
namespace ba {
constexpr int BM = 256, BN = 256, BK = 32, NST = 4;
constexpr int A_BYTES = BM * 64;       // 16 KB
constexpr int B_BYTES = BK * BN * 2;   // 16 KB
constexpr int STAGE = A_BYTES + B_BYTES, LDS = NST * STAGE;  // 128 KB
constexpr int LOADS = 4;               // direct loads per wave and stage
}  // namespace ba

template <int KIND>
__global__ __launch_bounds__(512, 1) void ffn_bwd_act_kernel(BwArgs a, const MTile* __restrict__ mtiles,
                                                             const int32_t* __restrict__ n_mtiles_ptr) {
  using namespace ba;
  static_assert(KIND == bw::DH || KIND == bw::DX, "activation kinds");
  static_assert(BM == kBmBwd, "the M-tile list is the backward permutation's");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[LDS];
  const int ncols = KIND == bw::DH ? a.I : a.d;
  const int n_nt = a.n_ntiles;
  // (M-tile, n-tile) unit, XCD-aware as in the forward
  const int U = *n_mtiles_ptr * n_nt, per = (U + 7) >> 3;
  const int slot_w = blockIdx.x >> 3;
  if (slot_w >= per) return;
  const int u = (blockIdx.x & 7) * per + slot_w;
  if (u >= U) return;
  const MTile tb = mtiles[u / n_nt];
  const int mt = (a.offsets[tb.expert + 1] - a.offsets[tb.expert] + BM - 1) / BM;
  const int ul = u - tb.first_tile * n_nt;
  const int ntile = ul / mt;
  const MTile tile = mtiles[tb.first_tile + (ul - ntile * mt)];
  const int e = tile.expert, row0 = tile.row0, rows = tile.rows;
  const int n0 = ntile * BN;
  const int nk = (KIND == bw::DX ? 2 * a.I : a.d) / BK;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // ---- loads: wave w's A loads q = w, w + 8 fill rows 16 q .. 16 q + 15 (lane l: row
  // 16 q + l / 4, slot l % 4, global chunk (l % 4) ^ swz4(row)); its B loads q = w, w + 8
  // fill k rows 2 q, 2 q + 1 (lane l: row 2 q + l / 32, 16-byte slot l % 32 with logical
  // chunk 2 ((slot / 2) ^ 2 (row % 4)) + slot % 2)
  size_t arow_off[2];
  int acol[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = (wave + 8 * i) * 16 + (lane >> 2);
    arow_off[i] = size_t(row0 + (r < rows ? r : 0));
    acol[i] = ((lane & 3) ^ swz4(r)) * 8;
  }
  const int slot16 = lane & 31;
  auto issue = [&](int kt, int slot) {
    unsigned char* st = smem + slot * STAGE;
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const bf16_t* srca;
      if constexpr (KIND == bw::DH) srca = a.dyp + arow_off[i] * a.d + k0 + acol[i];
      else srca = (k0 < a.I ? a.dg + arow_off[i] * a.I + k0 : a.du + arow_off[i] * a.I + (k0 - a.I)) + acol[i];
      dma16(srca, st + (wave + 8 * i) * 1024);
      const int kr = 2 * (wave + 8 * i) + (lane >> 5);
      const int c = 2 * ((slot16 >> 1) ^ (2 * (kr & 3))) + (slot16 & 1);
      const int n = n0 + c * 8;
      const int k = k0 + kr;
      const bf16_t* srcb;
      if constexpr (KIND == bw::DH) srcb = a.wd + (size_t(e) * a.d + k) * a.I + n;  // W_down[e] as [d][I]
      else srcb = (k < a.I ? a.wg + (size_t(e) * a.I + k) * a.d : a.wu + (size_t(e) * a.I + (k - a.I)) * a.d) + n;
      dma16(n < ncols ? srcb : a.zero, st + A_BYTES + (wave + 8 * i) * 1024);
    }
  };

  // ---- fragments -------------------------------------------------------------------------
  const int l32 = lane & 31, khalf = lane >> 5, sw = swz4(l32);
  const int tr_j = (lane >> 2) & 3, tr_row = 8 * (lane >> 5) + tr_j, tr_g = (lane >> 4) & 1;
  const int tr_byte = 8 * (lane & 3);
  typedef __attribute__((address_space(3))) unsigned char lds_u8;
  auto lds_addr = [&](const unsigned char* p) -> uint32_t {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(reinterpret_cast<const lds_u8*>(
        reinterpret_cast<uintptr_t>(p))));
  };
  auto b_addr = [&](const unsigned char* bop, int base, int ks) -> uint32_t {
    const int lg = (base >> 4) + tr_g;
    return lds_addr(bop + (ks + tr_row) * 512 + ((lg ^ (2 * tr_j)) << 5) + tr_byte);
  };
  auto frags = [&](const unsigned char* st, int ks, bf16x8 (&fa)[2], bf16x8 (&fb)[4]) {
    const int c = ks / 8 + khalf;  // the lane's 16-byte chunk of the A rows
#pragma unroll
    for (int i = 0; i < 2; ++i)
      fa[i] = *reinterpret_cast<const bf16x8*>(st + (wm * 64 + i * 32 + l32) * 64 + ((c ^ sw) << 4));
    const unsigned char* bop = st + A_BYTES;
    const uint32_t b0 = b_addr(bop, wn * 128, ks), b1 = b_addr(bop, wn * 128 + 32, ks);
    const uint32_t b2 = b_addr(bop, wn * 128 + 64, ks), b3 = b_addr(bop, wn * 128 + 96, ks);
    uint64_t r[8];
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n"
        "ds_read_b64_tr_b16 %1, %8 offset:2048\n"
        "ds_read_b64_tr_b16 %2, %9\n"
        "ds_read_b64_tr_b16 %3, %9 offset:2048\n"
        "ds_read_b64_tr_b16 %4, %10\n"
        "ds_read_b64_tr_b16 %5, %10 offset:2048\n"
        "ds_read_b64_tr_b16 %6, %11\n"
        "ds_read_b64_tr_b16 %7, %11 offset:2048\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]),
          "=&v"(r[7])
        : "v"(b0), "v"(b1), "v"(b2), "v"(b3)
        : "memory");
    typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[j] = __builtin_bit_cast(bf16x8, u64x2{r[2 * j], r[2 * j + 1]});
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  const int npro = nk < NST - 1 ? nk : NST - 1;
  for (int s2 = 0; s2 < npro; ++s2) issue(s2, s2);
  int issued = npro;
  for (int kt = 0; kt < nk; ++kt) {
    wait_vmcnt((issued - 1 - kt) * LOADS);  // this wave's loads of stage kt landed
    wait_lds_reads();
    block_barrier();  // every wave's loads of stage kt visible; stage kt-1 read by all
    if (issued < nk) {
      issue(issued, issued % NST);  // stage kt+NST-1 into stage kt-1's slot
      ++issued;
    }
    const unsigned char* st = smem + (kt % NST) * STAGE;
#pragma unroll
    for (int ks = 0; ks < BK; ks += 16) {
      bf16x8 fa[2], fb[4];
      frags(st, ks, fa, fb);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  }

  // ---- epilogue: 4-lane transposes (see ffn_wgrad_kernel), one row of 4 columns per lane --
  const int q4 = lane & 3;
  // dH: the gates of the lane's 8 rows, loaded before the first store (a load between the
  // stores would wait for every store before it)
  float grow[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int m = wm * 64 + i * 32 + 8 * rq + 4 * (lane >> 5) + q4;
      grow[i][rq] = KIND == bw::DH && m < rows ? a.g_row[row0 + m] : 0.f;
    }
  // the loads complete here, not next to their first use among the stores
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) asm volatile("" : "+v"(grow[i][rq]));
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        float v[4], w[4];
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) v[t4] = acc[i][j][rq * 4 + t4];
        quad_transpose(v, q4, w);
        const int m = wm * 64 + i * 32 + 8 * rq + 4 * (lane >> 5) + q4;
        const int n = n0 + wn * 128 + j * 32 + (lane & 28);
        if (m < rows && n < ncols) {
          const size_t r = size_t(row0 + m);
          if constexpr (KIND == bw::DH) {
            const float g = grow[i][rq];
            *reinterpret_cast<float4*>(a.dh + r * a.I + n) = make_float4(w[0] * g, w[1] * g, w[2] * g, w[3] * g);
          } else {
            const uint32_t lo = f2bf(w[0]) | (uint32_t(f2bf(w[1])) << 16);
            const uint32_t hi = f2bf(w[2]) | (uint32_t(f2bf(w[3])) << 16);
            *reinterpret_cast<uint2*>(a.dxp + r * a.d + n) = make_uint2(lo, hi);
          }
        }
      }
}

// gate of each FFN row: g_row[slot_row[t][k]] = gate[t][k]; and the 16 zero bytes
__global__ __launch_bounds__(256) void row_gates_kernel(const int32_t* __restrict__ slot_row,
                                                        const float* __restrict__ gate,
                                                        float* __restrict__ g_row, size_t tk,
                                                        uint4* __restrict__ zero) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *zero = make_uint4(0, 0, 0, 0);
  for (size_t i = size_t(blockIdx.x) * 256 + threadIdx.x; i < tk; i += size_t(gridDim.x) * 256) {
    const int r = slot_row[i];
    if (r >= 0) g_row[r] = gate[i];
  }
}

// dx_t = sum over the token's FFN picks, in pick order, of dX[row] + (zero picks' gates,
// summed in pick order) * dy_t; fp32, one rounding.  One workgroup per token.
__global__ __launch_bounds__(256) void dx_combine_kernel(const bf16_t* __restrict__ dxp,
                                                         const bf16_t* __restrict__ dy,
                                                         const int32_t* __restrict__ slot_row,
                                                         const float* __restrict__ gate,
                                                         bf16_t* __restrict__ dx, int d, int K) {
  const int t = blockIdx.x;
  for (int c = threadIdx.x * 8; c < d; c += 256 * 8) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float gz = 0.f;
    for (int k = 0; k < K; ++k) {
      const int r = slot_row[size_t(t) * K + k];
      if (r < 0) {
        gz += gate[size_t(t) * K + k];
        continue;
      }
      const uint4 q = *reinterpret_cast<const uint4*>(dxp + size_t(r) * d + c);
      const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += __uint_as_float(w[i] << 16);
        acc[2 * i + 1] += __uint_as_float(w[i] & 0xFFFF0000u);
      }
    }
    if (gz != 0.f) {
      const uint4 q = *reinterpret_cast<const uint4*>(dy + size_t(t) * d + c);
      const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = fmaf(gz, __uint_as_float(w[i] << 16), acc[2 * i]);
        acc[2 * i + 1] = fmaf(gz, __uint_as_float(w[i] & 0xFFFF0000u), acc[2 * i + 1]);
      }
    }
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = f2bf(acc[2 * i]) | (uint32_t(f2bf(acc[2 * i + 1])) << 16);
    *reinterpret_cast<uint4*>(dx + size_t(t) * d + c) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

hipError_t launch_ffn_backward(const lc_moe_shape& s, const BwPlan& p, void* ws, const void* x,
                               const void* w_gate, const void* w_up, const void* w_down,
                               const int32_t* idx, const float* gate, const void* dy, void* dx,
                               void* dw_gate, void* dw_up, void* dw_down, hipStream_t st) {
  using namespace bw;
  char* w = static_cast<char*>(ws);
  BwArgs a{};
  a.d = s.d;
  a.I = s.I;
  a.N = s.N;
  a.x = static_cast<const bf16_t*>(x);
  a.dy = static_cast<const bf16_t*>(dy);
  a.wg = static_cast<const bf16_t*>(w_gate);
  a.wu = static_cast<const bf16_t*>(w_up);
  a.wd = static_cast<const bf16_t*>(w_down);
  a.perm_token = reinterpret_cast<const int32_t*>(w + p.perm_token);
  a.g_row = reinterpret_cast<const float*>(w + p.g_row);
  a.offsets = reinterpret_cast<const int32_t*>(w + p.offsets);
  a.dh = reinterpret_cast<float*>(w + p.dh);
  a.gh = reinterpret_cast<bf16_t*>(w + p.gh);
  a.dg = reinterpret_cast<bf16_t*>(w + p.dg);
  a.du = reinterpret_cast<bf16_t*>(w + p.du);
  a.dxp = reinterpret_cast<bf16_t*>(w + p.dxp);
  a.dwg = static_cast<bf16_t*>(dw_gate);
  a.dwu = static_cast<bf16_t*>(dw_up);
  a.dwd = static_cast<bf16_t*>(dw_down);
  a.xp = reinterpret_cast<const bf16_t*>(w + p.xp);
  a.dyp = reinterpret_cast<const bf16_t*>(w + p.dyp);
  a.zero = reinterpret_cast<const bf16_t*>(w + p.zero);

  const size_t tk = size_t(s.T) * s.K;
  hipLaunchKernelGGL(row_gates_kernel, dim3(unsigned(tk / 256 + 1 < 4096 ? tk / 256 + 1 : 4096)), dim3(256), 0,
                     st, reinterpret_cast<const int32_t*>(w + p.slot_row), gate, reinterpret_cast<float*>(w + p.g_row),
                     tk, reinterpret_cast<uint4*>(w + p.zero));
  auto grid_of = [](size_t units) { return dim3(unsigned((units + 7) / 8 * 8)); };
  // x and dy rows in FFN-row order (dH, dW_down and dW_gate / dW_up read them contiguously)
  hipError_t err = launch_gather_rows(s, x, a.perm_token, a.offsets, w + p.xp, st);
  if (err != hipSuccess) return err;
  err = launch_gather_rows(s, dy, a.perm_token, a.offsets, w + p.dyp, st);
  if (err != hipSuccess) return err;
  // the M-tile lists: the permutation's (256 rows) for dH and dX, one at the pipelined
  // gate/up kernel's height for G, U
  const MTile* act_mtiles = reinterpret_cast<const MTile*>(w + p.mtiles);
  const int32_t* act_n = reinterpret_cast<const int32_t*>(w + p.n_mtiles);
  MTile* pipe_mtiles = reinterpret_cast<MTile*>(w + p.pipe_mtiles);
  int32_t* pipe_n = reinterpret_cast<int32_t*>(w + p.pipe_n_mtiles);
  err = launch_mtile_list(s, a.offsets, p.pipe_bm, pipe_mtiles, pipe_n, st);
  if (err != hipSuccess) return err;
  // dH
  a.n_ntiles = (s.I + ba::BN - 1) / ba::BN;
  hipLaunchKernelGGL(ffn_bwd_act_kernel<DH>, grid_of(size_t(p.mt_max) * a.n_ntiles), dim3(512), 0, st, a,
                     act_mtiles, act_n);
  // G and U recomputed on the forward's pipelined gate/up kernel: g*H, dG, dU
  err = launch_ffn_gate_up_grad(s, x, a.perm_token, w_gate, w_up, GuGrad{a.dh, a.g_row, a.dg, a.du}, a.gh,
                                pipe_mtiles, a.offsets, pipe_n, p.pipe_mt_max, st);
  if (err != hipSuccess) return err;
  // dX
  a.n_ntiles = (s.d + ba::BN - 1) / ba::BN;
  hipLaunchKernelGGL(ffn_bwd_act_kernel<DX>, grid_of(size_t(p.mt_max) * a.n_ntiles), dim3(512), 0, st, a,
                     act_mtiles, act_n);
  // weight gradients: every expert (an expert without rows gets zero gradients), one
  // persistent workgroup per CU
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return hipErrorInvalidDevice;
  const dim3 pgrid(unsigned(cus >= 8 ? cus / 8 * 8 : 8));
  hipLaunchKernelGGL(ffn_wgrad_kernel<DWD>, pgrid, dim3(512), 0, st, a);
  hipLaunchKernelGGL(ffn_wgrad_kernel<DWGU>, pgrid, dim3(512), 0, st, a);
  hipLaunchKernelGGL(dx_combine_kernel, dim3(s.T), dim3(256), 0, st, a.dxp, a.dy,
                     reinterpret_cast<const int32_t*>(w + p.slot_row), gate, static_cast<bf16_t*>(dx), s.d, s.K);
  return hipGetLastError();
}

}  // namespace lcm

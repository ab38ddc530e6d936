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
//   dW_down_e = sum_r dy_r^T gH_r               (kind DWD)
//   dW_gate_e = sum_r dG_r^T x_r, dW_up_e = sum_r dU_r^T x_r        (kind DWGU)
//   dx_t = sum over the token's FFN picks, in pick order, of dX_r + (zero picks' gate sum) dy_t
//
// The other four products run on one grouped GEMM kernel, C[m][n] = sum_k A(m, k) B(n, k), bf16 on
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation.  Each operand is either K-contiguous
// ("row": element (m, k) at row m, column k, as the forward's weights and activations) or
// M-contiguous ("col": for a fixed k the m run contiguously, as W_down read along its
// rows, or an activation matrix read along its tokens).  Both are staged in LDS as they lie
// in memory (16-byte loads, 16-byte LDS writes); a row tile is read by the MFMA with one
// 16-byte LDS read per fragment, a col tile with eight 2-byte reads.  So no operand needs
// a transposed copy.  Tile 128 x 128, K step 32, 256 threads (2 x 2 waves of 64 x 64),
// two LDS stages with the next step's loads in registers.  No atomics: every output
// element is written once, by one workgroup, so the results are deterministic.
#include "common.h"

namespace lcm {

namespace bw {
constexpr int BM = 128, BN = 128, BK = 32;
constexpr int LDR = BK + 8;    // row tile: [128][40] bf16 (80-byte rows)
// col tile: [32][160] bf16 (320-byte rows: a transposing read's four 16-lane groups read
// rows 16 dwords apart, 32 bytes each, on 64 distinct banks)
constexpr int LDC = BM + 32;
constexpr int TILE = BM * LDR; // elements per operand and stage (both forms: 128 x 40 = 32 x 160)
static_assert(BK * LDC <= TILE, "col tile must fit the stage");
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
  const MTile* mtiles;
  const int32_t* n_mtiles;
  float* dh;
  bf16_t* gh;
  bf16_t* dg;
  bf16_t* du;
  bf16_t* dxp;
  bf16_t* dwg;
  bf16_t* dwu;
  bf16_t* dwd;
  int n_ntiles;  // N-tiles per M-tile (activation kinds) or per expert and matrix (weight kinds)
  int n_mt;      // weight kinds: M-tiles per matrix
  int n_units;   // weight kinds: units in all
};

template <int KIND>
__global__ __launch_bounds__(256, 4) void ffn_backward_kernel(BwArgs a) {
  using namespace bw;
  constexpr bool A_COL = KIND == DWD || KIND == DWGU;  // B is M-contiguous in every kind
  __shared__ __attribute__((aligned(16))) bf16_t As[2][TILE];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2][TILE];

  // ---- the work unit ------------------------------------------------------------------
  int e, mrows, m0 = 0, n0, ktot, row0 = 0, mat = 0;
  if constexpr (KIND == DH || KIND == DX) {
    // (M-tile of an expert's rows, N-tile); XCD-aware order as in the forward
    const int nmt = *a.n_mtiles, U = nmt * a.n_ntiles, per = (U + 7) >> 3;
    const int slot = blockIdx.x >> 3;
    if (slot >= per) return;
    const int u = (blockIdx.x & 7) * per + slot;
    if (u >= U) return;
    const MTile tb = a.mtiles[u / a.n_ntiles];
    const int mt = (a.offsets[tb.expert + 1] - a.offsets[tb.expert] + BM - 1) / BM;
    const int ul = u - tb.first_tile * a.n_ntiles;
    const int nt = ul / mt;
    const MTile t = a.mtiles[tb.first_tile + (ul - nt * mt)];
    e = t.expert;
    row0 = t.row0;
    mrows = t.rows;
    n0 = nt * BN;
    ktot = KIND == DX ? 2 * a.I : a.d;
  } else {
    // (expert, matrix, M-tile, N-tile), expert-major; K = the expert's rows
    const int U = a.n_units, per = (U + 7) >> 3;
    const int slot = blockIdx.x >> 3;
    if (slot >= per) return;
    const int u = (blockIdx.x & 7) * per + slot;
    if (u >= U) return;
    const int per_mat = a.n_mt * a.n_ntiles;
    const int per_exp = per_mat * (KIND == DWGU ? 2 : 1);
    e = u / per_exp;
    int ul = u - e * per_exp;
    mat = ul / per_mat;
    ul -= mat * per_mat;
    m0 = (ul / a.n_ntiles) * BM;
    n0 = (ul % a.n_ntiles) * BN;
    row0 = a.offsets[e];
    ktot = a.offsets[e + 1] - row0;
    mrows = (KIND == DWD ? a.d : a.I) - m0;
  }
  const int ncols = KIND == DH ? a.I : KIND == DX ? a.d : KIND == DWD ? a.I : a.d;
  const int tid = threadIdx.x;

  // ---- load assignment ----------------------------------------------------------------
  // row tile: chunk q = tid + 256 i (i < 2): row q / 4, k offset (q % 4) * 8
  // col tile: chunk q: line k = q / 16, m offset (q % 16) * 8
  const bf16_t* arow[2] = {nullptr, nullptr};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = tid + 256 * i;
    if constexpr (!A_COL) {
      const int r = q >> 2;
      if (r < mrows) {
        const size_t grow = size_t(row0 + r);
        if (KIND == DH) arow[i] = a.dy + size_t(a.perm_token[grow]) * a.d;
        else arow[i] = a.dg + grow * a.I;  // DX: dG for k < I, dU after (switched below)
      }
    }
  }
  uint4 ra[2], rb[2];
  auto line_ptr = [&](int which, int k) -> const bf16_t* {
    // which 0: A, 1: B; the start of line k (k < ktot) of a col operand, at column m0 / n0
    if constexpr (KIND == DH) {  // B: W_down[e] as [K = d][N = I]
      return a.wd + (size_t(e) * a.d + k) * a.I + n0;
    } else if constexpr (KIND == DX) {  // B: W_gate[e] then W_up[e] as [K = I][N = d]
      const bf16_t* w = k < a.I ? a.wg : a.wu;
      const int kk = k < a.I ? k : k - a.I;
      return w + (size_t(e) * a.I + kk) * a.d + n0;
    } else if constexpr (KIND == DWD) {
      if (which == 0) return a.dy + size_t(a.perm_token[row0 + k]) * a.d + m0;  // (m = j, k = r)
      return a.gh + size_t(row0 + k) * a.I + n0;                                 // (n = i, k = r)
    } else {  // DWGU
      if (which == 0) return (mat == 0 ? a.dg : a.du) + size_t(row0 + k) * a.I + m0;  // (m = i, k = r)
      return a.x + size_t(a.perm_token[row0 + k]) * a.d + n0;                         // (n = j, k = r)
    }
  };
  const int mlim = KIND == DWD || KIND == DWGU ? mrows : 0;  // col A: valid m < mlim
  const int nlim = ncols - n0;                                // col B: valid n < nlim
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = tid + 256 * i;
      // A
      if constexpr (!A_COL) {
        const int kc = (q & 3) * 8;
        const bf16_t* p = arow[i];
        if (KIND == DX && p && k0 >= a.I) p = a.du + (p - a.dg) - a.I;  // dU row, same offset
        ra[i] = p ? *reinterpret_cast<const uint4*>(p + k0 + kc) : make_uint4(0, 0, 0, 0);
      } else {
        const int k = k0 + (q >> 4), mc = (q & 15) * 8;
        ra[i] = (k < ktot && mc < mlim) ? *reinterpret_cast<const uint4*>(line_ptr(0, k) + mc)
                                        : make_uint4(0, 0, 0, 0);
      }
      // B
      {
        const int k = k0 + (q >> 4), nc = (q & 15) * 8;
        rb[i] = (k < ktot && nc < nlim) ? *reinterpret_cast<const uint4*>(line_ptr(1, k) + nc)
                                        : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = tid + 256 * i;
      if constexpr (!A_COL) *reinterpret_cast<uint4*>(&As[buf][(q >> 2) * LDR + (q & 3) * 8]) = ra[i];
      else *reinterpret_cast<uint4*>(&As[buf][(q >> 4) * LDC + (q & 15) * 8]) = ra[i];
      *reinterpret_cast<uint4*>(&Bs[buf][(q >> 4) * LDC + (q & 15) * 8]) = rb[i];
    }
  };

  // ---- MFMA -----------------------------------------------------------------------------
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lk = (lane >> 5) * 8;
  // tile rows of the wave's two A blocks and two B blocks
  const int am[2] = {wm * 64, wm * 64 + 32};
  const int bn[2] = {wn * 64, wn * 64 + 32};
  // fragment of one 32-row block at k offset kk: 8 consecutive k of row (base + lane % 32).
  // A col tile holds [k][m]; gfx950's transposing LDS read (ds_read_b64_tr_b16) gives lane
  // 16g + 4a + b element b of the 8 bytes addressed by lanes 16g + 4j + a, j = 0..3, as its
  // element j.  So lane 16g + 4j + a points at k row kk + 8 (g / 2) + 4 h + j, m column
  // base + 16 (g % 2) + 4 a: two reads (h = 0, 1) give the lane's 8 k values of row
  // base + lane % 32.
  const int tr_k = 8 * (lane >> 5) + ((lane >> 2) & 3), tr_m = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  auto frag = [&](const bf16_t* tile, bool colform, int base, int kk) -> bf16x8 {
    if (!colform) return *reinterpret_cast<const bf16x8*>(tile + (base + lr) * LDR + kk + lk);
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const bf16_t* p = tile + (kk + tr_k) * LDC + base + tr_m;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * LDC));
    return __builtin_bit_cast(bf16x8, (short __attribute__((ext_vector_type(8)))){lo[0], lo[1], lo[2], lo[3],
                                                                                hi[0], hi[1], hi[2], hi[3]});
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = (ktot + BK - 1) / BK;
  if (nk > 0) {
    load(0);
    store(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < nk) load((kt + 1) * BK);
#pragma unroll
      for (int ks = 0; ks < BK; ks += 16) {
        bf16x8 fa[2], fb[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) fa[i] = frag(As[buf], A_COL, am[i], ks);
#pragma unroll
        for (int j = 0; j < 2; ++j) fb[j] = frag(Bs[buf], true, bn[j], ks);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
      }
      if (kt + 1 < nk) store(buf ^ 1);
      __syncthreads();
    }
  }

  // ---- epilogue; 32x32 D layout: column lane % 32, rows 8 (r / 4) + 4 (lane / 32) + r % 4 --
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = am[i] + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (m >= mrows) continue;
      {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = n0 + bn[j] + lr;
          if (col >= ncols) continue;
          const float v = acc[i][j][r];
          if constexpr (KIND == DH) {
            a.dh[size_t(row0 + m) * a.I + col] = v * a.g_row[row0 + m];
          } else if constexpr (KIND == DX) {
            a.dxp[size_t(row0 + m) * a.d + col] = f2bf(v);
          } else if constexpr (KIND == DWD) {
            a.dwd[(size_t(e) * a.d + m0 + m) * a.I + col] = f2bf(v);
          } else {
            bf16_t* dw = mat == 0 ? a.dwg : a.dwu;
            dw[(size_t(e) * a.I + m0 + m) * a.d + col] = f2bf(v);
          }
        }
      }
    }
  }
}

// gate of each FFN row: g_row[slot_row[t][k]] = gate[t][k]
__global__ __launch_bounds__(256) void row_gates_kernel(const int32_t* __restrict__ slot_row,
                                                        const float* __restrict__ gate,
                                                        float* __restrict__ g_row, size_t tk) {
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
  a.mtiles = reinterpret_cast<const MTile*>(w + p.mtiles);
  a.n_mtiles = reinterpret_cast<const int32_t*>(w + p.n_mtiles);
  a.dh = reinterpret_cast<float*>(w + p.dh);
  a.gh = reinterpret_cast<bf16_t*>(w + p.gh);
  a.dg = reinterpret_cast<bf16_t*>(w + p.dg);
  a.du = reinterpret_cast<bf16_t*>(w + p.du);
  a.dxp = reinterpret_cast<bf16_t*>(w + p.dxp);
  a.dwg = static_cast<bf16_t*>(dw_gate);
  a.dwu = static_cast<bf16_t*>(dw_up);
  a.dwd = static_cast<bf16_t*>(dw_down);

  const size_t tk = size_t(s.T) * s.K;
  hipLaunchKernelGGL(row_gates_kernel, dim3(unsigned(tk / 256 + 1 < 4096 ? tk / 256 + 1 : 4096)), dim3(256), 0,
                     st, reinterpret_cast<const int32_t*>(w + p.slot_row), gate, reinterpret_cast<float*>(w + p.g_row),
                     tk);
  auto grid_of = [](size_t units) { return dim3(unsigned((units + 7) / 8 * 8)); };
  // activation kinds: units over the M-tile list
  a.n_ntiles = (s.I + BN - 1) / BN;
  hipLaunchKernelGGL(ffn_backward_kernel<DH>, grid_of(size_t(p.mt_max) * a.n_ntiles), dim3(256), 0, st, a);
  // G and U recomputed on the forward's pipelined gate/up kernel (its own M-tile height)
  MTile* pipe_mtiles = reinterpret_cast<MTile*>(w + p.pipe_mtiles);
  int32_t* pipe_n = reinterpret_cast<int32_t*>(w + p.pipe_n_mtiles);
  hipError_t err = launch_mtile_list(s, a.offsets, p.pipe_bm, pipe_mtiles, pipe_n, st);
  if (err != hipSuccess) return err;
  err = launch_ffn_gate_up_grad(s, x, a.perm_token, w_gate, w_up, GuGrad{a.dh, a.g_row, a.dg, a.du}, a.gh,
                                pipe_mtiles, a.offsets, pipe_n, p.pipe_mt_max, st);
  if (err != hipSuccess) return err;
  a.n_ntiles = (s.d + BN - 1) / BN;
  hipLaunchKernelGGL(ffn_backward_kernel<DX>, grid_of(size_t(p.mt_max) * a.n_ntiles), dim3(256), 0, st, a);
  // weight kinds: every expert (an expert without rows gets zero gradients)
  a.n_mt = (s.d + BM - 1) / BM;
  a.n_ntiles = (s.I + BN - 1) / BN;
  a.n_units = s.N * a.n_mt * a.n_ntiles;
  hipLaunchKernelGGL(ffn_backward_kernel<DWD>, grid_of(size_t(a.n_units)), dim3(256), 0, st, a);
  a.n_mt = (s.I + BM - 1) / BM;
  a.n_ntiles = (s.d + BN - 1) / BN;
  a.n_units = s.N * 2 * a.n_mt * a.n_ntiles;
  hipLaunchKernelGGL(ffn_backward_kernel<DWGU>, grid_of(size_t(a.n_units)), dim3(256), 0, st, a);
  hipLaunchKernelGGL(dx_combine_kernel, dim3(s.T), dim3(256), 0, st, a.dxp, a.dy,
                     reinterpret_cast<const int32_t*>(w + p.slot_row), gate, static_cast<bf16_t*>(dx), s.d, s.K);
  return hipGetLastError();
}

}  // namespace lcm

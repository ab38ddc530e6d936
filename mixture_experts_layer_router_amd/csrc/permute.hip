// Expert load histogram, prefix scan and stable scatter of the FFN picks into
// expert-contiguous rows.  Zero-computation picks (index >= N) are counted in the load
// but get no row: they need no compute (LongCat-Flash article, itouyu.top, section
// "Zero-computation experts"); the load histogram is the "recent expert usage" signal
// the bias adjustment of that section consumes.
//
// Order: rows of expert e are ffn_offsets[e] .. ffn_offsets[e+1]-1 in (token, pick)
// order.  Tokens are cut into blocks of 256; a block's rank of token t for expert e is
//   (picks of e in earlier blocks) + (picks of e by earlier waves of the block)
//   + popcount(64-lane mask of e in t's wave, lanes below t),
// all integer, so the result is independent of thread timing.  The masks hold one bit per
// token, which ranks correctly only while a token picks an expert at most once (as the
// router's top-K always does).  A caller's topk_idx may repeat an expert within a token:
// the mask's atomicOr then returns the bit already set, and the block ranks its picks one
// by one in (token, pick) order instead, so every pick still gets its own row.
#include "common.h"
#include "topk.h"

namespace lcm {

__global__ __launch_bounds__(256) void histogram_kernel(const int32_t* __restrict__ idx,
                                                        int32_t* __restrict__ block_counts,
                                                        int32_t* __restrict__ ffn_cnt, int T,
                                                        int K, int E, int N) {
  __shared__ int cnt[kMaxE];
  const int tid = threadIdx.x, b = blockIdx.x;
  for (int e = tid; e < E; e += 256) cnt[e] = 0;
  __syncthreads();
  const int t = b * kTokBlock + tid;
  if (t < T) {
    int f = 0;
    for (int k = 0; k < K; ++k) {
      const int e = idx[size_t(t) * K + k];
      if (static_cast<unsigned>(e) < static_cast<unsigned>(E)) {
        atomicAdd(&cnt[e], 1);  // integer: exact whatever the order
        f += e < N;
      }
    }
    if (ffn_cnt) ffn_cnt[t] = f;
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256) block_counts[size_t(b) * E + e] = cnt[e];
}

// One workgroup of 1024 threads.
__global__ __launch_bounds__(1024) void scan_kernel(const int32_t* __restrict__ block_counts,
                                                    int nblocks, int E, int N,
                                                    int32_t* __restrict__ load,
                                                    int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ block_base,
                                                    MTile* __restrict__ mtiles,
                                                    int32_t* __restrict__ n_mtiles, int bm) {
  __shared__ int tot[kMaxN];
  __shared__ int part[1024], part2[1024];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 1024) {
    int s = 0;
    for (int b = 0; b < nblocks; ++b) s += block_counts[size_t(b) * E + e];
    load[e] = s;
    if (e < N) tot[e] = s;
  }
  __syncthreads();
  // exclusive scans over the N FFN experts of rows and of M-tiles: thread tid owns the
  // consecutive experts [tid*per, tid*per + per)
  const int per = (N + 1023) / 1024;
  int rs = 0, ms = 0;
  for (int i = 0; i < per; ++i) {
    const int e = tid * per + i;
    if (e < N) {
      rs += tot[e];
      ms += (tot[e] + bm - 1) / bm;
    }
  }
  part[tid] = rs;
  part2[tid] = ms;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {  // Hillis-Steele inclusive scan
    const int a = tid >= o ? part[tid - o] : 0;
    const int c = tid >= o ? part2[tid - o] : 0;
    __syncthreads();
    part[tid] += a;
    part2[tid] += c;
    __syncthreads();
  }
  int r = tid > 0 ? part[tid - 1] : 0;
  int m = tid > 0 ? part2[tid - 1] : 0;
  for (int i = 0; i < per; ++i) {
    const int e = tid * per + i;
    if (e < N) {
      offsets[e] = r;
      const int rows = tot[e];
      const int nt = (rows + bm - 1) / bm;
      for (int j = 0; j < nt; ++j) {
        MTile mt;
        mt.expert = e;
        mt.row0 = r + j * bm;
        mt.rows = min(bm, rows - j * bm);
        mt.first_tile = m;
        mtiles[m + j] = mt;
      }
      r += rows;
      m += nt;
    }
  }
  if (tid == 1023) {
    offsets[N] = part[1023];
    *n_mtiles = part2[1023];
  }
  __syncthreads();
  // per-(block, expert) first row
  for (int e = tid; e < N; e += 1024) {
    int run = offsets[e];
    for (int b = 0; b < nblocks; ++b) {
      block_base[size_t(b) * N + e] = run;
      run += block_counts[size_t(b) * E + e];
    }
  }
}

// Ranks the FFN picks of tokens t0..t1-1 one by one in (token, pick) order, run[e] holding
// the next row of expert e; one thread, for token blocks with repeated picks.
__device__ void scatter_serial(const int32_t* __restrict__ idx, int t0, int t1, int K, int N,
                               int* run, int32_t* __restrict__ slot_row,
                               int32_t* __restrict__ perm_token) {
  for (int t = t0; t < t1; ++t)
    for (int k = 0; k < K; ++k) {
      const int e = idx[size_t(t) * K + k];
      int row = -1;
      if (static_cast<unsigned>(e) < static_cast<unsigned>(N)) {
        row = run[e]++;
        perm_token[row] = t;
      }
      slot_row[size_t(t) * K + k] = row;
    }
}

// 256 threads = 4 waves; wave w owns tokens b*256 + w*64 + lane.  Dynamic LDS: 4*N masks.
__global__ __launch_bounds__(256) void scatter_kernel(const int32_t* __restrict__ idx,
                                                      const int32_t* __restrict__ block_base,
                                                      int32_t* __restrict__ slot_row,
                                                      int32_t* __restrict__ perm_token, int T,
                                                      int K, int N) {
  extern __shared__ unsigned long long masks[];  // [4][N]; reused as int run[N]
  __shared__ int repeated;                       // a token of the block picks an expert twice
  const int tid = threadIdx.x, b = blockIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  for (int i = tid; i < 4 * N; i += 256) masks[i] = 0ull;
  if (tid == 0) repeated = 0;
  __syncthreads();
  const int t = b * kTokBlock + tid;
  if (t < T) {
    for (int k = 0; k < K; ++k) {
      const int e = idx[size_t(t) * K + k];
      if (static_cast<unsigned>(e) < static_cast<unsigned>(N)) {
        const unsigned long long bit = 1ull << lane;
        if (atomicOr(&masks[w * N + e], bit) & bit) repeated = 1;
      }
    }
  }
  __syncthreads();
  if (repeated) {  // uniform over the block
    int* run = reinterpret_cast<int*>(masks);
    for (int e = tid; e < N; e += 256) run[e] = block_base[size_t(b) * N + e];
    __syncthreads();
    if (tid == 0) scatter_serial(idx, b * kTokBlock, min(T, (b + 1) * kTokBlock), K, N, run, slot_row, perm_token);
    return;
  }
  if (t < T) {
    const unsigned long long below_lane = (1ull << lane) - 1ull;
    for (int k = 0; k < K; ++k) {
      const int e = idx[size_t(t) * K + k];
      int row = -1;
      if (static_cast<unsigned>(e) < static_cast<unsigned>(N)) {
        int rank = __popcll(masks[w * N + e] & below_lane);
        for (int ww = 0; ww < w; ++ww) rank += __popcll(masks[ww * N + e]);
        row = block_base[size_t(b) * N + e] + rank;
        perm_token[row] = t;
      }
      slot_row[size_t(t) * K + k] = row;
    }
  }
}

// Layers of one token block (T <= 256, decode): histogram, scan and scatter in one
// workgroup, with the counts, the wave masks and the offsets in LDS; the three kernels
// above are each a few microseconds of mostly launch and latency at this size.  The same
// integer rules, so the same results: token t is thread t (wave t / 64, lane t % 64), its
// rank for expert e is popcount(mask of e in its wave, lanes below) plus the picks of e by
// earlier waves, and its row is offsets[e] + rank.  NT threads (NT >= 256: waves 0..3 hold
// the tokens).
struct BlockLds {
  int cnt[kMaxE];
  unsigned long long masks[4 * kMaxN];  // [wave][expert]
  int off[kMaxN];
  int part[1024], part2[1024];
  int repeated;  // a token picks an expert twice: rank one by one (as scatter_kernel)
  int last;      // fused kernel: this workgroup finished last
};

template <int NT>
__device__ void permute_block(BlockLds& L, const int32_t* __restrict__ idx, int T, int K, int E,
                              int N, int bm, int32_t* __restrict__ load, int32_t* __restrict__ ffn_cnt,
                              int32_t* __restrict__ offsets, MTile* __restrict__ mtiles,
                              int32_t* __restrict__ n_mtiles, int32_t* __restrict__ slot_row,
                              int32_t* __restrict__ perm_token) {
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  for (int e = tid; e < E; e += NT) L.cnt[e] = 0;
  for (int i = tid; i < 4 * N; i += NT) L.masks[i] = 0ull;
  if (tid == 0) L.repeated = 0;
  __syncthreads();
  const int t = tid;  // T <= 256: tokens on waves 0..3
  if (t < T) {
    int f = 0;
    for (int k = 0; k < K; ++k) {
      const int e = idx[size_t(t) * K + k];
      if (static_cast<unsigned>(e) < static_cast<unsigned>(E)) {
        atomicAdd(&L.cnt[e], 1);  // integer: exact whatever the order
        if (e < N) {
          ++f;
          const unsigned long long bit = 1ull << lane;
          if (atomicOr(&L.masks[w * N + e], bit) & bit) L.repeated = 1;
        }
      }
    }
    if (ffn_cnt) ffn_cnt[t] = f;
  }
  __syncthreads();
  for (int e = tid; e < E; e += NT) load[e] = L.cnt[e];
  // exclusive scans over the N FFN experts of rows and of M-tiles (as in scan_kernel)
  const int per = (N + NT - 1) / NT;
  int rs = 0, ms = 0;
  for (int i = 0; i < per; ++i) {
    const int e = tid * per + i;
    if (e < N) {
      rs += L.cnt[e];
      ms += (L.cnt[e] + bm - 1) / bm;
    }
  }
  L.part[tid] = rs;
  L.part2[tid] = ms;
  __syncthreads();
  for (int o = 1; o < NT; o <<= 1) {  // Hillis-Steele inclusive scan
    const int a = tid >= o ? L.part[tid - o] : 0;
    const int c = tid >= o ? L.part2[tid - o] : 0;
    __syncthreads();
    L.part[tid] += a;
    L.part2[tid] += c;
    __syncthreads();
  }
  int r = tid > 0 ? L.part[tid - 1] : 0;
  int m = tid > 0 ? L.part2[tid - 1] : 0;
  for (int i = 0; i < per; ++i) {
    const int e = tid * per + i;
    if (e < N) {
      L.off[e] = r;
      offsets[e] = r;
      const int rows = L.cnt[e];
      const int nt = (rows + bm - 1) / bm;
      for (int j = 0; j < nt; ++j) {
        MTile mt;
        mt.expert = e;
        mt.row0 = r + j * bm;
        mt.rows = min(bm, rows - j * bm);
        mt.first_tile = m;
        mtiles[m + j] = mt;
      }
      r += rows;
      m += nt;
    }
  }
  if (tid == NT - 1) {
    offsets[N] = L.part[NT - 1];
    *n_mtiles = L.part2[NT - 1];
  }
  __syncthreads();
  if (L.repeated) {  // uniform over the workgroup
    if (tid == 0) scatter_serial(idx, 0, T, K, N, L.off, slot_row, perm_token);
    return;
  }
  if (t < T) {
    const unsigned long long below_lane = (1ull << lane) - 1ull;
    for (int k = 0; k < K; ++k) {
      const int e = idx[size_t(t) * K + k];
      int row = -1;
      if (static_cast<unsigned>(e) < static_cast<unsigned>(N)) {
        int rank = __popcll(L.masks[w * N + e] & below_lane);
        for (int ww = 0; ww < w; ++ww) rank += __popcll(L.masks[ww * N + e]);
        row = L.off[e] + rank;
        perm_token[row] = t;
      }
      slot_row[size_t(t) * K + k] = row;
    }
  }
}

__global__ __launch_bounds__(1024) void permute_small_kernel(
    const int32_t* __restrict__ idx, int T, int K, int E, int N, int bm,
    int32_t* __restrict__ load, int32_t* __restrict__ ffn_cnt, int32_t* __restrict__ offsets,
    MTile* __restrict__ mtiles, int32_t* __restrict__ n_mtiles, int32_t* __restrict__ slot_row,
    int32_t* __restrict__ perm_token) {
  __shared__ BlockLds L;
  permute_block<1024>(L, idx, T, K, E, N, bm, load, ffn_cnt, offsets, mtiles, n_mtiles, slot_row,
                      perm_token);
}

// Top-K and the one-block permutation in one kernel, for the forward of layers of one token
// block (T <= 256): the top-K runs as in router_topk_kernel, one wavefront per token and
// four tokens per workgroup; then each workgroup counts itself done on a device-scope
// counter, and the workgroup that finishes last runs the permutation above on every
// token's picks.  The counter is zeroed by the router-logits kernel that runs just before
// on the same stream, so no memset is needed (the kernel can be captured into a graph).
// Same picks, gates and permutation as the separate kernels, bit for bit.
template <int EPL>
__global__ __launch_bounds__(256) void topk_permute_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias, int T, int K, int E, int N,
    int bm, int32_t* __restrict__ idx, float* __restrict__ gate, int32_t* __restrict__ done,
    int32_t* __restrict__ load, int32_t* __restrict__ offsets, MTile* __restrict__ mtiles,
    int32_t* __restrict__ n_mtiles, int32_t* __restrict__ slot_row, int32_t* __restrict__ perm_token) {
  __shared__ BlockLds L;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t < T)
    router_topk_token<EPL>(logits + size_t(t) * E, bias, E, K, threadIdx.x & 63, idx + size_t(t) * K,
                           gate + size_t(t) * K);
  __threadfence();  // this workgroup's picks are visible device-wide before it counts itself
  __syncthreads();
  if (threadIdx.x == 0) L.last = atomicAdd(done, 1) == int(gridDim.x) - 1;
  __syncthreads();
  if (!L.last) return;
  __threadfence();  // the other workgroups' picks, published before their increments
  permute_block<256>(L, idx, T, K, E, N, bm, load, nullptr, offsets, mtiles, n_mtiles, slot_row,
                     perm_token);
}

// One workgroup per row; rows from offsets[N] on exit at once.
template <typename V>
__global__ __launch_bounds__(256) void gather_rows_kernel(const V* __restrict__ x,
                                                          const int32_t* __restrict__ perm_token,
                                                          const int32_t* __restrict__ offsets,
                                                          V* __restrict__ x_perm, int vec_per_row,
                                                          int N) {
  const int r = blockIdx.x;
  if (r >= offsets[N]) return;
  const V* src = x + size_t(perm_token[r]) * vec_per_row;
  V* dst = x_perm + size_t(r) * vec_per_row;
  for (int i = threadIdx.x; i < vec_per_row; i += 256) dst[i] = src[i];
}

__global__ void copy_i32_kernel(const int32_t* __restrict__ src, int32_t* __restrict__ dst, size_t n) {
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += size_t(gridDim.x) * blockDim.x)
    dst[i] = src[i];
}
__global__ void copy_f32_kernel(const float* __restrict__ src, float* __restrict__ dst, size_t n) {
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += size_t(gridDim.x) * blockDim.x)
    dst[i] = src[i];
}

hipError_t launch_histogram(const lc_moe_shape& s, const int32_t* idx, int32_t* block_counts,
                            int32_t* ffn_cnt, int nblocks, hipStream_t st) {
  hipLaunchKernelGGL(histogram_kernel, dim3(nblocks), dim3(256), 0, st, idx, block_counts,
                     ffn_cnt, s.T, s.K, s.N + s.Z, s.N);
  return hipGetLastError();
}

hipError_t launch_scan(const lc_moe_shape& s, const int32_t* block_counts, int nblocks,
                       int32_t* load, int32_t* offsets, int32_t* block_base, MTile* mtiles,
                       int32_t* n_mtiles, int bm, hipStream_t st) {
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, st, block_counts, nblocks,
                     s.N + s.Z, s.N, load, offsets, block_base, mtiles, n_mtiles, bm);
  return hipGetLastError();
}

hipError_t launch_permute_small(const lc_moe_shape& s, const int32_t* idx, int32_t* load,
                                int32_t* ffn_cnt, int32_t* offsets, MTile* mtiles,
                                int32_t* n_mtiles, int bm, int32_t* slot_row, int32_t* perm_token,
                                hipStream_t st) {
  hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(1024), 0, st, idx, s.T, s.K, s.N + s.Z, s.N,
                     bm, load, ffn_cnt, offsets, mtiles, n_mtiles, slot_row, perm_token);
  return hipGetLastError();
}

hipError_t launch_topk_permute(const lc_moe_shape& s, const float* logits, const float* bias,
                               int32_t* idx, float* gate, int32_t* done, int32_t* load,
                               int32_t* offsets, MTile* mtiles, int32_t* n_mtiles, int bm,
                               int32_t* slot_row, int32_t* perm_token, hipStream_t st) {
  const int E = s.N + s.Z;
  const int epl = (E + 63) / 64;
  const dim3 grid((s.T + 3) / 4), block(256);
#define LCM_TOPK(n)                                                                        \
  hipLaunchKernelGGL(topk_permute_kernel<n>, grid, block, 0, st, logits, bias, s.T, s.K, E, s.N, \
                     bm, idx, gate, done, load, offsets, mtiles, n_mtiles, slot_row, perm_token)
  if (epl <= 2) LCM_TOPK(2);
  else if (epl <= 4) LCM_TOPK(4);
  else if (epl <= 8) LCM_TOPK(8);
  else if (epl <= 16) LCM_TOPK(16);
  else if (epl <= 32) LCM_TOPK(32);
  else LCM_TOPK(64);
#undef LCM_TOPK
  return hipGetLastError();
}

hipError_t launch_scatter(const lc_moe_shape& s, const int32_t* idx, const int32_t* block_base,
                          int nblocks, int32_t* slot_row, int32_t* perm_token, hipStream_t st) {
  const size_t lds = size_t(4) * s.N * sizeof(unsigned long long);
  hipLaunchKernelGGL(scatter_kernel, dim3(nblocks), dim3(256), lds, st, idx, block_base,
                     slot_row, perm_token, s.T, s.K, s.N);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const lc_moe_shape& s, const void* x, const int32_t* perm_token,
                              const int32_t* offsets, void* x_perm, hipStream_t st) {
  const size_t row_bytes = size_t(s.d) * (s.dtype == LC_MOE_BF16 ? 2 : 4);
  const unsigned grid = static_cast<unsigned>(size_t(s.T) * s.K);
  if (row_bytes % 16 == 0) {
    hipLaunchKernelGGL(gather_rows_kernel<uint4>, dim3(grid), dim3(256), 0, st,
                       static_cast<const uint4*>(x), perm_token, offsets,
                       static_cast<uint4*>(x_perm), int(row_bytes / 16), s.N);
  } else {
    hipLaunchKernelGGL(gather_rows_kernel<uint2>, dim3(grid), dim3(256), 0, st,
                       static_cast<const uint2*>(x), perm_token, offsets,
                       static_cast<uint2*>(x_perm), int(row_bytes / 8), s.N);
  }
  return hipGetLastError();
}

hipError_t launch_copy_i32(const int32_t* src, int32_t* dst, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  unsigned grid = static_cast<unsigned>(n / 256 + 1 < 4096 ? n / 256 + 1 : 4096);
  hipLaunchKernelGGL(copy_i32_kernel, dim3(grid), dim3(256), 0, st, src, dst, n);
  return hipGetLastError();
}

hipError_t launch_copy_f32(const float* src, float* dst, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  unsigned grid = static_cast<unsigned>(n / 256 + 1 < 4096 ? n / 256 + 1 : 4096);
  hipLaunchKernelGGL(copy_f32_kernel, dim3(grid), dim3(256), 0, st, src, dst, n);
  return hipGetLastError();
}

// M-tile list of height bm over the FFN experts' rows given by offsets [N+1]: expert e's
// rows offsets[e] .. offsets[e+1]-1 in tiles of bm rows, experts in order (the list the scan
// kernel builds at that height).  One 1024-thread workgroup; thread tid owns consecutive
// experts, whose tile counts it scans with the others'.
__global__ __launch_bounds__(1024) void mtile_list_kernel(const int32_t* __restrict__ offsets, int N, int bm,
                                                          MTile* __restrict__ mtiles,
                                                          int32_t* __restrict__ n_mtiles) {
  __shared__ int part[1024];
  const int tid = threadIdx.x;
  const int per = (N + 1023) / 1024;
  int ms = 0;
  for (int i = 0; i < per; ++i) {
    const int e = tid * per + i;
    if (e < N) ms += (offsets[e + 1] - offsets[e] + bm - 1) / bm;
  }
  part[tid] = ms;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {  // Hillis-Steele inclusive scan
    const int a = tid >= o ? part[tid - o] : 0;
    __syncthreads();
    part[tid] += a;
    __syncthreads();
  }
  int m = tid > 0 ? part[tid - 1] : 0;
  for (int i = 0; i < per; ++i) {
    const int e = tid * per + i;
    if (e < N) {
      const int r0 = offsets[e], rows = offsets[e + 1] - r0;
      const int nt = (rows + bm - 1) / bm;
      for (int j = 0; j < nt; ++j) {
        MTile mt;
        mt.expert = e;
        mt.row0 = r0 + j * bm;
        mt.rows = min(bm, rows - j * bm);
        mt.first_tile = m;
        mtiles[m + j] = mt;
      }
      m += nt;
    }
  }
  if (tid == 1023) *n_mtiles = part[1023];
}

hipError_t launch_mtile_list(const lc_moe_shape& s, const int32_t* offsets, int bm, MTile* mtiles,
                             int32_t* n_mtiles, hipStream_t st) {
  hipLaunchKernelGGL(mtile_list_kernel, dim3(1), dim3(1024), 0, st, offsets, s.N, bm, mtiles, n_mtiles);
  return hipGetLastError();
}

}  // namespace lcm

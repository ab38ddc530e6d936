// bf16 expert weights re-laid for the pipelined FFN kernel: every (expert, n-tile, K step)
// becomes one contiguous 16 KB block holding exactly the LDS image of that stage's 256
// weight rows (layout in common.h, plan_packed).  The kernel then fills a stage with 16
// one-kilobyte contiguous loads instead of 256 row segments 64 bytes long.  The values are
// copied bit for bit; where the row-major weights run the same pipelined kernel (layers of
// more than 256 tokens) the layer computed on the packed weights is the same, to the bit.
#include "common.h"

namespace lcm {

// One workgroup per 16 KB block (grid: K step, n-tile, expert).  Thread q of the block's
// 1024 16-byte chunks writes chunk q: row q/4, slot q%4, which holds the row's column
// chunk (q%4) ^ swz4(row).  GU: rows 0..127 from w0 (gate), 128..255 from w1 (up), rows
// nt*128 + (r % 128); otherwise rows nt*256 + r of w0 (down).  Rows past `rows` are zero.
template <bool GU>
__global__ __launch_bounds__(256) void pack_kernel(const bf16_t* __restrict__ w0,
                                                   const bf16_t* __restrict__ w1,
                                                   unsigned char* __restrict__ out, int rows,
                                                   int kdim, int n_ntiles) {
  const int kt = blockIdx.x, nt = blockIdx.y, e = blockIdx.z;
  const int nk = kdim / 32;
  uint4* blk = reinterpret_cast<uint4*>(out + ((size_t(e) * n_ntiles + nt) * nk + kt) * 16384);
  for (int q = threadIdx.x; q < 1024; q += 256) {
    const int r = q >> 2, c = (q & 3) ^ swz4(r);
    const int row = GU ? nt * 128 + (r & 127) : nt * 256 + r;
    const bf16_t* m = GU && r >= 128 ? w1 : w0;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row < rows) v = *reinterpret_cast<const uint4*>(m + (size_t(e) * rows + row) * kdim + kt * 32 + c * 8);
    blk[q] = v;
  }
}

hipError_t launch_pack_weights(const lc_moe_shape& s, const void* w_gate, const void* w_up,
                               const void* w_down, void* packed, hipStream_t st) {
  const PackPlan p = plan_packed(s);
  unsigned char* out = static_cast<unsigned char*>(packed);
  const int nt_gu = (s.I + 127) / 128, nt_d = (s.d + 255) / 256;
  hipLaunchKernelGGL(pack_kernel<true>, dim3(unsigned(s.d / 32), unsigned(nt_gu), unsigned(s.N)), dim3(256),
                     0, st, static_cast<const bf16_t*>(w_gate), static_cast<const bf16_t*>(w_up),
                     out + p.gu, s.I, s.d, nt_gu);
  hipLaunchKernelGGL(pack_kernel<false>, dim3(unsigned(s.I / 32), unsigned(nt_d), unsigned(s.N)), dim3(256),
                     0, st, static_cast<const bf16_t*>(w_down), nullptr, out + p.d, s.d, s.I, nt_d);
  return hipGetLastError();
}

}  // namespace lcm

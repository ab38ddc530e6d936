// Cross-lane helpers for the MFMA epilogues.
#pragma once

namespace lcm {

// 4 x 4 transpose among lanes 4q .. 4q+3 of a wave: lane q4 holds column q4 of a block as
// v[0..3] (rows 0..3) and receives row q4 as w[0..3] (columns 0..3).  Its own v[q4] is
// column q4; in round s column q4 ^ s comes from lane q4 ^ s, which sends its v[q4].
__device__ __forceinline__ void quad_transpose(const float (&v)[4], int q4, float (&w)[4]) {
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) {
    float send = v[0];
#pragma unroll
    for (int t4 = 1; t4 < 4; ++t4) send = (q4 ^ s4) == t4 ? v[t4] : send;
    const float got = s4 == 0 ? send : __shfl_xor(send, s4);
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) w[c4] = c4 == (q4 ^ s4) ? got : (s4 == 0 ? 0.f : w[c4]);
  }
}

}  // namespace lcm

// Expert-bias controller: one PID update of the selection bias from the expert loads of
// the last step (LongCat-Flash article, itouyu.top, section "Zero-computation experts",
// bias paragraph: the expert bias follows recent usage and is adjusted in real time by a
// PID controller).  The error is the gap between each expert's target share and its
// share of the T*K picks; every expert is independent, so one thread per expert.
#include "common.h"

namespace lcm {

__global__ __launch_bounds__(256) void bias_update_kernel(int E, float tk, float kp, float ki,
                                                          float kd, const int32_t* __restrict__ load,
                                                          const float* __restrict__ target,
                                                          float* __restrict__ bias,
                                                          float* __restrict__ integral,
                                                          float* __restrict__ prev_err) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= E) return;
  const float e = target[i] - static_cast<float>(load[i]) / tk;
  const float acc = integral[i] + e;
  const float de = e - prev_err[i];
  // kp*e + ki*acc + kd*de, evaluated left to right with separate roundings
  const float step = __fadd_rn(__fadd_rn(__fmul_rn(kp, e), __fmul_rn(ki, acc)), __fmul_rn(kd, de));
  bias[i] = bias[i] + step;
  integral[i] = acc;
  prev_err[i] = e;
}

hipError_t launch_bias_update(int E, long long tk, float kp, float ki, float kd,
                              const int32_t* load, const float* target, float* bias,
                              float* integral, float* prev_err, hipStream_t st) {
  hipLaunchKernelGGL(bias_update_kernel, dim3((E + 255) / 256), dim3(256), 0, st, E,
                     static_cast<float>(tk), kp, ki, kd, load, target, bias, integral, prev_err);
  return hipGetLastError();
}

}  // namespace lcm

// Direct global->LDS loads and the explicit waits around them, shared by the pipelined
// GEMM kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>

namespace lcm {

typedef __attribute__((address_space(3))) void lds_void;

// One wave-wide direct global->LDS load: lane l copies 16 bytes from g to lds + 16*l.
__device__ __forceinline__ void dma16(const void* g, unsigned char* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 16, 0, 0);
}

// The same with the non-temporal hint (cache-policy bit NT): for data read exactly once
// in whole 128-byte lines, such as weights stored in the order a kernel streams them.
// The hint keeps the stream from displacing reused lines; a stream that reads half a line
// per load and the other half a step later (row-major weights, 64-byte segments) must
// not take it, or each line is fetched twice.
__device__ __forceinline__ void dma16_stream(const void* g, unsigned char* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 16, 0, 2);
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
#define LCM_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt((((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14)))

// s_waitcnt vmcnt(n) for a run-time n.  The counter holds at most 63 loads, and a wave
// cannot issue a 64th, so a wait for a load older than 63 later loads is already met.
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n < 63 ? n : 63) {
#define LCM_CASE(k) case k: LCM_WAIT_VMCNT(k); break;
#define LCM_CASE8(k) LCM_CASE(k) LCM_CASE(k + 1) LCM_CASE(k + 2) LCM_CASE(k + 3) \
                     LCM_CASE(k + 4) LCM_CASE(k + 5) LCM_CASE(k + 6) LCM_CASE(k + 7)
    LCM_CASE8(0) LCM_CASE8(8) LCM_CASE8(16) LCM_CASE8(24) LCM_CASE8(32) LCM_CASE8(40)
    LCM_CASE8(48) LCM_CASE(56) LCM_CASE(57) LCM_CASE(58) LCM_CASE(59) LCM_CASE(60)
    LCM_CASE(61) LCM_CASE(62)
#undef LCM_CASE8
#undef LCM_CASE
    default: LCM_WAIT_VMCNT(63); break;
  }
}

// s_waitcnt lgkmcnt(0) alone: this wave's LDS reads have returned.
__device__ __forceinline__ void wait_lds_reads() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup barrier without the vmcnt(0) that __syncthreads implies: the direct loads of
// later stages stay in flight across it.
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace lcm

// Matrix-core throughput probe for gfx950 (MI355X).
//
// Measures what the matrix cores deliver with no memory traffic at all, the
// ceiling that the decode kernel's MFMA work is compared against: every wave
// keeps four independent accumulator chains of 32x32 MFMAs in flight (fp8
// 32x32x64, 131072 FLOP per instruction, or bf16 32x32x16, 32768 FLOP), so
// issue never waits on a dependent result.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace mla {

namespace {

typedef int p_i32x4 __attribute__((ext_vector_type(4)));
typedef int p_i32x8 __attribute__((ext_vector_type(8)));
typedef float p_f32x16 __attribute__((ext_vector_type(16)));

template <bool FP8>
__global__ __launch_bounds__(256) void mfma_peak_kernel(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  p_f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const p_i32x8 a = {lane, lane + 1, lane + 2, lane + 3, lane + 4, lane + 5, lane + 6, lane + 7};
  const p_i32x8 b = {7 - lane, 6, 5, 4, 3, 2, 1, lane};
  asm volatile("s_nop 4" ::: "memory");   // operands were just written by VALU
  for (int it = 0; it < iters; ++it) {
    if constexpr (FP8) {
      asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %4, %5, %0\n\t"
                   "v_mfma_f32_32x32x64_f8f6f4 %1, %4, %5, %1\n\t"
                   "v_mfma_f32_32x32x64_f8f6f4 %2, %4, %5, %2\n\t"
                   "v_mfma_f32_32x32x64_f8f6f4 %3, %4, %5, %3"
                   : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3) : "v"(a), "v"(b));
    } else {
      const p_i32x4 a4 = {a[0], a[1], a[2], a[3]}, b4 = {b[0], b[1], b[2], b[3]};
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %4, %5, %0\n\t"
                   "v_mfma_f32_32x32x16_bf16 %1, %4, %5, %1\n\t"
                   "v_mfma_f32_32x32x16_bf16 %2, %4, %5, %2\n\t"
                   "v_mfma_f32_32x32x16_bf16 %3, %4, %5, %3"
                   : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3) : "v"(a4), "v"(b4));
    }
  }
  // results of the last MFMAs are read by VALU below: cover their latency
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3));
  float acc = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc += c0[r] + c1[r] + c2[r] + c3[r];
  sink[(long)blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace

hipError_t launch_mfma_peak(int dot, int iters, int blocks, float* sink, hipStream_t st) {
  if (dot == 1)   // fp8 (the header's MLA_DOT_FP8)
    hipLaunchKernelGGL(mfma_peak_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, st, iters, sink);
  else
    hipLaunchKernelGGL(mfma_peak_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, st, iters, sink);
  return hipGetLastError();
}

}  // namespace mla

// Quantize-on-write of the paged FP8 latent cache for gfx950 (MI355X).
//
// The step before the decode (InfiniCore PR #1568, Summary, FP8 KV cache
// bullet: the per-tensor scale is amax / 448, 448 being the largest finite
// e4m3fn value): new latent rows (512 bf16 "nope" values and 64 bf16 rope
// values per token) are written into their cache rows, the nope part as OCP
// e4m3fn codes of value / scale (round to nearest even, saturating at +-448),
// the rope part copied unchanged. The cache row is the decode's: 512 code
// bytes, then the 64 rope values (640 bytes; 512 rope-free). A token's row is
// slot_mapping[token] = page * 64 + slot; tokens with a negative or
// out-of-range slot are not written.
//
// Two kernels, both HBM-bound streams:
//  * amax: each workgroup reduces |value| over its share of the written
//    tokens' nope values and stores one partial (no atomics);
//  * encode: every workgroup reduces the partials (at most kAmaxGroups
//    floats), so all of them derive the same scale; workgroup 0 stores it to
//    k_scale and v_scale. With a given scale the amax kernel is skipped and
//    the scale is read from k_scale. Each thread then turns 16 input values
//    into one 16-byte store of the cache row (40 stores per 640-byte row, so
//    a wave's stores cover whole rows contiguously).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace mla {

namespace {

typedef int q_i32x4 __attribute__((ext_vector_type(4)));

constexpr int kAmaxGroups = 1024;   // partials in the workspace (<= 1024 floats)
constexpr int kQThreads = 256;
constexpr float kE4m3Max = 448.f;

__device__ inline float bf16_lo_f(unsigned w) { return __builtin_bit_cast(float, w << 16); }
__device__ inline float bf16_hi_f(unsigned w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

__device__ inline bool slot_ok(int slot, long rows) { return slot >= 0 && (long)slot < rows; }

// Max of x over the workgroup (256 threads = 4 waves); valid in thread 0.
__device__ inline float block_max(float x, float* red) {
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) x = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  return x;
}

// Partial amax of workgroup blockIdx.x: 16-byte chunks (8 bf16) of the nope
// values of written tokens, grid-strided, four chunks per thread in flight.
// The value and slot loads do not depend on each other (a chunk past the end
// re-reads the last one and is masked), so both go out together.
__global__ __launch_bounds__(kQThreads) void kv_amax_kernel(const uint16_t* __restrict__ ckv,
                                                            const int32_t* __restrict__ slots,
                                                            int num_tokens, long cache_rows,
                                                            float* __restrict__ partials) {
  __shared__ float red[4];
  const long chunks = (long)num_tokens * 64;   // 512 values = 64 chunks per token
  const long stride = (long)gridDim.x * kQThreads;
  float m = 0.f;
  for (long c0 = (long)blockIdx.x * kQThreads + threadIdx.x; c0 < chunks; c0 += 4 * stride) {
    q_i32x4 v[4];
    int sl[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const long c = c0 + u * stride < chunks ? c0 + u * stride : chunks - 1;
      v[u] = *reinterpret_cast<const q_i32x4*>(ckv + c * 8);
      sl[u] = c0 + u * stride < chunks ? slots[c >> 6] : -1;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float mu = 0.f;
#pragma unroll
      for (int d = 0; d < 4; ++d)
        mu = fmaxf(mu, fmaxf(fabsf(bf16_lo_f((unsigned)v[u][d])), fabsf(bf16_hi_f((unsigned)v[u][d]))));
      m = slot_ok(sl[u], cache_rows) ? fmaxf(m, mu) : m;
    }
  }
  m = block_max(m, red);
  if (threadIdx.x == 0) partials[blockIdx.x] = m;
}

// 4 floats -> 4 e4m3fn bytes, round to nearest even (hardware conversion;
// the inputs are already within +-448).
__device__ inline int enc4(float a, float b, float c, float d) {
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
}

__device__ inline float qv(float x, float scale) {
  const float y = __fdiv_rn(x, scale);   // correctly rounded f32 division
  return fminf(fmaxf(y, -kE4m3Max), kE4m3Max);
}

template <int ROPE>
__global__ __launch_bounds__(kQThreads) void kv_encode_kernel(const uint16_t* __restrict__ ckv,
                                                              const uint16_t* __restrict__ rope,
                                                              const int32_t* __restrict__ slots,
                                                              int num_tokens, long cache_rows,
                                                              uint8_t* __restrict__ kv,
                                                              float* __restrict__ k_scale,
                                                              float* __restrict__ v_scale,
                                                              const float* __restrict__ partials,
                                                              int num_partials) {
  constexpr int RB = 512 + 2 * ROPE;          // cache row bytes
  constexpr int CPR = RB / 16;                // 16-byte stores per row
  __shared__ float red[4];
  __shared__ float s_scale;
  if (partials != nullptr) {
    float m = 0.f;
    for (int i = threadIdx.x; i < num_partials; i += kQThreads) m = fmaxf(m, partials[i]);
    m = block_max(m, red);
    if (threadIdx.x == 0) {
      const float sc = m > 0.f ? __fdiv_rn(m, kE4m3Max) : 1.f;
      s_scale = sc;
      if (blockIdx.x == 0) {
        *k_scale = sc;
        *v_scale = sc;
      }
    }
  } else if (threadIdx.x == 0) {
    s_scale = *k_scale;
  }
  __syncthreads();
  const float scale = s_scale;

  const long chunks = (long)num_tokens * CPR;
  for (long c = (long)blockIdx.x * kQThreads + threadIdx.x; c < chunks; c += (long)gridDim.x * kQThreads) {
    const long tok = c / CPR;
    const int part = (int)(c - tok * CPR);
    // the slot is only needed for the store: the value loads below do not
    // wait for it
    const int slot = slots[tok];
    q_i32x4 o;
    if (part < 32) {
      // nope values 16 part .. +15 -> 16 code bytes
      const q_i32x4* src = reinterpret_cast<const q_i32x4*>(ckv + tok * 512 + 16 * part);
      const q_i32x4 a = src[0], b = src[1];
      const unsigned w[8] = {(unsigned)a[0], (unsigned)a[1], (unsigned)a[2], (unsigned)a[3],
                             (unsigned)b[0], (unsigned)b[1], (unsigned)b[2], (unsigned)b[3]};
#pragma unroll
      for (int k = 0; k < 4; ++k)
        o[k] = enc4(qv(bf16_lo_f(w[2 * k]), scale), qv(bf16_hi_f(w[2 * k]), scale),
                    qv(bf16_lo_f(w[2 * k + 1]), scale), qv(bf16_hi_f(w[2 * k + 1]), scale));
    } else {
      // rope values 8 (part - 32) .. +7, copied
      o = *reinterpret_cast<const q_i32x4*>(rope + tok * ROPE + 8 * (part - 32));
    }
    if (slot_ok(slot, cache_rows)) *reinterpret_cast<q_i32x4*>(kv + (long)slot * RB + 16 * part) = o;
  }
}

// Per-token scales: one wave per token. Lane l holds nope values 8l .. 8l+7;
// the row's amax is a wave reduction, its scale amax / 448 (1 if 0) is stored
// at the row's slot in k_scale and v_scale, and lanes 0-7 copy the rope.
template <int ROPE>
__global__ __launch_bounds__(kQThreads) void kv_encode_per_token_kernel(const uint16_t* __restrict__ ckv,
                                                                        const uint16_t* __restrict__ rope,
                                                                        const int32_t* __restrict__ slots,
                                                                        int num_tokens, long cache_rows,
                                                                        uint8_t* __restrict__ kv,
                                                                        float* __restrict__ k_scale,
                                                                        float* __restrict__ v_scale) {
  constexpr int RB = 512 + 2 * ROPE;
  const int lane = threadIdx.x & 63;
  const long tok = (long)blockIdx.x * (kQThreads / 64) + (threadIdx.x >> 6);
  if (tok >= num_tokens) return;
  const int slot = slots[tok];
  if (!slot_ok(slot, cache_rows)) return;   // wave-uniform
  const q_i32x4 v = *reinterpret_cast<const q_i32x4*>(ckv + tok * 512 + 8 * lane);
  float m = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d) m = fmaxf(m, fmaxf(fabsf(bf16_lo_f((unsigned)v[d])), fabsf(bf16_hi_f((unsigned)v[d]))));
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  const float scale = m > 0.f ? __fdiv_rn(m, kE4m3Max) : 1.f;
  const int c0 = enc4(qv(bf16_lo_f((unsigned)v[0]), scale), qv(bf16_hi_f((unsigned)v[0]), scale),
                      qv(bf16_lo_f((unsigned)v[1]), scale), qv(bf16_hi_f((unsigned)v[1]), scale));
  const int c1 = enc4(qv(bf16_lo_f((unsigned)v[2]), scale), qv(bf16_hi_f((unsigned)v[2]), scale),
                      qv(bf16_lo_f((unsigned)v[3]), scale), qv(bf16_hi_f((unsigned)v[3]), scale));
  uint8_t* row = kv + (long)slot * RB;
  *reinterpret_cast<uint2*>(row + 8 * lane) = uint2{(unsigned)c0, (unsigned)c1};
  if constexpr (ROPE > 0) {
    if (lane < 8) *reinterpret_cast<q_i32x4*>(row + 512 + 16 * lane) =
        *reinterpret_cast<const q_i32x4*>(rope + tok * ROPE + 8 * lane);
  }
  if (lane == 0) {
    k_scale[slot] = scale;
    v_scale[slot] = scale;
  }
}

int grid_for(long work, int cap) {
  long g = (work + kQThreads - 1) / kQThreads;
  if (g < 1) g = 1;
  return (int)(g < cap ? g : cap);
}

}  // namespace

size_t quantize_workspace_bytes() { return kAmaxGroups * sizeof(float); }

hipError_t launch_quantize_kv(const QuantizeLaunch& d, hipStream_t st) {
  const long rows = (long)d.num_pages * 64;
  if (d.per_token) {
    const dim3 grid((unsigned)((d.num_tokens + kQThreads / 64 - 1) / (kQThreads / 64)));
    if (d.d_rope == 64)
      hipLaunchKernelGGL((kv_encode_per_token_kernel<64>), grid, dim3(kQThreads), 0, st, d.ckv, d.rope, d.slots,
                         d.num_tokens, rows, d.kv, d.k_scale, d.v_scale);
    else
      hipLaunchKernelGGL((kv_encode_per_token_kernel<0>), grid, dim3(kQThreads), 0, st, d.ckv, d.rope, d.slots,
                         d.num_tokens, rows, d.kv, d.k_scale, d.v_scale);
    return hipGetLastError();
  }
  float* partials = nullptr;
  int np = 0;
  if (d.compute_scale) {
    partials = d.workspace;
    np = grid_for((long)d.num_tokens * 64, kAmaxGroups);
    hipLaunchKernelGGL(kv_amax_kernel, dim3((unsigned)np), dim3(kQThreads), 0, st, d.ckv, d.slots, d.num_tokens,
                       rows, partials);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const long work = (long)d.num_tokens * ((512 + 2 * d.d_rope) / 16);
  const int g = grid_for(work, 4096);
  if (d.d_rope == 64)
    hipLaunchKernelGGL((kv_encode_kernel<64>), dim3((unsigned)g), dim3(kQThreads), 0, st, d.ckv, d.rope, d.slots,
                       d.num_tokens, rows, d.kv, d.k_scale, d.v_scale, partials, np);
  else
    hipLaunchKernelGGL((kv_encode_kernel<0>), dim3((unsigned)g), dim3(kQThreads), 0, st, d.ckv, d.rope, d.slots,
                       d.num_tokens, rows, d.kv, d.k_scale, d.v_scale, partials, np);
  return hipGetLastError();
}

}  // namespace mla

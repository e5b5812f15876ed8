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

// Partial amax of workgroup blockIdx.x. A token's 512 nope values are one
// wave-wide 16-byte load (lane l: values 8 l .. 8 l + 7); each wave takes
// tokens grid-strided, eight in flight. The eight slots come first, as one
// load (lane l reads the slot of token l % 8), and are read out lane by lane
// once the value loads are in flight.
__global__ __launch_bounds__(kQThreads) void kv_amax_kernel(const uint16_t* __restrict__ ckv,
                                                            const int32_t* __restrict__ slots,
                                                            int num_tokens, long cache_rows,
                                                            float* __restrict__ partials) {
  constexpr int kInFlight = 8;
  __shared__ float red[4];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int waves = gridDim.x * (kQThreads / 64);
  float m = 0.f;
  for (int t0 = blockIdx.x * (kQThreads / 64) + wave; t0 < num_tokens; t0 += kInFlight * waves) {
    const int tl = t0 + (lane % kInFlight) * waves;
    const int sl = slots[tl < num_tokens ? tl : num_tokens - 1];
    q_i32x4 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      const int t = t0 + u * waves;
      const int tc = t < num_tokens ? t : num_tokens - 1;   // past the end: re-read, masked
      v[u] = reinterpret_cast<const q_i32x4*>(ckv + (long)tc * 512)[lane];   // cached: see the encode order
    }
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      float mu = 0.f;
#pragma unroll
      for (int d = 0; d < 4; ++d)
        mu = fmaxf(mu, fmaxf(fabsf(bf16_lo_f((unsigned)v[u][d])), fabsf(bf16_hi_f((unsigned)v[u][d]))));
      const bool ok = t0 + u * waves < num_tokens && slot_ok(__builtin_amdgcn_readlane(sl, u), cache_rows);
      m = ok ? fmaxf(m, mu) : m;
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

// The same code through the reciprocal: y = RN(1 / scale) (correctly
// rounded, computed once), q0 = RN(x y) within an ulp or two of x / scale,
// then two residual corrections q <- RN(q + (x - q scale) y) with the
// residual exact under an fma. By Markstein's theorem (the correction of a
// quotient within an ulp by the correctly rounded reciprocal gives the
// correctly rounded quotient) the second step yields RN(x / scale), the
// division above, for scales in [2^-100, 2^100] (no overflow of y, no
// underflow of a residual that decides a code). The sign is taken from x (the
// quotient's, a -0 input stays -0); a quotient past +-448, inf or NaN comes
// from q0 and saturates as above.
__device__ inline float qv_rcp(float x, float scale, float y) {
  const float q0 = x * y;
  const float q1 = fmaf(fmaf(-q0, scale, x), y, q0);
  const float q2 = fmaf(fmaf(-q1, scale, x), y, q1);
  const float q = fabsf(q0) <= kE4m3Max ? copysignf(q2, x) : q0;
  return fminf(fmaxf(q, -kE4m3Max), kE4m3Max);
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
  const float rcp = __fdiv_rn(1.f, scale);
  const bool by_rcp = scale >= 0x1p-100f && scale <= 0x1p100f;   // uniform

  // two chunks per thread per step, both loaded before either is encoded
  const long chunks = (long)num_tokens * CPR;
  const long stride = (long)gridDim.x * kQThreads;
  // Steps in reverse: the amax pass reads the tokens in rising order with
  // ordinary (cached) loads, so the last of them may still sit in the
  // memory-side cache when this pass starts, and are read again first
  // (benchmark cache: 292 -> 271 us per call with the scale computed).
  const long first = (long)blockIdx.x * kQThreads + threadIdx.x;
  const long nsteps = first < chunks ? (chunks - 1 - first) / (2 * stride) + 1 : 0;
  for (long k = nsteps - 1; k >= 0; --k) {
    const long c0 = first + k * (2 * stride);
    long tok[2];
    int part[2], slot[2];
    q_i32x4 a[2], b[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const long c = c0 + u * stride < chunks ? c0 + u * stride : c0;   // past the end: chunk c0 again
      tok[u] = c / CPR;
      part[u] = (int)(c - tok[u] * CPR);
      // the slot is only needed for the store: the value loads do not wait for it
      slot[u] = c0 + u * stride < chunks ? slots[tok[u]] : -1;
      if (part[u] < 32) {   // nope values 16 part .. +15
        const q_i32x4* src = reinterpret_cast<const q_i32x4*>(ckv + tok[u] * 512 + 16 * part[u]);
        a[u] = __builtin_nontemporal_load(src);
        b[u] = __builtin_nontemporal_load(src + 1);
      } else {              // rope values 8 (part - 32) .. +7, copied
        a[u] = __builtin_nontemporal_load(reinterpret_cast<const q_i32x4*>(rope + tok[u] * ROPE + 8 * (part[u] - 32)));
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      q_i32x4 o = a[u];
      if (part[u] < 32) {   // 16 values -> 16 code bytes
        const unsigned w[8] = {(unsigned)a[u][0], (unsigned)a[u][1], (unsigned)a[u][2], (unsigned)a[u][3],
                               (unsigned)b[u][0], (unsigned)b[u][1], (unsigned)b[u][2], (unsigned)b[u][3]};
        if (by_rcp) {
#pragma unroll
          for (int k = 0; k < 4; ++k)
            o[k] = enc4(qv_rcp(bf16_lo_f(w[2 * k]), scale, rcp), qv_rcp(bf16_hi_f(w[2 * k]), scale, rcp),
                        qv_rcp(bf16_lo_f(w[2 * k + 1]), scale, rcp), qv_rcp(bf16_hi_f(w[2 * k + 1]), scale, rcp));
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k)
            o[k] = enc4(qv(bf16_lo_f(w[2 * k]), scale), qv(bf16_hi_f(w[2 * k]), scale),
                        qv(bf16_lo_f(w[2 * k + 1]), scale), qv(bf16_hi_f(w[2 * k + 1]), scale));
        }
      }
      if (slot_ok(slot[u], cache_rows))
        __builtin_nontemporal_store(o, reinterpret_cast<q_i32x4*>(kv + (long)slot[u] * RB + 16 * part[u]));
    }
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
  // the value and rope loads go out with the slot's (all in bounds for any
  // slot); a row that is not written is dropped once the slot is known
  const int slot = slots[tok];
  const q_i32x4 v = *reinterpret_cast<const q_i32x4*>(ckv + tok * 512 + 8 * lane);
  q_i32x4 rv{};
  if constexpr (ROPE > 0) {
    if (lane < 8) rv = *reinterpret_cast<const q_i32x4*>(rope + tok * ROPE + 8 * lane);
  }
  if (!slot_ok(slot, cache_rows)) return;   // wave-uniform
  float m = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d) m = fmaxf(m, fmaxf(fabsf(bf16_lo_f((unsigned)v[d])), fabsf(bf16_hi_f((unsigned)v[d]))));
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  const float scale = m > 0.f ? __fdiv_rn(m, kE4m3Max) : 1.f;
  int c0, c1;
  if (scale >= 0x1p-100f && scale <= 0x1p100f) {   // wave-uniform
    const float rcp = __fdiv_rn(1.f, scale);
    c0 = enc4(qv_rcp(bf16_lo_f((unsigned)v[0]), scale, rcp), qv_rcp(bf16_hi_f((unsigned)v[0]), scale, rcp),
              qv_rcp(bf16_lo_f((unsigned)v[1]), scale, rcp), qv_rcp(bf16_hi_f((unsigned)v[1]), scale, rcp));
    c1 = enc4(qv_rcp(bf16_lo_f((unsigned)v[2]), scale, rcp), qv_rcp(bf16_hi_f((unsigned)v[2]), scale, rcp),
              qv_rcp(bf16_lo_f((unsigned)v[3]), scale, rcp), qv_rcp(bf16_hi_f((unsigned)v[3]), scale, rcp));
  } else {
    c0 = enc4(qv(bf16_lo_f((unsigned)v[0]), scale), qv(bf16_hi_f((unsigned)v[0]), scale),
              qv(bf16_lo_f((unsigned)v[1]), scale), qv(bf16_hi_f((unsigned)v[1]), scale));
    c1 = enc4(qv(bf16_lo_f((unsigned)v[2]), scale), qv(bf16_hi_f((unsigned)v[2]), scale),
              qv(bf16_lo_f((unsigned)v[3]), scale), qv(bf16_hi_f((unsigned)v[3]), scale));
  }
  uint8_t* row = kv + (long)slot * RB;
  *reinterpret_cast<uint2*>(row + 8 * lane) = uint2{(unsigned)c0, (unsigned)c1};
  if constexpr (ROPE > 0) {
    if (lane < 8) *reinterpret_cast<q_i32x4*>(row + 512 + 16 * lane) = rv;
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

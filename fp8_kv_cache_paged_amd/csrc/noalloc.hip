// Allocation-free decode entry point (mla_fp8_decode_noalloc in
// include/mla_fp8.h): the same host checks, split plan and kernels as
// mla_fp8_decode, with the split partials in a fixed device array of this file
// instead of a caller-supplied workspace.
//
// The array's name is only a host-side handle: its device address on each GPU
// comes from hipGetSymbolAddress, taken once per device with that device
// current and kept per device; the kernels receive that address, never the
// name. Nothing here allocates.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/mla_fp8.h"
#include "launch.h"

// One per GPU, held until the process ends. Contents need no clearing: the
// split kernel writes every partial the combine reads.
static __device__ __align__(256) uint8_t scratch[MLA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch array's device address on the current device.
int32_t scratch_ptr(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MLA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return MLA_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MLA_OK;
}

int32_t supply_scratch(size_t need, void** ws, size_t* ws_bytes) {
  if (need > MLA_NOALLOC_SCRATCH_BYTES) return MLA_ERR_SCRATCH;
  *ws = nullptr;
  *ws_bytes = 0;
  if (need == 0) return MLA_OK;
  const int32_t st = scratch_ptr(ws);
  if (st != MLA_OK) return st;
  *ws_bytes = MLA_NOALLOC_SCRATCH_BYTES;
  return MLA_OK;
}

}  // namespace

extern "C" MLA_API int32_t mla_fp8_decode_noalloc(const mla_params* p, const void* q, const void* kv_cache,
                                                  const int32_t* block_table, const int32_t* seq_lens,
                                                  const float* k_scale, const float* v_scale, int32_t num_splits,
                                                  void* out, float* lse, const int32_t* indices,
                                                  void* hip_stream) {
  return mla::decode_impl(p, q, kv_cache, block_table, seq_lens, k_scale, v_scale, num_splits, out, lse, indices,
                          nullptr, 0, hip_stream, true, 0, supply_scratch);
}

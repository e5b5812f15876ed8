// Internal interface between the C-ABI host layer (host.cpp, noalloc.hip) and
// the HIP kernels (mla_decode.hip, mla_decode_ws.hip). Not installed; include/mla_fp8.h is the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/mla_fp8.h"

namespace mla {

// Supplies the workspace of a decode once its size is known (need bytes, 0
// when the resolved split count is 1): sets *ws and *ws_bytes, or returns a
// status that ends the call before any launch.
using WorkspaceFn = int32_t (*)(size_t need, void** ws, size_t* ws_bytes);

// The decode entry points' common body (host.cpp): host checks, split plan,
// launches. supply may be null (the caller's ws, ws_bytes are used as given).
int32_t decode_impl(const mla_params* p, const void* q, const void* kv_cache, const int32_t* block_table,
                    const int32_t* seq_lens, const float* k_scale, const float* v_scale, int32_t num_splits,
                    void* out, float* lse, const int32_t* indices, void* ws, size_t ws_bytes, void* stream,
                    bool with_combine, int32_t variant, WorkspaceFn supply);

// Everything a decode launch needs, resolved and validated on the host.
struct DecodeLaunch {
  const uint16_t* q;
  const uint8_t* kv;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* indices;
  const float* k_scale;
  const float* v_scale;
  uint16_t* out;
  float* lse;
  uint16_t* part_o; // workspace, splits > 1: fp16 partial outputs
  float* part_lse;  // workspace, splits > 1
  int32_t batch, s_q, h_q, d_rope;
  int32_t num_pages, max_pages, topk, causal, dot;
  int32_t groups;      // batch (dense) or batch * s_q (sparse)
  int32_t rows;        // query rows sharing one key stream: s_q*h_q (dense) or h_q (sparse)
  int32_t row_blocks;  // ceil(rows / 32)
  int32_t splits;
  float softmax_scale;
  bool gather_v;       // debug: byte-gather V^T fragments instead of transposed LDS reads
  bool rows_kernel;    // fp8 dots: P.V split by row block (as for bf16 dots) instead of by dv
  bool dv_split_kernel;  // fp8 dots: the four-wave dv-split kernel instead of the default
  bool per_token;      // k_scale, v_scale: one per cache row ([num_pages, 64])
  bool fnuz;           // e4m3fnuz cache codes (bf16 dots, per-tensor scales)
  bool debug_print;
};

// Bytes of the partial-output workspace for the given geometry.
// Split partials: fp16 values in the accumulator layout, then an f32 log2-lse
// per row, then (per-token scales only) an f32 scale per row that multiplies
// the row's stored values (part_row_scale).
size_t partials_bytes(int32_t splits, int32_t groups, int32_t row_blocks, bool per_token);

hipError_t launch_decode(const DecodeLaunch& d, hipStream_t stream);
hipError_t launch_combine(const DecodeLaunch& d, hipStream_t stream);

// A quantize-on-write launch, validated on the host.
struct QuantizeLaunch {
  const uint16_t* ckv;     // bf16 [num_tokens, 512]
  const uint16_t* rope;    // bf16 [num_tokens, d_rope] (d_rope = 64) or null
  const int32_t* slots;    // [num_tokens] cache row = page * 64 + slot
  uint8_t* kv;             // [num_pages, 64, 1, 512 + 2 d_rope]
  float* k_scale;
  float* v_scale;
  float* workspace;        // quantize_workspace_bytes(), compute_scale only
  int32_t num_tokens, d_rope, num_pages;
  bool compute_scale;
  bool per_token;          // compute_scale: one scale per written row
};

size_t quantize_workspace_bytes();
hipError_t launch_quantize_kv(const QuantizeLaunch& d, hipStream_t stream);

hipError_t launch_debug_decode_e4m3fn(const uint8_t* codes, float* out_f32, uint16_t* out_bf16,
                                      int32_t n, hipStream_t stream);
hipError_t launch_debug_fnuz_to_ocp(const uint8_t* codes, uint8_t* out, int32_t n, hipStream_t stream);
hipError_t launch_debug_quantize_q(const uint16_t* q, int32_t rows, int32_t row_len,
                                   uint8_t* codes, int32_t* exps, hipStream_t stream);
hipError_t launch_debug_gather(const uint8_t* kv, const int32_t* block_table,
                               const int32_t* seq_lens, int32_t batch, int32_t max_pages,
                               int32_t num_pages, int32_t d_rope, uint8_t* dense_out,
                               hipStream_t stream);
hipError_t launch_debug_gather_ws(const uint8_t* kv, const int32_t* block_table, const int32_t* seq_lens,
                                  int32_t batch, int32_t max_pages, int32_t num_pages, int32_t d_rope,
                                  uint8_t* dense_out, hipStream_t stream);
hipError_t launch_stream_read(const void* src, size_t bytes, float* sink, hipStream_t stream);
hipError_t launch_mfma_peak(int dot, int iters, int blocks, float* sink, hipStream_t stream);

}  // namespace mla

// C-ABI entry points of the FP8-KV paged MLA decode library (include/mla_fp8.h).
//
// Host-side work only: argument validation (no HIP call, so it runs and is
// tested without a GPU), the split plan, workspace sizing, and the launches.
// Validation follows the pages' conventions: a missing scale with an fp8
// cache is an error rather than a silent misread (InfiniCore PR #1568, the
// "F8 cache without scales fails loudly" commit); a one-byte encoding other
// than the native OCP e4m3fn is refused rather than decoded as e4m3fn
// (ROCm/aiter PR #6199, the foreign-encoding refusal commit).

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <mutex>

#include "../../include/mla_fp8.h"
#include "launch.h"

namespace {

constexpr int kPage = 64;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int32_t groups_of(const mla_params& p) { return p.topk > 0 ? p.batch * p.s_q : p.batch; }
int32_t rows_of(const mla_params& p) { return p.topk > 0 ? p.h_q : p.s_q * p.h_q; }
int32_t units_of(const mla_params& p) {
  // 64-key units one key stream spans at most: pages (dense) or 64-entry
  // chunks of the index list (sparse)
  return p.topk > 0 ? (p.topk + kPage - 1) / kPage : p.max_pages_per_seq;
}

int32_t validate(const mla_params* p) {
  if (p == nullptr) return MLA_ERR_NULL;
  switch (p->kv_dtype) {
    case MLA_KV_FP8_E4M3FN:
    case MLA_KV_UINT8:
      break;
    case MLA_KV_FP8_E4M3FNUZ:
      // per-tensor scales; bf16 dots decode the codes in registers, fp8 dots
      // transcode each landed tile to the e4m3fn codes of the same values
      if (p->kv_scale_per_token != 0) return MLA_ERR_UNSUPPORTED;
      break;
    case MLA_KV_FP8_E5M2:
    case MLA_KV_INT8:
    case MLA_KV_BF16:
      return MLA_ERR_UNSUPPORTED;
    default:
      return MLA_ERR_DTYPE;
  }
  // dense rows share a key stream per sequence (s_q * h_q of them); sparse
  // query tokens each carry their own index list, so a long prefill is many
  // independent groups
  if (p->batch < 1 || p->s_q < 1 || p->s_q > (p->topk > 0 ? 65536 : 1024) || p->h_q < 1 || p->h_q > 1024)
    return MLA_ERR_SHAPE;
  if (p->num_pages < 1 || p->max_pages_per_seq < 1 || p->topk < 0) return MLA_ERR_SHAPE;
  if (p->causal != 0 && p->causal != 1) return MLA_ERR_SHAPE;
  if (p->kv_scale_per_token != 0 && p->kv_scale_per_token != 1) return MLA_ERR_SHAPE;
  if (p->dot != MLA_DOT_BF16 && p->dot != MLA_DOT_FP8) return MLA_ERR_SHAPE;
  if (!(p->softmax_scale <= 0.f || isfinite(p->softmax_scale))) return MLA_ERR_SHAPE;
  if (p->h_kv != 1 || p->d_nope != 512 || p->dv != p->d_nope || p->page_block != kPage ||
      (p->d_rope != 0 && p->d_rope != 64))
    return MLA_ERR_UNSUPPORTED;
  // index arithmetic in the kernels is 32-bit on rows and 64-bit on bytes
  if ((int64_t)p->num_pages * kPage > INT32_MAX) return MLA_ERR_SHAPE;
  if ((int64_t)p->max_pages_per_seq * kPage > INT32_MAX) return MLA_ERR_SHAPE;
  if ((int64_t)p->batch * p->s_q * p->h_q > INT32_MAX / 1024) return MLA_ERR_SHAPE;
  return MLA_OK;
}

int32_t resolve(const mla_params& p, int32_t num_splits, int32_t cu_count) {
  if (num_splits < 0) return -MLA_ERR_SHAPE;
  const int32_t units = units_of(p);
  if (num_splits > 0) return num_splits > MLA_MAX_SPLITS ? MLA_MAX_SPLITS : num_splits;
  const char* env = getenv("MLA_FP8_NUM_SPLITS");
  if (env != nullptr) {
    const long v = strtol(env, nullptr, 10);
    if (v > 0) return v > MLA_MAX_SPLITS ? MLA_MAX_SPLITS : (int32_t)v;
  }
  // smallest s with (workgroups per split) * s >= CUs, capped at 16 and at the
  // units per stream; a split has one workgroup per key stream and group of
  // four 32-row blocks (a prefill chunk's many rows already fill the chip)
  const int32_t row_blocks = (rows_of(p) + 31) / 32;
  const int32_t g = groups_of(p) * ((row_blocks + 3) / 4);
  int32_t s = cu_count > 0 ? (cu_count + g - 1) / g : 1;
  if (s > 16) s = 16;
  if (s > units) s = units;
  return s < 1 ? 1 : s;
}

size_t workspace(const mla_params& p, int32_t splits) {
  if (splits <= 1) return 0;
  return mla::partials_bytes(splits, groups_of(p), (rows_of(p) + 31) / 32, p.kv_scale_per_token != 0);
}

std::mutex g_cu_mutex;
int g_cu_count[64] = {0};

int32_t device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (dev >= 0 && dev < 64) {
    std::lock_guard<std::mutex> lock(g_cu_mutex);
    if (g_cu_count[dev] == 0) {
      int cus = 0;
      if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
      g_cu_count[dev] = cus;
    }
    return g_cu_count[dev];
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  return cus;
}

}  // namespace

namespace mla {

int32_t decode_impl(const mla_params* p, const void* q, const void* kv_cache, const int32_t* block_table,
                    const int32_t* seq_lens, const float* k_scale, const float* v_scale, int32_t num_splits,
                    void* out, float* lse, const int32_t* indices, void* ws, size_t ws_bytes, void* stream,
                    bool with_combine, int32_t variant, WorkspaceFn supply) {
  int32_t st = validate(p);
  if (st != MLA_OK) return st;
  if (q == nullptr || kv_cache == nullptr || block_table == nullptr || seq_lens == nullptr || out == nullptr ||
      lse == nullptr)
    return MLA_ERR_NULL;
  if (k_scale == nullptr || v_scale == nullptr) return MLA_ERR_NULL;   // an fp8 cache needs its scales
  if (p->topk > 0 && indices == nullptr) return MLA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(kv_cache, 16) || !aligned(out, 16) || !aligned(lse, 4) ||
      !aligned(block_table, 4) || !aligned(seq_lens, 4) || !aligned(k_scale, 4) || !aligned(v_scale, 4) ||
      (indices != nullptr && !aligned(indices, 4)))
    return MLA_ERR_ALIGN;
  int32_t cus = 0;
  if (num_splits == 0) {
    cus = device_cu_count();
    if (cus < 0) return MLA_ERR_HIP;
  }
  const int32_t splits = resolve(*p, num_splits, cus);
  if (splits < 1) return -splits;
  const size_t need = workspace(*p, splits);
  if (supply != nullptr) {
    st = supply(need, &ws, &ws_bytes);
    if (st != MLA_OK) return st;
  }
  if (need > 0) {
    if (ws == nullptr || ws_bytes < need) return MLA_ERR_WORKSPACE;
    if (!aligned(ws, 16)) return MLA_ERR_ALIGN;
  }

  mla::DecodeLaunch d;
  d.q = static_cast<const uint16_t*>(q);
  d.kv = static_cast<const uint8_t*>(kv_cache);
  d.block_table = block_table;
  d.seq_lens = seq_lens;
  d.indices = p->topk > 0 ? indices : nullptr;
  d.k_scale = k_scale;
  d.v_scale = v_scale;
  d.out = static_cast<uint16_t*>(out);
  d.lse = lse;
  d.batch = p->batch;
  d.s_q = p->s_q;
  d.h_q = p->h_q;
  d.d_rope = p->d_rope;
  d.num_pages = p->num_pages;
  d.max_pages = p->max_pages_per_seq;
  d.topk = p->topk;
  d.causal = p->topk > 0 ? 0 : p->causal;
  d.dot = p->dot;
  d.groups = groups_of(*p);
  d.rows = rows_of(*p);
  d.row_blocks = (d.rows + 31) / 32;
  d.splits = splits;
  d.softmax_scale = p->softmax_scale > 0.f ? p->softmax_scale : 1.f / sqrtf((float)(p->d_nope + p->d_rope));
  const size_t frags = (size_t)splits * d.groups * d.row_blocks;
  d.part_o = need > 0 ? static_cast<uint16_t*>(ws) : nullptr;
  d.part_lse = need > 0 ? reinterpret_cast<float*>(static_cast<char*>(ws) + frags * 16 * 64 * 16 * sizeof(uint16_t))
                        : nullptr;
  // the fp8-dot read of an fnuz cache exists in the default kernel only
  if (variant != 0 && p->kv_dtype == MLA_KV_FP8_E4M3FNUZ && p->dot == MLA_DOT_FP8) return MLA_ERR_UNSUPPORTED;
  d.gather_v = (variant & MLA_VARIANT_GATHER_V) != 0;
  d.rows_kernel = (variant & MLA_VARIANT_ROWS) != 0;
  d.dv_split_kernel = (variant & MLA_VARIANT_DV_SPLIT) != 0;
  d.per_token = p->kv_scale_per_token != 0;
  d.fnuz = p->kv_dtype == MLA_KV_FP8_E4M3FNUZ;
  // read once per process (the split-count override, read per call, is meant
  // to be changed between calls; the plan print is not)
  static const bool debug_print = [] {
    const char* dbg = getenv("MLA_FP8_DEBUG");
    return dbg != nullptr && dbg[0] == '1';
  }();
  d.debug_print = debug_print;
  if (d.debug_print)
    fprintf(stderr, "[mla_fp8] plan: groups=%d rows=%d splits=%d workspace=%zu cus=%d\n", d.groups, d.rows, splits,
            need, cus);

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (mla::launch_decode(d, s) != hipSuccess) return MLA_ERR_HIP;
  if (splits > 1 && with_combine) {
    if (mla::launch_combine(d, s) != hipSuccess) return MLA_ERR_HIP;
  }
  return MLA_OK;
}

}  // namespace mla

extern "C" {

MLA_API int32_t mla_fp8_validate(const mla_params* p) { return validate(p); }

MLA_API int32_t mla_fp8_decode_resolve_splits(const mla_params* p, int32_t num_splits, int32_t cu_count) {
  const int32_t st = validate(p);
  if (st != MLA_OK) return -st;
  return resolve(*p, num_splits, cu_count);
}

MLA_API size_t mla_fp8_decode_workspace_size(const mla_params* p, int32_t splits) {
  if (validate(p) != MLA_OK || splits < 1) return 0;
  return workspace(*p, splits);
}

MLA_API int32_t mla_fp8_decode(const mla_params* p, const void* q, const void* kv_cache,
                               const int32_t* block_table, const int32_t* seq_lens, const float* k_scale,
                               const float* v_scale, int32_t num_splits, void* out, float* lse,
                               const int32_t* indices, void* workspace_ptr, size_t workspace_bytes,
                               void* hip_stream) {
  return mla::decode_impl(p, q, kv_cache, block_table, seq_lens, k_scale, v_scale, num_splits, out, lse, indices,
                     workspace_ptr, workspace_bytes, hip_stream, true, 0, nullptr);
}

MLA_API int32_t mla_fp8_debug_decode_variant(const mla_params* p, const void* q, const void* kv_cache,
                                             const int32_t* block_table, const int32_t* seq_lens,
                                             const float* k_scale, const float* v_scale, int32_t num_splits,
                                             void* out, float* lse, const int32_t* indices, void* workspace_ptr,
                                             size_t workspace_bytes, int32_t variant, void* hip_stream) {
  if (variant & ~(MLA_VARIANT_GATHER_V | MLA_VARIANT_ROWS | MLA_VARIANT_DV_SPLIT)) return MLA_ERR_SHAPE;
  return mla::decode_impl(p, q, kv_cache, block_table, seq_lens, k_scale, v_scale, num_splits, out, lse, indices,
                     workspace_ptr, workspace_bytes, hip_stream, true, variant, nullptr);
}

MLA_API int32_t mla_fp8_decode_partials(const mla_params* p, const void* q, const void* kv_cache,
                                        const int32_t* block_table, const int32_t* seq_lens,
                                        const float* k_scale, const float* v_scale, int32_t num_splits,
                                        void* out, float* lse, const int32_t* indices, void* workspace_ptr,
                                        size_t workspace_bytes, void* hip_stream) {
  return mla::decode_impl(p, q, kv_cache, block_table, seq_lens, k_scale, v_scale, num_splits, out, lse, indices,
                     workspace_ptr, workspace_bytes, hip_stream, false, 0, nullptr);
}

MLA_API const char* mla_fp8_status_string(int32_t status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL: return "a required pointer is NULL";
    case MLA_ERR_SHAPE: return "a size is out of range or inconsistent";
    case MLA_ERR_DTYPE: return "unknown kv_dtype code";
    case MLA_ERR_UNSUPPORTED: return "unsupported encoding or dimension";
    case MLA_ERR_WORKSPACE: return "workspace missing or too small";
    case MLA_ERR_ALIGN: return "a pointer is misaligned";
    case MLA_ERR_HIP: return "HIP runtime error";
    case MLA_ERR_SCRATCH: return "the call needs more workspace than the fixed scratch of the allocation-free entry point";
    default: return "unknown status";
  }
}

MLA_API size_t mla_fp8_quantize_kv_workspace_size(void) { return mla::quantize_workspace_bytes(); }

MLA_API int32_t mla_fp8_quantize_kv(int32_t num_tokens, int32_t d_rope, int32_t num_pages, const void* ckv,
                                    const void* k_rope, const int32_t* slot_mapping, void* kv_cache,
                                    float* k_scale, float* v_scale, int32_t compute_scale, void* workspace_ptr,
                                    size_t workspace_bytes, void* hip_stream) {
  if (num_tokens < 0 || num_pages < 1 || compute_scale < 0 || compute_scale > 2) return MLA_ERR_SHAPE;
  if (d_rope != 0 && d_rope != 64) return MLA_ERR_UNSUPPORTED;
  if ((int64_t)num_pages * kPage > INT32_MAX) return MLA_ERR_SHAPE;
  if (k_scale == nullptr || v_scale == nullptr || kv_cache == nullptr) return MLA_ERR_NULL;
  if (num_tokens > 0 && (ckv == nullptr || slot_mapping == nullptr || (d_rope > 0 && k_rope == nullptr)))
    return MLA_ERR_NULL;
  if (compute_scale == 1 && (workspace_ptr == nullptr || workspace_bytes < mla::quantize_workspace_bytes()))
    return MLA_ERR_WORKSPACE;
  if (!aligned(kv_cache, 16) || (ckv != nullptr && !aligned(ckv, 16)) ||
      (d_rope > 0 && k_rope != nullptr && !aligned(k_rope, 16)) ||
      (slot_mapping != nullptr && !aligned(slot_mapping, 4)) || !aligned(k_scale, 4) || !aligned(v_scale, 4) ||
      (workspace_ptr != nullptr && !aligned(workspace_ptr, 4)))
    return MLA_ERR_ALIGN;
  if (num_tokens == 0 && compute_scale != 1) return MLA_OK;   // nothing to write
  mla::QuantizeLaunch d;
  d.ckv = static_cast<const uint16_t*>(ckv);
  d.rope = d_rope > 0 ? static_cast<const uint16_t*>(k_rope) : nullptr;
  d.slots = slot_mapping;
  d.kv = static_cast<uint8_t*>(kv_cache);
  d.k_scale = k_scale;
  d.v_scale = v_scale;
  d.workspace = compute_scale == 1 ? static_cast<float*>(workspace_ptr) : nullptr;
  d.num_tokens = num_tokens;
  d.d_rope = d_rope;
  d.num_pages = num_pages;
  d.compute_scale = compute_scale != 0;
  d.per_token = compute_scale == 2;
  return mla::launch_quantize_kv(d, static_cast<hipStream_t>(hip_stream)) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

MLA_API int32_t mla_fp8_debug_decode_e4m3fn(const uint8_t* codes, float* out_f32, uint16_t* out_bf16, int32_t n,
                                            void* hip_stream) {
  if (codes == nullptr || (out_f32 == nullptr && out_bf16 == nullptr)) return MLA_ERR_NULL;
  if (n < 0) return MLA_ERR_SHAPE;
  if (n == 0) return MLA_OK;
  return mla::launch_debug_decode_e4m3fn(codes, out_f32, out_bf16, n, static_cast<hipStream_t>(hip_stream)) ==
                 hipSuccess
             ? MLA_OK
             : MLA_ERR_HIP;
}

MLA_API int32_t mla_fp8_debug_fnuz_to_e4m3fn(const uint8_t* codes, uint8_t* out, int32_t n, void* hip_stream) {
  if (codes == nullptr || out == nullptr) return MLA_ERR_NULL;
  if (n < 0) return MLA_ERR_SHAPE;
  if (n == 0) return MLA_OK;
  return mla::launch_debug_fnuz_to_ocp(codes, out, n, static_cast<hipStream_t>(hip_stream)) == hipSuccess
             ? MLA_OK
             : MLA_ERR_HIP;
}

MLA_API int32_t mla_fp8_debug_quantize_q(const void* q, int32_t rows, int32_t row_len, uint8_t* codes,
                                         int32_t* exps, void* hip_stream) {
  if (q == nullptr || codes == nullptr || exps == nullptr) return MLA_ERR_NULL;
  if (rows < 0 || row_len < 512 || row_len % 8 != 0) return MLA_ERR_SHAPE;
  if (!aligned(q, 16) || !aligned(codes, 4) || !aligned(exps, 4)) return MLA_ERR_ALIGN;
  if (rows == 0) return MLA_OK;
  return mla::launch_debug_quantize_q(static_cast<const uint16_t*>(q), rows, row_len, codes, exps,
                                      static_cast<hipStream_t>(hip_stream)) == hipSuccess
             ? MLA_OK
             : MLA_ERR_HIP;
}

MLA_API int32_t mla_fp8_debug_gather(const mla_params* p, const void* kv_cache, const int32_t* block_table,
                                     const int32_t* seq_lens, void* dense_out, void* hip_stream) {
  const int32_t st = validate(p);
  if (st != MLA_OK) return st;
  if (kv_cache == nullptr || block_table == nullptr || seq_lens == nullptr || dense_out == nullptr)
    return MLA_ERR_NULL;
  if (!aligned(kv_cache, 16) || !aligned(dense_out, 16)) return MLA_ERR_ALIGN;
  return mla::launch_debug_gather(static_cast<const uint8_t*>(kv_cache), block_table, seq_lens, p->batch,
                                  p->max_pages_per_seq, p->num_pages, p->d_rope, static_cast<uint8_t*>(dense_out),
                                  static_cast<hipStream_t>(hip_stream)) == hipSuccess
             ? MLA_OK
             : MLA_ERR_HIP;
}

MLA_API int32_t mla_fp8_debug_gather_ws(const mla_params* p, const void* kv_cache, const int32_t* block_table,
                                        const int32_t* seq_lens, void* dense_out, void* hip_stream) {
  const int32_t st = validate(p);
  if (st != MLA_OK) return st;
  if (kv_cache == nullptr || block_table == nullptr || seq_lens == nullptr || dense_out == nullptr)
    return MLA_ERR_NULL;
  if (!aligned(kv_cache, 16) || !aligned(dense_out, 16)) return MLA_ERR_ALIGN;
  return mla::launch_debug_gather_ws(static_cast<const uint8_t*>(kv_cache), block_table, seq_lens, p->batch,
                                     p->max_pages_per_seq, p->num_pages, p->d_rope,
                                     static_cast<uint8_t*>(dense_out), static_cast<hipStream_t>(hip_stream)) ==
                 hipSuccess
             ? MLA_OK
             : MLA_ERR_HIP;
}

MLA_API int32_t mla_fp8_bench_mfma(int32_t dot, int32_t iters, int32_t blocks, float* sink, void* hip_stream) {
  if (sink == nullptr) return MLA_ERR_NULL;
  if ((dot != MLA_DOT_BF16 && dot != MLA_DOT_FP8) || iters < 1 || blocks < 1) return MLA_ERR_SHAPE;
  if (!aligned(sink, 4)) return MLA_ERR_ALIGN;
  return mla::launch_mfma_peak(dot, iters, blocks, sink, static_cast<hipStream_t>(hip_stream)) == hipSuccess
             ? MLA_OK
             : MLA_ERR_HIP;
}

MLA_API int32_t mla_fp8_bench_stream_read(const void* src, size_t bytes, float* sink, void* hip_stream) {
  if (src == nullptr || sink == nullptr) return MLA_ERR_NULL;
  if (bytes % 16 != 0) return MLA_ERR_SHAPE;
  if (!aligned(src, 16)) return MLA_ERR_ALIGN;
  if (bytes == 0) return MLA_OK;
  return mla::launch_stream_read(src, bytes, sink, static_cast<hipStream_t>(hip_stream)) == hipSuccess
             ? MLA_OK
             : MLA_ERR_HIP;
}

}  // extern "C"

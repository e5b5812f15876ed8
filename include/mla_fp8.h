/*
 * mla_fp8.h -- C ABI of the MI355X (gfx950) FP8-KV paged MLA decode library.
 *
 * The operation (FlashMLA PR #82 "update fp8 support", description and the H800
 * test report; ROCm/aiter PR #6199, Technical details; InfiniCore PR #1568,
 * Summary, paged attention bullets): multi-head latent attention decode. For
 * every query token (s_q of them per sequence, 2 with multi-token prediction)
 * h_q query heads attend to ONE shared latent KV head (h_kv = 1) per cached
 * token. A cached token row holds 512 OCP e4m3fn "nope" bytes followed by 64
 * little-endian bf16 rope values (or no rope). K = [nope * k_scale, rope],
 * V = nope * v_scale. The output is softmax(scale * Q K^T) V over the 512-wide
 * latent, plus the natural-log log-sum-exp of the scaled logits. Long key
 * ranges are cut into splits whose partials are merged by a log-sum-exp
 * combine (InfiniCore PR #1568, split-kv commit).
 *
 * Tensor layouts (all device memory, row-major, caller-owned):
 *   q            bf16   [batch, s_q, h_q, d_nope + d_rope]
 *   kv_cache     bytes  [num_pages, page_block, h_kv=1, d_nope + 2*d_rope]
 *                       page_block must be 64; 16-byte aligned base
 *   block_table  int32  [batch, max_pages_per_seq]   physical page ids
 *   seq_lens     int32  [batch]                      cached tokens per sequence
 *   k_scale      f32[1] device pointer (as the FlashInfer XQA launcher's
 *   v_scale      f32[1]  kvCacheScale, FlashInfer PR #1769): never read on the host
 *   indices      int32  [batch, s_q, topk]  sparse variant only: logical token
 *                       positions; entries < 0 or >= seq_len are skipped
 *   out          bf16   [batch, s_q, h_q, dv]      (dv = d_nope = 512)
 *   lse          f32    [batch, s_q, h_q]          natural log; -inf for a row
 *                                                  with no visible key (out = 0)
 *   workspace    device scratch of mla_fp8_decode_workspace_size() bytes when
 *                the resolved split count is > 1 (may be NULL otherwise);
 *                calls that share a workspace must be ordered on one stream
 *
 * Semantics not fixed by the source pages, as implemented:
 *   softmax_scale <= 0 selects 1/sqrt(d_nope + d_rope); causal rows are
 *   bottom-right aligned (token i of s_q sees keys 0 .. seq_len - s_q + i);
 *   k_scale scales only the fp8 part of K; sparse rows take no causal mask.
 *   MLA_DOT_FP8 quantizes each query row's nope part to e4m3fn with its own
 *   power-of-two scale (the smallest 2^e with amax <= 448 * 2^e), and P,
 *   taken against a running row max that is only raised when a tile exceeds
 *   it by more than 3 in log2 units (so p <= 8), to e4m3fn after scaling it
 *   by 32 (values <= 256); MLA_DOT_BF16 keeps Q in bf16 and
 *   converts the cache bytes to bf16 exactly. With at most 16 query rows per
 *   key stream (s_q * h_q dense, h_q sparse) both modes multiply the exact
 *   bf16 query, on the fp8 matrix cores, as two terms: each row's nope part
 *   as 2^e (c1 + c2 / 16), c1 and c2 e4m3fn codes, equal to the bf16 query
 *   for every element of magnitude >= 2^(e-6) (e as above). MLA_DOT_FP8 then
 *   packs P as above; MLA_DOT_BF16 (e4m3fn cache) packs P as two terms too,
 *   c1 + c2 / 16 with c1 = e4m3fn(p), about 8 significant bits (as a bf16 P)
 *   for p down to 2^-14 of the running max, which is then raised at every
 *   larger tile max, with P scaled by 256.
 *
 * Ownership, streams and threads: the library never allocates, frees or
 * synchronizes device memory, apart from one fixed device array per GPU that
 * the loader reserves for mla_fp8_decode_noalloc (MLA_NOALLOC_SCRATCH_BYTES,
 * held until the process ends). Every kernel is enqueued on the caller's
 * hip_stream (NULL = the default stream). No mutable global state beyond a
 * per-device cache of the compute-unit count; calls are thread-safe. Results
 * are deterministic: the same inputs and split count give bitwise equal
 * output (no atomics).
 *
 * Errors: every entry point returns an int32 status (MLA_OK = 0). All host
 * checks run before any launch, so a failing call enqueues nothing and writes
 * nothing. Device-side values (seq_lens, block_table entries, indices,
 * scales) cannot be checked without a synchronization: the kernels clamp
 * seq_len to [0, max_pages_per_seq * 64] and skip keys whose page id lies
 * outside [0, num_pages), which keeps every access in bounds; results for
 * such inputs are otherwise unspecified, as are non-finite or non-positive
 * scales.
 */
#ifndef MLA_FP8_H
#define MLA_FP8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_API __attribute__((visibility("default")))

/* status codes */
#define MLA_OK 0
#define MLA_ERR_NULL 1         /* a required pointer is NULL (incl. scales with an fp8 cache) */
#define MLA_ERR_SHAPE 2        /* a size is out of range or inconsistent */
#define MLA_ERR_DTYPE 3        /* kv_dtype is not a known code */
#define MLA_ERR_UNSUPPORTED 4  /* a known but unsupported encoding or dimension */
#define MLA_ERR_WORKSPACE 5    /* workspace missing or too small */
#define MLA_ERR_ALIGN 6        /* a pointer is not aligned as required */
#define MLA_ERR_HIP 7          /* the HIP runtime reported an error */
#define MLA_ERR_SCRATCH 8      /* mla_fp8_decode_noalloc: the call needs more
                                  workspace than MLA_NOALLOC_SCRATCH_BYTES */

/* kv_dtype codes. The OCP e4m3fn encoding (or a uint8 view of it) is read
 * by both dot modes. gfx942's e4m3fnuz (bias 8, largest magnitude 240, NaN
 * only at 0x80; ROCm/aiter PR #6199, Technical details) is read with
 * per-tensor scales only. MLA_DOT_BF16 decodes its codes exactly to bf16 in
 * registers. MLA_DOT_FP8 (dense and sparse) turns
 * each landed tile's codes into the e4m3fn codes of the same values for the
 * OCP fp8 matrix cores: exact for every magnitude from 2^-6 to 240 (in units
 * of the scale); the fnuz magnitudes below 2^-6 (steps of 2^-10) go to
 * e4m3fn's (steps of 2^-9) by round to nearest even, moving by at most
 * 2^-10. In both modes 0x80, the NaN code, reads as zero. Per-token scales
 * with an fnuz cache are MLA_ERR_UNSUPPORTED. The other one-byte encodings are refused rather than
 * misread (ROCm/aiter PR #6199, the foreign-encoding refusal commit). */
#define MLA_KV_FP8_E4M3FN 0
#define MLA_KV_UINT8 1          /* raw bytes, taken to be e4m3fn */
#define MLA_KV_FP8_E4M3FNUZ 2   /* per-tensor scales */
#define MLA_KV_FP8_E5M2 3       /* refused: MLA_ERR_UNSUPPORTED */
#define MLA_KV_INT8 4           /* refused: MLA_ERR_UNSUPPORTED */
#define MLA_KV_BF16 5           /* refused: MLA_ERR_UNSUPPORTED */

/* contraction precision */
#define MLA_DOT_BF16 0
#define MLA_DOT_FP8 1

#define MLA_MAX_SPLITS 64

/* Host-side description of the tensors. */
typedef struct mla_params {
  int32_t batch;              /* sequences, >= 1 */
  int32_t s_q;                /* query tokens per sequence: 1..1024 dense (2 with MTP;
                                 up to 16 for multi-token decode, more for a causal
                                 prefill chunk: the last s_q tokens of the sequence);
                                 1..65536 sparse, where every token carries its own
                                 index list (a sparse prefill, ROCm/aiter PR #6199,
                                 Results: 16K tokens) */
  int32_t h_q;                /* query heads, 1..1024 */
  int32_t h_kv;               /* latent KV heads: must be 1 */
  int32_t d_nope;             /* must be 512 */
  int32_t d_rope;             /* 64 or 0 */
  int32_t dv;                 /* must equal d_nope */
  int32_t page_block;         /* tokens per page: must be 64 */
  int32_t num_pages;          /* pages in kv_cache, >= 1 */
  int32_t max_pages_per_seq;  /* block_table row length, >= 1 */
  int32_t kv_dtype;           /* MLA_KV_* */
  int32_t causal;             /* 0 or 1 (dense only) */
  int32_t dot;                /* MLA_DOT_BF16 or MLA_DOT_FP8 */
  int32_t topk;               /* 0 = dense paged; > 0 = sparse, indices required */
  float softmax_scale;        /* <= 0 selects 1/sqrt(d_nope + d_rope) */
  int32_t kv_scale_per_token; /* 0: k_scale, v_scale are f32[1] (per tensor);
                                 1: f32 [num_pages, 1, 64], one k and one v scale
                                 per cache row (InfiniCore PR #1568, Summary: the
                                 [num_blocks, h_kv, block_size] layout) */
} mla_params;

/* Host-only validation of *p (no HIP call). Returns MLA_OK or the first
 * failing check's code. */
MLA_API int32_t mla_fp8_validate(const mla_params* p);

/* Split count the decode will use. The split-KV scheme is InfiniCore PR #1568's
 * split-kv commit: the token range of a sequence is sharded over several
 * workgroups, the split count comes from an automatic occupancy ("waves")
 * heuristic that leaves an already large grid unsplit, and an environment
 * variable overrides it. Here: num_splits > 0 is taken as given (capped at
 * MLA_MAX_SPLITS); 0 selects the smallest s with groups * row_groups * s >=
 * cu_count, capped at 16 and at the number of 64-key units per sequence,
 * where groups is batch (dense) or batch * s_q (sparse) and row_groups is
 * ceil(rows / 128), rows = s_q * h_q (dense) or h_q (sparse): the workgroups
 * one split launches. The environment variable
 * MLA_FP8_NUM_SPLITS, when set to a positive integer, replaces the automatic
 * choice. Returns a value >= 1, or a negative status on invalid *p. Host-only,
 * no HIP call. */
MLA_API int32_t mla_fp8_decode_resolve_splits(const mla_params* p, int32_t num_splits,
                                              int32_t cu_count);

/* Workspace bytes needed for a resolved split count (0 when splits == 1).
 * As in InfiniCore PR #1568's split-kv commit, where the decode's workspace
 * grows from zero to splits x sequences x heads x (value size + 2) floats,
 * the workspace holds one partial per split and query row: here the 512
 * partial output values in fp16 and one f32 log-sum-exp, padded to 32-row
 * blocks: splits * groups * ceil(rows / 32) * (32 KiB + 128 B); with per-token
 * scales also one f32 per row that scales its stored values (+128 B per
 * block; the values stay within fp16's normal range at any scale). The caller
 * owns it; its contents need no initialization and are overwritten by every
 * call. Returns 0 for invalid *p or splits < 1. Host-only, no HIP call. */
MLA_API size_t mla_fp8_decode_workspace_size(const mla_params* p, int32_t splits);

/* The decode. Enqueues one kernel (splits == 1) or the split kernel and the
 * combine kernel on hip_stream. num_splits as for resolve_splits, with the
 * current device's compute-unit count. indices may be NULL unless topk > 0;
 * workspace may be NULL when the resolved split count is 1. */
MLA_API int32_t mla_fp8_decode(const mla_params* p, const void* q, const void* kv_cache,
                               const int32_t* block_table, const int32_t* seq_lens,
                               const float* k_scale, const float* v_scale, int32_t num_splits,
                               void* out, float* lse, const int32_t* indices, void* workspace,
                               size_t workspace_bytes, void* hip_stream);

/* Allocation-free decode, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation). Arguments and results as for mla_fp8_decode, without the
 * workspace: the split partials go to a fixed device array of the library
 * (MLA_NOALLOC_SCRATCH_BYTES per GPU, 256-byte aligned, its address looked up
 * once per device on the first call that needs it). A call whose
 * mla_fp8_decode_workspace_size() exceeds that size returns MLA_ERR_SCRATCH
 * before any launch (a smaller explicit num_splits lowers the need; 1 needs
 * none). The call allocates nothing: no
 * hipMalloc, no library routine that allocates. Every call on one GPU shares
 * that GPU's array, whose contents need no clearing (each call overwrites the
 * partials it reads): calls that overlap on one GPU (two streams, or two
 * threads without ordering) race on it and give unspecified results; calls
 * ordered on one stream are safe. */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
MLA_API int32_t mla_fp8_decode_noalloc(const mla_params* p, const void* q, const void* kv_cache,
                                       const int32_t* block_table, const int32_t* seq_lens,
                                       const float* k_scale, const float* v_scale, int32_t num_splits,
                                       void* out, float* lse, const int32_t* indices, void* hip_stream);

/* First stage only (timing and tests): with a resolved split count > 1 it
 * writes the per-split partials into the workspace and launches no combine;
 * with 1 split it is the whole decode. Arguments as for mla_fp8_decode. */
MLA_API int32_t mla_fp8_decode_partials(const mla_params* p, const void* q, const void* kv_cache,
                                        const int32_t* block_table, const int32_t* seq_lens,
                                        const float* k_scale, const float* v_scale,
                                        int32_t num_splits, void* out, float* lse,
                                        const int32_t* indices, void* workspace,
                                        size_t workspace_bytes, void* hip_stream);

/* Quantize-on-write of the paged latent cache, the step that fills the cache
 * the decode reads (InfiniCore PR #1568, Summary, FP8 KV cache bullet: a
 * per-tensor scale amax / 448, 448 being the largest finite e4m3fn value).
 *
 *   ckv           bf16  [num_tokens, 512]     new latent ("nope") rows
 *   k_rope        bf16  [num_tokens, d_rope]  their rope values (NULL if d_rope = 0)
 *   slot_mapping  int32 [num_tokens]          cache row of each token: page * 64 +
 *                                             slot within the page; a negative or
 *                                             out-of-range entry is skipped (not
 *                                             written); each row at most once
 *   kv_cache      bytes [num_pages, 64, 1, 512 + 2 * d_rope], the decode's layout;
 *                 only the rows named by slot_mapping are written
 *   k_scale, v_scale  f32[1] device pointers
 *   compute_scale 2: per token: each written row gets its own scale, amax of
 *                 its 512 nope values / 448 (1 if 0), stored at its cache row in
 *                 k_scale and v_scale, here f32 [num_pages, 1, 64] arrays (the
 *                 layout of kv_scale_per_token); no workspace.
 *   compute_scale 1: scale = amax / 448 over the nope values of the written
 *                 tokens (1 when that amax is 0), computed in f32 and stored to
 *                 both k_scale and v_scale; needs a workspace of
 *                 mla_fp8_quantize_kv_workspace_size() bytes.
 *                 0: the scale is read from k_scale (nothing is stored to the
 *                 scales; workspace may be NULL).
 *
 * A written row holds, for each nope value x, the e4m3fn code of x / scale
 * (f32, correctly rounded division), clamped to [-448, 448] and rounded to
 * nearest even; then the d_rope bf16 values copied unchanged. Two kernels
 * (amax, encode) on hip_stream; no atomics, deterministic. Host checks as for
 * the decode; a non-finite or non-positive given scale and NaN inputs give
 * unspecified codes. */
MLA_API size_t mla_fp8_quantize_kv_workspace_size(void);
MLA_API int32_t mla_fp8_quantize_kv(int32_t num_tokens, int32_t d_rope, int32_t num_pages, const void* ckv,
                                    const void* k_rope, const int32_t* slot_mapping, void* kv_cache,
                                    float* k_scale, float* v_scale, int32_t compute_scale, void* workspace,
                                    size_t workspace_bytes, void* hip_stream);

/* Static description of a status code. Never NULL. The codes follow the
 * pages' failure conventions: an F8 cache without its scales fails loudly as
 * a bad parameter rather than being read unscaled (InfiniCore PR #1568, the
 * commit that makes a scale-less F8 cache fail with Bad Parameter), and a
 * configuration the library does not implement is refused with its own code
 * rather than misread (InfiniCore PR #1568, the backends commit returning
 * NOT_IMPLEMENTED for F8 caches; ROCm/aiter PR #6199, the foreign-encoding
 * refusal). */
MLA_API const char* mla_fp8_status_string(int32_t status);

/* --- test and measurement exports (device pointers, caller's stream) --- */

/* The decode (arguments as for mla_fp8_decode) with an internal kernel
 * variant forced, so that tests can compare the variants on the same inputs:
 *   MLA_VARIANT_GATHER_V    V^T operands by byte gathers instead of the
 *                           transposing LDS reads
 *   MLA_VARIANT_ROWS        fp8 dots: the row-block kernel (P.V split by row
 *                           block) instead of the default
 *   MLA_VARIANT_DV_SPLIT    fp8 dots: the four-wave dv-split kernel instead of
 *                           the default
 * 0 is the production choice. Unknown bits are MLA_ERR_SHAPE. */
#define MLA_VARIANT_GATHER_V 1
#define MLA_VARIANT_ROWS 2
#define MLA_VARIANT_DV_SPLIT 4
MLA_API int32_t mla_fp8_debug_decode_variant(const mla_params* p, const void* q, const void* kv_cache,
                                             const int32_t* block_table, const int32_t* seq_lens,
                                             const float* k_scale, const float* v_scale,
                                             int32_t num_splits, void* out, float* lse,
                                             const int32_t* indices, void* workspace,
                                             size_t workspace_bytes, int32_t variant, void* hip_stream);

/* Decodes n e4m3fn bytes with the same device routines the decode kernels
 * use: to f32 (out_f32, may be NULL) and to bf16 bits (out_bf16, may be NULL). */
MLA_API int32_t mla_fp8_debug_decode_e4m3fn(const uint8_t* codes, float* out_f32,
                                            uint16_t* out_bf16, int32_t n, void* hip_stream);

/* The fp8-dot path's transcoding of an e4m3fnuz cache byte to the e4m3fn
 * code of the same value (rounded to nearest even below 2^-6, 0x80 to 0x80;
 * see the kv_dtype codes) on n bytes. */
MLA_API int32_t mla_fp8_debug_fnuz_to_e4m3fn(const uint8_t* codes, uint8_t* out, int32_t n, void* hip_stream);

/* Runs the fp8-dot path's query quantization on `rows` bf16 rows of length
 * row_len (the first 512 entries of each row are quantized): writes 512 codes
 * per row and the power-of-two exponent e per row (q ~ code * 2^e). The
 * decode kernels quantize with two lane layouts (a row per lane quad, or half
 * a row per lane); the codes written are the first's, and a row on which the
 * second disagrees reports e = INT32_MIN. */
MLA_API int32_t mla_fp8_debug_quantize_q(const void* q, int32_t rows, int32_t row_len,
                                         uint8_t* codes, int32_t* exps, void* hip_stream);

/* Copies, through the decode kernel's paged gather (global -> LDS -> global),
 * the first seq_len rows of every sequence into dense_out
 * [batch, max_pages_per_seq * 64, row_bytes]; rows at or past seq_len, and
 * rows of out-of-range pages, come back as zeros. */
MLA_API int32_t mla_fp8_debug_gather(const mla_params* p, const void* kv_cache,
                                     const int32_t* block_table, const int32_t* seq_lens,
                                     void* dense_out, void* hip_stream);

/* The same check for the tile loader of the role-split fp8 kernel (its nope
 * bytes in 4 KiB dv slices): copies through that loader (global -> LDS ->
 * global) in the layout and with the zero-fill of mla_fp8_debug_gather. */
MLA_API int32_t mla_fp8_debug_gather_ws(const mla_params* p, const void* kv_cache,
                                        const int32_t* block_table, const int32_t* seq_lens,
                                        void* dense_out, void* hip_stream);

/* Matrix-core throughput probe: `blocks` workgroups of 256 threads, each wave
 * issuing 4 * iters independent 32x32 MFMAs (MLA_DOT_FP8: 32x32x64 fp8,
 * 131072 FLOP each; MLA_DOT_BF16: 32x32x16 bf16, 32768 FLOP each) with no
 * memory traffic; writes one f32 per thread to sink (blocks * 256 floats). */
MLA_API int32_t mla_fp8_bench_mfma(int32_t dot, int32_t iters, int32_t blocks, float* sink, void* hip_stream);

/* Streams `bytes` (a multiple of 16) of device memory and writes one f32 per
 * workgroup to sink (>= 65536 floats): an HBM read-bandwidth probe. */
MLA_API int32_t mla_fp8_bench_stream_read(const void* src, size_t bytes, float* sink,
                                          void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_FP8_H */

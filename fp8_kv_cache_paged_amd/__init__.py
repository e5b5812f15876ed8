"""Python binding of the MI355X FP8-KV paged MLA decode library.

Argument marshalling only: every step of the decode runs in the HIP kernels
of libmla_fp8.so, reached through its C ABI (include/mla_fp8.h) with ctypes.
torch supplies device memory and the current HIP stream. There is no CPU or
eager fallback: if the library is missing, every entry point raises.
"""

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libmla_fp8.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG_DIR), "include", "mla_fp8.h")

# status codes
MLA_OK = 0
MLA_ERR_NULL = 1
MLA_ERR_SHAPE = 2
MLA_ERR_DTYPE = 3
MLA_ERR_UNSUPPORTED = 4
MLA_ERR_WORKSPACE = 5
MLA_ERR_ALIGN = 6
MLA_ERR_HIP = 7
MLA_ERR_SCRATCH = 8

# fixed device scratch of mla_fp8_decode_noalloc, per GPU
MLA_NOALLOC_SCRATCH_BYTES = 64 << 20

# kv_dtype codes
MLA_KV_FP8_E4M3FN = 0
MLA_KV_UINT8 = 1
MLA_KV_FP8_E4M3FNUZ = 2
MLA_KV_FP8_E5M2 = 3
MLA_KV_INT8 = 4
MLA_KV_BF16 = 5

MLA_DOT_BF16 = 0
MLA_DOT_FP8 = 1
MLA_MAX_SPLITS = 64

# kernel variants of the test-only decode export
MLA_VARIANT_GATHER_V = 1
MLA_VARIANT_ROWS = 2
MLA_VARIANT_DV_SPLIT = 4

_KV_DTYPES = {
    torch.float8_e4m3fn: MLA_KV_FP8_E4M3FN,
    torch.uint8: MLA_KV_UINT8,
    torch.float8_e4m3fnuz: MLA_KV_FP8_E4M3FNUZ,
    torch.float8_e5m2: MLA_KV_FP8_E5M2,
    torch.int8: MLA_KV_INT8,
    torch.bfloat16: MLA_KV_BF16,
}


class MlaParams(ctypes.Structure):
    """Mirror of `mla_params` in include/mla_fp8.h."""
    _fields_ = [(name, ctypes.c_int32) for name in (
        "batch", "s_q", "h_q", "h_kv", "d_nope", "d_rope", "dv", "page_block", "num_pages",
        "max_pages_per_seq", "kv_dtype", "causal", "dot", "topk")] + [("softmax_scale", ctypes.c_float),
                                                                          ("kv_scale_per_token", ctypes.c_int32)]


class MlaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_string(status)})")


_lib = None


def library_available() -> bool:
    return os.path.exists(LIB_PATH)


def lib() -> ctypes.CDLL:
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "(or python -m fp8_kv_cache_paged_amd._build)")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(MlaParams)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.mla_fp8_validate.argtypes = [P]
        L.mla_fp8_validate.restype = i32
        L.mla_fp8_decode_resolve_splits.argtypes = [P, i32, i32]
        L.mla_fp8_decode_resolve_splits.restype = i32
        L.mla_fp8_decode_workspace_size.argtypes = [P, i32]
        L.mla_fp8_decode_workspace_size.restype = sz
        dec_args = [P, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, sz, vp]
        L.mla_fp8_decode.argtypes = dec_args
        L.mla_fp8_decode.restype = i32
        L.mla_fp8_decode_noalloc.argtypes = dec_args[:11] + [vp]
        L.mla_fp8_decode_noalloc.restype = i32
        L.mla_fp8_decode_partials.argtypes = dec_args
        L.mla_fp8_decode_partials.restype = i32
        L.mla_fp8_debug_decode_variant.argtypes = dec_args[:-1] + [i32, vp]
        L.mla_fp8_debug_decode_variant.restype = i32
        L.mla_fp8_status_string.argtypes = [i32]
        L.mla_fp8_status_string.restype = ctypes.c_char_p
        L.mla_fp8_debug_decode_e4m3fn.argtypes = [vp, vp, vp, i32, vp]
        L.mla_fp8_debug_decode_e4m3fn.restype = i32
        L.mla_fp8_debug_fnuz_to_e4m3fn.argtypes = [vp, vp, i32, vp]
        L.mla_fp8_debug_fnuz_to_e4m3fn.restype = i32
        L.mla_fp8_debug_quantize_q.argtypes = [vp, i32, i32, vp, vp, vp]
        L.mla_fp8_debug_quantize_q.restype = i32
        L.mla_fp8_debug_gather.argtypes = [P, vp, vp, vp, vp, vp]
        L.mla_fp8_debug_gather.restype = i32
        L.mla_fp8_debug_gather_ws.argtypes = [P, vp, vp, vp, vp, vp]
        L.mla_fp8_debug_gather_ws.restype = i32
        L.mla_fp8_bench_stream_read.argtypes = [vp, sz, vp, vp]
        L.mla_fp8_bench_stream_read.restype = i32
        L.mla_fp8_bench_mfma.argtypes = [i32, i32, i32, vp, vp]
        L.mla_fp8_bench_mfma.restype = i32
        L.mla_fp8_quantize_kv_workspace_size.argtypes = []
        L.mla_fp8_quantize_kv_workspace_size.restype = sz
        L.mla_fp8_quantize_kv.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp, vp, i32, vp, sz, vp]
        L.mla_fp8_quantize_kv.restype = i32
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().mla_fp8_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != MLA_OK:
        raise MlaError(status, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def make_params(*, batch: int, s_q: int, h_q: int, d_nope: int = 512, d_rope: int = 64,
                num_pages: int, max_pages_per_seq: int, kv_dtype=torch.uint8, causal: bool = True,
                dot: str = "fp8", topk: int = 0, softmax_scale: float = 0.0, h_kv: int = 1,
                page_block: int = 64, dv: Optional[int] = None, per_token_scales: bool = False) -> MlaParams:
    code = kv_dtype if isinstance(kv_dtype, int) else _KV_DTYPES.get(kv_dtype, 99)
    return MlaParams(batch, s_q, h_q, h_kv, d_nope, d_rope, d_nope if dv is None else dv, page_block,
                     num_pages, max_pages_per_seq, code, int(bool(causal)),
                     MLA_DOT_FP8 if dot == "fp8" else MLA_DOT_BF16, topk, float(softmax_scale),
                     int(bool(per_token_scales)))


def validate(params: MlaParams) -> int:
    return lib().mla_fp8_validate(ctypes.byref(params))


def resolve_splits(params: MlaParams, num_splits: int, cu_count: int) -> int:
    return lib().mla_fp8_decode_resolve_splits(ctypes.byref(params), int(num_splits), int(cu_count))


def workspace_size(params: MlaParams, splits: int) -> int:
    return lib().mla_fp8_decode_workspace_size(ctypes.byref(params), int(splits))


def cu_count(device=None) -> int:
    return torch.cuda.get_device_properties(device if device is not None else torch.cuda.current_device()).multi_processor_count


def params_for(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor, *, causal: bool = True,
               dot: str = "fp8", indices: Optional[torch.Tensor] = None, softmax_scale: float = 0.0,
               per_token_scales: bool = False) -> MlaParams:
    """mla_params describing the given tensors (layouts as in include/mla_fp8.h)."""
    b, s_q, h_q, d = q.shape
    row_bytes = kv_cache.shape[-1] * kv_cache.element_size()
    d_nope = 512
    d_rope = (row_bytes - d_nope) // 2
    if kv_cache.dim() == 4:
        h_kv = kv_cache.shape[2]
    else:
        h_kv = 1
    return make_params(batch=b, s_q=s_q, h_q=h_q, d_nope=d_nope, d_rope=d_rope, num_pages=kv_cache.shape[0],
                       max_pages_per_seq=block_table.shape[1], kv_dtype=kv_cache.dtype, causal=causal,
                       dot=dot, topk=0 if indices is None else indices.shape[-1],
                       softmax_scale=softmax_scale, h_kv=h_kv, page_block=kv_cache.shape[1],
                       dv=d_nope if d == d_nope + d_rope else -1, per_token_scales=per_token_scales)


def decode(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
           k_scale: torch.Tensor, v_scale: torch.Tensor, *, num_splits: int = 0, dot: str = "fp8",
           causal: bool = True, softmax_scale: float = 0.0, indices: Optional[torch.Tensor] = None,
           out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None, stream=None,
           partials_only: bool = False, per_token_scales: bool = False,
           variant: int = 0) -> Tuple[torch.Tensor, torch.Tensor]:
    """MLA decode over the paged fp8 cache; returns (out bf16 [b,s_q,h_q,512], lse f32 [b,s_q,h_q]).

    q bf16 [b, s_q, h_q, 576|512]; kv_cache uint8/float8_e4m3fn [pages, 64, (1,) 640|512];
    block_table, seq_lens int32; k_scale, v_scale f32 device tensors of one element;
    indices int32 [b, s_q, topk] selects the sparse variant. ``variant`` (tests
    only) forces an internal kernel variant, MLA_VARIANT_* bits.
    """
    p = params_for(q, kv_cache, block_table, causal=causal, dot=dot, indices=indices,
                   softmax_scale=softmax_scale, per_token_scales=per_token_scales)
    b, s_q, h_q, _ = q.shape
    if out is None:
        out = torch.empty((b, s_q, h_q, 512), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((b, s_q, h_q), dtype=torch.float32, device=q.device)
    L = lib()
    splits = num_splits
    if splits == 0:
        splits = L.mla_fp8_decode_resolve_splits(ctypes.byref(p), 0, cu_count(q.device))
        if splits < 0:
            _check(-splits, "mla_fp8_decode_resolve_splits")
    need = L.mla_fp8_decode_workspace_size(ctypes.byref(p), splits) if splits > 0 else 0
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    args = (ctypes.byref(p), _ptr(q), _ptr(kv_cache), _ptr(block_table), _ptr(seq_lens), _ptr(k_scale),
            _ptr(v_scale), int(splits), _ptr(out), _ptr(lse), _ptr(indices), _ptr(workspace),
            0 if workspace is None else workspace.numel() * workspace.element_size())
    if variant:
        if partials_only:
            raise ValueError("variant and partials_only cannot be combined")
        st = L.mla_fp8_debug_decode_variant(*args, int(variant), _stream(stream))
    else:
        fn = L.mla_fp8_decode_partials if partials_only else L.mla_fp8_decode
        st = fn(*args, _stream(stream))
    _check(st, "mla_fp8_decode")
    return out, lse


def decode_noalloc(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
                   k_scale: torch.Tensor, v_scale: torch.Tensor, out: torch.Tensor, lse: torch.Tensor, *,
                   num_splits: int = 0, dot: str = "fp8", causal: bool = True, softmax_scale: float = 0.0,
                   indices: Optional[torch.Tensor] = None, stream=None,
                   per_token_scales: bool = False) -> Tuple[torch.Tensor, torch.Tensor]:
    """mla_fp8_decode_noalloc: the decode with its split partials in the library's fixed
    per-GPU scratch (MLA_NOALLOC_SCRATCH_BYTES) instead of a workspace. The caller
    passes `out` (bf16 [b, s_q, h_q, 512]) and `lse` (f32 [b, s_q, h_q]); nothing is
    allocated. Calls that overlap on one GPU race on the scratch."""
    p = params_for(q, kv_cache, block_table, causal=causal, dot=dot, indices=indices,
                   softmax_scale=softmax_scale, per_token_scales=per_token_scales)
    st = lib().mla_fp8_decode_noalloc(ctypes.byref(p), _ptr(q), _ptr(kv_cache), _ptr(block_table),
                                      _ptr(seq_lens), _ptr(k_scale), _ptr(v_scale), int(num_splits), _ptr(out),
                                      _ptr(lse), _ptr(indices), _stream(stream))
    _check(st, "mla_fp8_decode_noalloc")
    return out, lse


def debug_decode_e4m3fn(codes: torch.Tensor, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Device decode of e4m3fn bytes (uint8 tensor) -> (f32 values, bf16 bit patterns as int16)."""
    n = codes.numel()
    f = torch.empty(n, dtype=torch.float32, device=codes.device)
    bb = torch.empty(n, dtype=torch.int16, device=codes.device)
    _check(lib().mla_fp8_debug_decode_e4m3fn(_ptr(codes), _ptr(f), _ptr(bb), n, _stream(stream)),
           "mla_fp8_debug_decode_e4m3fn")
    return f, bb


def debug_fnuz_to_e4m3fn(codes: torch.Tensor, stream=None) -> torch.Tensor:
    """The fp8-dot path's e4m3fnuz -> e4m3fn byte transcoding on a uint8 device tensor."""
    out = torch.empty_like(codes)
    _check(lib().mla_fp8_debug_fnuz_to_e4m3fn(_ptr(codes), _ptr(out), codes.numel(), _stream(stream)),
           "mla_fp8_debug_fnuz_to_e4m3fn")
    return out


def debug_quantize_q(q: torch.Tensor, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """The fp8-dot path's per-row query quantization: q bf16 [..., D>=512] -> (codes uint8 [..., 512], exps int32 [...])."""
    rows = q.numel() // q.shape[-1]
    codes = torch.empty((*q.shape[:-1], 512), dtype=torch.uint8, device=q.device)
    exps = torch.empty(q.shape[:-1], dtype=torch.int32, device=q.device)
    _check(lib().mla_fp8_debug_quantize_q(_ptr(q), rows, q.shape[-1], _ptr(codes), _ptr(exps), _stream(stream)),
           "mla_fp8_debug_quantize_q")
    return codes, exps


def debug_gather(kv_cache: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
                 stream=None, loader: str = "dense") -> torch.Tensor:
    """Dense copy [b, max_pages*64, row_bytes] of the cache rows through the decode's paged gather
    (loader "dense": the tile loader of mla_decode.hip's kernels; "ws": the sliced loader of the
    role-split fp8 kernel)."""
    row_bytes = kv_cache.shape[-1] * kv_cache.element_size()
    d_rope = (row_bytes - 512) // 2
    b, mp = block_table.shape
    p = make_params(batch=b, s_q=1, h_q=1, d_rope=d_rope, num_pages=kv_cache.shape[0], max_pages_per_seq=mp,
                    kv_dtype=kv_cache.dtype)
    dense = torch.empty((b, mp * 64, row_bytes), dtype=torch.uint8, device=kv_cache.device)
    fn = lib().mla_fp8_debug_gather_ws if loader == "ws" else lib().mla_fp8_debug_gather
    _check(fn(ctypes.byref(p), _ptr(kv_cache), _ptr(block_table), _ptr(seq_lens), _ptr(dense), _stream(stream)),
           "mla_fp8_debug_gather")
    return dense


def stream_read(src: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """HBM read-bandwidth probe: streams all of `src` (sink: f32 device tensor of >= 65536 elements)."""
    nbytes = src.numel() * src.element_size()
    _check(lib().mla_fp8_bench_stream_read(_ptr(src), nbytes - nbytes % 16, _ptr(sink), _stream(stream)),
           "mla_fp8_bench_stream_read")


def mfma_probe(dot: str, iters: int, blocks: int, sink: torch.Tensor, stream=None) -> int:
    """Matrix-core throughput probe: blocks x 4 waves, each issuing 4 * iters
    independent 32x32 MFMAs (dot "fp8": 32x32x64, "bf16": 32x32x16); sink: f32
    device tensor of >= blocks * 256 elements. Returns the FLOP it executes."""
    if dot not in ("fp8", "bf16"):
        raise ValueError(f"dot must be 'fp8' or 'bf16', got {dot!r}")
    if sink.dtype != torch.float32 or not sink.is_cuda or sink.numel() < blocks * 256:
        raise ValueError("sink must be a float32 device tensor of >= blocks * 256 elements")
    code = MLA_DOT_FP8 if dot == "fp8" else MLA_DOT_BF16
    _check(lib().mla_fp8_bench_mfma(code, iters, blocks, _ptr(sink), _stream(stream)), "mla_fp8_bench_mfma")
    return blocks * 4 * iters * 4 * (131072 if dot == "fp8" else 32768)


def quantize_kv(ckv: torch.Tensor, k_rope: Optional[torch.Tensor], slot_mapping: torch.Tensor,
                kv_cache: torch.Tensor, k_scale: torch.Tensor, v_scale: torch.Tensor, *,
                compute_scale=True, workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Quantize-on-write of new latent rows into the paged cache (in place).

    ckv bf16 [n, 512], k_rope bf16 [n, 64] or None, slot_mapping int32 [n]
    (page * 64 + slot; negative or out of range = skipped), kv_cache uint8
    [pages, 64, 1, 512 + 2 d_rope], k_scale / v_scale f32 [1] on the device.
    compute_scale: True (or 1) stores amax / 448 of the written rows to both
    scales; "per_token" (or 2) gives every written row its own scale, stored
    at its cache row in k_scale / v_scale f32 [pages, 64]; False encodes with
    k_scale as given.
    """
    mode = 2 if compute_scale == "per_token" or compute_scale == 2 else (1 if compute_scale else 0)
    n = int(slot_mapping.shape[0])
    d_rope = 0 if k_rope is None else int(k_rope.shape[1])
    if ckv.dtype != torch.bfloat16 or ckv.dim() != 2 or ckv.shape[1] != 512 or ckv.shape[0] != n:
        raise ValueError("ckv must be bf16 [n, 512] with n = len(slot_mapping)")
    if k_rope is not None and (k_rope.dtype != torch.bfloat16 or k_rope.shape[0] != n):
        raise ValueError("k_rope must be bf16 [n, d_rope]")
    if kv_cache.dim() != 4 or kv_cache.shape[1] != 64 or kv_cache.shape[3] != 512 + 2 * d_rope:
        raise ValueError("kv_cache must be [pages, 64, 1, 512 + 2 * d_rope]")
    for t in (ckv, k_rope, slot_mapping, kv_cache):
        if t is not None and not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    if mode == 1 and workspace is None:
        workspace = torch.empty(lib().mla_fp8_quantize_kv_workspace_size(), dtype=torch.uint8,
                                device=kv_cache.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().mla_fp8_quantize_kv(n, d_rope, int(kv_cache.shape[0]), _ptr(ckv), _ptr(k_rope),
                                     _ptr(slot_mapping), _ptr(kv_cache), _ptr(k_scale), _ptr(v_scale),
                                     mode, _ptr(workspace), ws_bytes, _stream(stream)),
           "mla_fp8_quantize_kv")

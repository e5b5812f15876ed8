"""CPU oracle for FP8-KV paged MLA decode.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It is a plain, slow, obviously
correct float64 implementation written from the source pages, and it shares no
code, headers, tables or helpers with the HIP library in
``fp8_kv_cache_paged_amd/``.

Modules
  fp8   OCP e4m3fn codec from the format definition, bf16 helpers.
  attn  attention over the dequantized paged cache (dense and sparse), the
        split-KV partial form and its log-sum-exp combine, and the per-row
        power-of-two query quantization the fp8-dot path uses.
  cache quantize-on-write of new latent rows into the paged cache
        (per-tensor amax / 448 scale, e4m3fn encode, rope copy).

Parity status (pins live in tests/test_oracle_*.py):
  fp8.decode_e4m3fn, fp8.encode_e4m3fn, fp8.bf16 helpers  -- pinned
  attn.mla_decode, attn.split_partials, attn.combine       -- pinned
  attn.quantize_q_rows                                      -- pinned
  cache.kv_scale, cache.encode_rows, cache.quantize_kv      -- pinned
  The GPU's rounding of Q' and of P inside the fp8-dot path is not modelled
  here; for that path only the tolerance bound is checked ("parity unpinned"
  beyond the bound), see attn.mla_decode's docstring.
"""

from . import fp8, attn, cache  # noqa: F401

"""Byte-level paths of the HIP library, bit-exact against the oracle: the
e4m3fn decode of all 256 codes, the fp8-dot query quantization, and the paged
gather (global -> LDS -> global)."""

import numpy as np
import pytest
import torch

import fp8_kv_cache_paged_amd as mla
import workloads
from oracle import attn, fp8

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def test_decode_all_256_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).to(DEV)
    f, bb = mla.debug_decode_e4m3fn(codes)
    f = f.cpu().numpy().astype(np.float64)
    ref = fp8.E4M3FN_TABLE
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(f), nan)
    assert np.array_equal(f[~nan], ref[~nan])
    assert np.array_equal(np.signbit(f[~nan]), np.signbit(ref[~nan]))
    bits = bb.cpu().numpy().view(np.uint16)
    ref_bits = fp8.f32_to_bf16_bits(ref[~nan].astype(np.float32))
    assert np.array_equal(bits[~nan], ref_bits)


def test_decode_odd_length_tail():
    codes = torch.tensor([0x38, 0x7E, 0x01, 0x80, 0x49], dtype=torch.uint8, device=DEV)
    f, _ = mla.debug_decode_e4m3fn(codes)
    assert f.cpu().tolist() == [1.0, 448.0, 2.0 ** -9, -0.0, 4.5]


@pytest.mark.parametrize("shape", [(1, 1, 16, 576), (2, 2, 64, 576), (3, 2, 16, 512)])
def test_query_quantization_matches_oracle(shape):
    w = workloads.make("tiny", batch=shape[0], s_q=shape[1], h_q=shape[2],
                       d_rope=shape[3] - 512, seq_len=64, seed=sum(shape))
    qb = w.q_bits.copy()
    flat = qb.reshape(-1, shape[3])
    flat[0, :512] = 0                                           # an all-zero row
    flat[-1, :512] = fp8.f32_to_bf16_bits(np.float32(1e-30))   # a tiny row (large 2^-e)
    if flat.shape[0] > 2:
        flat[1, :512] = fp8.f32_to_bf16_bits(np.float32(448.0))
    if flat.shape[0] > 4:
        # amax 1e-37: 2^-e lies beyond float32's range; bf16 subnormals
        flat[2, :512] = fp8.f32_to_bf16_bits(np.linspace(-1e-37, 1e-37, 512, dtype=np.float32))
        flat[3, :512] = np.arange(512, dtype=np.uint16) % 0x7F + 1
    q = torch.from_numpy(qb.view(np.int16)).view(torch.bfloat16).to(DEV)
    codes, exps = mla.debug_quantize_q(q)
    ref_codes, ref_exps = attn.quantize_q_rows(fp8.bf16_bits_to_f64(qb)[..., :512])
    assert np.array_equal(exps.cpu().numpy(), ref_exps)
    assert np.array_equal(codes.cpu().numpy(), ref_codes)
    # the decode on the same rows stays finite (the tiny rows give uniform weights)
    if flat.shape[0] > 4:
        assert np.all(np.abs(ref_exps.reshape(-1)[2:4]) > 127)


@pytest.mark.parametrize("name,kw", [("tiny", {}), ("mtp", {"batch": 3, "seq_len": [8196, 65, 0]}),
                                     ("sparse", {"batch": 2, "seq_len": 4096, "topk": 64}),
                                     ("tiny", {"batch": 2, "seq_len": [1, 127]})])
@pytest.mark.parametrize("loader", ["dense", "ws"])
def test_paged_gather_is_bytewise_exact(name, kw, loader):
    w = workloads.make(name, **kw)
    kv = torch.from_numpy(w.kv_cache).to(DEV)
    dense = mla.debug_gather(kv, torch.from_numpy(w.block_table).to(DEV),
                             torch.from_numpy(w.seq_lens).to(DEV), loader=loader).cpu().numpy()
    b, mp = w.block_table.shape
    for bi in range(b):
        sk = int(w.seq_lens[bi])
        pos = np.arange(sk)
        ref = w.kv_cache[w.block_table[bi, pos // 64], pos % 64]
        assert np.array_equal(dense[bi, :sk], ref), f"sequence {bi}"
        assert np.all(dense[bi, sk:] == 0), "rows past seq_len must come back zero-filled"

"""Pins of the oracle's e4m3fn codec and bf16 helpers (CPU only)."""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import fp8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)


def _anchors():
    with open(os.path.join(GOLDEN, "e4m3fn_anchors.json")) as f:
        return json.load(f)


def test_definition_anchor_codes():
    a = _anchors()["definition_anchors"]
    for code, val in a["codes"].items():
        got = fp8.E4M3FN_TABLE[int(code, 16)]
        assert got == val and math.copysign(1, got) == math.copysign(1, val), code
    for code in a["nan_codes"]:
        assert math.isnan(fp8.E4M3FN_TABLE[int(code, 16)])
    assert int(np.isnan(fp8.E4M3FN_TABLE).sum()) == 2


def test_page_facts():
    facts = _anchors()["page_facts"]
    assert np.nanmax(fp8.E4M3FN_TABLE) == facts[0]["value"] == fp8.E4M3FN_MAX
    # fnuz's 240 is a finite e4m3fn value but not the top of the range here
    assert facts[3]["fnuz_max"] in fp8.E4M3FN_TABLE and facts[3]["fnuz_max"] < fp8.E4M3FN_MAX


def test_bf16_bit_placement_second_derivation():
    """InfiniCore's bit-placement identity, applied to all 254 finite codes."""
    factor = _anchors()["page_facts"][1]["bf16_factor_log2"]
    c = FINITE.astype(np.uint32)
    bits = (((c & 0x80) << 8) | ((c & 0x7F) << 4)).astype(np.uint16)
    placed = fp8.bf16_bits_to_f64(bits)
    np.testing.assert_array_equal(placed * 2.0 ** (-factor), fp8.E4M3FN_TABLE[FINITE])
    np.testing.assert_array_equal(fp8.e4m3fn_by_bf16_bit_placement(FINITE), fp8.E4M3FN_TABLE[FINITE])


def test_f16_bit_placement_third_derivation():
    factor = _anchors()["page_facts"][2]["f16_factor_log2"]
    c = FINITE.astype(np.uint32)
    bits = (((c & 0x80) << 8) | ((c & 0x7F) << 7)).astype(np.uint16)
    placed = bits.view(np.float16).astype(np.float64)
    np.testing.assert_array_equal(placed * 2.0 ** (-factor), fp8.E4M3FN_TABLE[FINITE])


def test_decode_matches_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = fp8.decode_e4m3fn(np.arange(256, dtype=np.uint8))
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])
    np.testing.assert_array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


def test_values_strictly_increase_over_positive_codes():
    v = fp8.E4M3FN_TABLE[:0x7F]
    assert np.all(np.diff(v) > 0)
    np.testing.assert_array_equal(fp8.E4M3FN_TABLE[0x80:0xFF], -v)


def test_encode_roundtrip_all_finite_codes():
    np.testing.assert_array_equal(fp8.encode_e4m3fn(fp8.E4M3FN_TABLE[FINITE]), FINITE)


def test_encode_ties_go_to_even_mantissa():
    v = fp8.E4M3FN_TABLE[:0x7F]
    mids = (v[:-1] + v[1:]) / 2
    got = fp8.encode_e4m3fn(mids).astype(np.int64)
    lo = np.arange(0x7E)
    expect = np.where(lo % 2 == 0, lo, lo + 1)
    np.testing.assert_array_equal(got, expect)
    # just off the midpoint goes to the nearer side
    np.testing.assert_array_equal(fp8.encode_e4m3fn(np.nextafter(mids, 0)), lo)
    np.testing.assert_array_equal(fp8.encode_e4m3fn(np.nextafter(mids, 1e9)), lo + 1)


def test_encode_saturates_and_keeps_sign():
    got = fp8.encode_e4m3fn(np.array([448.0, 449.0, 500.0, 1e30, -1e30, -0.0, -1e-9, 1e-9, np.nan]))
    np.testing.assert_array_equal(got, [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x80, 0x80, 0x00, 0x7F])


def test_encode_matches_torch_cast_in_range():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(100000) * 40, rng.standard_normal(10000) * 1e-3,
                        rng.uniform(-448, 448, 10000)]).astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(fp8.encode_e4m3fn(x), ref)


def test_bf16_helpers_match_torch():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(50000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1e-40, 3.4e38, np.inf, -np.inf], dtype=np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(fp8.f32_to_bf16_bits(x), ref)
    back = torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(fp8.bf16_bits_to_f64(ref), back)


@pytest.mark.parametrize("code", [0x01, 0x07, 0x08, 0x38, 0x7E])
def test_every_e4m3fn_value_is_exact_in_bf16(code):
    """The bf16-dot path converts cache bytes to bf16; that must be exact."""
    v = np.float32(fp8.E4M3FN_TABLE[code])
    assert fp8.bf16_bits_to_f64(fp8.f32_to_bf16_bits(v)) == v
    allv = fp8.E4M3FN_TABLE[FINITE].astype(np.float32)
    np.testing.assert_array_equal(fp8.bf16_bits_to_f64(fp8.f32_to_bf16_bits(allv)), allv)


# ---- e4m3fnuz (gfx942's encoding) ------------------------------------------


def test_fnuz_page_fact_largest_value_240():
    # ROCm/aiter PR #6199 quantizes to 240 for gfx942's fnuz code
    facts = _anchors()["page_facts"]
    assert np.nanmax(fp8.E4M3FNUZ_TABLE) == facts[3]["fnuz_max"] == fp8.E4M3FNUZ_MAX
    assert fp8.E4M3FNUZ_TABLE[0x7F] == 240.0 and fp8.E4M3FNUZ_TABLE[0xFF] == -240.0


def test_fnuz_decode_matches_torch_float8_e4m3fnuz():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fnuz).to(torch.float64).numpy()
    got = fp8.decode_e4m3fnuz(np.arange(256, dtype=np.uint8))
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])
    np.testing.assert_array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


def test_fnuz_special_codes():
    t = fp8.E4M3FNUZ_TABLE
    assert int(np.isnan(t).sum()) == 1 and math.isnan(t[0x80])   # the only NaN
    assert int((t == 0).sum()) == 1 and not np.signbit(t[0x00])   # no negative zero
    assert not np.isinf(t).any()
    assert t[0x01] == 2.0 ** -10                                   # smallest subnormal


def test_fnuz_is_half_of_fn_away_from_the_special_codes():
    # exponent bias 8 instead of 7 with the same bit fields: each code other
    # than 0x80 (fnuz NaN, fn -0) and 0x7F / 0xFF (fnuz +-240, fn NaN) means
    # half its e4m3fn value
    c = np.array([x for x in range(256) if x not in (0x7F, 0x80, 0xFF)], dtype=np.uint8)
    np.testing.assert_array_equal(fp8.E4M3FNUZ_TABLE[c] * 2.0, fp8.E4M3FN_TABLE[c])


def test_kv_code_dispatch():
    c = np.arange(256, dtype=np.uint8)
    assert np.array_equal(fp8.decode_kv_codes(c, "e4m3fn"), fp8.E4M3FN_TABLE, equal_nan=True)
    assert np.array_equal(fp8.decode_kv_codes(c, "e4m3fnuz"), fp8.E4M3FNUZ_TABLE, equal_nan=True)
    with pytest.raises(ValueError):
        fp8.decode_kv_codes(c, "e5m2")


def test_fnuz_as_e4m3fn_keeps_values_from_2_pow_minus_6_up():
    # every fnuz magnitude in [2**-6, 240] is an e4m3fn value: the transcoding
    # keeps it; 240 (0x7F) is e4m3fn 0x77, one exponent lower in the code
    codes = np.arange(256, dtype=np.uint8)
    out = fp8.fnuz_as_e4m3fn(codes)
    v_in = fp8.decode_e4m3fnuz(codes)
    v_out = fp8.decode_e4m3fn(out)
    big = (codes & 0x7F) >= 0x10
    assert np.array_equal(v_out[big], v_in[big])
    assert out[0x7F] == 0x77 and out[0xFF] == 0xF7 and fp8.decode_e4m3fn(np.uint8(0x77)) == 240.0
    # and the code is the fnuz code 8 lower (bias 8 against 7, same mantissa)
    assert np.array_equal(out[big], codes[big] - 8)


def test_fnuz_as_e4m3fn_rounds_the_smallest_magnitudes_to_even():
    # fnuz exponent field 0 or 1: k * 2**-10 (k = 0..15); e4m3fn subnormals are
    # m * 2**-9, then 2**-6: k rounds to 2 m with ties to the even mantissa
    for k in range(16):
        out = int(fp8.fnuz_as_e4m3fn(np.uint8(k)))
        exact = k * 2.0 ** -10
        got = float(fp8.decode_e4m3fn(np.uint8(out)))
        assert abs(got - exact) <= 2.0 ** -10
        if k % 2 == 0:
            assert got == exact
        else:
            assert (out & 1) == 0, (k, out)     # the tie went to the even code
    assert fp8.fnuz_as_e4m3fn(np.uint8(15)) == 0x08      # 15 * 2**-10 -> 2**-6, the smallest normal
    assert fp8.fnuz_as_e4m3fn(np.uint8(0x89)) == 0x84    # sign kept: -9 * 2**-10 -> -4 * 2**-9
    assert fp8.fnuz_as_e4m3fn(np.uint8(0x80)) == 0x80    # fnuz NaN read as zero


def test_fnuz_as_e4m3fn_against_torch_casts():
    # an outside check: torch's fnuz decode, then torch's e4m3fn cast (RNE)
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    vals = codes.view(torch.float8_e4m3fnuz).to(torch.float32)
    vals = torch.where(torch.isnan(vals), torch.tensor(-0.0), vals)
    ref = vals.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fp8.fnuz_as_e4m3fn(np.arange(256, dtype=np.uint8)), ref)

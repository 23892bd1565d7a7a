"""Pins of the oracle's number formats against torch's own casts (library routines) and against
values fixed by the formats' definitions (bf16; OCP 8-bit floating point E4M3FN).
"""
import numpy as np
import pytest
import torch

from oracle import codecs


def _normal_fp32_patterns():
    """Every bf16-normal high half (sign, exponent 1..254, 7 mantissa bits) combined with low halves
    that cover every rounding case: exact, just above/below the midpoint, the midpoint, max."""
    hi = np.arange(1 << 16, dtype=np.uint32)
    exp = (hi >> 7) & 0xFF
    hi = hi[(exp >= 1) & (exp <= 253)]               # keep clear of overflow on round-up
    rng = np.random.default_rng(5)
    lows = np.concatenate([np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000],
                                    dtype=np.uint32),
                           rng.integers(0, 1 << 16, size=24).astype(np.uint32)])
    return ((hi[:, None] << 16) | lows[None, :]).ravel()


def test_bf16_round_matches_torch_cast_on_fp32_patterns():
    bits = _normal_fp32_patterns()
    f32 = bits.view(np.float32)
    mine = codecs.bf16_round(f32.astype(np.float64))
    ref = torch.from_numpy(f32.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(mine, ref)


def test_bf16_round_float64_midpoints():
    """Exact float64 midpoints tie to even; one float64 ulp off the midpoint rounds away from it.
    Rounding is sign-symmetric, so the negated cases must mirror the positive ones."""
    rng = np.random.default_rng(6)
    base = np.abs(codecs.bf16_round(rng.standard_normal(5000) * 10.0 ** rng.integers(-20, 20, 5000)))
    ulp = np.exp2(np.floor(np.log2(base)) - 7)
    mid = base + ulp / 2                                  # exact in float64
    up = base + ulp
    lower_is_even = ((base.view(np.uint64) >> np.uint64(45)) & np.uint64(1)) == 0
    for sgn in (1.0, -1.0):
        assert np.array_equal(codecs.bf16_round(sgn * mid), sgn * np.where(lower_is_even, base, up))
        assert np.array_equal(codecs.bf16_round(sgn * np.nextafter(mid, np.inf)), sgn * up)
        assert np.array_equal(codecs.bf16_round(sgn * np.nextafter(mid, 0)), sgn * base)


def test_bf16_round_rejects_out_of_range():
    for bad in [np.nan, np.inf, 1e-40, 1e39]:
        with pytest.raises(ValueError):
            codecs.bf16_round(np.array([bad]))
    assert codecs.bf16_round(np.array([0.0]))[0] == 0.0


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = codecs.e4m3_decode(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    assert np.array_equal(np.signbit(mine[ok]), np.signbit(ref[ok]))


def test_e4m3_definition_values():
    """Values fixed by the format: largest finite, smallest normal, smallest subnormal, NaN codes."""
    d = codecs.e4m3_decode(np.array([0x7E, 0x08, 0x01, 0x38, 0x7F, 0xFF, 0x80, 0xFE], dtype=np.uint8))
    assert d[0] == 448.0 and d[1] == 2.0 ** -6 and d[2] == 2.0 ** -9 and d[3] == 1.0
    assert np.isnan(d[4]) and np.isnan(d[5])
    assert d[6] == 0.0 and np.signbit(d[6]) and d[7] == -448.0


def test_e4m3_encode_matches_torch_in_range():
    """All midpoints between adjacent finite codes, points just off them, and a dense sweep."""
    vals = codecs.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))       # 0 .. 448 ascending
    mids = (vals[:-1] + vals[1:]) / 2
    pts = np.concatenate([vals, mids, np.nextafter(mids, 0), np.nextafter(mids, 1000),
                          np.linspace(0, 448, 200001)])
    pts = np.concatenate([pts, -pts]).astype(np.float32)
    mine = codecs.e4m3_encode(pts.astype(np.float64))
    ref = torch.from_numpy(pts.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mine, ref)


def test_e4m3_encode_saturates():
    c = codecs.e4m3_encode(np.array([448.0, 449.0, 463.9, 464.0, 1e9, -500.0, -1e30]))
    assert list(c) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]


def test_quant_rows_fp8_properties():
    rng = np.random.default_rng(7)
    rows = (rng.standard_normal((64, 2560)) * 3).astype(np.float32)
    rows = torch.from_numpy(rows).to(torch.bfloat16).to(torch.float32).numpy()
    codes, scale = codecs.quant_rows_fp8(rows)
    # the element of largest magnitude lands on +-448
    j = np.argmax(np.abs(rows), axis=1)
    top = codes[np.arange(64), j]
    assert np.all((top & 0x7F) == 0x7E)
    # dequantised values are within half a step of E4M3 (relative 2^-4 for normals)
    deq = codecs.e4m3_decode(codes) * scale[:, None].astype(np.float64)
    err = np.abs(deq - rows)
    bound = np.maximum(np.abs(rows) * 2.0 ** -4, scale[:, None] * 2.0 ** -10) * (1 + 1e-6)
    assert np.all(err <= bound)
    # scaling a row by a power of two scales the scale and keeps the codes
    codes2, scale2 = codecs.quant_rows_fp8(rows * np.float32(8.0))
    assert np.array_equal(codes, codes2) and np.array_equal(scale2, scale * np.float32(8.0))
    # zero rows
    codes0, scale0 = codecs.quant_rows_fp8(np.zeros((2, 16), dtype=np.float32))
    assert np.all(codes0 == 0) and np.all(scale0 == 1.0)


def test_quant_rows_fp8_exact_power_of_two_case():
    """amax = 448 * 2^-3 gives scale 2^-3 exactly, and values on the E4M3 grid encode exactly."""
    row = np.array([[56.0, -1.0, 0.5, 3.5, 0.0, -56.0, 2.0 ** -12]], dtype=np.float32)
    codes, scale = codecs.quant_rows_fp8(row)
    assert scale[0] == np.float32(0.125)
    assert list(codecs.e4m3_decode(codes[0])) == [448.0, -8.0, 4.0, 28.0, 0.0, -448.0, 2.0 ** -9]

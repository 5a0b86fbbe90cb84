"""Pins of the oracle's 8-bit float (OCP E4M3) row quantizer, from the
format's definition: special codes, the value table's structure, round trip,
ties to even, the scale rule and the error bound."""
import math

import numpy as np
import pytest

from oracle import fp8


def test_special_codes():
    assert fp8.e4m3_decode(0x7E) == 448.0                # S.1111.110: largest finite
    assert math.isnan(fp8.e4m3_decode(0x7F)) and math.isnan(fp8.e4m3_decode(0xFF))
    assert fp8.e4m3_decode(0x38) == 1.0                  # exponent field 7 = bias
    assert fp8.e4m3_decode(0x08) == 2.0 ** -6            # smallest normal
    assert fp8.e4m3_decode(0x07) == 7 * 2.0 ** -9        # largest subnormal
    assert fp8.e4m3_decode(0x01) == 2.0 ** -9            # smallest subnormal
    assert fp8.e4m3_decode(0x00) == 0.0 and math.copysign(1.0, fp8.e4m3_decode(0x80)) < 0
    assert fp8.e4m3_decode(0xB8) == -1.0
    assert fp8.e4m3_decode(0x70) == 128.0                # exponent field 14, mantissa 0
    assert fp8.e4m3_decode(0x77) == 240.0                # 1.875 * 2^7
    assert fp8.e4m3_decode(0x78) == 256.0                # exponent field 15


def test_value_table_structure():
    vals = [fp8.e4m3_decode(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(vals, vals[1:]))      # strictly increasing codes
    # inside each binade the 8 codes are equally spaced by 2^(E-10)
    for E in range(1, 16):
        codes = [c for c in range(0x7F) if (c >> 3) == E]
        steps = {fp8.e4m3_decode(b) - fp8.e4m3_decode(a) for a, b in zip(codes, codes[1:])}
        assert steps == {2.0 ** (E - 10)}
    assert len([v for v in vals if v > 0]) == 126


def test_round_trip_and_ties_to_even():
    for c in list(range(0x7F)) + list(range(0x80, 0xFF)):
        assert fp8.e4m3_encode(fp8.e4m3_decode(c)) == c
    # the midpoint of two neighbours goes to the even mantissa
    for c in range(0x7E):
        lo, hi = fp8.e4m3_decode(c), fp8.e4m3_decode(c + 1)
        got = fp8.e4m3_encode((lo + hi) / 2)
        assert got == (c if c % 2 == 0 else c + 1)
        assert fp8.e4m3_encode(lo + (hi - lo) * 0.49) == c
        assert fp8.e4m3_encode(lo + (hi - lo) * 0.51) == c + 1
    with pytest.raises(ValueError):
        fp8.e4m3_encode(449.0)


@pytest.mark.parametrize("amax", [448.0, 448.0 * 2 ** -20, 1.0, 3.5, 0.001, 1e4, 224.0, 224.0001])
def test_scale_rule(amax):
    e = fp8.row_scale_exponent(amax)
    assert amax <= 448.0 * 2.0 ** e
    assert amax > 448.0 * 2.0 ** (e - 1)                   # smallest such e


def test_quantize_row_error_bound():
    """Every element is within half a code spacing of its value; the largest
    element uses the top binade (no headroom is wasted)."""
    rng = np.random.default_rng(0)
    for scale in (1e-3, 0.3, 1.0, 57.0):
        c = rng.standard_normal(512) * scale
        codes, e = fp8.quantize_row(c)
        d = fp8.dequantize_row(codes, e)
        # spacing of the code grid at |c|: 2^(floor(log2|c| 2^-e) - 3) 2^e, subnormal floor 2^-9 2^e
        a = np.abs(c) * 2.0 ** -e
        spacing = np.where(a >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(a, 1e-300))) - 3),
                           2.0 ** -9) * 2.0 ** e
        assert np.all(np.abs(d - c) <= spacing / 2 * (1 + 1e-12))
        assert np.abs(d).max() > 224.0 * 2.0 ** e * 0.99 or np.abs(c).max() <= 224.0 * 2.0 ** e
    codes, e = fp8.quantize_row(np.zeros(8))
    assert e == 0 and not codes.any()


def test_array_encoder_is_the_scalar_definition():
    rng = np.random.default_rng(1)
    mids = [(fp8.e4m3_decode(c) + fp8.e4m3_decode(c + 1)) / 2 for c in range(0x7E)]
    x = np.concatenate([rng.uniform(-448, 448, 2000), rng.standard_normal(2000) * 0.01,
                        np.array(mids), -np.array(mids), [0.0, -0.0, 448.0, -448.0, 2.0 ** -10]])
    got = fp8.e4m3_encode_array(x)
    want = np.array([fp8.e4m3_encode(v) for v in x], dtype=np.uint8)
    assert np.array_equal(got, want)
    assert np.array_equal(fp8.dequantize_row(np.arange(256, dtype=np.uint8), 3)[:0x7F],
                          np.array([fp8.e4m3_decode(c) * 8.0 for c in range(0x7F)]))


def test_fp8_rows_quantizes_only_the_latent():
    """A hand-built row with d_c = 4 and a 2-wide rope block.  max|c| = 500
    needs e = 1 (448 < 500 <= 896); c * 2^-1 = (0.5, -1.75, 0.15, 250):
    0.5 and -1.75 are codes, 0.15 lies between 0.140625 and 0.15625 (spacing
    2^-6 in [1/8, 1/4)) and rounds up, 250 lies between 240 and 256 (spacing
    16 in [128, 256)) and rounds up.  The rope part comes back unchanged
    ("Multi-head Latent Attention and KV Cache Compression", section "Moving
    a trained MHA model over": it is the latent that is quantized further)."""
    row = np.array([[1.0, -3.5, 0.3, 500.0, 0.123456789, -7.7]])
    got = fp8.fp8_rows(row, 4)
    assert got[0, :4].tolist() == [1.0, -3.5, 0.3125, 512.0]
    assert got[0, 4:].tobytes() == row[0, 4:].tobytes()
    # a second row with a different scale leaves the first alone
    rows = np.vstack([row, [[0.001, 0.0, -0.002, 0.0015, 3.0, 4.0]]])
    got2 = fp8.fp8_rows(rows, 4)
    assert got2[0].tobytes() == got[0].tobytes()
    codes, e = fp8.quantize_row(rows[1, :4])
    assert got2[1, :4].tolist() == fp8.dequantize_row(codes, e).tolist()
    assert got2[1, 4:].tolist() == [3.0, 4.0]
    assert rows[0, 2] == 0.3   # the input is not modified in place

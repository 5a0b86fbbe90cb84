"""8-bit float (OCP E4M3) row quantization of the latent, plain Python/NumPy.

TEST INFRASTRUCTURE ONLY (see ``oracle/mla_oracle.py``).

Source: "Multi-head Latent Attention and KV Cache Compression" (jongkwan.dev),
section "Moving a trained MHA model over": the cached latent can be quantized
further, with scale correction; the pages name no format, so the reading
taken here is the OCP 8-bit float E4M3: 1 sign bit, 4
exponent bits with bias 7, 3 mantissa bits; exponent field 0 encodes
subnormals m * 2^-9; no infinities; only S.1111.111 is NaN, so the largest
finite magnitude is 1.75 * 2^8 = 448.  One power-of-two scale per row:
c ~= 2^e * code with e the smallest integer such that max|c| <= 448 * 2^e,
codes rounded to nearest, ties to even.
"""
from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(code: int) -> float:
    """Value of one 8-bit code (NaN for S.1111.111)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def _finite_magnitudes():
    """(value, code) for the 127 non-negative finite codes, ascending."""
    return [(e4m3_decode(c), c) for c in range(0x7F)]


_MAGS = _finite_magnitudes()


def e4m3_encode(x: float) -> int:
    """Nearest code to x (|x| <= 448), ties to the code with an even
    mantissa; the sign of zero is kept.  Written as a search over the
    finite codes so that it follows the definition, not bit tricks."""
    x = float(x)
    if not math.isfinite(x) or abs(x) > E4M3_MAX:
        raise ValueError("outside the E4M3 range")
    sign = 0x80 if math.copysign(1.0, x) < 0 else 0
    a = abs(x)
    best, best_code = None, None
    for v, c in _MAGS:
        d = abs(v - a)
        if best is None or d < best or (d == best and (c & 1) == 0):
            best, best_code = d, c
    return sign | best_code


_MAG_VALUES = np.array([v for v, _ in _MAGS])   # ascending; index = code


def e4m3_encode_array(x) -> np.ndarray:
    """e4m3_encode over an array: the two codes around |x| by a sorted
    search, the nearer one, ties to the even code, sign bit from x."""
    x = np.asarray(x, dtype=np.float64)
    if x.size and (not np.all(np.isfinite(x)) or np.abs(x).max() > E4M3_MAX):
        raise ValueError("outside the E4M3 range")
    a = np.abs(x)
    hi = np.minimum(np.searchsorted(_MAG_VALUES, a, side="left"), len(_MAG_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _MAG_VALUES[lo]
    dhi = _MAG_VALUES[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return code | (np.signbit(x).astype(np.uint8) << 7)


DECODE_TABLE = np.array([e4m3_decode(c) for c in range(256)])


def row_scale_exponent(amax: float) -> int:
    """Smallest integer e with amax <= 448 * 2^e (0 when amax is 0)."""
    if amax == 0.0:
        return 0
    e = math.ceil(math.log2(amax / E4M3_MAX))
    # guard the float log against an off-by-one at exact powers of two
    while amax > E4M3_MAX * 2.0 ** e:
        e += 1
    while amax <= E4M3_MAX * 2.0 ** (e - 1):
        e -= 1
    return e


def quantize_row(c) -> tuple[np.ndarray, int]:
    """Codes (uint8) and scale exponent of one latent row."""
    c = np.asarray(c, dtype=np.float64)
    e = row_scale_exponent(float(np.abs(c).max()) if c.size else 0.0)
    return e4m3_encode_array(c * 2.0 ** -e), e


def dequantize_row(codes, e: int) -> np.ndarray:
    return DECODE_TABLE[np.asarray(codes, dtype=np.uint8)] * 2.0 ** e


def fp8_rows(rows: np.ndarray, d_c: int) -> np.ndarray:
    """What a quantized cache holds for float64 rows [n][d_c + d_rope]: the
    latent dequantized from its codes, the rope part unchanged (it is stored
    in bf16 and rounded like a bf16 cache)."""
    out = np.array(rows, dtype=np.float64, copy=True)
    for i in range(out.shape[0]):
        codes, e = quantize_row(out[i, :d_c])
        out[i, :d_c] = dequantize_row(codes, e)
    return out

"""Round float64 values to bfloat16 (nearest, ties to even), float64 math.

TEST INFRASTRUCTURE ONLY (see ``oracle/mla_oracle.py``).

Used where the expected value of a stored bf16 element is known exactly
(integer-valued sums) and the comparison is bit for bit.  bfloat16 keeps 8
significant bits, so a finite nonzero v with 2**e <= |v| < 2**(e+1) is
rounded to a multiple of 2**(e-7); numpy's ``rint`` rounds halves to even.
"""
from __future__ import annotations

import numpy as np


def rne_bf16_value(v) -> np.ndarray:
    """float64 -> nearest bfloat16 value (as float64).  Normal range only."""
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros_like(v)
    nz = v != 0
    e = np.floor(np.log2(np.abs(v[nz])))
    ulp = np.exp2(e - 7.0)
    out[nz] = np.rint(v[nz] / ulp) * ulp
    return out


def bf16_value_to_bits(v) -> np.ndarray:
    """Exact bfloat16 value (float64) -> its 16-bit pattern."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)   # exact for bf16 values
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)

"""Decoders for the storage formats of the attention inputs and outputs (fp64 results).

TEST INFRASTRUCTURE ONLY -- see oracle/__init__.py.

Each format is decoded from its bit-level definition by one generic minifloat
routine: sign bit, ``e`` exponent bits with bias ``2**(e-1) - 1``, ``m`` mantissa
bits, subnormals when the exponent field is zero.

* bf16: 1-8-7, the upper half of an IEEE binary32 (infinities and NaNs as IEEE);
* fp16: IEEE binary16, 1-5-10;
* fp8 e4m3 (the ``float_e4m3_t`` output type named by the CUTLASS Blackwell FMHA
  walk-through, trdm.cn, section on the fp8 element types): the OCP "E4M3FN"
  variant, 1-4-3 with bias 7, no infinities, and only S.1111.111 is NaN, so the
  largest finite value is 448.
"""
from __future__ import annotations

import numpy as np

_FORMATS = {
    # name: (exponent bits, mantissa bits, ieee_special)  ieee_special: all-ones exponent is inf/NaN
    "bf16": (8, 7, True),
    "f16": (5, 10, True),
    "f8e4m3": (4, 3, False),
}


def decode_minifloat(bits: np.ndarray, exp_bits: int, man_bits: int, ieee_special: bool) -> np.ndarray:
    b = np.asarray(bits).astype(np.int64)
    sign = np.where((b >> (exp_bits + man_bits)) & 1, -1.0, 1.0)
    e = (b >> man_bits) & ((1 << exp_bits) - 1)
    m = (b & ((1 << man_bits) - 1)).astype(np.float64)
    bias = (1 << (exp_bits - 1)) - 1
    frac = m / float(1 << man_bits)
    normal = sign * np.ldexp(1.0 + frac, (e - bias).astype(np.int64))
    subnormal = sign * np.ldexp(frac, 1 - bias)
    out = np.where(e == 0, subnormal, normal)
    e_max = (1 << exp_bits) - 1
    if ieee_special:
        out = np.where((e == e_max) & (m == 0), sign * np.inf, out)
        out = np.where((e == e_max) & (m != 0), np.nan, out)
    else:
        out = np.where((e == e_max) & (m == float((1 << man_bits) - 1)), np.nan, out)
    return out


def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Raw storage bits (uint16 for bf16/fp16, uint8 for fp8) -> float64, exactly."""
    e, m, special = _FORMATS[dtype]
    return decode_minifloat(bits, e, m, special)

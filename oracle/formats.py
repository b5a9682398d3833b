"""Exact decoders from raw storage bits to float64 (test infrastructure, never the product path).

Each decoder widens without rounding: every bf16, fp16 and fp8-e4m3 value is exactly
representable in float64.

* bf16: the upper 16 bits of an IEEE binary32; widen by shifting into a float32.
* fp16: IEEE binary16, widened through numpy's float16.
* fp8 e4m3 (the OCP "e4m3fn" variant): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
  exponent field 0 holds subnormals m * 2**-9; exponent 15 with mantissa 7 is NaN; there are no
  infinities, so the largest finite magnitude is 1.75 * 2**8 = 448.
  The FP8 KV cache is named on the babushkai.com "GPU推論の内部構造" page (KV-cache ledger and
  quantization sections); the bit layout is the format's own definition.
"""

from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):        # signalling-NaN patterns widen to NaN
        return b.view(np.float32).astype(np.float64)


def f16_to_f64(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def _e4m3fn_value(code: int) -> float:
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * man * 2.0**-9
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


E4M3FN_TABLE = np.array([_e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def e4m3fn_to_f64(bits: np.ndarray) -> np.ndarray:
    return E4M3FN_TABLE[np.asarray(bits, dtype=np.uint8)]


_E4M3FN_CODE_OF = {float(E4M3FN_TABLE[c]): c for c in range(0x7F)}   # finite, non-negative


def e4m3fn_encode(y: np.ndarray) -> np.ndarray:
    """Round values to OCP e4m3fn codes: saturate to +-448 (the largest finite magnitude; the
    format has no infinities), then round to the nearest representable value, ties to the even
    mantissa.  NaN gives 0x7F.  The sign of a value that rounds to zero is kept (0x80 = -0).

    The grid spacing in the binade [2**e, 2**(e+1)) is 2**(e-3) (3 mantissa bits); below 2**-6
    (the smallest normal) the subnormal spacing 2**-9 continues down to zero.
    """
    y = np.asarray(y, dtype=np.float64)
    nan = np.isnan(y)
    neg = np.signbit(y)
    a = np.minimum(np.abs(np.where(nan, 0.0, y)), 448.0)
    _, ex = np.frexp(a)                          # a = f * 2**ex with f in [0.5, 1)
    e = np.maximum(ex.astype(np.float64) - 1.0, -6.0)
    q = np.exp2(e - 3.0)
    r = np.round(a / q) * q                      # numpy rounds halves to even; a / q is exact
    codes = np.vectorize(lambda v: _E4M3FN_CODE_OF[float(v)], otypes=[np.uint8])(r)
    codes = np.where(neg, codes | 0x80, codes).astype(np.uint8)
    return np.where(nan, np.uint8(0x7F), codes).astype(np.uint8)


def to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_to_f64(bits)
    if dtype == "f16":
        return f16_to_f64(bits)
    if dtype == "fp8_e4m3":
        return e4m3fn_to_f64(bits)
    raise ValueError(f"unknown dtype {dtype!r}")

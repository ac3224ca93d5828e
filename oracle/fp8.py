"""FP8 E4M3 codes for a quantised KV cache — test infrastructure, never product code.

The pages name FP8 as a serving precision (the "Serving engine internals" lesson quotes Llama 3.3
70B in FP8 on an H100; the "Inference optimization" lesson lists FP8 quantization among kernel
optimizations; the vLLM-on-H100 article names FP8 precision as a further lever) but do not fix the
format.  This oracle takes the OCP 8-bit floating-point E4M3 format, the one FP8 KV caches use:
1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no infinities, and NaN only for the
codes with all exponent and mantissa bits set (0x7F, 0xFF).  Its largest finite magnitude is
1.75 * 2**8 = 448 and its smallest subnormal 2**-9.

Encoding is defined here by the value table: a real number becomes the code of the nearest finite
E4M3 value, with a tie going to the code whose lowest mantissa bit is zero (round to nearest
even); magnitudes beyond 448 saturate to 448.  The sign is kept, so a negative value that rounds
to zero gives the negative-zero code 0x80.

Quantisation of a cache row with a per-tensor scale s: code = encode(fp32(x) / fp32(s)), the
division being the correctly rounded fp32 quotient.  The cached value the attention sees is then
s * decode(code), exact in float64.
"""

from __future__ import annotations

import numpy as np

MAX_FINITE = 448.0


def decode_table() -> np.ndarray:
    """float64 value of each of the 256 codes (NaN for 0x7F and 0xFF), from the format's fields."""
    codes = np.arange(256)
    sign = np.where(codes >> 7, -1.0, 1.0)
    e = (codes >> 3) & 0xF
    m = (codes & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e.astype(np.float64) - 7))
    val = sign * mag
    val[(e == 0xF) & (codes & 0x7 == 0x7)] = np.nan
    return val


_TABLE = decode_table()
# Non-negative finite codes 0x00 .. 0x7E in increasing order of value.
_POS_CODES = np.arange(0x7F)
_POS_VALUES = _TABLE[:0x7F]


def decode(codes: np.ndarray) -> np.ndarray:
    """float64 values of uint8 codes."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def encode(x: np.ndarray) -> np.ndarray:
    """uint8 E4M3 codes of real values: nearest finite value, ties to the even code, saturating
    at +-448.  NaN inputs give 0x7F with the input's sign bit."""
    x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x)
    a = np.minimum(np.abs(x), MAX_FINITE)
    hi = np.searchsorted(_POS_VALUES, a, side="left")  # first value >= a
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    code = np.where(np.isnan(x), 0x7F, code)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def quantize(bf16_bits: np.ndarray, scale: float) -> np.ndarray:
    """Codes of bf16 values divided by a per-tensor scale (correctly rounded fp32 quotient)."""
    u = np.asarray(bf16_bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    x = u.view(np.float32)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        y = x / np.float32(scale)
    return encode(y.astype(np.float64))

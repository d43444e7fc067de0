"""Oracle for an fp8 KV cache: the e4m3 code, per-tensor scales, the cache
write that quantises and the attention that reads dequantised values.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Pages cited in this file:
  [1] "PagedAttention - how vLLM stopped wasting 80% of your GPU memory"
      (shivam2003.com/posts/pagedattention.html)
  [3] "PagedAttention and vLLM: Virtual Memory for the KV Cache" (passgenai.com)

What the pages fix: storing K and V in 8 bits (int8 or fp8) instead of 16
halves the bytes per element and composes with paging ([1], "How does this
relate to quantization?"; [3], the KV-size formula's bytes_per_element term).

Readings where the pages leave the scheme open:
  * the 8-bit format is the OCP "E4M3" float (the variant without
    infinities): sign, 4 exponent bits with bias 7, 3 mantissa bits;
    exponent field 0 encodes subnormals m * 2^-9; 0x7F and 0xFF are NaN;
    the largest finite magnitude is 448;
  * one fp32 scale per pool (per layer, K and V separately). A stored value x
    (any of f32, f16, bf16, widened exactly to fp32) is written as the code
    of y = fp32(x / scale): division in fp32 rounded to nearest even, then
    rounding to the nearest E4M3 value, ties to the even code; magnitudes
    beyond 448 (infinities included) saturate to 448; NaN is written as 0x7F;
    the sign of a zero result is kept;
  * the value read back is code_value * scale, exactly (in float64 here);
    attention is the plain definition over those values.
"""
from __future__ import annotations

from typing import Sequence

import numpy as np

E4M3_MAX = 448.0
E4M3_NAN = 0x7F


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 code as float64 (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


# the 127 non-negative finite values in code order (codes 0x00..0x7E)
_POS_VALUES = e4m3_decode(np.arange(0x7F))


def e4m3_encode(y) -> np.ndarray:
    """Nearest E4M3 code of each fp32 value, ties to the even code; beyond
    448 saturates; NaN gives 0x7F; the sign bit follows the input's sign."""
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y.astype(np.float64))
    nan = np.isnan(a)
    sat = a >= E4M3_MAX
    a = np.where(nan | sat, 0.0, a)
    # neighbours: the first value >= a, and the one below it
    hi = np.minimum(np.searchsorted(_POS_VALUES, a, side="left"), 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    even = np.where(lo % 2 == 0, lo, hi)
    pick = np.where(d_hi == 0, hi, np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, even)))
    pick = np.where(sat, 0x7E, pick)
    code = np.where(np.signbit(y), pick | 0x80, pick)
    return np.where(nan, E4M3_NAN, code).astype(np.uint8)


def to_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp32 view of stored f32 / f16 / bf16 (bit pattern) values."""
    x = np.asarray(x)
    if dtype == "bf16":
        return (x.astype(np.uint32) << 16).view(np.float32)
    if dtype in ("f32", "f16"):
        return x.astype(np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def quantize(x: np.ndarray, dtype: str, scale: float) -> np.ndarray:
    """E4M3 codes of stored values x under a per-tensor scale."""
    y = to_f32(x, dtype) / np.float32(scale)  # one fp32 division per element
    return e4m3_encode(y.astype(np.float32))


def dequantize(codes: np.ndarray, scale: float) -> np.ndarray:
    """Values an fp8 pool holds, as float64: code value times the scale."""
    return e4m3_decode(codes) * float(np.float32(scale))


def reshape_and_cache_fp8(k_new, v_new, k_pool, v_pool, slots: Sequence[int], dtype: str,
                          k_scale: float, v_scale: float, block_size: int = 16) -> None:
    """Write each new token's K and V rows, quantised, into its slot of the
    uint8 pools ([3], "The allocation lifecycle": the step's token goes into
    the last block). Slots < 0 are skipped."""
    for i, s in enumerate(slots):
        s = int(s)
        if s < 0:
            continue
        k_pool[s // block_size, :, s % block_size, :] = quantize(k_new[i], dtype, k_scale)
        v_pool[s // block_size, :, s % block_size, :] = quantize(v_new[i], dtype, v_scale)

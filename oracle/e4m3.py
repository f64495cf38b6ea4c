"""OCP FP8 E4M3 (E4M3FN) codec, written from the format definition.

The pages fix the format only as "e4m3" (lpnh.cn guide, section 3, [fp8] block;
zhihu infra commentary: E4M3 in both passes). The reading taken is the OCP 8-bit
E4M3FN format: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent
field 0 is subnormal (m/8 * 2^-6); no infinities; S.1111.111 is NaN; the largest
finite magnitude is 1.75 * 2^8 = 448.

Encoding is the plain definition: the nearest finite E4M3 value, ties to the code
with an even mantissa, magnitudes above 448 clamped to 448, the sign kept (so -0
and negative values that round to zero give 0x80), NaN -> 0x7F with its sign.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

E4M3_MAX = 448.0


def _code_value(code: int) -> float:
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * (m / 8.0) * 2.0 ** (-6)
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_TABLE = np.array([_code_value(c) for c in range(256)], dtype=np.float64)
# codes 0x00..0x7E are the non-negative finite values, strictly increasing
_POS = _TABLE[:127].copy()
assert np.all(np.diff(_POS) > 0)


def finite_values() -> np.ndarray:
    """The 127 non-negative finite E4M3 values, indexed by their code 0x00..0x7E."""
    return _POS.copy()


def decode(codes: np.ndarray) -> np.ndarray:
    """E4M3 codes (uint8) -> float64 values (NaN for 0x7F/0xFF)."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def _encode_chunk(x: np.ndarray) -> np.ndarray:
    pos = _POS
    nan = np.isnan(x)
    neg = np.signbit(x)
    a = np.abs(x.astype(np.float64))
    a = np.where(nan, 0.0, np.minimum(a, E4M3_MAX))
    hi = np.searchsorted(pos, a, side="left")      # pos[hi-1] < a <= pos[hi]
    hi = np.minimum(hi, 126)
    lo_i = np.maximum(hi - 1, 0)
    d_lo = a - pos[lo_i]
    d_hi = pos[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo_i).astype(np.uint8)
    code = np.where(nan, np.uint8(0x7F), code)
    return code | (neg.astype(np.uint8) << 7)


def encode(v: np.ndarray, chunk: int = 1 << 20) -> np.ndarray:
    """float32 values -> E4M3 codes (uint8): nearest value, ties to even, saturating.

    Large inputs are cut into chunks encoded on a thread pool (same arithmetic)."""
    v = np.asarray(v, dtype=np.float32)
    flat = v.reshape(-1)
    if flat.size <= chunk:
        return _encode_chunk(flat).reshape(v.shape)
    out = np.empty(flat.shape, dtype=np.uint8)
    starts = range(0, flat.size, chunk)

    def job(lo):
        out[lo:lo + chunk] = _encode_chunk(flat[lo:lo + chunk])
    with ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(job, starts))
    return out.reshape(v.shape)

"""fp8 E4M3 codec for the oracle (test infrastructure, CPU only).

The pages say only that a KV cache may be stored in "FP8", halving its bytes
at some cost in long-context accuracy ([nano-vllm blog §1.1, §6.3]).  The
format taken here is the OCP 8-bit floating point E4M3 variant ("E4M3FN"):

  bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa;
  exponent 0      -> subnormal  (m / 8) * 2^-6;
  exponent 1..15  -> normal     (1 + m / 8) * 2^(e - 7);
  exponent 15 with mantissa 7 (codes 0x7F, 0xFF) -> NaN; no infinities.
  Largest finite magnitude: 1.75 * 2^8 = 448.

Encoding (a reading the pages leave open): round to the nearest
representable value, ties to the even code, saturate magnitudes beyond 448 to
448 (infinities included), NaN stays NaN with its sign bit.  The stored code
represents ``code_value * scale`` for a per-tensor fp32 scale, and the value
written is ``float32(x) / float32(scale)`` computed in IEEE float32.

The encoder below is a nearest-neighbour search over the 127 non-negative
finite values of the format: slow, but it follows the definition directly.
"""
from __future__ import annotations

import numpy as np

MAX_FINITE = 448.0
NAN_CODE = 0x7F


def e4m3_value(code: int) -> float:
    """The real number an E4M3 code stands for (float('nan') for the NaN codes)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e4m3_decode_table() -> np.ndarray:
    """float64 value of every one of the 256 codes."""
    return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


_TABLE = e4m3_decode_table()
_GRID = _TABLE[:0x7F]            # codes 0x00..0x7E: 0 .. 448, strictly increasing


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Codes (uint8) -> float64 values."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """float32 values -> E4M3 codes (uint8): nearest, ties to even, saturating."""
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y.astype(np.float64))
    sign = np.signbit(y).astype(np.uint8) << np.uint8(7)
    # Neighbours in the grid: _GRID[hi_idx - 1] <= a <= _GRID[hi_idx].
    hi_idx = np.clip(np.searchsorted(_GRID, a, side="left"), 1, len(_GRID) - 1)
    lo_idx = hi_idx - 1
    d_lo = a - _GRID[lo_idx]
    d_hi = _GRID[hi_idx] - a
    lo_even = (lo_idx % 2) == 0
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & lo_even)
    mag = np.where(pick_lo, lo_idx, hi_idx).astype(np.int64)
    mag = np.where(a >= MAX_FINITE, 0x7E, mag)                # saturate (inf included)
    code = (mag.astype(np.uint8) | sign).astype(np.uint8)
    code = np.where(np.isnan(y), NAN_CODE | sign, code).astype(np.uint8)
    return code


def e4m3_quantise(x_f32: np.ndarray, scale: float) -> np.ndarray:
    """Codes for ``float32(x) / float32(scale)``; the division is IEEE float32."""
    x = np.asarray(x_f32, dtype=np.float32)
    y = (x / np.float32(scale)).astype(np.float32)
    return e4m3_encode(y)

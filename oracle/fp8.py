"""FP8 KV rows: the quantize step and its inverse (oracle; test infrastructure only).

The engine quantizes each new K/V row to FP8 before storing it in the cache, and
the attention reads the quantized rows ([P-DS4] "Architecture Deep Dive",
Whole-Model Graph Execution, where the layer schedule puts an FP8 quantize step
between the Q/KV projections and the raw KV store; "GPU Backend Architecture"
counts an FP8 KV quantization among the GPU operations).  The pages do not give
the format.  Readings taken:

* element format: OCP FP8 E4M3 ("e4m3fn"): 1 sign, 4 exponent bits (bias 7), 3
  mantissa bits; exponent field 0 is subnormal (m/8 * 2^-6); 0x7F / 0xFF are NaN;
  there are no infinities; the largest finite value is 448;
* one float32 scale per row of D elements (per K row and per V row), so that a
  row can be quantized the moment it is written; value = decode(code) * scale;
* quantize: amax = max |x| over the row (x widened to float32), scale =
  amax / 448 in float32; each element y = x / scale in float32, clamped to
  [-448, 448], rounded to the nearest E4M3 value, ties to even mantissa; the code
  keeps the sign bit of y (so -0.0 becomes 0x80);
* a row whose scale is 0 (all zeros, or an amax so small that amax / 448
  underflows) gets scale 0 and every code 0x00;
* rows must be finite; values are expected within the float16 range.

Float32 is the precision the pages' engine stores and divides in; both sides
take the rounding decisions in float32, so codes and scales compare bit for bit.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
_MIN_NORMAL = 2.0 ** -6     # smallest normal E4M3 value
_SUB_STEP = 2.0 ** -9       # spacing of the subnormals


def _round_half_even(a):
    return np.rint(a)


def _clamp(y):
    return np.clip(y, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))


def _sign_bit(y):
    return np.signbit(y)


def decode(codes: np.ndarray) -> np.ndarray:
    """float64 values of E4M3 codes (NaN for 0x7F and 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * _SUB_STEP, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def encode(y: np.ndarray) -> np.ndarray:
    """E4M3 codes of float32 values with |y| <= 448: nearest value, ties to even."""
    y = np.asarray(y, dtype=np.float32)
    if not np.all(np.abs(y) <= E4M3_MAX):
        raise ValueError("encode takes finite values within [-448, 448]")
    a = np.abs(y).astype(np.float64)                 # exact
    sign = _sign_bit(y).astype(np.int64) << 7
    # binade exponent, with everything below the smallest normal sharing the
    # subnormal spacing 2^-9
    _, ex = np.frexp(np.where(a > 0, a, 1.0))        # a = f * 2^ex with f in [0.5, 1), exactly
    e = np.where(a >= _MIN_NORMAL, ex - 1.0, -6.0)
    step = np.exp2(e - 3.0)                          # spacing of the values in that binade
    q = _round_half_even(a / step)                   # exact quotient, rounded half to even
    # q counts steps: 8..16 in a normal binade (16 carries into the next one),
    # 0..8 below the smallest normal (8 is the smallest normal itself)
    normal = a >= _MIN_NORMAL
    ef = np.where(normal, e + 7.0, 0.0)
    mant = np.where(normal, q - 8.0, q)
    carry = mant >= 8.0
    ef = np.where(carry, ef + 1.0, ef)
    mant = np.where(carry, mant - 8.0, mant)
    code = sign | (ef.astype(np.int64) << 3) | mant.astype(np.int64)
    return code.astype(np.uint8)


def quantize_rows(x: np.ndarray):
    """(codes uint8 [..., D], scales float32 [...]) of rows x [..., D] (float16 or float32)."""
    xf = np.asarray(x).astype(np.float32)
    amax = np.max(np.abs(xf), axis=-1) if xf.shape[-1] else np.zeros(xf.shape[:-1], np.float32)
    scale = (amax.astype(np.float32) / np.float32(E4M3_MAX)).astype(np.float32)
    codes = np.zeros(xf.shape, dtype=np.uint8)
    nz = scale != 0
    if np.any(nz):
        with np.errstate(divide="ignore", invalid="ignore"):
            y = (xf / np.where(nz, scale, np.float32(1))[..., None]).astype(np.float32)
        y = _clamp(y)
        codes = np.where(nz[..., None], encode(y), np.uint8(0)).astype(np.uint8)
    return codes, scale


def dequantize_rows(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """float64 rows decode(code) * scale."""
    return decode(codes) * np.asarray(scales, dtype=np.float64)[..., None]

"""Number formats used by the paged KV cache, written from their definitions.

TEST INFRASTRUCTURE: part of the CPU oracle.  Only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import it; the library's GPU path never does.

* bf16: the upper 16 bits of an IEEE-754 binary32 value.  Widening a bf16
  is exact: the 16 bits are shifted into the high half of a binary32.
* e4m3 (the OCP 8-bit "E4M3FN" variant, the one gfx950 implements): one
  sign bit, four exponent bits with bias 7, three mantissa bits.  Exponent
  field 0 holds subnormals ``m * 2^-9``; exponent field 15 with mantissa 7
  is NaN; there are no infinities, so the largest finite value is
  ``2^8 * 1.75 = 448``.

* int4: a signed integer in [-8, 7] stored offset by 8 as a 4-bit code
  0..15, two codes per byte: element 2i in the low nibble of byte i,
  element 2i+1 in the high nibble.  A value x is stored as the code of
  clamp(round_half_even(float32(x) / float32(scale)), -8, 7).

The pages only name "fp8" as a KV-cache type ("17 · 连续批处理与
PagedAttention", section 四, the ``kv_cache_dtype`` knob, which is said to
roughly double the batch) and compare FP16 / FP8 / INT4 KV in an exercise
("推理优化", section 五, exercise 1: INT4 about 4x the concurrency); the
e4m3 variant, round-to-nearest-even, saturation at +-448, and the int4
layout above are the readings of them taken here.  The pages fix neither
the variant nor the layout; the pins check these functions against the
format definitions (exhaustively) and torch's float8_e4m3fn cast.
"""
from __future__ import annotations

import numpy as np

E4M3_BIAS = 7
E4M3_MAX = 448.0
E4M3_NAN = 0x7F


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def e4m3_value(code: int) -> float:
    """Value of one e4m3 code, straight from the field definition."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * man * 2.0 ** (1 - E4M3_BIAS - 3)      # subnormal: m/8 * 2^(1-bias)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - E4M3_BIAS)


def e4m3_table() -> np.ndarray:
    """float64[256]: the value of every code (NaN for 0x7F and 0xFF)."""
    return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


_E4M3_TABLE = e4m3_table()


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    return _E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Saturating round-to-nearest-even encode of float32 values to e4m3 codes.

    The quantum of e4m3 in the binade [2^e, 2^(e+1)) is 2^(e-3) for normal
    exponents e >= -6 and 2^-9 below 2^-6 (subnormals).  A value is divided
    by its quantum (exact: a power of two), rounded half-to-even to an
    integer, and multiplied back; magnitudes at or above 448 saturate to 448.
    NaN maps to the NaN code (with the input's sign).
    """
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x).astype(np.float64)
    sign = np.signbit(x)
    nan = np.isnan(x)
    a = np.where(nan, 0.0, a)
    sat = a >= E4M3_MAX
    # binade exponent of a (floor(log2 a)), exact via frexp: a = f * 2^k, f in [0.5, 1)
    _, k = np.frexp(a)
    e = np.maximum(k - 1, -6)                     # subnormals share the quantum of e = -6
    quantum = np.ldexp(1.0, e - 3)
    y = np.round(a / quantum) * quantum           # np.round: half to even
    y = np.where(sat | (y > E4M3_MAX), E4M3_MAX, y)
    # code bits of the (now representable) magnitude y
    f, k2 = np.frexp(y)
    ey = k2 - 1
    normal = y >= 2.0 ** -6
    exp_field = np.where(normal, ey + E4M3_BIAS, 0)
    man_field = np.where(normal, np.rint((y / np.ldexp(1.0, ey) - 1.0) * 8.0),
                         np.rint(y / 2.0 ** -9))
    code = (exp_field.astype(np.int64) << 3) | man_field.astype(np.int64)
    code = np.where(y == 0.0, 0, code)
    code = np.where(nan, E4M3_NAN, code)
    code = code | np.where(sign, 0x80, 0)
    return code.astype(np.uint8)


def e4m3_quantize(x: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Code of ``float32(x) / float32(scale)`` (IEEE binary32 division), saturating RNE."""
    q = np.asarray(x, dtype=np.float32) / np.asarray(scale, dtype=np.float32)
    return e4m3_encode(q.astype(np.float32))


INT4_MIN, INT4_MAX, INT4_OFFSET = -8, 7, 8


def int4_unpack(packed: np.ndarray) -> np.ndarray:
    """[..., n] bytes -> [..., 2n] codes 0..15 (element 2i = low nibble of byte i)."""
    b = np.asarray(packed, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = b & 0x0F
    out[..., 1::2] = b >> 4
    return out


def int4_pack(codes: np.ndarray) -> np.ndarray:
    """[..., 2n] codes 0..15 -> [..., n] bytes."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def int4_to_f64(packed: np.ndarray) -> np.ndarray:
    """Values (code - 8) of packed int4 bytes, unpacked along the last axis."""
    return int4_unpack(packed).astype(np.float64) - INT4_OFFSET


def int4_encode(x: np.ndarray) -> np.ndarray:
    """Codes of float32 values: round half to even, clamp to [-8, 7], offset by 8
    (NaN, which has no int4 code, takes the code of -8)."""
    r = np.rint(np.asarray(x, dtype=np.float32).astype(np.float64))   # np.rint: half to even
    r = np.where(np.isnan(r), INT4_MIN, r)
    return (np.clip(r, INT4_MIN, INT4_MAX) + INT4_OFFSET).astype(np.uint8)


def int4_quantize(x: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Packed codes of ``float32(x) / float32(scale)`` (IEEE binary32 division)."""
    q = np.asarray(x, dtype=np.float32) / np.asarray(scale, dtype=np.float32)
    return int4_pack(int4_encode(q.astype(np.float32)))

"""Number formats used by the path, written out from their definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* OCP FP8 E4M3 ("e4m3fn"): 1 sign, 4 exponent (bias 7), 3 mantissa bits; no
  infinity; S.1111.111 is NaN; largest finite 448; subnormals m * 2**-9.
  The pages quantise to it with scale amax / 448 (vLLM "mega_moe" page,
  hidden_block docstring; "shared_expert" page, _group_scale docstring), so
  448 is the format's largest finite value. Encoding here is round to nearest,
  ties to even, saturating to +-448 (the reading the pages leave open for the
  off-page pack_fp8; with scale amax/448 saturation never triggers on finite
  data anyway).
* BF16: FP32 with the low 16 mantissa bits rounded off, nearest-even.
* f32: IEEE binary32 round-to-nearest-even of a float64 value.

All values are carried as float64 arrays holding exactly representable values
of the narrower format.
"""

from __future__ import annotations

import numpy as np

FP8_MAX = 448.0


def f32(v) -> np.ndarray:
    """Round float64 values to the nearest binary32 (ties to even)."""
    return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)


def e4m3_decode(codes) -> np.ndarray:
    """Value of each e4m3 byte: (-1)**s * (8 + m) * 2**(e - 10) for e > 0,
    (-1)**s * m * 2**-9 for e == 0, NaN for exponent 15 with mantissa 7."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0**-9, (8 + m) * np.exp2(e - 10.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return s * mag


E4M3_VALUES = e4m3_decode(np.arange(256))


def e4m3_encode(v) -> np.ndarray:
    """e4m3 byte nearest to each value, ties to the even mantissa, magnitudes
    that round above 448 saturating to 448 (code 0x7E)."""
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("e4m3_encode: non-finite input")
    a = np.abs(v)
    _, ex = np.frexp(a)                      # a = f * 2**ex, f in [0.5, 1)
    E = np.maximum(ex.astype(np.int64) - 1, -6)  # binade; below 2**-6 the grid is 2**-9
    q = np.rint(a / np.exp2(E - 3.0))        # 3 fraction bits; rint is ties-to-even
    carry = q >= 16                          # rounded up into the next binade
    E = np.where(carry, E + 1, E)
    q = np.where(carry, 8, q).astype(np.int64)
    value = q * np.exp2(E - 3.0)
    normal = q >= 8
    code = np.where(normal, ((E + 7) << 3) | (q - 8), q)
    code = np.where(value > FP8_MAX, 0x7E, code)
    code = code | np.where(np.signbit(v), 0x80, 0)
    return code.astype(np.uint8)


def bf16_round(v) -> np.ndarray:
    """Round to binary32 first, then to the nearest BF16 (8 significant bits,
    ties to even)."""
    x = f32(v)
    m, e = np.frexp(x)                       # x = m * 2**e, |m| in [0.5, 1)
    return np.ldexp(np.rint(m * 256.0), e - 8)

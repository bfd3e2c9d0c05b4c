"""Number formats used by the oracle (test infrastructure only).

The pages fix the storage formats of the path but not their arithmetic: keys and
values are "stored INT8, computed BF16" ("Hy-Nomas auf einer RTX 4090",
inferencekey.com, section "Das Single-GPU-Preset"). The oracle therefore holds
every value in float64 and rounds explicitly wherever a value is *stored* in a
narrower format:

* ``to_bf16``  -- round a float64 to the nearest bfloat16 (8 significant bits,
  exponent range of fp32, subnormals kept, ties to even, overflow to inf). This
  is one rounding from the exact value, written from the definition of
  round-to-nearest-even, not through fp32.
* ``to_f32``   -- round to the nearest float32 (numpy's cast, ties to even).
* ``bf16_bits`` / ``from_bf16_bits`` -- the 16-bit pattern of a bfloat16, the
  top half of the fp32 pattern of the same value.
"""

import numpy as np

# bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 stored mantissa bits.
BF16_PRECISION = 8          # significant bits including the implicit one
BF16_EMIN = -126            # exponent of the smallest normal
BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def to_bf16(x):
    """Nearest bfloat16 value of ``x`` (float64 in, float64 out), ties to even.

    For |x| with exponent e (x = f * 2**e, 0.5 <= |f| < 1) the quantum is
    2**(e - 8), but never below the subnormal quantum 2**(-126 - 7).
    ``np.rint`` rounds half to even; the scaling by powers of two is exact.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, dtype=np.float64, copy=True)
    finite = np.isfinite(x) & (x != 0)
    xf = x[finite]
    _, e = np.frexp(xf)                       # xf = f * 2**e, 0.5 <= |f| < 1
    q = np.maximum(e - BF16_PRECISION, BF16_EMIN - (BF16_PRECISION - 1))
    y = np.ldexp(np.rint(np.ldexp(xf, -q)), q)
    y = np.where(np.abs(y) > BF16_MAX, np.copysign(np.inf, xf), y)
    out[finite] = y
    return out


def to_f32(x):
    """Nearest float32 value of ``x`` as float64 (ties to even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def bf16_bits(x):
    """uint16 pattern of bfloat16 values ``x`` (x must already be bf16-exact)."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    if not np.array_equal(x32.astype(np.float64), np.asarray(x, np.float64), equal_nan=True):
        raise ValueError("bf16_bits: input is not representable in float32")
    u = x32.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("bf16_bits: input is not bfloat16-exact")
    return (u >> 16).astype(np.uint16)


def from_bf16_bits(u):
    """float64 values of uint16 bfloat16 patterns ``u``."""
    u = np.asarray(u).astype(np.uint32)
    return (u << 16).view(np.float32).astype(np.float64)


def bf16_ulp(y):
    """Spacing of bfloat16 numbers at magnitude |y| (the ulp of a bf16 value y)."""
    y = np.abs(np.asarray(y, dtype=np.float64))
    _, e = np.frexp(np.where(y == 0, 1.0, y))
    q = np.maximum(e - BF16_PRECISION, BF16_EMIN - (BF16_PRECISION - 1))
    return np.where(y == 0, 2.0 ** (BF16_EMIN - (BF16_PRECISION - 1)), np.ldexp(1.0, q))

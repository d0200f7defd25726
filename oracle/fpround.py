"""Round-to-nearest-even conversions to the two 16-bit formats the pages use.

The pack-unpack-run page stores the group scale as fp16 and reconstructs
weights as bf16, with "nearest-even ties" ("Three values and a shared
scale").  These routines round a float64 value to the nearest member of the
target format, ties to even, by working on values rather than bits: find the
spacing of the format at the value's binade, divide (exact, a power of two),
round to an integer with numpy's rint (IEEE ties-to-even), multiply back.
Only then is the (now exactly representable) value turned into its bit
pattern.
"""

import numpy as np


def _round_to_format(x, emin, frac_bits, overflow_at):
    """Nearest value of a binary format with `frac_bits` fraction bits and
    smallest normal exponent `emin`; ties to even; |result| >= overflow_at
    becomes +-inf.  Subnormals use the spacing of the smallest normal binade.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e2 = np.frexp(np.abs(x))            # |x| = f * 2**e2, 0.5 <= f < 1
    e = np.maximum(e2 - 1, emin)            # binade exponent, clamped at emin
    spacing = np.ldexp(1.0, e - frac_bits)
    with np.errstate(invalid="ignore", over="ignore"):
        r = np.rint(x / spacing) * spacing
        r = np.where(np.abs(r) >= overflow_at, np.copysign(np.inf, x), r)
    return r


def f64_to_f16_bits(x):
    """fp16 bits of the nearest-even fp16 value of float64 `x` (one rounding).

    fp16: 10 fraction bits, smallest normal 2**-14, largest finite 65504; a
    value that rounds to 2**16 overflows to infinity.
    """
    r = _round_to_format(x, -14, 10, 65536.0)
    return np.asarray(r, dtype=np.float16).view(np.uint16)


def f16_bits_to_f64(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def f64_to_bf16_bits(x):
    """bf16 bits of the nearest-even bf16 value of float64 `x` (one rounding).

    bf16: 7 fraction bits, smallest normal 2**-126; a value that rounds to
    2**128 overflows to infinity.  NaN stays NaN.
    """
    r = _round_to_format(x, -126, 7, 2.0 ** 128)
    bits32 = np.asarray(r, dtype=np.float32).view(np.uint32)
    return (bits32 >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f64(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def f64_to_f32(x):
    """Nearest-even fp32 value of float64 `x` (one rounding), as float32."""
    r = _round_to_format(x, -126, 23, 2.0 ** 128)
    return np.asarray(r, dtype=np.float32)

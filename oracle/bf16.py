"""bfloat16 bit patterns <-> float64 (oracle; test infrastructure only).

bfloat16 is the upper half of an IEEE-754 binary32: 1 sign bit, 8 exponent
bits, 7 stored mantissa bits (8 significant bits for normal numbers). The
pages' logits, conv inputs and KV caches are bf16 (PR #1377 "LFM2:
shared-round decode", the GPU-pick commit: 128,000 bf16 logits per row).

``round_f64`` rounds a float64 straight to the nearest bf16, ties to even,
in ONE rounding step (never via float32, which would round twice).
"""

import numpy as np

_QNAN_BITS = 0x7FC0


def to_f64(bits):
    """uint16 bf16 bit patterns -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def round_f64(x):
    """float64 values -> uint16 bf16 bit patterns, round to nearest, ties to even.

    The quantum of the bf16 grid at |x| in [2^(E-1), 2^E) is 2^(E-8) for normal
    numbers and 2^-133 below the smallest normal 2^-126. Dividing by the
    quantum is exact in float64, ``np.rint`` rounds half to even, and the
    rounded value is exactly representable in bf16 (hence in float32). A
    value that rounds to 2^128 or beyond overflows to infinity.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros(x.shape, dtype=np.uint16)
    nan = np.isnan(x)
    inf = np.isinf(x)
    fin = ~(nan | inf)
    xf = np.where(fin, x, 0.0)
    _, e = np.frexp(xf)                      # |x| = f * 2^e, 0.5 <= f < 1
    e = np.maximum(e, -125)                  # subnormal range shares one quantum
    quantum = np.ldexp(1.0, e - 8)
    y = np.rint(xf / quantum) * quantum
    over = np.abs(y) >= 2.0 ** 128
    y32 = np.where(over, 0.0, y).astype(np.float32)
    bits = (y32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    sign = np.signbit(x)
    inf_bits = np.where(sign, 0xFF80, 0x7F80).astype(np.uint16)
    bits = np.where(fin & over, inf_bits, bits)
    bits = np.where(inf, inf_bits, bits)
    bits = np.where(nan, np.uint16(_QNAN_BITS), bits)
    # keep the sign of zero results (e.g. -1e-50 rounds to -0)
    zero = fin & (y == 0.0)
    bits = np.where(zero & sign, np.uint16(0x8000), bits)
    bits = np.where(zero & ~sign, np.uint16(0x0000), bits)
    out[...] = bits
    return out


def is_nonfinite_bits(bits):
    """True where a bf16 bit pattern is NaN or +-Inf (exponent all ones)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b & np.uint16(0x7F80)) == np.uint16(0x7F80)


def is_nan_bits(bits):
    b = np.asarray(bits, dtype=np.uint16)
    return ((b & np.uint16(0x7F80)) == np.uint16(0x7F80)) & ((b & np.uint16(0x007F)) != 0)

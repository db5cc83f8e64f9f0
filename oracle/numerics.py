"""bfloat16 <-> fp64 for the oracle (test infrastructure only).

bfloat16 is the top half of an IEEE binary32: 1 sign bit, 8 exponent bits and
7 stored mantissa bits (8 significant bits).  The GPU path stores activations
in bfloat16 with round-to-nearest-even; the oracle rounds its fp64 values to
the same format at the same points, directly from fp64 (no detour through
float32, so there is no double rounding).
"""

import numpy as np

_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def bf16_decode(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> fp64, exactly."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def round_bf16(x) -> np.ndarray:
    """Round fp64 values to the nearest bfloat16 value (ties to even).

    Write |x| = m * 2**e with m in [0.5, 1).  A normal bfloat16 keeps 8
    significant bits, so the spacing there is 2**(e - 8); below the smallest
    normal (2**-126, i.e. e < -125) the spacing stays at 2**-133.  Scaling by a
    power of two is exact, and ``numpy.round`` rounds halves to even.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    q = np.maximum(e, -125) - 8
    r = np.ldexp(np.round(np.ldexp(x, -q)), q)
    r = np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, x), r)
    return np.where(np.isfinite(x), r, x)

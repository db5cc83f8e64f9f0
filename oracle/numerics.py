"""bfloat16 <-> fp64 for the oracle (test infrastructure only).

bfloat16 is the top half of an IEEE binary32: 1 sign bit, 8 exponent bits and
7 stored mantissa bits (8 significant bits).  The GPU path stores activations
in bfloat16 with round-to-nearest-even; the oracle rounds its fp64 values to
the same format at the same points, directly from fp64 (no detour through
float32, so there is no double rounding).
"""

import numpy as np

_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127
_CHUNK = 1 << 16  # elements per pass (cache-sized)


def bf16_decode(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> fp64, exactly."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def round_bf16(x) -> np.ndarray:
    """Round fp64 values to the nearest bfloat16 value (ties to even).

    A normal bfloat16 keeps the sign, the exponent and the top 7 of fp64's 52
    stored mantissa bits.  Round to nearest even on the fp64 bit pattern:
    add 2**44 - 1 plus the lowest kept bit, then clear the 45 dropped bits (a
    carry out of the mantissa correctly bumps the exponent).  Below the
    smallest normal bfloat16 (2**-126) the spacing stays at 2**-133: there the
    value is scaled by a power of two (exact) and rounded with numpy.round,
    which rounds halves to even.  Results above the largest bfloat16 become
    infinities; NaN and infinities pass through.
    """
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty_like(x)
    xf, of = x.reshape(-1), out.reshape(-1)
    keep = np.uint64(45)
    bias = np.uint64((1 << 44) - 1)
    for s in range(0, xf.size, _CHUNK):
        xc = xf[s:s + _CHUNK]
        t = xc.view(np.uint64) >> keep
        t &= np.uint64(1)
        t += bias
        t += xc.view(np.uint64)
        t >>= keep
        t <<= keep
        r = t.view(np.float64)
        a = np.abs(xc)
        if not (np.all(a >= 2.0 ** -126) and np.all(a <= _BF16_MAX)):  # rare: tiny, huge, inf, nan
            small = a < 2.0 ** -126
            r = np.where(small, np.ldexp(np.round(np.ldexp(xc, 133)), -133), r)
            r = np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, xc), r)
            r = np.where(np.isfinite(xc), r, xc)
        of[s:s + _CHUNK] = r
    return out

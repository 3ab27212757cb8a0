"""A brute-force MXFP4 element quantiser for the oracle's pins, written from
the format definitions alone: the block scale 2^(floor(log2 amax) - 2)
(floor(log2) from math.frexp, clamped below at 2^-127), and the code of the
nearest E2M1 magnitude by exhaustive search over the eight magnitudes, an
exact tie going to the even code, the sign kept in bit 3."""
import math

MAGS = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]   # E2M1 magnitudes, codes 0..7


def scale_exp(amax):
    """Exponent e of the block scale 2^e for a finite block maximum."""
    if amax == 0.0:
        return -127
    return max(math.frexp(amax)[1] - 1 - 2, -127)


def nearest_code(v, e):
    """Code (0..15) of v / 2^e rounded to the nearest E2M1 value."""
    y = abs(v) / 2.0 ** e
    best = None
    for code, m in enumerate(MAGS):
        d = abs(y - m)
        if best is None or d < best[0] or (d == best[0] and code % 2 == 0):
            best = (d, code)
    return best[1] | (8 if math.copysign(1.0, v) < 0 else 0)


def code_value(code, e):
    m = MAGS[code & 7] * 2.0 ** e
    return -m if code & 8 else m

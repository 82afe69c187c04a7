"""Direct float64 -> bfloat16 rounding (round to nearest, ties to even).

bfloat16 keeps 8 significant bits (1 implicit + 7 stored) and float32's
exponent range. A value in the binade [2^(e-1), 2^e) has a spacing of
2^(e-8); below the smallest normal (2^-126) the spacing is fixed at 2^-133.
Rounding is done in one step from float64 (scale to an integer grid, np.rint,
which rounds half to even, scale back), never via float32: two roundings can
differ from one on values just above a tie.

Used only by the storage-emulating oracle, to model values a bf16 device cache
holds.
"""
import numpy as np

_BF16_MAX = float.fromhex("0x1.fep127")          # largest finite bfloat16
_OVERFLOW = float.fromhex("0x1.ffp127")          # halfway to 2^128: rounds to inf


def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, returned as float64."""
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, dtype=np.float64, copy=True)
    fin = np.isfinite(x) & (x != 0.0)
    if np.any(fin):
        v = x[fin]
        _, e = np.frexp(v)                        # v = m * 2^e, 0.5 <= |m| < 1
        spacing_exp = np.maximum(e - 8, -133)     # bf16 spacing in this binade
        r = np.ldexp(np.rint(np.ldexp(v, -spacing_exp)), spacing_exp)
        big = np.abs(v) >= _OVERFLOW
        r[big] = np.copysign(np.inf, v[big])
        out[fin] = r
    return out


def is_bf16_exact(x) -> bool:
    """True when every value is representable in bfloat16."""
    x = np.asarray(x, dtype=np.float64)
    return bool(np.all((round_bf16(x) == x) | np.isnan(x)))

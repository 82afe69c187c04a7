"""Direct float64 -> 8-bit float rounding in the E4M3 format of the OCP 8-bit
floating point specification, saturating (round to nearest, ties to even).

E4M3 holds a sign, 4 exponent bits with bias 7 and 3 stored mantissa bits. It has no
infinities: exponent 15 with mantissa 7 is NaN, so the largest finite magnitude is
1.75 * 2^8 = 448. A normal value has 4 significant bits, so in the binade
[2^(e-1), 2^e) the spacing is 2^(e-4); the smallest normal is 2^-6, and below it the
subnormals m * 2^-9 (m = 1..7) keep the spacing 2^-9.

Rounding is one step from float64 onto that grid (scale, np.rint -- half to even --,
scale back). Magnitudes beyond 448 saturate to +-448: the conversion this models
clamps its input to [-448, 448] first, which gives the same result. The sign of a
value that rounds to zero is kept.

Used only by the storage-emulating oracle, to model values an fp8 device cache holds.
"""
import numpy as np

E4M3_MAX = 448.0
E4M3_MIN_NORMAL = 2.0 ** -6
E4M3_SUBNORMAL_SPACING = 2.0 ** -9


def round_e4m3(x) -> np.ndarray:
    """Round float64 values to the nearest E4M3 value (saturating), returned as float64."""
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, dtype=np.float64, copy=True)
    fin = np.isfinite(x) & (x != 0.0)
    if np.any(fin):
        v = np.clip(x[fin], -E4M3_MAX, E4M3_MAX)
        _, e = np.frexp(v)                        # v = m * 2^e, 0.5 <= |m| < 1
        spacing_exp = np.maximum(e - 4, -9)       # E4M3 spacing in this binade
        r = np.ldexp(np.rint(np.ldexp(v, -spacing_exp)), spacing_exp)
        out[fin] = np.clip(r, -E4M3_MAX, E4M3_MAX)
    inf = np.isinf(x)
    out[inf] = np.copysign(E4M3_MAX, x[inf])
    return out


def is_e4m3_exact(x) -> bool:
    """True when every value is representable in E4M3."""
    x = np.asarray(x, dtype=np.float64)
    return bool(np.all((round_e4m3(x) == x) | np.isnan(x)))

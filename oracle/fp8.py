"""Plain fp8 group quantisation (test infrastructure only; see the package docstring).

WarpDrive page, kernel 1 (fp8_quant): float32 activations are cut into groups
of 64-128 elements; per group the absolute maximum gives the scale
absmax / 448.0, the elements are divided by it and clamped to [-448, 448], and
stored as FP8. Readings where the page is silent: groups run along the last
axis; the FP8 format is E4M3 with 448 as its largest finite value (the "fn"
variant: no infinities), reached by round-to-nearest-even; the division and
the scale are float32 operations (the activations are float32); a group whose
absolute maximum is 0 gets scale 0 and all-zero codes.
"""

import numpy as np

FP8_MAX = 448.0


def e4m3_encode(y):
    """E4M3 ("fn") codes of float32 values with |y| <= 448, round to nearest even.

    Format: sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0
    holds the subnormals m * 2^-9; 0x7F / 0xFF are NaN (never produced here).
    Returns uint8 codes.
    """
    y = np.asarray(y, dtype=np.float32)
    if np.any(np.abs(y) > FP8_MAX) or not np.all(np.isfinite(y)):
        raise ValueError("e4m3_encode takes finite values within [-448, 448]")
    a = np.abs(y).astype(np.float64)  # exact
    sign = np.signbit(y).astype(np.uint8) << 7
    code = np.zeros(y.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    # subnormals (and the step up to the smallest normal): multiples of 2^-9
    code[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)
    # normals: a = 2^e (1 + f), f in [0, 1); 3 fraction bits, ties to even
    nrm = ~sub
    frac, ex = np.frexp(a[nrm])        # a = frac * 2^ex, frac in [0.5, 1)
    e = ex - 1
    m = np.rint((frac * 2.0 - 1.0) * 8.0).astype(np.int64)
    carry = m == 8
    m[carry] = 0
    e[carry] += 1
    code[nrm] = ((e + 7) << 3) | m
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def e4m3_decode(codes):
    """Values of E4M3 ("fn") codes (NaN codes excluded), as float64."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    ef, m = (c >> 3) & 0xF, c & 0x7
    val = np.where(ef == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (ef - 7.0))
    return s * val


def fp8_quant(x, group):
    """Group quantisation of float32 ``x`` [..., C] (C a multiple of ``group``).

    Returns (codes uint8 [..., C], scales float32 [..., C / group]).
    """
    x = np.asarray(x, dtype=np.float32)
    C = x.shape[-1]
    if C % group:
        raise ValueError("the last dimension must be a multiple of the group size")
    xg = x.reshape(*x.shape[:-1], C // group, group)
    absmax = np.max(np.abs(xg), axis=-1)
    scale = (absmax / np.float32(FP8_MAX)).astype(np.float32)  # float32 division
    with np.errstate(divide="ignore", invalid="ignore"):
        y = np.where(scale[..., None] > 0, xg / scale[..., None], np.float32(0.0)).astype(np.float32)
    y = np.clip(y, -FP8_MAX, FP8_MAX).astype(np.float32)
    return e4m3_encode(y).reshape(x.shape), scale

"""Number formats: bfloat16, E4M3 (OCP FP8, "fn" variant) and E2M1 (FP4).

Test infrastructure only (see the package docstring). Plain definitions, each
written out in full: a value table plus nearest-with-ties-to-even selection.
"""
from __future__ import annotations

import numpy as np

# E2M1 magnitudes by code 0..7: the value set that NVFP4 element codes take.
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float32)
# Midpoints between consecutive magnitudes; midpoint k separates code k from k+1.
_E2M1_MID = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bits -> float32 by placing the 16 bits in the top half of a word.

    PR, Optimization item 6: bfloat16 is float32 with the low half dropped, so
    widening is an exact 16-bit left shift.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bits, round to nearest, ties to even (finite inputs).

    Blog, QK Norm: the normalized value is cast back to the input element type;
    the cast is read as IEEE round-to-nearest-even.
    """
    x = np.asarray(x, dtype=np.float32)
    assert np.all(np.isfinite(x)), "oracle inputs must be finite"
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def f64_to_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> bfloat16 bits with a single round-to-nearest-even step.

    bfloat16 keeps 8 significant bits for binary exponents >= -126 and a fixed
    quantum of 2**-133 below that. The value is divided by its quantum (exact,
    a power of two), rounded to an integer with ties to even (``np.rint``) and
    scaled back; the result is then exactly a bfloat16 value.
    """
    x = np.asarray(x, dtype=np.float64)
    assert np.all(np.isfinite(x)), "oracle inputs must be finite"
    a = np.abs(x)
    _, e = np.frexp(a)            # a = m * 2**e with m in [0.5, 1)
    e = e.astype(np.int64) - 1     # binary exponent: a in [2**e, 2**(e+1))
    e = np.maximum(e, -126)
    q = np.ldexp(np.ones_like(a), (e - 7).astype(np.int32))
    r = np.rint(a / q) * q
    r = np.where(a == 0.0, 0.0, r)
    out = np.copysign(r, x).astype(np.float32)   # exact: r is a bfloat16 value
    assert np.all(np.isfinite(out)), "bfloat16 overflow"
    return (out.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _e4m3_table() -> np.ndarray:
    """Values of the 127 non-negative finite E4M3 codes 0x00..0x7E (bias 7)."""
    vals = np.zeros(127, dtype=np.float64)
    for c in range(127):
        e, m = c >> 3, c & 7
        vals[c] = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_E4M3 = _e4m3_table()          # increasing in code
E4M3_MAX = 448.0


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """E4M3 codes (non-negative, 0x00..0x7E) -> float32 values."""
    c = np.asarray(codes, dtype=np.int64)
    assert np.all((c >= 0) & (c <= 0x7E)), "only non-negative finite scale codes occur"
    return _E4M3[c].astype(np.float32)


def e4m3_encode(s: np.ndarray) -> np.ndarray:
    """Non-negative float32 -> E4M3 code: nearest value, ties to even code, saturate at 448.

    Reading R-bscale: the pages name only the E2M1 conversion as saturating;
    the FP8 block scale is read as round-to-nearest-even with saturation to
    the largest finite value and subnormals kept.
    """
    s = np.asarray(s, dtype=np.float32).astype(np.float64)
    assert np.all(np.isfinite(s) | (s == np.inf)) and np.all(s >= 0)
    s = np.minimum(s, E4M3_MAX)
    hi = np.searchsorted(_E4M3, s, side="left")          # first value >= s
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    exact = _E4M3[hi] == s
    d_lo = s - _E4M3[lo]
    d_hi = _E4M3[hi] - s
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(exact, hi, np.where(pick_hi, hi, lo))
    return code.astype(np.uint8)


def e2m1_encode(v: np.ndarray) -> np.ndarray:
    """float32 -> 4-bit E2M1 code, round to nearest, ties to even, saturate, keep sign.

    PR, Optimization item 3 (the saturating round-to-nearest conversion). The
    magnitude code is the number of midpoints strictly below |v| plus one for a
    tie at an odd midpoint (moving the tie to the even code); |v| > 6 exceeds
    all seven midpoints and lands on 6 (code 7). Reading R-e2m1: the sign bit
    (0x8) follows the sign of v, so -0 and small negatives give 0x8.
    """
    v = np.asarray(v, dtype=np.float32)
    assert not np.any(np.isnan(v)), "oracle inputs must not be NaN"
    a = np.abs(v)[..., None]
    mid = _E2M1_MID
    k = np.arange(7)
    mag = np.sum(a > mid, axis=-1) + np.sum((a == mid) & (k % 2 == 1), axis=-1)
    sign = np.signbit(v).astype(np.uint8) << np.uint8(3)
    return (mag.astype(np.uint8) | sign).astype(np.uint8)


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """4-bit E2M1 codes -> float32 values (code 0x8 decodes to -0.0)."""
    c = np.asarray(codes, dtype=np.uint8)
    mag = E2M1_VALUES[c & 7]
    return np.where((c & 8) != 0, -mag, mag).astype(np.float32)


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """[..., 2n] 4-bit codes -> [..., n] bytes; reading R-nibble: element 2i in the low nibble.

    PR, Correctness: the nibble order is part of the format and a wrong order
    must fail the comparison loudly.
    """
    c = np.asarray(codes, dtype=np.uint8)
    assert c.shape[-1] % 2 == 0
    return (c[..., 0::2] | (c[..., 1::2] << np.uint8(4))).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """Inverse of :func:`pack_nibbles`."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & np.uint8(0xF)
    out[..., 1::2] = p >> np.uint8(4)
    return out

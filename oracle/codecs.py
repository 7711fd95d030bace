"""Element codecs: e4m3fn, e2m1, e8m0 and bf16 (oracle; test infrastructure).

The pages name the formats only (NVFP4 = e2m1 elements with an e4m3 scale per
16, MXFP8 = e4m3 elements with an e8m0 scale per 32: [MegaMoE drop workflow,
§3 "kernel_helpers.py", the per-block-16 / per-block-32 quantise helpers]).
Their bit-level definitions are the OCP 8-bit floating point and OCP
Microscaling (MX) v1.0 formats:

* e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities;
  S.1111.111 is NaN; largest finite 448; subnormals m/8 * 2^-6.
* e2m1: 1 sign, 2 exponent (bias 1), 1 mantissa bit: {0, .5, 1, 1.5, 2, 3, 4, 6}.
* e8m0: unsigned power of two 2^(b-127); 0xFF is NaN.
* bf16: the top 16 bits of an IEEE fp32.

Encoders round to nearest, ties to the even code, and saturate to the largest
finite magnitude (satfinite).  Reading (the pages are silent): the sign bit is
always carried over, so a value that rounds to zero keeps its sign.

Everything here works on float64 numpy arrays holding exact values; the table
look-ups and midpoint comparisons are exact, so no rounding other than the
one being defined happens.
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------- e4m3fn


def _e4m3_magnitude_table() -> np.ndarray:
    """Values of the 127 finite non-negative e4m3fn codes 0x00..0x7E (ascending)."""
    vals = np.empty(127, np.float64)
    for c in range(127):
        e, m = c >> 3, c & 7
        vals[c] = (m / 8.0) * 2.0**-6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


E4M3_MAG = _e4m3_magnitude_table()
E4M3_MAX = 448.0

# e2m1 magnitudes, index = 3-bit magnitude code
E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E2M1_MAX = 6.0


def _rne_index_small(a: np.ndarray, mags: np.ndarray, scale=None) -> np.ndarray:
    """Index of the entry of the short ascending table `mags` (times `scale`)
    nearest to a >= 0; ties go to the even index; saturates at the last entry.

    The index is the number of midpoints that a lies beyond: midpoint i sits
    between entries i and i+1, and a value exactly on it moves up only when
    i + 1 is even.  With a per-element scale the midpoints are mid_i * scale,
    which is exact for the short dyadic tables used here.
    """
    a = np.asarray(a, np.float64)
    mids = (mags[:-1] + mags[1:]) * 0.5
    s = 1.0 if scale is None else np.asarray(scale, np.float64)
    idx = np.zeros(a.shape, np.int64)
    for i, m in enumerate(mids):
        t = m * s
        idx += (a > t) | ((a == t) & (i % 2 == 1))
    return idx


def _check_finite(v: np.ndarray) -> None:
    if not np.all(np.isfinite(v)):
        raise ValueError("codec input must be finite")


def e4m3_decode(codes) -> np.ndarray:
    c = np.asarray(codes, np.uint8).astype(np.int64)
    mag = c & 0x7F
    val = E4M3_MAG[np.minimum(mag, 126)]
    val = np.where(mag == 0x7F, np.nan, val)
    return np.where(c & 0x80, -val, val)


def e4m3_encode(v) -> np.ndarray:
    """Round-to-nearest-even, saturating e4m3fn encoding of exact values."""
    v = np.asarray(v, np.float64)
    _check_finite(v)
    a = np.abs(v)
    # ascending table: mags[idx] <= a < mags[idx + 1]; round to the nearer of
    # the two, ties to the even code; a >= 448 saturates to code 0x7E.
    idx = np.clip(np.searchsorted(E4M3_MAG, a, side="right") - 1, 0, 126)
    nxt = np.minimum(idx + 1, 126)
    mid = (E4M3_MAG[idx] + E4M3_MAG[nxt]) * 0.5  # exact
    up = (a > mid) | ((a == mid) & (idx % 2 == 1))
    mag = np.where(idx >= 126, 126, idx + up)
    sign = np.signbit(v).astype(np.int64) << 7
    return (mag | sign).astype(np.uint8)


# ----------------------------------------------------------------- e2m1


def e2m1_decode(codes) -> np.ndarray:
    c = np.asarray(codes, np.uint8).astype(np.int64) & 0xF
    val = E2M1_MAG[c & 7]
    return np.where(c & 8, -val, val)


def e2m1_encode(v, scale=None) -> np.ndarray:
    """e2m1 code (0..15) of v / scale, rounded to nearest even, saturating.

    With a scale, |v| is compared against the exact scaled table
    {0, .5, 1, 1.5, 2, 3, 4, 6} * scale (and its midpoints), so no division
    rounding enters.  scale must be > 0 where given.
    """
    v = np.asarray(v, np.float64)
    _check_finite(v)
    mag = _rne_index_small(np.abs(v), E2M1_MAG, scale)
    sign = np.signbit(v).astype(np.int64) << 3
    return (mag | sign).astype(np.uint8)


def pack_e2m1(codes: np.ndarray) -> np.ndarray:
    """Two e2m1 codes per byte along the last axis: element 2i in the low nibble."""
    c = np.asarray(codes, np.uint8)
    assert c.shape[-1] % 2 == 0
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def unpack_e2m1(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


# ----------------------------------------------------------------- e8m0


def e8m0_decode(b) -> np.ndarray:
    b = np.asarray(b, np.uint8).astype(np.int64)
    return np.where(b == 255, np.nan, np.ldexp(1.0, b - 127))


# ----------------------------------------------------------------- bf16

BF16_MAX = (2.0 - 2.0**-7) * 2.0**127


def bf16_decode(bits) -> np.ndarray:
    b = np.asarray(bits, np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):  # NaN payloads widen to NaN
        return b.view(np.float32).astype(np.float64)


def bf16_encode(v) -> np.ndarray:
    """Nearest bf16 (8 significant bits, fp32 exponent range), ties to even.

    Written from the definition: v = m * 2^e with m in [0.5, 1); the bf16
    quantum at that binade is 2^(e-8) (never below the subnormal quantum
    2^-133); round v / quantum to the nearest integer, ties to even (numpy
    rint), and scale back.  Overflow beyond the largest finite bf16 after
    rounding gives infinity, as an IEEE cast does.
    """
    v = np.asarray(v, np.float64)
    if np.any(np.isnan(v)):
        raise ValueError("bf16_encode: NaN input")
    a = np.abs(v)
    _, e = np.frexp(a)
    q = np.maximum(e - 8, -133)
    n = np.rint(np.ldexp(a, -q))
    r = np.ldexp(n, q)
    r = np.where(r > BF16_MAX, np.inf, r)
    r = np.where(np.signbit(v), -r, r)
    bits = r.astype(np.float32).view(np.uint32) >> 16  # r is bf16-exact
    return bits.astype(np.uint16)

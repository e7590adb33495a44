"""Number formats: bf16 storage, OCP FP8 E4M3 ("E4M3FN", max 448), E8M0.

Test infrastructure (see the package docstring): never used by the product path.

The pages name the formats only: FP8 and MXFP8 in "NVIDIA TransformerEngine
PyTorch Ext Normalization" (Overview, Description) and MXFP8Tensor in
"core.tensor_parallel.inference_layers" (``_apply_linear``). The maximum 448
used by the per-tensor scale fixes the E4M3 variant as OCP E4M3 (not the
"FNUZ" variant whose maximum is 240). Definitions below follow the OCP OFP8
specification rev. 1.0 (E4M3: bias 7, no infinities, S.1111.111 is NaN) and
OCP MX v1.0 (E8M0: an unsigned biased power of two, bias 127, 0xFF is NaN).
"""

import numpy as np

E4M3_MAX = 448.0
E4M3_BIAS = 7


# ---------------------------------------------------------------- bf16 -----
def bf16_to_f64(bits):
    """Exact value of bf16 numbers stored as uint16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def bf16_to_f32(bits):
    """bf16 bit patterns widened to float32 (exact)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f64_to_bf16(v):
    """Round finite fp64 values to the nearest bf16, ties to even (IEEE round-to-nearest-even),
    returned as uint16 bit patterns.

    bf16 keeps 8 significand bits (7 stored) and fp32's exponent range: a value of magnitude
    in [2^e, 2^(e+1)) sits on a grid of spacing 2^(e-7), subnormals (e < -126) on the grid
    2^-133. The value is divided by its grid spacing (exact: a power of two), rounded to the
    nearest integer with ties to even (numpy rint), and multiplied back (exact); the result
    is a bf16 value, read off as the top half of its fp32 bits. Magnitudes at or above
    2^128 - 2^119 round to infinity; zeros keep their sign.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, e2 = np.frexp(np.where(a > 0, a, 1.0))           # a = f * 2^e2, f in [0.5, 1)
    e = np.maximum(e2.astype(np.int64) - 1, -126)       # floor(log2 a), subnormals share -126
    ulp = np.ldexp(1.0, e - 7)
    r = np.rint(v / ulp) * ulp                          # exact: |v/ulp| < 2^9
    r = np.where(a > 0, r, v)                           # keep signed zeros
    with np.errstate(over="ignore"):
        f = r.astype(np.float32)                        # exact (r is a bf16 value) or +-inf
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ---------------------------------------------------------------- E4M3 -----
def e4m3_decode(codes):
    """Value of each E4M3 byte (OCP OFP8: sign, 4-bit exponent bias 7, 3-bit mantissa).

    normal (e > 0):    (-1)^s * 2^(e-7) * (1 + m/8)
    subnormal (e = 0): (-1)^s * 2^-6 * (m/8)
    S.1111.111:        NaN (the only non-finite code; no infinities)
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - E4M3_BIAS))
    val = np.where(s == 1, -mag, mag)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


# The 127 finite non-negative E4M3 values, indexed by their code 0x00..0x7E.
# Codes of one sign are ordered like their magnitudes, so this is ascending.
_E4M3_GRID = e4m3_decode(np.arange(0x7F, dtype=np.uint8))


def e4m3_encode(v):
    """Round float32 values to E4M3 codes.

    Rounding: to the nearest representable magnitude, ties to the code with an
    even mantissa (round-to-nearest-even). Overflow: magnitudes at or above
    448 give +-448 (code 0x7E | sign), the saturating conversion OCP OFP8
    allows for E4M3 (the pages are silent; saturation is the reading taken).
    Signed zero: the sign bit is kept, so tiny negatives give 0x80.
    NaN gives 0x7F | sign.
    """
    x = np.asarray(v, dtype=np.float32)
    a = np.abs(x.astype(np.float64))
    neg = np.signbit(x)
    nan = np.isnan(x)
    a = np.where(nan, 0.0, np.minimum(a, E4M3_MAX))
    hi = np.searchsorted(_E4M3_GRID, a, side="left")          # first grid value >= a
    hi = np.minimum(hi, len(_E4M3_GRID) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _E4M3_GRID[lo]
    d_hi = _E4M3_GRID[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == _E4M3_GRID[hi], hi, code)             # exact hits
    code = code.astype(np.uint8) | np.where(neg, 0x80, 0).astype(np.uint8)
    return np.where(nan, np.uint8(0x7F) | np.where(neg, 0x80, 0).astype(np.uint8), code).astype(np.uint8)


# ---------------------------------------------------------------- E8M0 -----
def e8m0_decode(s):
    """E8M0 shared scale (OCP MX v1.0): 2^(s-127); 0xFF is NaN."""
    b = np.asarray(s, dtype=np.uint8).astype(np.int64)
    return np.where(b == 0xFF, np.nan, np.ldexp(1.0, b - 127))

"""Pins of the oracle's MXFP8 grouped forward and its bf16 encoder.

The encoder is pinned against every bf16 pattern, exact midpoints (ties to even) and torch's
float32 -> bfloat16 conversion. The composed MXFP8 grouped MLP forward is pinned against a
brute-force pure-Python evaluation on tiny shapes: exact rationals for the roundings, a scan
over all 256 E4M3 codes for the nearest code, and math.fsum for the dot products.
"""

import math
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

import synth
from oracle import grouped
from oracle.codecs import bf16_to_f64, f64_to_bf16

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ------------------------------------------------------------- bf16 encoder
def test_bf16_encoder_round_trips_every_finite_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = bf16_to_f64(bits)
    fin = np.isfinite(v)
    assert np.array_equal(f64_to_bf16(v[fin]), bits[fin])        # includes -0 and subnormals


def test_bf16_encoder_ties_to_even_and_nearest():
    rng = np.random.default_rng(3)
    b = rng.integers(0x0080, 0x7F00, size=2000, dtype=np.uint16)   # positive normals, not the largest
    lo, hi = bf16_to_f64(b), bf16_to_f64(b + 1)
    mid = (lo + hi) / 2                                             # exact in fp64
    even = np.where(b % 2 == 0, b, b + 1).astype(np.uint16)
    assert np.array_equal(f64_to_bf16(mid), even)
    assert np.array_equal(f64_to_bf16(-mid), even | 0x8000)
    up, down = np.nextafter(mid, np.inf), np.nextafter(mid, -np.inf)
    assert np.array_equal(f64_to_bf16(up), (b + 1).astype(np.uint16))
    assert np.array_equal(f64_to_bf16(down), b)


def test_bf16_encoder_matches_torch_on_float32_values():
    rng = np.random.default_rng(4)
    x = np.concatenate([rng.standard_normal(50000), rng.standard_normal(20000) * 1e-38,
                        rng.standard_normal(20000) * 1e30]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f64_to_bf16(x.astype(np.float64)), ref)


# --------------------------------------------------- brute-force MX pipeline
def _e4m3_values():
    """All finite E4M3FN codes and their values, from the format: bias 7, 3 mantissa bits,
    exponent field 0 subnormal, S.1111.111 NaN."""
    out = []
    for code in range(256):
        s, e, m = code >> 7, (code >> 3) & 15, code & 7
        if e == 15 and m == 7:
            continue
        mag = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
        out.append((code, -mag if s else mag))
    return out


E4M3 = _e4m3_values()
E4M3_MAX = Fraction(448)


def _e4m3_nearest(v):
    """Nearest code by scan (saturating at +-448; ties to the even code; signed zero kept)."""
    v = Fraction(v)
    if v > E4M3_MAX:
        v = E4M3_MAX
    if v < -E4M3_MAX:
        v = -E4M3_MAX
    best = None
    for code, val in E4M3:
        d = abs(v - val)
        if best is None or d < best[0] or (d == best[0] and code % 2 == 0 and best[1] % 2 == 1):
            best = (d, code)
    code = best[1]
    if v == 0 or (code & 0x7F) == 0:                                # zero keeps the input's sign
        return 0x80 if (v < 0 or (v == 0 and math.copysign(1, float(v)) < 0)) else 0x00
    return code


def _bf16_value(bits):
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def _bf16_nearest_bits(v):
    """Nearest bf16 by comparing the two neighbours found from the float32 truncation."""
    f = struct.unpack("<I", struct.pack("<f", float(np.float32(v))))[0] >> 16
    cands = {(f + d) & 0xFFFF for d in (-1, 0, 1)}
    cands = [c for c in cands if math.isfinite(_bf16_value(c))]
    vv = Fraction(v)
    best = min(cands, key=lambda c: (abs(vv - Fraction(_bf16_value(c))), c % 2))
    return best


def _mx_block(vals):
    """E8M0 exponent and codes of one block (bf16 values): X = floor(log2 amax) - 8, clamped."""
    amax = max(abs(Fraction(v)) for v in vals)
    if amax == 0:
        X = -127
    else:
        e = 0
        while Fraction(2) ** (e + 1) <= amax:
            e += 1
        while Fraction(2) ** e > amax:
            e -= 1
        X = max(-127, min(127, e - 8))
    return X, [_e4m3_nearest(Fraction(v) / Fraction(2) ** X) for v in vals]


def _mx_rows(mat):
    """Rowwise MX of a list of rows of bf16 values -> dequantized rows, codes, exponents."""
    deq, codes, exps = [], [], []
    for row in mat:
        dr, cr, er = [], [], []
        for b0 in range(0, len(row), 32):
            X, cs = _mx_block(row[b0:b0 + 32])
            er.append(X + 127)
            cr.extend(cs)
            dr.extend(float(dict(E4M3)[c] * Fraction(2) ** X) if (c & 0x7F) else 0.0 for c in cs)
        deq.append(dr), codes.append(cr), exps.append(er)
    return deq, codes, exps


def test_mxfp8_grouped_forward_matches_brute_force():
    T, G, H, F = 6, 2, 32, 32
    splits = [4, 2]
    inp = synth.grouped(T, G, H, F, seed=5, splits=splits)
    base = np.concatenate([[0], np.cumsum(splits)])
    got = grouped.grouped_mlp_fwd_mxfp8(inp["x"], inp["w1"], inp["w2"], inp["p"], base)

    xs = [[_bf16_value(b) for b in r] for r in inp["x"]]
    xd, _, _ = _mx_rows(xs)
    yq_ref, ys_ref, out_ref = [], [], []
    for t in range(T):
        g = 0 if t < splits[0] else 1
        w1d, _, _ = _mx_rows([[_bf16_value(b) for b in r] for r in inp["w1"][g]])
        h = [math.fsum(xd[t][k] * w1d[n][k] for k in range(H)) for n in range(2 * F)]
        y = [float(inp["p"][t]) * (h[j] / (1 + math.exp(-h[j]))) * h[F + j] for j in range(F)]
        ybits = [_bf16_nearest_bits(v) for v in y]
        yd, yc, ye = _mx_rows([[_bf16_value(b) for b in ybits]])
        yq_ref.append(yc[0]), ys_ref.append(ye[0])
        w2d, _, _ = _mx_rows([[_bf16_value(b) for b in r] for r in inp["w2"][g]])
        out_ref.append([math.fsum(yd[0][k] * w2d[n][k] for k in range(F)) for n in range(H)])
    assert np.array_equal(got["y_q"], np.array(yq_ref, np.uint8))
    assert np.array_equal(got["y_s"], np.array(ys_ref, np.uint8))
    np.testing.assert_allclose(got["out"], np.array(out_ref), rtol=1e-12, atol=1e-12)

"""Pins of the oracle's quantized grouped path: MXFP8 forward and backward, FP8 current
scaling per group, and the bf16 encoder they round through.

The encoder is pinned against every bf16 pattern, exact midpoints (ties to even) and torch's
float32 -> bfloat16 conversion. The group layout is pinned on hand-worked offsets. Everything
else is pinned against brute-force pure-Python evaluations on tiny shapes: exact rationals for
the roundings, a scan over all 256 E4M3 codes for the nearest code, blocks and scales rebuilt
group by group, and math.fsum for the dot products.
"""

import math
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

import synth
from oracle import grouped, quant
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


# ------------------------------------------ MXFP8 grouped backward (token-blocked) ------
def test_mx_group_layout_hand_worked():
    # splits 300, 0, 211, 9, 0, 40: aligned lengths 384, 0, 256, 128, 0, 128
    base = [0, 300, 300, 511, 520, 520, 560]
    c, pad = quant.mx_group_layout(base, 560)
    assert c.tolist() == base
    assert pad.tolist() == [0, 384, 384, 640, 768, 768, 896]
    # out-of-order / out-of-range offsets are read as the grouped kernels read them
    c, pad = quant.mx_group_layout([5, -3, 10, 7, 100], 20)
    assert c.tolist() == [5, 5, 10, 10, 20]
    assert pad.tolist() == [0, 0, 128, 128, 256]
    c, pad = quant.mx_group_layout([0, 128, 256], 256)
    assert pad.tolist() == [0, 128, 256]                      # aligned groups are not padded


def _bf16_col(bits, j):
    return [_bf16_value(b) for b in bits[:, j]]


def _brute_token_blocks(bits, base, j):
    """{(g, b): (X, codes)} of column j: blocks of 32 from each group's first token."""
    col = _bf16_col(bits, j)
    out = {}
    for g in range(len(base) - 1):
        lo, hi = base[g], base[g + 1]
        for b, t0 in enumerate(range(lo, hi, 32)):
            out[(g, b)] = _mx_block(col[t0:min(t0 + 32, hi)])
    return out


def test_mxfp8_colwise_grouped_vs_brute_force():
    splits = [20, 0, 64, 7]
    base = [0, 20, 20, 84, 91]
    T, C = 91, 3
    r = synth.streams(8)
    x = synth.normal_bf16(r["x"], (T, C), 1.0, r["outliers_x"], outlier_rate=0.05)
    c, pad = quant.mx_group_layout(base, T)
    assert pad.tolist() == [0, 128, 128, 256, 384]
    q, s = quant.mxfp8_colwise_grouped(x, c, pad, 512)
    for j in range(C):
        blocks = _brute_token_blocks(x, base, j)
        want_q = np.zeros(512, np.uint8)
        want_s = np.zeros(16, np.uint8)                        # all-zero blocks: X = -127
        for (g, b), (X, codes) in blocks.items():
            p0 = pad[g] + 32 * b
            want_q[p0:p0 + len(codes)] = codes
            want_s[p0 // 32] = X + 127
        assert np.array_equal(q[j], want_q), j
        assert np.array_equal(s[j], want_s), j
    assert sum(splits) == T


def _deq(X, codes):
    table = dict(E4M3)
    return [float(table[cd] * Fraction(2) ** X) if (cd & 0x7F) else 0.0 for cd in codes]


def _token_blocked_values(bits, base, j):
    """Dequantized column j, token by token, from the brute-force token blocks."""
    vals = [0.0] * bits.shape[0]
    for (g, b), (X, codes) in _brute_token_blocks(bits, base, j).items():
        t0 = base[g] + 32 * b
        for i, v in enumerate(_deq(X, codes)):
            vals[t0 + i] = v
    return vals


def test_grouped_wgrad_mxfp8_vs_brute_force():
    base = [0, 40, 40, 75]
    T, N, K = 75, 2, 3
    r = synth.streams(9)
    dy = synth.normal_bf16(r["dy"], (T, N), 1e-2, r["outliers_dy"], outlier_rate=0.05)
    x = synth.normal_bf16(r["x"], (T, K), 1.0)
    got = grouped.grouped_linear_wgrad_mxfp8(dy, x, base, alpha=0.25)
    dyv = [_token_blocked_values(dy, base, n) for n in range(N)]
    xv = [_token_blocked_values(x, base, k) for k in range(K)]
    for g in range(3):
        for n in range(N):
            for k in range(K):
                ref = 0.25 * math.fsum(dyv[n][t] * xv[k][t] for t in range(base[g], base[g + 1]))
                assert got[g, n, k] == pytest.approx(ref, rel=1e-12, abs=1e-300), (g, n, k)
    assert not got[1].any()                                   # the empty group


def test_grouped_dgrad_mxfp8_vs_brute_force():
    base = [0, 3, 5]
    T, G, N, K = 5, 2, 64, 3
    r = synth.streams(10)
    dy = synth.normal_bf16(r["dy"], (T, N), 1.0, r["outliers_dy"], outlier_rate=0.05)
    w = synth.normal_bf16(r["w"], (G, N, K), 0.02, r["outliers_w"], outlier_rate=0.05)
    got = grouped.grouped_linear_dgrad_mxfp8(dy, w, base, alpha=-0.5)
    dyd, _, _ = _mx_rows([[_bf16_value(b) for b in row] for row in dy])
    for g in range(G):
        # W_g blocked along N: the rowwise blocks of its transpose
        wtd, _, _ = _mx_rows([[_bf16_value(b) for b in w[g][:, k]] for k in range(K)])
        for t in range(base[g], base[g + 1]):
            for k in range(K):
                ref = -0.5 * math.fsum(dyd[t][n] * wtd[k][n] for n in range(N))
                assert got[t, k] == pytest.approx(ref, rel=1e-12, abs=1e-300), (t, k)


def test_single_aligned_group_wgrad_equals_dense_mx_wgrad():
    T, N, K = 256, 64, 96
    r = synth.streams(11)
    dy = synth.normal_bf16(r["dy"], (T, N), 1.0)
    x = synth.normal_bf16(r["x"], (T, K), 1.0)
    got = grouped.grouped_linear_wgrad_mxfp8(dy, x, [0, T])[0]
    ref = quant.mx_dequantize(*quant.mxfp8_colwise(dy)) @ quant.mx_dequantize(*quant.mxfp8_colwise(x)).T
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-15)


def test_mxfp8_grouped_backward_matches_brute_force():
    T, G, H, F = 6, 2, 32, 32
    splits = [4, 2]
    base = [0, 4, 6]
    inp = synth.grouped(T, G, H, F, seed=6, splits=splits)
    got = grouped.grouped_mlp_bwd_mxfp8(inp["x"], inp["w1"], inp["w2"], inp["p"], base, inp["dout"])

    bits = lambda m: [[_bf16_value(b) for b in r] for r in m]   # noqa: E731
    xd, _, _ = _mx_rows(bits(inp["x"]))
    doutd, _, _ = _mx_rows(bits(inp["dout"]))
    grp = [0, 0, 0, 0, 1, 1]
    h_bits, y_bits, dh_bits, dh_q, dh_s, dp = [], [], [], [], [], []
    for t in range(T):
        g = grp[t]
        w1d, _, _ = _mx_rows(bits(inp["w1"][g]))
        h = [math.fsum(xd[t][k] * w1d[n][k] for k in range(H)) for n in range(2 * F)]
        hb = [_bf16_nearest_bits(v) for v in h]
        pt = float(inp["p"][t])
        y = [pt * (h[j] / (1 + math.exp(-h[j]))) * h[F + j] for j in range(F)]
        y_bits.append([_bf16_nearest_bits(v) for v in y])
        # fc2 dgrad: W2_g [H, F] blocked along H (rowwise blocks of its transpose)
        w2t, _, _ = _mx_rows([[_bf16_value(b) for b in inp["w2"][g][:, f]] for f in range(F)])
        gy = [math.fsum(doutd[t][n] * w2t[f][n] for n in range(H)) for f in range(F)]
        a = [_bf16_value(b) for b in hb[:F]]
        bb = [_bf16_value(b) for b in hb[F:]]
        sg = [1 / (1 + math.exp(-v)) for v in a]
        da = [gy[j] * pt * bb[j] * sg[j] * (1 + a[j] * (1 - sg[j])) for j in range(F)]
        db = [gy[j] * pt * a[j] * sg[j] for j in range(F)]
        dp.append(math.fsum(gy[j] * a[j] * sg[j] * bb[j] for j in range(F)))
        row = [_bf16_nearest_bits(v) for v in da + db]
        dh_bits.append(row)
        _, cq, ce = _mx_rows([[_bf16_value(b) for b in row]])
        dh_q.append(cq[0]), dh_s.append(ce[0])
    dh_bits = np.array(dh_bits, np.uint16)
    assert np.array_equal(got["dh_bits"], dh_bits)
    assert np.array_equal(got["dh_q"], np.array(dh_q, np.uint8))
    assert np.array_equal(got["dh_s"], np.array(dh_s, np.uint8))
    np.testing.assert_allclose(got["dp"], dp, rtol=1e-12, atol=1e-15)

    # fc1 dgrad: dh rowwise, W1_g [2F, H] blocked along 2F
    dhd, _, _ = _mx_rows(bits(dh_bits))
    for t in range(T):
        w1t, _, _ = _mx_rows([[_bf16_value(b) for b in inp["w1"][grp[t]][:, k]] for k in range(H)])
        ref = [math.fsum(dhd[t][n] * w1t[k][n] for n in range(2 * F)) for k in range(H)]
        np.testing.assert_allclose(got["dx"][t], ref, rtol=1e-12, atol=1e-15)
    # wgrads: token-blocked per group
    y_bits = np.array(y_bits, np.uint16)
    dov = [_token_blocked_values(inp["dout"], base, n) for n in range(H)]
    yv = [_token_blocked_values(y_bits, base, f) for f in range(F)]
    dhv = [_token_blocked_values(dh_bits, base, n) for n in range(2 * F)]
    xv = [_token_blocked_values(inp["x"], base, k) for k in range(H)]
    for g in range(G):
        ts = range(base[g], base[g + 1])
        dw2 = [[math.fsum(dov[n][t] * yv[f][t] for t in ts) for f in range(F)] for n in range(H)]
        dw1 = [[math.fsum(dhv[n][t] * xv[k][t] for t in ts) for k in range(H)] for n in range(2 * F)]
        np.testing.assert_allclose(got["dw2"][g], dw2, rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(got["dw1"][g], dw1, rtol=1e-12, atol=1e-15)


# ------------------------------------------ FP8 current scaling per group (grouped path) ------
def _f32(v):
    return float(np.float32(v))


def _fp8_tensor(vals):
    """Brute-force current scaling of a list of rows sharing one scale: (codes, dequantized rows,
    scale_inv). amax by Python max; scale = fp32(448 / amax); codes by a scan of fp32(v * scale)."""
    flat = [v for r in vals for v in r]
    a = max((abs(v) for v in flat), default=0.0)
    s = np.float32(1.0) if a == 0 else np.float32(448.0) / np.float32(a)
    sinv = _f32(np.float32(1.0) / s)
    codes = [[_e4m3_nearest(_f32(np.float32(v) * s)) for v in r] for r in vals]
    table = dict(E4M3)
    deq = [[float(table[cd]) * sinv if (cd & 0x7F) else 0.0 for cd in r] for r in codes]
    return codes, deq, sinv


def test_fp8_current_scaling_grouped_vs_brute_force():
    base = [0, 20, 20, 57, 60]
    T, C = 60, 5
    r = synth.streams(16)
    x = synth.normal_bf16(r["x"], (T, C), 1.0, r["outliers_x"], outlier_rate=0.05)
    c, pad = quant.mx_group_layout(base, T)
    got = quant.fp8_current_scaling_grouped(x, c, pad, 512)
    want_t = np.zeros((C, 512), np.uint8)
    for g in range(4):
        lo, hi = base[g], base[g + 1]
        codes, _, sinv = _fp8_tensor([[_bf16_value(b) for b in row] for row in x[lo:hi]])
        if hi > lo:
            assert np.array_equal(got["q"][lo:hi], np.array(codes, np.uint8)), g
            want_t[:, pad[g]:pad[g] + hi - lo] = np.array(codes, np.uint8).T
        assert got["scale_inv"][g] == np.float32(sinv), g
    assert got["scale"][1] == 1.0 and got["amax"][1] == 0.0               # the empty group
    assert np.array_equal(got["q_t"], want_t)


def test_fp8_grouped_mlp_fwd_bwd_match_brute_force():
    T, G, H, F = 5, 2, 32, 32
    splits = [3, 2]
    base = [0, 3, 5]
    grp = [0, 0, 0, 1, 1]
    inp = synth.grouped(T, G, H, F, seed=7, splits=splits)
    fwd = grouped.grouped_mlp_fwd_fp8(inp["x"], inp["w1"], inp["w2"], inp["p"], base)
    got = grouped.grouped_mlp_bwd_fp8(inp["x"], inp["w1"], inp["w2"], inp["p"], base, inp["dout"], fwd=fwd)

    vals = lambda m: [[_bf16_value(b) for b in r] for r in m]   # noqa: E731
    xd = [None] * T
    dod = [None] * T
    for g in range(G):
        lo, hi = base[g], base[g + 1]
        _, d, _ = _fp8_tensor(vals(inp["x"][lo:hi]))
        xd[lo:hi] = d
        _, d, _ = _fp8_tensor(vals(inp["dout"][lo:hi]))
        dod[lo:hi] = d
    w1d = [_fp8_tensor(vals(inp["w1"][g]))[1] for g in range(G)]
    w2d = [_fp8_tensor(vals(inp["w2"][g]))[1] for g in range(G)]
    h = [[math.fsum(xd[t][k] * w1d[grp[t]][n][k] for k in range(H)) for n in range(2 * F)] for t in range(T)]
    y_bits = [[_bf16_nearest_bits(float(inp["p"][t]) * (h[t][j] / (1 + math.exp(-h[t][j]))) * h[t][F + j])
               for j in range(F)] for t in range(T)]
    assert np.array_equal(fwd["y_bits"], np.array(y_bits, np.uint16))
    yd = [None] * T
    for g in range(G):
        lo, hi = base[g], base[g + 1]
        yd[lo:hi] = _fp8_tensor(vals(np.array(y_bits[lo:hi], np.uint16)))[1]
    out = [[math.fsum(yd[t][k] * w2d[grp[t]][n][k] for k in range(F)) for n in range(H)] for t in range(T)]
    np.testing.assert_allclose(fwd["out"], out, rtol=1e-12, atol=1e-15)

    dh_bits, dp = [], []
    for t in range(T):
        g = grp[t]
        gy = [math.fsum(dod[t][n] * w2d[g][n][f] for n in range(H)) for f in range(F)]
        hb = [_bf16_value(_bf16_nearest_bits(v)) for v in h[t]]
        a, b = hb[:F], hb[F:]
        pt = float(inp["p"][t])
        sg = [1 / (1 + math.exp(-v)) for v in a]
        da = [gy[j] * pt * b[j] * sg[j] * (1 + a[j] * (1 - sg[j])) for j in range(F)]
        db = [gy[j] * pt * a[j] * sg[j] for j in range(F)]
        dp.append(math.fsum(gy[j] * a[j] * sg[j] * b[j] for j in range(F)))
        dh_bits.append([_bf16_nearest_bits(v) for v in da + db])
    assert np.array_equal(got["dh_bits"], np.array(dh_bits, np.uint16))
    np.testing.assert_allclose(got["dp"], dp, rtol=1e-12, atol=1e-15)
    dhd = [None] * T
    for g in range(G):
        lo, hi = base[g], base[g + 1]
        dhd[lo:hi] = _fp8_tensor(vals(np.array(dh_bits[lo:hi], np.uint16)))[1]
    for t in range(T):
        w1 = w1d[grp[t]]
        ref = [math.fsum(dhd[t][n] * w1[n][k] for n in range(2 * F)) for k in range(H)]
        np.testing.assert_allclose(got["dx"][t], ref, rtol=1e-12, atol=1e-15)
    for g in range(G):
        ts = range(base[g], base[g + 1])
        dw2 = [[math.fsum(dod[t][n] * yd[t][f] for t in ts) for f in range(F)] for n in range(H)]
        dw1 = [[math.fsum(dhd[t][n] * xd[t][k] for t in ts) for k in range(H)] for n in range(2 * F)]
        np.testing.assert_allclose(got["dw2"][g], dw2, rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(got["dw1"][g], dw1, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("act", ["swiglu", "srelu"])
def test_requantized_bar_covers_fp32_accumulation(act):
    """The bar that the FP8 grouped MLP's GPU test puts on outputs fed by a requantized bf16
    intermediate, exercised on the CPU: fc1 accumulated in fp32 (as a GPU kernel does) instead
    of fp64 moves some bf16 activations by one step, and per-group E4M3 quantization can turn
    such a step into a neighbouring code; fc2's wgrad on those codes stays inside the bar."""
    from oracle import offsets
    from oracle.grouped import _ACTS, _fp8_experts_hat, _fp8_groups_hat, grouped_linear_wgrad
    from .helpers import TAU_FP8, assert_close_requantized

    splits = [300, 0, 211, 9, 0, 40]
    T, G = sum(splits), len(splits)
    inp = synth.grouped(T, G, 256, 256, seed=33, splits=splits, gated=act == "swiglu")
    base = offsets.base_offsets(inp["splits"])
    fwd = grouped.grouped_mlp_fwd_fp8(inp["x"], inp["w1"], inp["w2"], inp["p"], base, act)
    bwd = grouped.grouped_mlp_bwd_fp8(inp["x"], inp["w1"], inp["w2"], inp["p"], base, inp["dout"], fwd=fwd, act=act)
    c, _ = quant.mx_group_layout(base, T)
    xh = _fp8_groups_hat(inp["x"], c).astype(np.float32)
    w1h = _fp8_experts_hat(inp["w1"]).astype(np.float32)
    h32 = np.zeros((T, w1h.shape[1]), np.float32)
    for g in range(G):
        h32[base[g]:base[g + 1]] = xh[base[g]:base[g + 1]] @ w1h[g].T
    y_bits = f64_to_bf16(_ACTS[act][0](h32.astype(np.float64), inp["p"]).astype(np.float32).astype(np.float64))
    assert np.count_nonzero(y_bits != fwd["y_bits"]) > 0               # the case exercises the rounding
    dw2 = grouped_linear_wgrad(_fp8_groups_hat(inp["dout"], c), _fp8_groups_hat(y_bits, c), base)
    assert_close_requantized(dw2, bwd["dw2"], TAU_FP8, what="dw2")

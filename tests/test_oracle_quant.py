"""Pins of the oracle's quantizers: hand-derived golden blocks, library routines, invariants."""

import json
import math
import os

import numpy as np
import torch

from oracle import codecs, quant
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bf16(vals):
    return synth.f32_to_bf16_bits(np.asarray(vals, dtype=np.float32))


# ----------------------------------------------------------- per tensor -----
def test_fp8_current_scaling_golden():
    for case in _golden("fp8_current_scaling.json")["cases"]:
        x = _bf16(case["x"])[None, :]
        r = quant.fp8_current_scaling(x)
        assert float(r["amax"]) == case["amax"]
        if "scale_bits" in case:
            assert int(np.float32(r["scale"]).view(np.uint32)) == int(case["scale_bits"], 16)
        else:
            assert float(r["scale"]) == case["scale"]
            assert float(r["scale_inv"]) == case["scale_inv"]
        assert [int(c) for c in r["q"][0]] == [int(c, 16) for c in case["q"]], case["why"]


def test_amax_vs_torch():
    rng = np.random.default_rng(1)
    x = _bf16(rng.standard_normal((37, 53)).astype(np.float32) * 3)
    ref = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).float().abs().max().item()
    assert float(quant.amax(x)) == ref
    assert float(quant.amax(np.zeros((4, 4), np.uint16))) == 0.0


def test_fp8_scale_exhaustive_over_bf16_amax_vs_torch_division():
    """scale = 448/amax in fp32 for every positive finite bf16 amax (normals and subnormals)."""
    bits = np.arange(1, 0x7F80, dtype=np.uint16)            # +min subnormal .. +max finite
    a = codecs.bf16_to_f32(bits)
    ref = (torch.tensor(448.0, dtype=torch.float32) / torch.from_numpy(a)).numpy()
    ref = np.where(np.isfinite(ref), ref, np.finfo(np.float32).max).astype(np.float32)
    ours = np.array([quant.fp8_scale(v) for v in a], dtype=np.float32)
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))
    inv_ref = (torch.tensor(1.0) / torch.from_numpy(ref)).numpy()
    inv = np.array([quant.fp8_scale_inv(s) for s in ours], dtype=np.float32)
    assert np.array_equal(inv.view(np.uint32), inv_ref.view(np.uint32))


def test_fp8_amax_element_reaches_448():
    """x_amax * fp32(448/x_amax) is within an fp32 ulp of 448, so it encodes to +-448.

    Holds whenever the quotient does not overflow (amax >= 2^-119)."""
    bits = np.arange(0x0400, 0x7F80, dtype=np.uint16)        # 2^-119 .. max finite
    a = codecs.bf16_to_f32(bits)
    for sign in (1, -1):
        for v in a[::7]:
            q = quant.fp8_quantize_with_scale(_bf16([sign * v]), quant.fp8_scale(v))
            assert int(q[0]) == (0x7E | (0x80 if sign < 0 else 0)), v


def test_fp8_current_scaling_vs_torch_pipeline():
    for seed, (R, C), std in [(0, (64, 96), 1.0), (1, (33, 17), 1e-2), (2, (5, 300), 0.02)]:
        x = synth.normal_bf16(np.random.default_rng(seed), (R, C), std)
        r = quant.fp8_current_scaling(x)
        xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).float()
        amax = xt.abs().max()
        scale = torch.tensor(448.0) / amax
        q = (xt * scale).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert float(r["amax"]) == amax.item()
        assert np.float32(r["scale"]) == np.float32(scale.item())
        assert np.array_equal(r["q"], q)
        assert np.array_equal(r["q_t"], q.T)


def test_fp8_dequantize_within_half_step():
    x = synth.normal_bf16(np.random.default_rng(3), (50, 70), 1.0)
    r = quant.fp8_current_scaling(x)
    deq = quant.fp8_dequantize(r["q"], r["scale_inv"])
    xs = codecs.bf16_to_f64(x) * np.float64(r["scale"])
    # relative half-step of a 3-bit mantissa is 2^-4; below 2^-6 the step is 2^-9
    err = np.abs(deq * np.float64(r["scale"]) - xs)
    assert np.all(err <= np.maximum(np.abs(xs) * 2.0 ** -4, 2.0 ** -10) * (1 + 1e-6))


# ----------------------------------------------------------------- MX -------
def _golden_blocks():
    out = []
    for b in _golden("mx_blocks.json")["blocks"]:
        vals = np.full(32, b["fill"], dtype=np.float64)
        codes = np.full(32, int(b["codes"]["fill"], 16), dtype=np.uint8)
        for k, v in b["set"].items():
            vals[int(k)] = v
        for k, c in b["codes"].items():
            if k != "fill":
                codes[int(k)] = int(c, 16)
        out.append((b, vals, codes))
    return out


def test_mx_golden_blocks_rowwise():
    for b, vals, codes in _golden_blocks():
        x = _bf16(vals)
        assert np.array_equal(codecs.bf16_to_f64(x), vals), ("fixture not exact in bf16", b["name"])
        q, s = quant.mxfp8_rowwise(x[None, :])
        assert int(s[0, 0]) == b["scale"], (b["name"], b["why"])
        assert np.array_equal(q[0], codes), (b["name"], q[0], codes, b["why"])


def test_mx_golden_blocks_colwise_orientation():
    """Blocks placed down the columns of a [64, 3] matrix come back in q_colT rows."""
    blocks = _golden_blocks()
    cols = [(blocks[i], blocks[j]) for i, j in [(0, 6), (7, 1), (9, 4)]]
    mat = np.zeros((64, 3), np.float64)
    for c, (top, bot) in enumerate(cols):
        mat[:32, c] = top[1]
        mat[32:, c] = bot[1]
    qT, sT = quant.mxfp8_colwise(_bf16(mat))
    assert qT.shape == (3, 64) and sT.shape == (3, 2)
    for c, (top, bot) in enumerate(cols):
        assert int(sT[c, 0]) == top[0]["scale"] and int(sT[c, 1]) == bot[0]["scale"]
        assert np.array_equal(qT[c, :32], top[2]) and np.array_equal(qT[c, 32:], bot[2])


def test_mx_e8m0_decode_of_scales_matches_torch():
    x = synth.normal_bf16(np.random.default_rng(4), (8, 64), 1.0)
    _, s = quant.mxfp8_rowwise(x)
    ref = torch.from_numpy(s.copy()).view(torch.float8_e8m0fnu).double().numpy()
    assert np.array_equal(codecs.e8m0_decode(s), ref)


def test_mx_idempotent_requantization():
    rng = np.random.default_rng(5)
    x = synth.normal_bf16(rng, (16, 128), 1.0, outlier_rng=np.random.default_rng(6))
    q, s = quant.mxfp8_rowwise(x)
    deq = quant.mx_dequantize(q, s)
    x2 = _bf16(deq.astype(np.float32))
    assert np.array_equal(codecs.bf16_to_f64(x2), deq)      # E4M3 * 2^k is exact in bf16
    q2, s2 = quant.mxfp8_rowwise(x2)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)


def test_mx_error_bound_and_scale_minimality():
    """Each element is within half an E4M3 step of v/2^X (or saturated); the block max lands in [256, 448]."""
    rng = np.random.default_rng(7)
    x = synth.normal_bf16(rng, (32, 256), 1.0, outlier_rng=np.random.default_rng(8))
    q, s = quant.mxfp8_rowwise(x)
    v = codecs.bf16_to_f64(x).reshape(32, 8, 32)
    X = s.astype(np.int64) - 127
    scaled = v / np.ldexp(1.0, X)[:, :, None]
    deq = codecs.e4m3_decode(q).reshape(32, 8, 32)
    sat = np.abs(scaled) > 448
    err = np.abs(deq - scaled)
    bound = np.maximum(np.abs(scaled) * 2.0 ** -4, 2.0 ** -10)
    assert np.all(err[~sat] <= bound[~sat] * (1 + 1e-12))
    assert np.all(np.abs(deq[sat]) == 448)
    bmax = np.max(np.abs(scaled), axis=2)
    assert np.all((bmax >= 256) & (bmax < 512))


def test_mx_shared_exponent_vs_math_floor_log2():
    vals = [1.0, 1.5, 2.0, 448.0, 511.0, 512.0, 3e-5, 6e37, 2.0 ** -126, 2.0 ** -130]
    for v in vals:
        expect = max(-127, min(127, math.floor(math.log2(v)) - 8))
        assert int(quant.mx_shared_exponent(np.float32(v))) == expect, v
    assert int(quant.mx_shared_exponent(np.float32(0.0))) == -127

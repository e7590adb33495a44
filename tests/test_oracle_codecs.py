"""Pins of the oracle's number formats against the OCP specification points and torch's casts."""

import json
import os

import numpy as np
import torch

from oracle import codecs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_e4m3_decode_spec_points():
    g = _golden("ocp_e4m3_points.json")
    for row in g["decode"]:
        v = codecs.e4m3_decode(np.uint8(int(row["code"], 16)))
        assert float(v) == row["value"], row
        assert np.signbit(v) == np.signbit(row["value"]), row
    for c in g["nan_codes"]:
        assert np.isnan(codes := codecs.e4m3_decode(np.uint8(int(c, 16)))), codes


def test_e4m3_decode_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = codecs.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.array_equal(ours[~both_nan], ref[~both_nan])
    assert np.array_equal(np.signbit(ours[~both_nan]), np.signbit(ref[~both_nan]))


def test_e4m3_encode_spec_points():
    for row in _golden("ocp_e4m3_points.json")["encode"]:
        got = codecs.e4m3_encode(np.float32(row["value"]))
        assert int(got) == int(row["code"], 16), row


def test_e4m3_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = codecs.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(codecs.e4m3_encode(vals), codes)


def _torch_e4m3_saturating(v32):
    t = torch.from_numpy(v32).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_e4m3_encode_exhaustive_bf16_times_scales_vs_torch():
    """Every bf16 value times several fp32 scales, against torch's RNE cast after a clamp.

    Clamping first then rounding equals rounding then saturating under RNE
    (the tie at 464 already goes to 448)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = codecs.bf16_to_f32(bits)
    finite = np.isfinite(x)
    scales = [1.0, float(np.float32(448.0) / np.float32(5.5)), 3.0] + [2.0 ** k for k in range(-12, 13, 3)]
    for s in scales:
        with np.errstate(over="ignore"):
            v = (x * np.float32(s)).astype(np.float32)
        ok = finite & np.isfinite(v)
        ours = codecs.e4m3_encode(v[ok])
        ref = _torch_e4m3_saturating(v[ok])
        bad = np.nonzero(ours != ref)[0]
        assert bad.size == 0, (s, v[ok][bad[:5]], ours[bad[:5]], ref[bad[:5]])


def test_e4m3_encode_nan_and_signed_zero():
    assert codecs.e4m3_encode(np.float32(np.nan)) & 0x7F == 0x7F
    assert codecs.e4m3_encode(np.float32(-0.0)) == 0x80
    assert codecs.e4m3_encode(np.float32(0.0)) == 0x00
    assert codecs.e4m3_encode(np.float32(np.inf)) == 0x7E
    assert codecs.e4m3_encode(np.float32(-np.inf)) == 0xFE


def test_bf16_decode_all_patterns_vs_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = codecs.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_e8m0_decode_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = codecs.e8m0_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    assert np.array_equal(ours[:255], ref[:255])
    assert ours[127] == 1.0 and ours[0] == 2.0 ** -127 and ours[254] == 2.0 ** 127

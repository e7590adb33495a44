"""Bit-exact parity of the HIP quantizers against the oracle."""

import numpy as np
import pytest
import torch

import scaled_gemm_epilogues_amd as sge
import synth
from oracle import codecs, quant

from .gpu_paths import quant_fp8, quant_mx
from .helpers import dev_bf16, host_u8

pytestmark = pytest.mark.gpu


def _f32bits(t):
    return int(t.detach().cpu().view(torch.int32).item()) & 0xFFFFFFFF


def _np_f32bits(v):
    return int(np.float32(v).view(np.uint32))


def _check_fp8(bits, got):
    ref = quant.fp8_current_scaling(bits)
    assert _f32bits(got["amax"]) == _np_f32bits(ref["amax"])
    assert _f32bits(got["scale"]) == _np_f32bits(ref["scale"])
    assert _f32bits(got["scale_inv"]) == _np_f32bits(ref["scale_inv"])
    if got["q"] is not None:
        q = host_u8(got["q"])
        bad = np.argwhere(q != ref["q"])
        assert bad.size == 0, (bad[:5], q[tuple(bad[0])], ref["q"][tuple(bad[0])])
    if got["q_t"] is not None:
        assert np.array_equal(host_u8(got["q_t"]), ref["q_t"])


@pytest.mark.parametrize("shape,std", [((608, 528), 1.0), ((64, 4096), 1e-2), ((16, 16), 0.02),
                                       ((4096, 64), 3.0)])
def test_fp8_current_scaling_bitexact(shape, std):
    print(f"case fp8 quant {shape}", flush=True)
    bits = synth.normal_bf16(np.random.default_rng(11), shape, std)
    _check_fp8(bits, quant_fp8(dev_bf16(bits)))


def _all_finite_bf16_upto(amax):
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = codecs.bf16_to_f64(allb)
    keep = np.isfinite(v) & (np.abs(v) <= amax)
    return allb[keep]


@pytest.mark.parametrize("amax", [1.0, 3.0, 5.5, 1e-3, 2.0 ** -120, 1e10, 3.3895313892515355e38])
def test_fp8_every_bf16_value_under_an_amax(amax):
    """All finite bf16 values with |v| <= amax, plus amax itself, in one tensor."""
    vals = _all_finite_bf16_upto(amax)
    top = synth.f32_to_bf16_bits(np.array([amax], np.float32))
    vals = np.concatenate([vals, top])
    n = ((len(vals) + 255) // 256) * 256
    bits = np.zeros(n, np.uint16)
    bits[:len(vals)] = np.random.default_rng(12).permutation(vals)
    bits = bits.reshape(-1, 16)
    _check_fp8(bits, quant_fp8(dev_bf16(bits)))


def test_fp8_scale_for_every_positive_bf16_amax():
    """scale, scale_inv and the amax element's code for each of the 32639 positive finite bf16 values."""
    amaxes = np.arange(1, 0x7F80, dtype=np.uint32).astype(np.uint16)
    t = torch.zeros(16, 16, dtype=torch.bfloat16, device="cuda")
    q = torch.empty(16, 16, dtype=torch.uint8, device="cuda")
    outs = torch.empty(len(amaxes), 3, dtype=torch.float32, device="cuda")
    codes = torch.empty(len(amaxes), dtype=torch.uint8, device="cuda")
    ws = torch.empty(sge.quantize_fp8_amax_workspace_size(16, 16), dtype=torch.uint8, device="cuda")
    flat = t.view(torch.int16).view(-1)
    vals = torch.from_numpy(amaxes.view(np.int16)).cuda()
    for i in range(len(amaxes)):
        flat[0] = vals[i]
        o = outs[i]
        sge.quantize_fp8_amax(t, q, None, o[0:1], o[1:2], o[2:3], ws)
        codes[i] = q[0, 0]
    outs = outs.cpu().numpy()
    codes = codes.cpu().numpy()
    for i, b in enumerate(amaxes):
        a = codecs.bf16_to_f32(b)
        s = quant.fp8_scale(a)
        assert outs[i, 0] == a
        assert outs[i, 1].view(np.uint32) == np.float32(s).view(np.uint32), (a, outs[i, 1], s)
        assert outs[i, 2].view(np.uint32) == quant.fp8_scale_inv(s).view(np.uint32)
        assert codes[i] == quant.fp8_quantize_with_scale(np.array([b], np.uint16), s)[0]


def test_fp8_zero_tensor_and_signed_zeros():
    bits = np.zeros((32, 32), np.uint16)
    bits[::2, ::3] = 0x8000
    _check_fp8(bits, quant_fp8(dev_bf16(bits)))


def _check_mx(bits, got):
    qr, sr = quant.mxfp8_rowwise(bits)
    qc, sc = quant.mxfp8_colwise(bits)
    assert np.array_equal(host_u8(got["s_row"]), sr)
    bad = np.argwhere(host_u8(got["q_row"]) != qr)
    assert bad.size == 0, bad[:5]
    assert np.array_equal(host_u8(got["s_colT"]), sc)
    assert np.array_equal(host_u8(got["q_colT"]), qc)


@pytest.mark.parametrize("shape", [(608, 544), (32, 32), (64, 96), (160, 64)])
def test_mxfp8_bitexact_with_outliers(shape):
    print(f"case mx quant {shape}", flush=True)
    bits = synth.normal_bf16(np.random.default_rng(13), shape, 1.0, outlier_rng=np.random.default_rng(14))
    _check_mx(bits, quant_mx(dev_bf16(bits)))


@pytest.mark.parametrize("shape", [(2048, 32), (32, 2048), (256, 256)])
def test_mxfp8_every_finite_bf16_value(shape):
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    fin = allb[np.isfinite(codecs.bf16_to_f64(allb))]
    bits = np.zeros(65536, np.uint16)
    bits[:len(fin)] = np.random.default_rng(15).permutation(fin)
    bits = bits.reshape(shape)
    _check_mx(bits, quant_mx(dev_bf16(bits)))


def test_mxfp8_golden_blocks_on_device():
    """The hand-derived blocks of the oracle's pins, quantized by the GPU."""
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "mx_blocks.json")) as f:
        blocks = json.load(f)["blocks"]
    mat = np.zeros((32, 32 * len(blocks)), np.float32)
    for b, blk in enumerate(blocks):
        vals = np.full(32, blk["fill"], np.float32)
        for k, v in blk["set"].items():
            vals[int(k)] = v
        mat[:, 32 * b:32 * (b + 1)] = vals[None, :]
    bits = synth.f32_to_bf16_bits(mat)
    got = quant_mx(dev_bf16(bits))
    s = host_u8(got["s_row"])
    for b, blk in enumerate(blocks):
        assert np.all(s[:, b] == blk["scale"]), blk["name"]
    _check_mx(bits, got)


def test_mxfp8_row_only_and_col_only():
    bits = synth.normal_bf16(np.random.default_rng(16), (64, 64), 1.0)
    r = quant_mx(dev_bf16(bits), row=True, col=False)
    c = quant_mx(dev_bf16(bits), row=False, col=True)
    qr, sr = quant.mxfp8_rowwise(bits)
    qc, sc = quant.mxfp8_colwise(bits)
    assert np.array_equal(host_u8(r["q_row"]), qr) and np.array_equal(host_u8(r["s_row"]), sr)
    assert np.array_equal(host_u8(c["q_colT"]), qc) and np.array_equal(host_u8(c["s_colT"]), sc)

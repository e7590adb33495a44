"""RMSNorm / LayerNorm on the GPU against the oracle: the bf16 output and saved statistics,
the fused quantized outputs (byte-identical to the oracle's quantizers applied to the same
launch's bf16 output and to the standalone quantizers on it, and close to the oracle's
quantization of its own output), and the backward."""

import numpy as np
import pytest
import torch

import scaled_gemm_epilogues_amd as sge
import synth
from oracle import norm, quant

from .gpu_paths import quant_fp8, quant_mx
from .helpers import (TAU_BF16, TAU_FP8, assert_close, assert_mx_dequant_close, assert_oracle_mx_rowwise, dev_bf16,
                      host_bits, host_f64, host_u8)

pytestmark = pytest.mark.gpu

SHAPES = [(37, 96), (300, 2048), (64, 16384), (256, 8192)]
KW = dict(rel_tight=2.0 ** -7, abs_tight=1e-3)


def _inputs(R, C, seed):
    r = synth.streams(seed)
    return {"x": synth.normal_bf16(r["x"], (R, C), 1.0, r["outliers_x"]),
            "gamma": synth.normal_bf16(r["w"], (C,), 0.5),
            "beta": synth.normal_bf16(r["residual"], (C,), 0.1),
            "dz": synth.normal_bf16(r["dy"], (R, C), 1.0)}


def _run_fwd(kind, d, zc, eps, fp8=False, mx=False):
    R, C = d["x"].shape
    k = sge.NORM_LAYER if kind == "ln" else sge.NORM_RMS
    X = dev_bf16(d["x"])
    out = {"y": torch.empty(R, C, dtype=torch.bfloat16, device="cuda"),
           "rsigma": torch.empty(R, dtype=torch.float32, device="cuda"),
           "mu": torch.empty(R, dtype=torch.float32, device="cuda") if kind == "ln" else None}
    kw = {}
    if fp8:
        f32 = dict(dtype=torch.float32, device="cuda")
        out["fp8"] = {"q": torch.empty(R, C, dtype=torch.uint8, device="cuda"),
                      "q_t": torch.empty(C, R, dtype=torch.uint8, device="cuda"),
                      "amax": torch.empty(1, **f32), "scale": torch.empty(1, **f32), "scale_inv": torch.empty(1, **f32)}
        kw["fp8"] = out["fp8"]
        kw["workspace"] = torch.empty(max(16, sge.norm_fwd_workspace_size(R, C)), dtype=torch.uint8, device="cuda")
    if mx:
        u8 = dict(dtype=torch.uint8, device="cuda")
        out["mx_row"] = (torch.empty(R, C, **u8), torch.empty(R, C // 32, **u8))
        out["mx_col"] = (torch.empty(C, R, **u8), torch.empty(C, R // 32, **u8))
        kw.update(mx_row=out["mx_row"], mx_col=out["mx_col"])
    sge.norm_fwd(k, X, dev_bf16(d["gamma"]), out["y"], out["rsigma"], beta=dev_bf16(d["beta"]) if kind == "ln" else None,
                 mu=out["mu"], eps=eps, zero_centered=zc, **kw)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("kind", ["rms", "ln"])
@pytest.mark.parametrize("shape", SHAPES)
def test_norm_forward(kind, shape):
    R, C = shape
    zc = C % 3 == 0
    print(f"case norm fwd {kind} {R}x{C} zc={zc}", flush=True)
    d = _inputs(R, C, 20)
    got = _run_fwd(kind, d, zc, 1e-5)
    ref = norm.norm_fwd(kind, d["x"], d["gamma"], d["beta"], 1e-5, zc)
    assert_close(host_f64(got["y"]), ref["y"], TAU_BF16, what="y", **KW)
    np.testing.assert_allclose(got["rsigma"].cpu().numpy(), ref["rsigma"], rtol=2e-6)
    if kind == "ln":
        np.testing.assert_allclose(got["mu"].cpu().numpy(), ref["mu"], rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("kind", ["rms", "ln"])
@pytest.mark.parametrize("shape", [(64, 96), (512, 4096)])
def test_norm_forward_fused_quantized_outputs(kind, shape):
    R, C = shape
    print(f"case norm fwd quantized {kind} {R}x{C}", flush=True)
    d = _inputs(R, C, 21)
    got = _run_fwd(kind, d, False, 1e-5, fp8=True, mx=True)
    # fused == the standalone quantizers on the same launch's bf16 output
    f8 = quant_fp8(got["y"])
    mxs = quant_mx(got["y"])
    torch.cuda.synchronize()
    for k in ("q", "q_t"):
        assert np.array_equal(host_u8(got["fp8"][k]), host_u8(f8[k])), k
    for k in ("amax", "scale", "scale_inv"):
        assert got["fp8"][k].item() == f8[k].item(), k
    assert np.array_equal(host_u8(got["mx_row"][0]), host_u8(mxs["q_row"]))
    assert np.array_equal(host_u8(got["mx_row"][1]), host_u8(mxs["s_row"]))
    assert np.array_equal(host_u8(got["mx_col"][0]), host_u8(mxs["q_colT"]))
    assert np.array_equal(host_u8(got["mx_col"][1]), host_u8(mxs["s_colT"]))
    # == the oracle's quantizers on the same launch's bf16 output (bit-exact: amax, scale,
    # scale_inv, codes, both MXFP8 copies)
    yb = host_bits(got["y"])
    rf = quant.fp8_current_scaling(yb)
    for k in ("amax", "scale", "scale_inv"):
        g = np.float32(got["fp8"][k].item())
        assert g.view(np.uint32) == np.float32(rf[k]).view(np.uint32), (k, g, rf[k])
    assert np.array_equal(host_u8(got["fp8"]["q"]), rf["q"])
    assert np.array_equal(host_u8(got["fp8"]["q_t"]), rf["q_t"])
    assert_oracle_mx_rowwise(yb, host_u8(got["mx_row"][0]), host_u8(got["mx_row"][1]), what="norm MXFP8 row")
    assert_oracle_mx_rowwise(np.ascontiguousarray(yb.T), host_u8(got["mx_col"][0]), host_u8(got["mx_col"][1]),
                             what="norm MXFP8 col")
    # and close to the oracle's quantization of its own output
    ref = norm.norm_fwd_quantized(kind, d["x"], d["gamma"], d["beta"], 1e-5)
    assert_close(got["fp8"]["amax"].item(), ref["fp8"]["amax"], TAU_BF16, what="amax", rel_tight=2.0 ** -7)
    deq = quant.fp8_dequantize(host_u8(got["fp8"]["q"]), got["fp8"]["scale_inv"].item())
    assert_mx_dequant_close(deq, quant.fp8_dequantize(ref["fp8"]["q"], ref["fp8"]["scale_inv"]), what="fp8 y")
    assert_mx_dequant_close(quant.mx_dequantize(host_u8(got["mx_row"][0]), host_u8(got["mx_row"][1])),
                            quant.mx_dequantize(*ref["mx_row"]), what="mx row y")


@pytest.mark.parametrize("kind", ["rms", "ln"])
@pytest.mark.parametrize("shape", [(37, 96), (300, 2048), (1100, 8192), (0, 64)])
def test_norm_backward(kind, shape):
    R, C = shape
    zc = R % 2 == 1
    print(f"case norm bwd {kind} {R}x{C} zc={zc}", flush=True)
    d = _inputs(R, C, 22)
    k = sge.NORM_LAYER if kind == "ln" else sge.NORM_RMS
    f = _run_fwd(kind, d, zc, 1e-5) if R else {"rsigma": torch.empty(0, device="cuda"),
                                              "mu": torch.empty(0, device="cuda")}
    bf = dict(dtype=torch.bfloat16, device="cuda")
    dx, dg, db = torch.empty(R, C, **bf), torch.empty(C, **bf), torch.empty(C, **bf)
    ws = torch.empty(max(16, sge.norm_bwd_workspace_size(R, C)), dtype=torch.uint8, device="cuda")
    X = dev_bf16(d["x"]) if R else torch.empty(0, C, **bf)
    DZ = dev_bf16(d["dz"]) if R else torch.empty(0, C, **bf)
    sge.norm_bwd(k, DZ, X, f["rsigma"], dev_bf16(d["gamma"]), dx, dg, ws, mu=f["mu"] if kind == "ln" else None,
                 dbeta=db if kind == "ln" else None, zero_centered=zc)
    torch.cuda.synchronize()
    if R == 0:
        assert not host_f64(dg).any() and (kind == "rms" or not host_f64(db).any())
        return
    ref_f = norm.norm_fwd(kind, d["x"], d["gamma"], d["beta"], 1e-5, zc)
    ref = norm.norm_bwd(kind, d["dz"], d["x"], ref_f["mu"], ref_f["rsigma"], d["gamma"], zc)
    assert_close(host_f64(dx), ref["dx"], TAU_BF16, what="dx", **KW)
    assert_close(host_f64(dg), ref["dgamma"], TAU_BF16, what="dgamma", **KW)
    if kind == "ln":
        assert_close(host_f64(db), ref["dbeta"], TAU_BF16, what="dbeta", **KW)


@pytest.mark.parametrize("kind", ["rms", "ln"])
def test_norm_backward_bitwise_repeatable(kind):
    """dgamma / dbeta are sums of per-block partials in a fixed order (and dx a per-row block
    reduction in a fixed order): two runs on the same inputs give the same bits. 3000 rows give
    every one of the 512 blocks several rows (the next-row loads alternate buffers)."""
    R, C = 3000, 4096
    print(f"case norm bwd repeatable {kind} {R}x{C}", flush=True)
    d = _inputs(R, C, 23)
    k = sge.NORM_LAYER if kind == "ln" else sge.NORM_RMS
    f = _run_fwd(kind, d, False, 1e-5)
    bf = dict(dtype=torch.bfloat16, device="cuda")
    X, DZ, gam = dev_bf16(d["x"]), dev_bf16(d["dz"]), dev_bf16(d["gamma"])
    ws = torch.empty(sge.norm_bwd_workspace_size(R, C), dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(2):
        dx, dg, db = torch.empty(R, C, **bf), torch.empty(C, **bf), torch.empty(C, **bf)
        ws.fill_(0xFF)                                   # partials rewritten on every run
        sge.norm_bwd(k, DZ, X, f["rsigma"], gam, dx, dg, ws, mu=f["mu"] if kind == "ln" else None,
                     dbeta=db if kind == "ln" else None, zero_centered=False)
        torch.cuda.synchronize()
        outs.append([host_bits(t) for t in ((dx, dg, db) if kind == "ln" else (dx, dg))])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)
    ref_f = norm.norm_fwd(kind, d["x"], d["gamma"], d["beta"], 1e-5, False)
    ref = norm.norm_bwd(kind, d["dz"], d["x"], ref_f["mu"], ref_f["rsigma"], d["gamma"], False)
    assert_close(host_f64(dg), ref["dgamma"], TAU_BF16, what="dgamma", **KW)

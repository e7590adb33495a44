"""Pins of the oracle's RMSNorm / LayerNorm: torch's fp64 routines and autograd (library
routines), closed forms, invariances, zero-centered gamma, the saved statistics, and the
quantized outputs against the pinned quantizers applied to a brute-force bf16 output."""

import math

import numpy as np
import pytest
import torch

import synth
from oracle import norm, quant
from oracle.codecs import bf16_to_f64, f64_to_bf16


def _inputs(R=7, C=96, seed=0):
    r = synth.streams(seed)
    return {"x": synth.normal_bf16(r["x"], (R, C), 1.0, r["outliers_x"], outlier_rate=0.05),
            "gamma": synth.normal_bf16(r["w"], (C,), 0.5),
            "beta": synth.normal_bf16(r["residual"], (C,), 0.1),
            "dz": synth.normal_bf16(r["dy"], (R, C), 1.0)}


@pytest.mark.parametrize("kind", ["rms", "ln"])
@pytest.mark.parametrize("zc", [False, True])
def test_forward_matches_torch_fp64(kind, zc):
    d = _inputs()
    eps = 1e-5
    got = norm.norm_fwd(kind, d["x"], d["gamma"], d["beta"], eps, zc)
    x = torch.from_numpy(bf16_to_f64(d["x"]))
    g = torch.from_numpy(bf16_to_f64(d["gamma"])) + (1.0 if zc else 0.0)
    if kind == "rms":
        ref = torch.nn.functional.rms_norm(x, (x.shape[1],), g, eps)
    else:
        ref = torch.nn.functional.layer_norm(x, (x.shape[1],), g, torch.from_numpy(bf16_to_f64(d["beta"])), eps)
    np.testing.assert_allclose(got["y"], ref.numpy(), rtol=1e-12, atol=1e-12)
    assert np.array_equal(got["y_bits"], f64_to_bf16(ref.numpy()))


@pytest.mark.parametrize("kind", ["rms", "ln"])
@pytest.mark.parametrize("zc", [False, True])
def test_backward_matches_torch_autograd(kind, zc):
    d = _inputs(seed=1)
    eps = 1e-5
    f = norm.norm_fwd(kind, d["x"], d["gamma"], d["beta"], eps, zc)
    # the backward uses the saved (fp32) statistics; torch recomputes them in fp64, so the
    # comparison is to the fp32 rounding of rsigma
    got = norm.norm_bwd(kind, d["dz"], d["x"], f["mu"], f["rsigma"], d["gamma"], zc)
    x = torch.from_numpy(bf16_to_f64(d["x"])).requires_grad_()
    gam = torch.from_numpy(bf16_to_f64(d["gamma"])).requires_grad_()
    bet = torch.from_numpy(bf16_to_f64(d["beta"])).requires_grad_()
    g = gam + (1.0 if zc else 0.0)
    y = torch.nn.functional.rms_norm(x, (x.shape[1],), g, eps) if kind == "rms" else \
        torch.nn.functional.layer_norm(x, (x.shape[1],), g, bet, eps)
    y.backward(torch.from_numpy(bf16_to_f64(d["dz"])))
    np.testing.assert_allclose(got["dx"], x.grad.numpy(), rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(got["dgamma"], gam.grad.numpy(), rtol=1e-6, atol=1e-6)
    if kind == "ln":
        np.testing.assert_allclose(got["dbeta"], bet.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_closed_forms_and_invariances():
    C = 64
    gamma = f64_to_bf16(np.full(C, 1.5))
    beta = f64_to_bf16(np.full(C, -0.25))
    const = f64_to_bf16(np.full((1, C), 3.0))
    r = norm.norm_fwd("rms", const, gamma, None, 1e-6)
    assert r["y"][0, 0] == pytest.approx(1.5 * 3.0 / math.sqrt(9.0 + 1e-6), rel=1e-14)
    l = norm.norm_fwd("ln", const, gamma, beta, 1e-6)
    assert np.all(l["y"] == -0.25) and l["mu"][0] == 3.0                # a constant row maps to beta
    d = _inputs(R=3, C=C, seed=2)
    base = norm.norm_fwd("rms", d["x"], d["gamma"], None, 0.0)["y"]
    scaled = norm.norm_fwd("rms", f64_to_bf16(bf16_to_f64(d["x"]) * 4.0), d["gamma"], None, 0.0)["y"]
    np.testing.assert_allclose(scaled, base, rtol=1e-13)                 # RMSNorm is scale-invariant
    lb = norm.norm_fwd("ln", d["x"], d["gamma"], d["beta"], 1e-5)["y"]
    ls = norm.norm_fwd("ln", f64_to_bf16(bf16_to_f64(d["x"]) + 8.0), d["gamma"], d["beta"], 1e-5)["y"]
    # the shift is exact in bf16 only for some values: compare where it was
    xs = bf16_to_f64(d["x"])
    exact = np.all(bf16_to_f64(f64_to_bf16(xs + 8.0)) - 8.0 == xs, axis=1)
    np.testing.assert_allclose(ls[exact], lb[exact], rtol=1e-10, atol=1e-12)
    zc = norm.norm_fwd("rms", d["x"], f64_to_bf16(bf16_to_f64(d["gamma"]) - 1.0), None, 1e-5, True)["y"]
    gm1 = bf16_to_f64(f64_to_bf16(bf16_to_f64(d["gamma"]) - 1.0)) + 1.0
    ref = norm.norm_fwd("rms", d["x"], f64_to_bf16(gm1), None, 1e-5)["y"]
    ok = bf16_to_f64(f64_to_bf16(gm1)) == gm1
    np.testing.assert_allclose(zc[:, ok], ref[:, ok], rtol=1e-14)


def test_backward_central_differences():
    d = _inputs(R=2, C=32, seed=3)
    eps = 1e-3
    x = bf16_to_f64(d["x"])
    g = bf16_to_f64(d["gamma"])
    bvec = bf16_to_f64(d["beta"])
    dz = bf16_to_f64(d["dz"])

    def loss(xv):
        mu = xv.mean(axis=1, keepdims=True)
        rs = 1 / np.sqrt(((xv - mu) ** 2).mean(axis=1, keepdims=True) + eps)
        return float(np.sum(dz * ((xv - mu) * rs * g + bvec)))

    f = norm.norm_fwd("ln", d["x"], d["gamma"], d["beta"], eps)
    # exact fp64 statistics (not the fp32 saved ones) for a tight comparison
    mu = x.mean(axis=1)
    rs = 1 / np.sqrt(((x - mu[:, None]) ** 2).mean(axis=1) + eps)
    got = norm.norm_bwd("ln", d["dz"], d["x"], mu, rs, d["gamma"])
    h = 1e-6
    for (i, j) in [(0, 0), (1, 5), (0, 31)]:
        xp, xm = x.copy(), x.copy()
        xp[i, j] += h
        xm[i, j] -= h
        assert got["dx"][i, j] == pytest.approx((loss(xp) - loss(xm)) / (2 * h), rel=1e-6, abs=1e-8)
    assert f["rsigma"].dtype == np.float32 and f["mu"].dtype == np.float32


def test_quantized_outputs_are_the_quantizers_of_the_bf16_output():
    d = _inputs(R=64, C=64, seed=4)
    r = norm.norm_fwd_quantized("rms", d["x"], d["gamma"], None, 1e-5)
    # brute-force bf16 output: per element, x * rsigma * gamma rounded once to bf16
    x = bf16_to_f64(d["x"])
    g = bf16_to_f64(d["gamma"])
    yb = np.empty_like(r["y_bits"])
    for i in range(x.shape[0]):
        rs = 1 / math.sqrt(math.fsum(v * v for v in x[i]) / x.shape[1] + 1e-5)
        yb[i] = f64_to_bf16(np.array([v * rs * gg for v, gg in zip(x[i], g)]))
    assert np.array_equal(r["y_bits"], yb)
    q, s = quant.mxfp8_rowwise(yb)
    assert np.array_equal(r["mx_row"][0], q) and np.array_equal(r["mx_row"][1], s)
    qc, sc = quant.mxfp8_colwise(yb)
    assert np.array_equal(r["mx_col"][0], qc) and np.array_equal(r["mx_col"][1], sc)
    f8 = quant.fp8_current_scaling(yb)
    assert np.array_equal(r["fp8"]["q"], f8["q"]) and r["fp8"]["scale_inv"] == f8["scale_inv"]

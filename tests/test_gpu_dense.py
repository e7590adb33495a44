"""Parity of the dense fused scaled linear (HIP path through the C ABI) against the oracle."""

import numpy as np
import pytest
import torch

import scaled_gemm_epilogues_amd as sge
import synth
from oracle import linear
from oracle.codecs import bf16_to_f64

from .gpu_paths import dense_operands, run_dense
from .helpers import TAU_BF16, TAU_FP8, assert_close, dev_bf16, host_bits, host_f64

pytestmark = pytest.mark.gpu

# Sizes spanning several 256x256 tiles with ragged edges in M, N and the contraction.
SMALL = {
    "bf16": (600, 520, 328),
    "fp8": (608, 528, 336),
    "mxfp8": (608, 544, 352),      # K % 128 != 0: the unaligned E8M0 scale path
}


def _oracle_dense(fmt, d, alpha):
    ops = linear.operands(fmt, d["x"], d["w"], d["dy"])
    return {
        "fwd": linear.linear_scale_add_fwd(*ops["fwd"], bf16_to_f64(d["residual"]), alpha),
        "dgrad": linear.linear_scale_dgrad(*ops["dgrad"], alpha),
        "wgrad": linear.linear_scale_wgrad(*ops["wgrad"], alpha),
    }


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mxfp8"])
def test_dense_parity_ragged(fmt):
    M, N, K = SMALL[fmt]
    print(f"case dense {fmt} M={M} N={N} K={K}", flush=True)
    d = synth.dense(M, N, K, seed=1, outliers=fmt == "mxfp8", w_std=1.0 if fmt == "mxfp8" else 0.02,
                    dy_std=1.0 if fmt == "mxfp8" else 1e-2)
    alpha = 0.5
    got = run_dense(fmt, d, alpha)
    ref = _oracle_dense(fmt, d, alpha)
    tau = TAU_BF16 if fmt == "bf16" else TAU_FP8
    for k in ("fwd", "dgrad", "wgrad"):
        assert_close(host_f64(got[k]), ref[k], tau, what=f"{fmt} {k}")


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mxfp8"])
def test_dense_parity_aligned_tiles(fmt):
    M, N, K = 512, 768, 512
    print(f"case dense aligned {fmt}", flush=True)
    d = synth.dense(M, N, K, seed=2, outliers=fmt == "mxfp8")
    got = run_dense(fmt, d, 0.25)
    ref = _oracle_dense(fmt, d, 0.25)
    tau = TAU_BF16 if fmt == "bf16" else TAU_FP8
    for k in ("fwd", "dgrad", "wgrad"):
        assert_close(host_f64(got[k]), ref[k], tau, what=f"{fmt} {k}")


# bf16 contraction lengths at the k-step (32) and k-tile (64) edges: shorter than a step, one step,
# one tile, a tile and a ragged step; the last case also gives dgrad (over N = 24) and wgrad (over
# M = 40) a single partial k-tile.
@pytest.mark.parametrize("M,N,K", [(264, 264, 8), (264, 264, 32), (264, 264, 64), (264, 264, 72), (40, 24, 96)])
def test_bf16_contraction_edges(M, N, K):
    print(f"case dense bf16 M={M} N={N} K={K}", flush=True)
    d = synth.dense(M, N, K, seed=5)
    got = run_dense("bf16", d, 0.75)
    ref = _oracle_dense("bf16", d, 0.75)
    for k in ("fwd", "dgrad", "wgrad"):
        assert_close(host_f64(got[k]), ref[k], TAU_BF16, what=f"bf16 {k} M={M} N={N} K={K}")


def test_forward_256x512x512_full_parity():
    """The small forward workload at its own size: every element against the oracle."""
    w = synth.WORKLOADS["bf16_fwd_256x512x512"]
    d = synth.workload_inputs("bf16_fwd_256x512x512", seed=0)
    got = run_dense("bf16", d, w["alpha"], passes=("fwd",))
    ops = linear.operands("bf16", d["x"], d["w"])
    ref = linear.linear_scale_add_fwd(*ops["fwd"], bf16_to_f64(d["residual"]), w["alpha"])
    assert_close(host_f64(got["fwd"]), ref, TAU_BF16, what="256x512x512 fwd")


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mxfp8"])
def test_alpha_zero_returns_residual_bitexact(fmt):
    d = synth.dense(96, 64, 64, seed=3)
    res = d["residual"].copy()
    res[0, 0] = 0x8000                                  # -0.0 survives
    d["residual"] = res
    got = run_dense(fmt, d, 0.0, passes=("fwd",))
    assert np.array_equal(host_bits(got["fwd"]), res)


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mxfp8"])
def test_alpha_zero_backward_writes_positive_zero(fmt):
    d = synth.dense(64, 64, 64, seed=4)
    got = run_dense(fmt, d, 0.0, passes=("dgrad", "wgrad"))
    for k in ("dgrad", "wgrad"):
        assert np.all(host_bits(got[k]) == 0)


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mxfp8"])
def test_zero_residual_alpha_one_is_plain_gemm(fmt):
    M, N = (300, 264) if fmt == "bf16" else (320, 288)
    d = synth.dense(M, N, 256, seed=5)
    d["residual"] = np.zeros_like(d["residual"])
    X, W = dev_bf16(d["x"]), dev_bf16(d["w"])
    ops = dense_operands(fmt, X, W)
    a = torch.zeros(M, N, dtype=torch.bfloat16, device="cuda")
    b = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    sge.linear_scale_add_fwd(*ops["fwd"], a, 1.0, accumulate=True)
    sge.linear_scale_add_fwd(*ops["fwd"], b, 1.0, accumulate=False)
    ha, hb = host_f64(a), host_f64(b)
    assert np.array_equal(ha, hb)                       # +-0 compare equal
    ref = linear.linear_scale_add_fwd(*linear.operands(fmt, d["x"], d["w"])["fwd"], None, 1.0, accumulate=False)
    assert_close(ha, ref, TAU_BF16 if fmt == "bf16" else TAU_FP8, what=f"{fmt} plain")


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mxfp8"])
def test_gradients_scale_linearly_in_alpha(fmt):
    d = synth.dense(256, 320, 128, seed=6)
    one = run_dense(fmt, d, 1.0, passes=("dgrad", "wgrad"))
    for a in (0.125, 0.25, 0.5):
        got = run_dense(fmt, d, a, passes=("dgrad", "wgrad"))
        for k in ("dgrad", "wgrad"):
            scaled = (one[k].float() * a).to(torch.bfloat16)     # exact: power-of-two scaling of bf16
            assert torch.equal(got[k].view(torch.int16), scaled.view(torch.int16)), (fmt, k, a)


def test_every_output_element_written():
    d = synth.dense(328, 264, 200, seed=7)
    X, W, DY = dev_bf16(d["x"]), dev_bf16(d["w"]), dev_bf16(d["dy"])
    ops = dense_operands("bf16", X, W, DY)
    dg = torch.full((328, 200), float("nan"), dtype=torch.bfloat16, device="cuda")
    wg = torch.full((264, 200), float("nan"), dtype=torch.bfloat16, device="cuda")
    sge.linear_scale_bwd(*ops["dgrad"], *ops["wgrad"], dg, wg, 0.5, 0.5)
    assert torch.isfinite(dg.float()).all() and torch.isfinite(wg.float()).all()


def test_outputs_respect_leading_dimension():
    """A residual view with a padded leading dimension: the padding is never touched."""
    d = synth.dense(200, 136, 64, seed=8)
    X, W = dev_bf16(d["x"]), dev_bf16(d["w"])
    big = torch.full((200, 160), 7.0, dtype=torch.bfloat16, device="cuda")
    view = big[:, :136]
    view.copy_(dev_bf16(d["residual"]))
    sge.linear_scale_add_fwd(sge.Operand.bf16(X), sge.Operand.bf16(W), view, 0.5)
    assert torch.all(big[:, 136:] == 7.0)
    ref = linear.linear_scale_add_fwd(bf16_to_f64(d["x"]), bf16_to_f64(d["w"]), bf16_to_f64(d["residual"]), 0.5)
    assert_close(host_f64(view), ref, TAU_BF16, what="ld view")


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mxfp8"])
def test_bitwise_repeatable(fmt):
    d = synth.dense(512, 512, 256, seed=9)
    a = run_dense(fmt, d, 0.5)
    b = run_dense(fmt, d, 0.5)
    for k in ("fwd", "dgrad", "wgrad"):
        assert torch.equal(a[k].view(torch.int16), b[k].view(torch.int16)), k


def test_fused_matches_unfused_composition():
    """Fused GEMM+scale+add against plain GEMM, then a scale, then an add (torch elementwise)."""
    d = synth.dense(384, 256, 512, seed=10)
    X, W = dev_bf16(d["x"]), dev_bf16(d["w"])
    res = dev_bf16(d["residual"])
    fused = res.clone()
    sge.linear_scale_add_fwd(sge.Operand.bf16(X), sge.Operand.bf16(W), fused, 0.125)
    plain = torch.empty_like(res)
    sge.linear_scale_add_fwd(sge.Operand.bf16(X), sge.Operand.bf16(W), plain, 1.0, accumulate=False)
    unfused = (res.float() + (plain.float() * 0.125).to(torch.bfloat16).float()).to(torch.bfloat16)
    f, u = host_f64(fused), host_f64(unfused)
    # one extra bf16 rounding of the product on the unfused side
    bound = 2.0 ** -7 * np.abs(f) + 2.0 ** -8 * 0.125 * np.abs(host_f64(plain)) + 1e-30
    assert np.all(np.abs(f - u) <= bound)


def test_empty_shapes_are_noops():
    x = torch.zeros(0, 64, dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(64, 64, dtype=torch.bfloat16, device="cuda")
    r = torch.zeros(0, 64, dtype=torch.bfloat16, device="cuda")
    sge.linear_scale_add_fwd(sge.Operand.bf16(x), sge.Operand.bf16(w), r, 0.5)
    torch.cuda.synchronize()

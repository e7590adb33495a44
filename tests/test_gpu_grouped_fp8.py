"""Grouped path on FP8 E4M3 operands with current scaling per group, against the oracle: the
per-group quantizer (bit-exact: amax, scale, scale_inv, codes and the transposed copy in the
aligned group layout), the grouped GEMMs with per-group scales and alpha, and the whole MLP
forward + backward (FP8 bar)."""

import numpy as np
import pytest
import torch

import synth
from oracle import grouped, offsets, quant

from .gpu_paths import mx_layout, quant_fp8_grouped, run_grouped_mlp_fp8
from .helpers import (TAU_FP8, assert_close, assert_close_requantized, assert_oracle_fp8_grouped, clamp_settled_h,
                      dev, dev_bf16, host_bits, host_f64, host_u8)

pytestmark = pytest.mark.gpu

# Clamped SwiGLU with a limit well inside the pre-activations' spread (both clamps engage)
CLAMPED = ("clamped_swiglu", 0.25, 1.702)

KW = dict(rel_tight=2.0 ** -3, abs_tight=0.1)

QUANT_CASES = {
    "ragged_with_empty_groups": ([300, 0, 211, 9, 0, 40], 96),
    "dirichlet_8": (None, 160),
    "one_group": ([513], 48),
}


def _host_f32(t):
    return t.detach().cpu().numpy().astype(np.float32)


@pytest.mark.parametrize("case", list(QUANT_CASES))
def test_quantize_fp8_grouped_tokens_exact(case):
    splits, C = QUANT_CASES[case]
    if splits is None:
        splits = synth.dirichlet_splits(np.random.default_rng(3), 8, 1000)
    T, G = int(sum(splits)), len(splits)
    print(f"case fp8 grouped quant {case} T={T} G={G} C={C}", flush=True)
    r = synth.streams(17)
    x = synth.normal_bf16(r["x"], (T, C), 1.0, r["outliers_x"])
    base = offsets.base_offsets(splits)
    lay = mx_layout(dev(base), T)
    got = quant_fp8_grouped(dev_bf16(x), G, lay, fill=0xAB)
    torch.cuda.synchronize()
    c, pad = quant.mx_group_layout(base, T)
    ref = quant.fp8_current_scaling_grouped(x, c, pad, got["ld"])
    for k in ("amax", "scale", "scale_inv"):
        assert np.array_equal(_host_f32(got[k]), ref[k]), k
    assert np.array_equal(host_u8(got["q"]), ref["q"])
    P = int(pad[-1])
    gt = host_u8(got["q_t"])
    assert np.array_equal(gt[:, :P], ref["q_t"][:, :P])
    assert np.all(gt[:, P:] == 0xAB)                                    # past the last group: untouched


def test_quantize_fp8_grouped_experts_exact():
    G, N, K = 3, 256, 96
    print(f"case fp8 grouped quant experts G={G} N={N} K={K}", flush=True)
    r = synth.streams(18)
    w = synth.normal_bf16(r["w"], (G * N, K), 0.02, r["outliers_w"])
    got = quant_fp8_grouped(dev_bf16(w), G)
    torch.cuda.synchronize()
    c = np.arange(G + 1, dtype=np.int64) * N
    ref = quant.fp8_current_scaling_grouped(w, c, c, G * N)
    for k in ("amax", "scale", "scale_inv"):
        assert np.array_equal(_host_f32(got[k]), ref[k]), k
    assert np.array_equal(host_u8(got["q"]), ref["q"])
    assert np.array_equal(host_u8(got["q_t"]), ref["q_t"])


def _hat(q, sinv, c):
    out = np.zeros(q.shape, np.float64)
    for g in range(len(c) - 1):
        out[c[g]:c[g + 1]] = quant.fp8_dequantize(q[c[g]:c[g + 1]], sinv[g])
    return out


@pytest.mark.parametrize("case", ["ragged_with_empty_group", "dirichlet"])
def test_grouped_gemms_fp8_per_group_scales_and_alpha(case):
    splits = [300, 0, 211, 9, 0, 40] if case == "ragged_with_empty_group" else \
        list(synth.dirichlet_splits(np.random.default_rng(6), 5, 700))
    T, G, N, K = int(sum(splits)), len(splits), 256, 384
    print(f"case fp8 grouped gemms {case} T={T} G={G} N={N} K={K}", flush=True)
    r = synth.streams(19)
    x = synth.normal_bf16(r["x"], (T, K), 1.0, r["outliers_x"])
    w = synth.normal_bf16(r["w"], (G, N, K), 0.02, r["outliers_w"])
    dy = synth.normal_bf16(r["dy"], (T, N), 1e-2)
    base = offsets.base_offsets(splits)
    b_dev = dev(base)
    lay = mx_layout(b_dev, T)
    qx, qdy = quant_fp8_grouped(dev_bf16(x), G, lay), quant_fp8_grouped(dev_bf16(dy), G, lay)
    qw = quant_fp8_grouped(dev_bf16(w.reshape(G * N, K)), G)
    import scaled_gemm_epilogues_amd as sge
    bf = dict(dtype=torch.bfloat16, device="cuda")
    out, dx, dw = torch.empty(T, N, **bf), torch.empty(T, K, **bf), torch.empty(G, N, K, **bf)
    sge.grouped_linear_fwd_fp8(qx["q"], qx["scale_inv"], qw["q"].view(G, N, K), qw["scale_inv"], b_dev, out,
                               alpha=0.5)
    sge.grouped_linear_dgrad_fp8(qdy["q"], qdy["scale_inv"], qw["q_t"], qw["scale_inv"], b_dev, alpha=-0.75, dx=dx)
    sge.grouped_linear_wgrad_fp8(qdy["q_t"], qdy["scale_inv"], qx["q_t"], qx["scale_inv"], lay, dw, alpha=0.25)
    torch.cuda.synchronize()
    c, _ = quant.mx_group_layout(base, T)
    cw = np.arange(G + 1, dtype=np.int64) * N
    rx = quant.fp8_current_scaling_grouped(x, c, c)
    rdy = quant.fp8_current_scaling_grouped(dy, c, c)
    rw = quant.fp8_current_scaling_grouped(w.reshape(G * N, K), cw, cw)
    x_hat, dy_hat = _hat(rx["q"], rx["scale_inv"], c), _hat(rdy["q"], rdy["scale_inv"], c)
    w_hat = _hat(rw["q"], rw["scale_inv"], cw).reshape(G, N, K)
    assert_close(host_f64(out), grouped.grouped_linear_fwd(x_hat, w_hat, base, 0.5), TAU_FP8, what="fwd", **KW)
    assert_close(host_f64(dx), grouped.grouped_linear_dgrad(dy_hat, w_hat, base, -0.75), TAU_FP8, what="dgrad", **KW)
    assert_close(host_f64(dw), grouped.grouped_linear_wgrad(dy_hat, x_hat, base, 0.25), TAU_FP8, what="wgrad", **KW)


MLP_CASES = {
    "ragged_with_empty_group": ([300, 0, 211, 9, 0, 40], 256, 256),
    "dirichlet_wide": (None, 512, 384),
}


@pytest.mark.parametrize("act", ["swiglu", "srelu", CLAMPED], ids=["swiglu", "srelu", "clamped_swiglu"])
@pytest.mark.parametrize("case", list(MLP_CASES))
def test_fp8_grouped_mlp_fwd_bwd(case, act):
    splits, hidden, ffn = MLP_CASES[case]
    T = 700 if splits is None else sum(splits)
    G = 5 if splits is None else len(splits)
    print(f"case fp8 grouped mlp {case} {act} T={T} G={G} hidden={hidden} ffn={ffn}", flush=True)
    inp = synth.grouped(T, G, hidden, ffn, seed=33, splits=splits, gated=act != "srelu")
    got = run_grouped_mlp_fp8(inp, act)
    base = offsets.base_offsets(inp["splits"])
    fwd = grouped.grouped_mlp_fwd_fp8(inp["x"], inp["w1"], inp["w2"], inp["p"], base, act)
    bwd = grouped.grouped_mlp_bwd_fp8(inp["x"], inp["w1"], inp["w2"], inp["p"], base, inp["dout"], fwd=fwd, act=act)
    # the amax fused into the epilogues, and the bytes quantized with it, == the oracle's per-group
    # current scaling of the same launch's bf16 y and dh
    c, pad = quant.mx_group_layout(base, T)
    assert_oracle_fp8_grouped(host_bits(got["y"]), got["qy"], c, pad, what="y (fused amax)")
    assert_oracle_fp8_grouped(host_bits(got["dh"]), got["qdh"], c, pad, what="dh (fused amax)")
    # and == the quantizer's own amax pass: identical bytes
    for fused, alone in (("qy", "qy_alone"), ("qdh", "qdh_alone")):
        for k in ("amax", "scale", "scale_inv"):
            assert np.array_equal(_host_f32(got[fused][k]), _host_f32(got[alone][k])), (fused, k)
        assert np.array_equal(host_u8(got[fused]["q"]), host_u8(got[alone]["q"])), fused
        P = int(quant.mx_group_layout(base, T)[1][-1])
        assert np.array_equal(host_u8(got[fused]["q_t"])[:, :P], host_u8(got[alone]["q_t"])[:, :P]), fused
    assert_close(host_f64(got["h"]), fwd["h"], TAU_FP8, what="h", **KW)
    assert_close(host_f64(got["y"]), fwd["y"], TAU_FP8, what="y", **KW)
    # out, dx and the weight gradients consume y or dh, quantized per group on each side
    assert_close_requantized(host_f64(got["out"]), fwd["out"], TAU_FP8, what="out", **KW)
    if isinstance(act, tuple):                             # clamps: settle the ambiguous decisions
        h_set, n_amb = clamp_settled_h(host_f64(got["dh"]), bwd["dh"], bwd["gy"], fwd["h"], inp["p"], act)
        assert n_amb <= 1e-3 * h_set.size
        bwd = grouped.grouped_mlp_bwd_fp8(inp["x"], inp["w1"], inp["w2"], inp["p"], base, inp["dout"],
                                          fwd=dict(fwd, h=h_set), act=act)
    assert_close(host_f64(got["dh"]), bwd["dh"], TAU_FP8, what="dh", **KW)
    assert_close(host_f64(got["dp"]), bwd["dp"], TAU_FP8, what="dprobs", **KW)
    assert_close_requantized(host_f64(got["dx"]), bwd["dx"], TAU_FP8, what="dx", **KW)
    assert_close_requantized(host_f64(got["dw2"]), bwd["dw2"], TAU_FP8, what="dw2", **KW)
    assert_close_requantized(host_f64(got["dw1"]), bwd["dw1"], TAU_FP8, what="dw1", **KW)

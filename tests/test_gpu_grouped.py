"""Parity of the grouped path (split offsets, grouped GEMMs, fused scaled SwiGLU) against the oracle."""

import numpy as np
import pytest
import torch

import scaled_gemm_epilogues_amd as sge
import synth
from oracle import grouped, offsets
from oracle.codecs import bf16_to_f64, f64_to_bf16

from .gpu_paths import run_grouped_mlp
from .helpers import TAU_BF16, assert_close, clamp_settled_h, dev_bf16, host_f64

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("G,T", [(1, 10), (8, 65536), (64, 1000), (4096, 100000), (300, 0)])
def test_splits_to_offsets_exact(G, T):
    rng = np.random.default_rng(G)
    s = synth.dirichlet_splits(rng, G, T)
    mults = [1, 2048, 4096]
    out = torch.empty(3, G + 1, dtype=torch.int64, device="cuda")
    err = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    sge.splits_to_offsets(torch.from_numpy(s).cuda(), mults, out, expected_total=T, err_flag=err)
    assert np.array_equal(out.cpu().numpy(), offsets.splits_to_offsets(s, mults))
    assert int(err.item()) == 0


def test_splits_to_offsets_flags_bad_totals_and_negatives():
    s = torch.tensor([3, 4, 5], dtype=torch.int64, device="cuda")
    out = torch.empty(1, 4, dtype=torch.int64, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    sge.splits_to_offsets(s, [1], out, expected_total=13, err_flag=err)
    assert int(err.item()) == 1
    sge.splits_to_offsets(torch.tensor([3, -1, 5], dtype=torch.int64, device="cuda"), [1], out, err_flag=err)
    assert int(err.item()) == 1
    sge.splits_to_offsets(s, [1], out, expected_total=-1, err_flag=err)
    assert int(err.item()) == 0


def _oracle_mlp(inp):
    base = offsets.base_offsets(inp["splits"])
    x, w1, w2 = bf16_to_f64(inp["x"]), bf16_to_f64(inp["w1"]), bf16_to_f64(inp["w2"])
    p = inp["p"].astype(np.float64)
    f = grouped.grouped_mlp_fwd(x, w1, w2, p, base)
    b = grouped.grouped_mlp_bwd(bf16_to_f64(inp["dout"]), x, w1, w2, p, base, h=f["h"], y=f["y"])
    return f, b


# splits (None: Dirichlet over T=520, G=5), hidden, ffn. The mid-size case gives the weight
# gradients 16 and 8 output tiles per group, so each XCD takes a slice of every group.
SPLIT_CASES = {
    "empty_and_single": ([0, 1, 300, 0, 211, 8], 256, 256),
    "dirichlet": (None, 256, 256),
    "mid_xcd_slices": ([700, 0, 333, 41, 210], 1024, 512),
}


@pytest.mark.parametrize("case", list(SPLIT_CASES))
def test_grouped_mlp_parity(case):
    splits, hidden, ffn = SPLIT_CASES[case]
    T = 520 if splits is None else sum(splits)
    G = 5 if splits is None else len(splits)
    print(f"case grouped mlp {case} T={T} G={G} hidden={hidden} ffn={ffn}", flush=True)
    inp = synth.grouped(T, G, hidden, ffn, seed=21, splits=splits)
    got = run_grouped_mlp(inp)
    f, b = _oracle_mlp(inp)
    assert int(got["err"].item()) == 0
    assert_close(host_f64(got["h"]), f["h"], TAU_BF16, what="h")
    assert_close(host_f64(got["y"]), f["y"], TAU_BF16, what="y", rel_tight=2.0 ** -7, abs_tight=2e-2)
    assert_close(host_f64(got["out"]), f["out"], TAU_BF16, what="out", rel_tight=2.0 ** -7, abs_tight=5e-2)
    assert_close(host_f64(got["dh"]), b["dh"], TAU_BF16, what="dh", rel_tight=2.0 ** -7, abs_tight=5e-2)
    assert_close(host_f64(got["dp"]), b["dp"], TAU_BF16, what="dp", rel_tight=2.0 ** -7, abs_tight=5e-2)
    assert_close(host_f64(got["dw2"]), b["dw2"], TAU_BF16, what="dw2", rel_tight=2.0 ** -7, abs_tight=5e-2)
    assert_close(host_f64(got["dx"]), b["dx"], TAU_BF16, what="dx", rel_tight=2.0 ** -7, abs_tight=5e-2)
    assert_close(host_f64(got["dw1"]), b["dw1"], TAU_BF16, what="dw1", rel_tight=2.0 ** -7, abs_tight=5e-2)
    if splits is not None:
        for g, n in enumerate(splits):
            if n == 0:
                assert torch.all(got["dw1"][g] == 0) and torch.all(got["dw2"][g] == 0)


def test_single_group_equals_dense_bitwise():
    T, N, K = 300, 256, 192
    d = synth.dense(T, N, K, seed=22, with_dy=False)
    X, W = dev_bf16(d["x"]), dev_bf16(d["w"])
    dense = torch.empty(T, N, dtype=torch.bfloat16, device="cuda")
    sge.linear_scale_add_fwd(sge.Operand.bf16(X), sge.Operand.bf16(W), dense, 1.0, accumulate=False)
    offs = torch.tensor([0, T], dtype=torch.int64, device="cuda")
    out = torch.empty(T, N, dtype=torch.bfloat16, device="cuda")
    sge.grouped_linear_fwd(X, W[None], offs, out)
    assert torch.equal(dense.view(torch.int16), out.view(torch.int16))


def test_fused_swiglu_matches_unfused():
    inp = synth.grouped(700, 3, 256, 256, seed=23, splits=[200, 0, 500])
    got = run_grouped_mlp(inp, with_backward=True)
    P = torch.from_numpy(inp["p"]).cuda()
    y2 = torch.empty_like(got["y"])
    sge.scaled_swiglu_fwd(got["h"], P, y2)
    a, b = host_f64(got["y"]), host_f64(y2)
    assert np.all(np.abs(a - b) <= 2.0 ** -6 * np.abs(a) + 1e-3 * np.sqrt(np.mean(a ** 2)))
    # backward: g from a plain grouped dgrad, then the unfused dSwiGLU
    W2 = dev_bf16(inp["w2"])
    DOUT = dev_bf16(inp["dout"])
    g = torch.empty(700, 256, dtype=torch.bfloat16, device="cuda")
    sge.grouped_linear_bwd(DOUT, None, W2, got["offsets"][0], dx=g)
    dh = torch.empty_like(got["dh"])
    dp = torch.empty_like(got["dp"])
    sge.scaled_swiglu_bwd(g, got["h"], P, dh, dp)
    fa, fb = host_f64(got["dh"]), host_f64(dh)
    assert np.all(np.abs(fa - fb) <= 2.0 ** -6 * np.abs(fa) + 1e-2 * np.sqrt(np.mean(fa ** 2)))
    pa, pb = host_f64(got["dp"]), host_f64(dp)
    assert np.all(np.abs(pa - pb) <= 2.0 ** -6 * np.abs(pa) + 1e-2 * np.sqrt(np.mean(pa ** 2)))


def test_unfused_swiglu_parity():
    rng = np.random.default_rng(24)
    T, F = 100, 264
    h = synth.normal_bf16(rng, (T, 2 * F), 2.0)
    p = rng.random(T, dtype=np.float32)
    gy = synth.normal_bf16(rng, (T, F), 1.0)
    H, P, GY = dev_bf16(h), torch.from_numpy(p).cuda(), dev_bf16(gy)
    y = torch.empty(T, F, dtype=torch.bfloat16, device="cuda")
    dh = torch.empty(T, 2 * F, dtype=torch.bfloat16, device="cuda")
    dp = torch.empty(T, dtype=torch.float32, device="cuda")
    sge.scaled_swiglu_fwd(H, P, y)
    sge.scaled_swiglu_bwd(GY, H, P, dh, dp)
    hf, pf = bf16_to_f64(h), p.astype(np.float64)
    assert_close(host_f64(y), grouped.scaled_swiglu_fwd(hf, pf), TAU_BF16, what="y")
    rdh, rdp = grouped.scaled_swiglu_bwd(bf16_to_f64(gy), hf, pf)
    assert_close(host_f64(dh), rdh, TAU_BF16, what="dh")
    assert_close(host_f64(dp), rdp, TAU_BF16, what="dp", rel_tight=1e-5, abs_tight=1e-5)


SRELU_CASES = {
    "empty_and_single": ([0, 1, 300, 0, 211, 8], 256, 256),
    "ragged_ffn": (None, 256, 264),                  # F not a multiple of the 256-column tile
}


@pytest.mark.parametrize("case", list(SRELU_CASES))
def test_grouped_srelu_mlp_parity(case):
    splits, hidden, ffn = SRELU_CASES[case]
    T = 520 if splits is None else sum(splits)
    G = 5 if splits is None else len(splits)
    print(f"case grouped srelu mlp {case} T={T} G={G} hidden={hidden} ffn={ffn}", flush=True)
    inp = synth.grouped(T, G, hidden, ffn, seed=23, splits=splits, gated=False)
    got = run_grouped_mlp(inp, act="srelu")
    base = offsets.base_offsets(inp["splits"])
    x, w1, w2 = bf16_to_f64(inp["x"]), bf16_to_f64(inp["w1"]), bf16_to_f64(inp["w2"])
    p = inp["p"].astype(np.float64)
    f = grouped.grouped_mlp_fwd(x, w1, w2, p, base, act="srelu")
    b = grouped.grouped_mlp_bwd(bf16_to_f64(inp["dout"]), x, w1, w2, p, base, h=f["h"], y=f["y"], act="srelu")
    kw = dict(rel_tight=2.0 ** -7, abs_tight=5e-2)
    assert_close(host_f64(got["h"]), f["h"], TAU_BF16, what="h")
    for k, ref in (("y", f["y"]), ("out", f["out"]), ("dh", b["dh"]), ("dp", b["dp"]), ("dw2", b["dw2"]),
                   ("dx", b["dx"]), ("dw1", b["dw1"])):
        assert_close(host_f64(got[k]), ref, TAU_BF16, what=k, **kw)


CLAMPED_CASES = {
    # limit well inside the pre-activations' spread: both clamps engage on many elements
    "engaged_empty_and_single": ([0, 1, 300, 0, 211, 8], 256, 256, 0.25, 1.702),
    # a limit no pre-activation reaches, alpha 1: only the up half's offset of one remains
    "not_engaged": (None, 256, 256, 64.0, 1.0),
}


@pytest.mark.parametrize("case", list(CLAMPED_CASES))
def test_grouped_clamped_swiglu_mlp_parity(case):
    """Grouped MLP with the clamped SwiGLU in fc1's epilogue and its backward in fc2's dgrad
    epilogue. The oracle's backward reads the pre-activation rounded to bf16, as the saved
    pre-activation the kernel reads (the clamps' pass-through decisions are taken on it)."""
    splits, hidden, ffn, limit, alpha = CLAMPED_CASES[case]
    act = ("clamped_swiglu", limit, alpha)
    T = 520 if splits is None else sum(splits)
    G = 5 if splits is None else len(splits)
    print(f"case grouped clamped swiglu mlp {case} T={T} G={G} hidden={hidden} ffn={ffn}", flush=True)
    inp = synth.grouped(T, G, hidden, ffn, seed=25, splits=splits)
    got = run_grouped_mlp(inp, act=act)
    base = offsets.base_offsets(inp["splits"])
    x, w1, w2 = bf16_to_f64(inp["x"]), bf16_to_f64(inp["w1"]), bf16_to_f64(inp["w2"])
    p = inp["p"].astype(np.float64)
    f = grouped.grouped_mlp_fwd(x, w1, w2, p, base, act=act)
    h_saved = bf16_to_f64(f64_to_bf16(f["h"]))
    b = grouped.grouped_mlp_bwd(bf16_to_f64(inp["dout"]), x, w1, w2, p, base, h=h_saved, y=f["y"], act=act)
    if limit < 1.0:                                        # the clamps engage on both halves
        F = ffn
        assert np.mean(f["h"][:, :F] > limit) > 0.05 and np.mean(np.abs(f["h"][:, F:]) > limit) > 0.05
    kw = dict(rel_tight=2.0 ** -7, abs_tight=5e-2)
    h_set, n_amb = clamp_settled_h(host_f64(got["dh"]), b["dh"], b["gy"], f["h"], p, act)
    assert n_amb <= 1e-3 * h_set.size
    b = grouped.grouped_mlp_bwd(bf16_to_f64(inp["dout"]), x, w1, w2, p, base, h=bf16_to_f64(f64_to_bf16(h_set)),
                                y=f["y"], act=act)
    assert_close(host_f64(got["h"]), f["h"], TAU_BF16, what="h")
    for k, ref in (("y", f["y"]), ("out", f["out"]), ("dh", b["dh"]), ("dp", b["dp"]), ("dw2", b["dw2"]),
                   ("dx", b["dx"]), ("dw1", b["dw1"])):
        assert_close(host_f64(got[k]), ref, TAU_BF16, what=k, **kw)


def test_single_group_quantized_equals_dense_bitwise():
    """One group spanning every token: the MXFP8 and FP8 (per-group current scaling) grouped
    forward, dgrad and wgrad equal the dense MXFP8 / FP8 linear bit for bit (same operands, same
    per-tile accumulation order)."""
    from .gpu_paths import mx_layout, quant_fp8, quant_fp8_grouped, quant_mx, quant_mx_grouped
    T, N, K = 384, 256, 256                                 # T a multiple of 128: no token padding
    d = synth.dense(T, N, K, seed=24, outliers=True, w_std=1.0, dy_std=1.0)
    X, W, DY = dev_bf16(d["x"]), dev_bf16(d["w"]), dev_bf16(d["dy"])
    bf = dict(dtype=torch.bfloat16, device="cuda")
    offs = torch.tensor([0, T], dtype=torch.int64, device="cuda")
    lay = mx_layout(offs, T)
    # MXFP8
    qx, qw, qd = quant_mx(X), quant_mx(W), quant_mx(DY)
    ref_f, ref_d, ref_w = torch.empty(T, N, **bf), torch.empty(T, K, **bf), torch.empty(N, K, **bf)
    sge.linear_scale_add_fwd(sge.Operand.mxfp8(qx["q_row"], qx["s_row"]), sge.Operand.mxfp8(qw["q_row"], qw["s_row"]),
                             ref_f, 0.5, accumulate=False)
    sge.linear_scale_bwd(sge.Operand.mxfp8(qd["q_row"], qd["s_row"]), sge.Operand.mxfp8(qw["q_colT"], qw["s_colT"]),
                         sge.Operand.mxfp8(qd["q_colT"], qd["s_colT"]), sge.Operand.mxfp8(qx["q_colT"], qx["s_colT"]),
                         ref_d, ref_w, 0.5, 0.5)
    out, dx, dw = torch.empty(T, N, **bf), torch.empty(T, K, **bf), torch.empty(1, N, K, **bf)
    sge.grouped_linear_fwd_mxfp8(qx["q_row"], qx["s_row"], qw["q_row"][None], qw["s_row"][None], offs, out=out,
                                 alpha=0.5)
    sge.grouped_linear_dgrad_mxfp8(qd["q_row"], qd["s_row"], qw["q_colT"], qw["s_colT"], offs, alpha=0.5, dx=dx)
    tx, td = quant_mx_grouped(X, lay), quant_mx_grouped(DY, lay)
    sge.grouped_linear_wgrad_mxfp8(td["q_colT"], td["s_colT"], tx["q_colT"], tx["s_colT"], lay, dw, alpha=0.5)
    torch.cuda.synchronize()
    for a, b in ((out, ref_f), (dx, ref_d), (dw[0], ref_w)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    # FP8 current scaling: one group's scale is the tensor's scale
    fx, fw, fd = quant_fp8(X), quant_fp8(W), quant_fp8(DY)
    gx, gw, gd = quant_fp8_grouped(X, 1, lay), quant_fp8_grouped(W, 1), quant_fp8_grouped(DY, 1, lay)
    sge.linear_scale_add_fwd(sge.Operand.e4m3(fx["q"], fx["scale_inv"]), sge.Operand.e4m3(fw["q"], fw["scale_inv"]),
                             ref_f, 0.5, accumulate=False)
    sge.linear_scale_bwd(sge.Operand.e4m3(fd["q"], fd["scale_inv"]), sge.Operand.e4m3(fw["q_t"], fw["scale_inv"]),
                         sge.Operand.e4m3(fd["q_t"], fd["scale_inv"]), sge.Operand.e4m3(fx["q_t"], fx["scale_inv"]),
                         ref_d, ref_w, 0.5, 0.5)
    sge.grouped_linear_fwd_fp8(gx["q"], gx["scale_inv"], gw["q"][None], gw["scale_inv"], offs, out, alpha=0.5)
    sge.grouped_linear_dgrad_fp8(gd["q"], gd["scale_inv"], gw["q_t"], gw["scale_inv"], offs, alpha=0.5, dx=dx)
    sge.grouped_linear_wgrad_fp8(gd["q_t"], gd["scale_inv"], gx["q_t"], gx["scale_inv"], lay, dw, alpha=0.5)
    torch.cuda.synchronize()
    assert torch.equal(gx["scale_inv"], fx["scale_inv"]) and torch.equal(gx["q"], fx["q"])
    for a, b in ((out, ref_f), (dx, ref_d), (dw[0], ref_w)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))

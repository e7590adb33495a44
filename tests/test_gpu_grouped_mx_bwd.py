"""MXFP8 grouped backward against the oracle: the token-blocked group layout and quantizer
(bit-exact), the grouped dgrad with the fused backward of the scaled activation (SwiGLU or
SReLU) and group quantize, the grouped wgrad on token-blocked operands, and the whole MLP
backward (FP8 bar)."""

import numpy as np
import pytest
import torch

import synth
from oracle import grouped, offsets, quant
from oracle.codecs import bf16_to_f64, f64_to_bf16
from oracle.quant import mx_dequantize

from .gpu_paths import (grouped_dgrad_mx, grouped_wgrad_mx, mx_layout, quant_mx, quant_mx_grouped,
                        run_grouped_mlp_bwd_mx, run_grouped_mlp_fwd_mx)
from .helpers import (TAU_FP8, assert_close, assert_mx_dequant_close, assert_oracle_mx_rowwise, clamp_settled_h, dev,
                      dev_bf16, host_bits, host_f64, host_u8)

pytestmark = pytest.mark.gpu

# Clamped SwiGLU with a limit well inside the pre-activations' spread (both clamps engage)
CLAMPED = ("clamped_swiglu", 0.25, 1.702)

KW = dict(rel_tight=2.0 ** -3, abs_tight=0.1)

LAYOUT_CASES = {
    "ragged_with_empty_groups": ([0, 300, 300, 511, 520, 520, 560], 560),
    "one_group": ([0, 1000], 1000),
    "unsorted_and_out_of_range": ([5, -3, 10, 7, 100], 20),
    "all_empty": ([0, 0, 0], 0),
}


@pytest.mark.parametrize("case", list(LAYOUT_CASES))
def test_mx_group_layout_exact(case):
    offs, T = LAYOUT_CASES[case]
    print(f"case mx layout {case}", flush=True)
    lay = mx_layout(dev(np.asarray(offs, np.int64)), T)
    c, pad = quant.mx_group_layout(offs, T)
    got = lay.cpu().numpy()
    assert np.array_equal(got[0], c) and np.array_equal(got[1], pad)


def test_mx_group_layout_4096_groups():
    print("case mx layout G=4096", flush=True)
    rng = np.random.default_rng(7)
    splits = synth.dirichlet_splits(rng, 4096, 65536)
    base = offsets.base_offsets(splits)
    lay = mx_layout(dev(base), 65536).cpu().numpy()
    c, pad = quant.mx_group_layout(base, 65536)
    assert np.array_equal(lay[0], c) and np.array_equal(lay[1], pad)


QUANT_CASES = {
    "ragged_with_empty_groups": ([300, 0, 211, 9, 0, 40], 96),
    "aligned_single_group": ([256], 64),
    "dirichlet_8": (None, 160),
    "no_tokens": ([0, 0], 32),
}


@pytest.mark.parametrize("case", list(QUANT_CASES))
def test_quantize_mxfp8_grouped_exact(case):
    splits, C = QUANT_CASES[case]
    if splits is None:
        splits = synth.dirichlet_splits(np.random.default_rng(3), 8, 1000)
    T = int(sum(splits))
    print(f"case mx grouped quant {case} T={T} C={C}", flush=True)
    r = synth.streams(12)
    x = synth.normal_bf16(r["x"], (T, C), 1.0, r["outliers_x"])
    base = offsets.base_offsets(splits)
    lay = mx_layout(dev(base), T)
    got = quant_mx_grouped(dev_bf16(x) if T else torch.empty(0, C, dtype=torch.bfloat16, device="cuda"), lay,
                           row=True, fill=0xAB)
    torch.cuda.synchronize()
    c, pad = quant.mx_group_layout(base, T)
    q, s = quant.mxfp8_colwise_grouped(x, c, pad, got["ld"])
    P = int(pad[-1])
    gq, gs = host_u8(got["q_colT"]), host_u8(got["s_colT"])
    assert np.array_equal(gq[:, :P], q[:, :P])
    assert np.array_equal(gs[:, :P // 32], s[:, :P // 32])
    assert np.all(gq[:, P:] == 0xAB) and np.all(gs[:, P // 32:] == 0xAB)     # past the last group: untouched
    if T:
        qr, sr = quant.mxfp8_rowwise(x)
        assert np.array_equal(host_u8(got["q_row"]), qr) and np.array_equal(host_u8(got["s_row"]), sr)


DGRAD_CASES = {
    "ragged_with_empty_group": ([300, 0, 211, 9, 0, 40], 256, 384),
    "dirichlet_5": (None, 512, 256),
}


@pytest.mark.parametrize("case", list(DGRAD_CASES))
def test_grouped_dgrad_mxfp8(case):
    splits, N, K = DGRAD_CASES[case]
    if splits is None:
        splits = synth.dirichlet_splits(np.random.default_rng(4), 5, 700)
    T, G = int(sum(splits)), len(splits)
    print(f"case mx grouped dgrad {case} T={T} G={G} N={N} K={K}", flush=True)
    r = synth.streams(13)
    dy = synth.normal_bf16(r["dy"], (T, N), 1.0, r["outliers_dy"])
    w = synth.normal_bf16(r["w"], (G, N, K), 0.02, r["outliers_w"])
    base = offsets.base_offsets(splits)
    W = dev_bf16(w)
    q_dy = quant_mx(dev_bf16(dy), col=False)
    w_col = quant_mx(W.reshape(G * N, K), row=False)
    out = grouped_dgrad_mx(q_dy, w_col, dev(base), alpha=-0.75)
    torch.cuda.synchronize()
    # operand bytes: W blocked along N per expert, stored [K][G*N]
    for g in range(G):
        qg, sg = quant.mxfp8_colwise(w[g])
        assert np.array_equal(host_u8(w_col["q_colT"])[:, g * N:(g + 1) * N], qg)
        assert np.array_equal(host_u8(w_col["s_colT"])[:, g * N // 32:(g + 1) * N // 32], sg)
    ref = grouped.grouped_linear_dgrad_mxfp8(dy, w, base, alpha=-0.75)
    assert_close(host_f64(out["dx"]), ref, TAU_FP8, what="dx", **KW)


@pytest.mark.parametrize("case", list(DGRAD_CASES))
def test_grouped_dgrad_mxfp8_dswiglu_fused_quantize(case):
    splits, N, K = DGRAD_CASES[case]
    if splits is None:
        splits = synth.dirichlet_splits(np.random.default_rng(4), 5, 700)
    T, G = int(sum(splits)), len(splits)
    print(f"case mx grouped dgrad dswiglu {case} T={T} G={G} N={N} F={K}", flush=True)
    r = synth.streams(14)
    dy = synth.normal_bf16(r["dy"], (T, N), 1e-2)
    w = synth.normal_bf16(r["w"], (G, N, K), 0.02)
    h = synth.normal_bf16(r["x"], (T, 2 * K), 1.0)
    p = r["p"].random(size=T, dtype=np.float32)
    base = offsets.base_offsets(splits)
    W = dev_bf16(w)
    q_dy = quant_mx(dev_bf16(dy), col=False)
    w_col = quant_mx(W.reshape(G * N, K), row=False)
    out = grouped_dgrad_mx(q_dy, w_col, dev(base), preact=dev_bf16(h), probs=dev(p), want_q=True)
    unfused = quant_mx(out["dact"], col=False)
    torch.cuda.synchronize()
    # fused group quantize == the oracle's MXFP8 of the same launch's bf16 dact, and the standalone
    # quantizer on it
    assert_oracle_mx_rowwise(host_bits(out["dact"]), host_u8(out["dact_q"]), host_u8(out["dact_s"]),
                             what="dact (fused MXFP8)")
    assert np.array_equal(host_u8(out["dact_q"]), host_u8(unfused["q_row"]))
    assert np.array_equal(host_u8(out["dact_s"]), host_u8(unfused["s_row"]))
    gy = grouped.grouped_linear_dgrad_mxfp8(dy, w, base)
    rdh, rdp = grouped.scaled_swiglu_bwd(gy, bf16_to_f64(h), p)
    assert_close(host_f64(out["dact"]), rdh, TAU_FP8, what="dact", **KW)
    assert_close(host_f64(out["dprobs"]), rdp, TAU_FP8, what="dprobs", **KW)
    rq, rs = quant.mxfp8_rowwise(f64_to_bf16(rdh))
    assert_mx_dequant_close(mx_dequantize(host_u8(out["dact_q"]), host_u8(out["dact_s"])), mx_dequantize(rq, rs),
                            what="dact (MXFP8)")


COLT_CASES = {
    "ragged_with_empty_groups": ([300, 0, 211, 9, 0, 40], 256, 384),
    # whole tiles, a group ending 127 rows into its second tile's aligned range, an empty one
    "tile_multiples": ([512, 256, 129, 0, 383], 128, 256),
    "dirichlet_6": (None, 256, 128),
    # many small groups (every tile a single partial pass), one exactly 128 and one exactly 256
    "many_small_groups": ([7, 0, 128, 33, 1, 256, 0, 90, 12, 5, 64, 31, 2, 0, 19, 40], 128, 128),
}


@pytest.mark.parametrize("act", ["swiglu", "srelu", CLAMPED], ids=["swiglu", "srelu", "clamped_swiglu"])
@pytest.mark.parametrize("case", list(COLT_CASES))
def test_grouped_dgrad_mxfp8_token_blocked_output(case, act):
    """The dgrad epilogue's token-blocked dact: bit-exact against the oracle's token blocking of
    the same launch's bf16 dact and against the standalone token-blocked quantizer, padding
    included; nothing written past the last group's range; the same bytes (and the same
    rowwise MXFP8) without the bf16 dact."""
    splits, N, K = COLT_CASES[case]
    if splits is None:
        splits = synth.dirichlet_splits(np.random.default_rng(6), 6, 900)
    T, G = int(sum(splits)), len(splits)
    hw = K if act == "srelu" else 2 * K
    print(f"case mx grouped dgrad token-blocked {case} {act} T={T} G={G} N={N} K={K}", flush=True)
    r = synth.streams(16)
    dy = synth.normal_bf16(r["dy"], (T, N), 1e-2)
    w = synth.normal_bf16(r["w"], (G, N, K), 0.02)
    h = synth.normal_bf16(r["x"], (T, hw), 1.0)
    p = r["p"].random(size=T, dtype=np.float32)
    base = offsets.base_offsets(splits)
    W = dev_bf16(w)
    q_dy = quant_mx(dev_bf16(dy), col=False)
    w_col = quant_mx(W.reshape(G * N, K), row=False)
    lay = mx_layout(dev(base), T)
    kw = dict(preact=dev_bf16(h), probs=dev(p), act=act, lay=lay)
    out = grouped_dgrad_mx(q_dy, w_col, dev(base), want_q=True, **kw)
    alone = grouped_dgrad_mx(q_dy, w_col, dev(base), want_q=True, want_bf16=False, fill=0x5C, **kw)
    std = quant_mx_grouped(out["dact"], lay)
    torch.cuda.synchronize()
    c, pad = quant.mx_group_layout(base, T)
    P = int(pad[-1])
    q, s = quant.mxfp8_colwise_grouped(host_bits(out["dact"]), c, pad, out["ld"])
    gq, gs = host_u8(out["q_colT"]), host_u8(out["s_colT"])
    assert np.array_equal(gq[:, :P], q[:, :P]) and np.array_equal(gs[:, :P // 32], s[:, :P // 32])
    assert np.all(gq[:, P:] == 0xAB) and np.all(gs[:, P // 32:] == 0xAB)
    assert np.array_equal(gq[:, :P], host_u8(std["q_colT"])[:, :P])
    assert np.array_equal(gs[:, :P // 32], host_u8(std["s_colT"])[:, :P // 32])
    aq, as_ = host_u8(alone["q_colT"]), host_u8(alone["s_colT"])
    assert np.array_equal(aq[:, :P], gq[:, :P]) and np.array_equal(as_[:, :P // 32], gs[:, :P // 32])
    assert np.all(aq[:, P:] == 0x5C) and np.all(as_[:, P // 32:] == 0x5C)
    assert np.array_equal(host_u8(alone["dact_q"]), host_u8(out["dact_q"]))
    assert np.array_equal(host_u8(alone["dact_s"]), host_u8(out["dact_s"]))
    assert np.array_equal(host_u8(alone["dprobs"]), host_u8(out["dprobs"]))


WGRAD_CASES = {
    "ragged_with_empty_groups": ([300, 0, 211, 9, 0, 40], 256, 192),
    "dirichlet_wide": (None, 512, 384),
    "mid_xcd_slices": ([700, 0, 333, 41, 210], 1024, 512),
}


@pytest.mark.parametrize("case", list(WGRAD_CASES))
def test_grouped_wgrad_mxfp8(case):
    splits, N, K = WGRAD_CASES[case]
    if splits is None:
        splits = synth.dirichlet_splits(np.random.default_rng(5), 6, 900)
    T, G = int(sum(splits)), len(splits)
    print(f"case mx grouped wgrad {case} T={T} G={G} N={N} K={K}", flush=True)
    r = synth.streams(15)
    dy = synth.normal_bf16(r["dy"], (T, N), 1e-2, r["outliers_dy"])
    x = synth.normal_bf16(r["x"], (T, K), 1.0, r["outliers_x"])
    base = offsets.base_offsets(splits)
    lay = mx_layout(dev(base), T)
    qa, qb = quant_mx_grouped(dev_bf16(dy), lay), quant_mx_grouped(dev_bf16(x), lay)
    dw = grouped_wgrad_mx(qa, qb, lay, G, alpha=0.5)
    torch.cuda.synchronize()
    c, pad = quant.mx_group_layout(base, T)
    P = int(pad[-1])
    for got, src in ((qa, dy), (qb, x)):
        q, s = quant.mxfp8_colwise_grouped(src, c, pad, got["ld"])
        assert np.array_equal(host_u8(got["q_colT"])[:, :P], q[:, :P])
        assert np.array_equal(host_u8(got["s_colT"])[:, :P // 32], s[:, :P // 32])
    ref = grouped.grouped_linear_wgrad_mxfp8(dy, x, base, alpha=0.5)
    assert_close(host_f64(dw), ref, TAU_FP8, what="dw", **KW)
    for g in range(G):
        if splits[g] == 0:
            assert not host_f64(dw[g]).any()                  # empty group: zero gradient


MLP_CASES = {
    "ragged_with_empty_group": ([300, 0, 211, 9, 0, 40], 256, 256),
    "dirichlet_wide": (None, 512, 384),
}


@pytest.mark.parametrize("act", ["swiglu", "srelu", CLAMPED], ids=["swiglu", "srelu", "clamped_swiglu"])
@pytest.mark.parametrize("case", list(MLP_CASES))
def test_mxfp8_grouped_mlp_backward(case, act):
    splits, hidden, ffn = MLP_CASES[case]
    T = 700 if splits is None else sum(splits)
    G = 5 if splits is None else len(splits)
    print(f"case mxfp8 grouped mlp bwd {case} {act} T={T} G={G} hidden={hidden} ffn={ffn}", flush=True)
    inp = synth.grouped(T, G, hidden, ffn, seed=32, splits=splits, gated=act != "srelu")
    fwd = run_grouped_mlp_fwd_mx(inp, act)
    got = run_grouped_mlp_bwd_mx(inp, fwd)
    base = offsets.base_offsets(inp["splits"])
    rf = grouped.grouped_mlp_fwd_mxfp8(inp["x"], inp["w1"], inp["w2"], inp["p"], base, act)
    ref = grouped.grouped_mlp_bwd_mxfp8(inp["x"], inp["w1"], inp["w2"], inp["p"], base, inp["dout"], fwd=rf,
                                        act=act)
    # fused activation backward + group quantize == the oracle's MXFP8 of the same launch's bf16
    # dh, and the standalone quantizer on it
    assert_oracle_mx_rowwise(host_bits(got["dh"]), host_u8(got["dhq"]), host_u8(got["dhs"]), what="dh (fused MXFP8)")
    assert np.array_equal(host_u8(got["dhq"]), host_u8(got["dh_unfused"]["q_row"]))
    assert np.array_equal(host_u8(got["dhs"]), host_u8(got["dh_unfused"]["s_row"]))
    # the token-blocked wgrad operands of y and dh, written by the producing epilogues: the
    # oracle's blocking of the same launches' bf16 tensors
    c, pad = quant.mx_group_layout(base, T)
    P = int(pad[-1])
    for key, src in (("q_y", fwd["y"]), ("q_dh", got["dh"])):
        q, s = quant.mxfp8_colwise_grouped(host_bits(src), c, pad, got[key]["ld"])
        assert np.array_equal(host_u8(got[key]["q_colT"])[:, :P], q[:, :P]), key
        assert np.array_equal(host_u8(got[key]["s_colT"])[:, :P // 32], s[:, :P // 32]), key
    if isinstance(act, tuple):                             # clamps: settle the ambiguous decisions
        h_set, n_amb = clamp_settled_h(host_f64(got["dh"]), ref["dh"], ref["gy"], rf["h"], inp["p"], act)
        assert n_amb <= 1e-3 * h_set.size
        ref = grouped.grouped_mlp_bwd_mxfp8(inp["x"], inp["w1"], inp["w2"], inp["p"], base, inp["dout"],
                                            fwd=dict(rf, h=h_set), act=act)
    assert_close(host_f64(got["dh"]), ref["dh"], TAU_FP8, what="dh", **KW)
    assert_close(host_f64(got["dp"]), ref["dp"], TAU_FP8, what="dprobs", **KW)
    assert_close(host_f64(got["dx"]), ref["dx"], TAU_FP8, what="dx", **KW)
    assert_close(host_f64(got["dw2"]), ref["dw2"], TAU_FP8, what="dw2", **KW)
    assert_close(host_f64(got["dw1"]), ref["dw1"], TAU_FP8, what="dw1", **KW)

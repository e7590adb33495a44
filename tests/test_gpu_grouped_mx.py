"""MXFP8 grouped MLP forward with the fused activation + group quantize, against the oracle.

The fused MXFP8 output of fc1 must equal, byte for byte, the oracle's MXFP8 quantization of the
same launch's bf16 output (the fusion of the activation and the group quantize; the standalone
quantizer on that output writes the same bytes); every
value is compared with the oracle's own pipeline from the same seeded inputs within the FP8 bar.
"""

import numpy as np
import pytest
import torch

import scaled_gemm_epilogues_amd as sge
import synth
from oracle import grouped, offsets, quant
from oracle.quant import mx_dequantize

from .gpu_paths import (_act_epilogues, _act_params, mx_layout, quant_mx, quant_mx_grouped,
                        run_grouped_mlp_fwd_mx)
from .helpers import (TAU_FP8, assert_close, assert_mx_dequant_close, assert_oracle_mx_rowwise, dev, dev_bf16,
                      host_bits, host_f64, host_u8)

pytestmark = pytest.mark.gpu

# Clamped SwiGLU with a limit well inside the pre-activations' spread (both clamps engage)
CLAMPED = ("clamped_swiglu", 0.25, 1.702)

KW = dict(rel_tight=2.0 ** -3, abs_tight=0.1)

CASES = {
    "ragged_with_empty_group": ([300, 0, 211, 9, 0, 40], 256, 256),
    "dirichlet_wide": (None, 512, 384),
}


@pytest.mark.parametrize("act", ["swiglu", "srelu", CLAMPED], ids=["swiglu", "srelu", "clamped_swiglu"])
@pytest.mark.parametrize("case", list(CASES))
def test_mxfp8_grouped_mlp_forward(case, act):
    splits, hidden, ffn = CASES[case]
    T = 700 if splits is None else sum(splits)
    G = 5 if splits is None else len(splits)
    print(f"case mxfp8 grouped fwd {case} {act} T={T} G={G} hidden={hidden} ffn={ffn}", flush=True)
    inp = synth.grouped(T, G, hidden, ffn, seed=31, splits=splits, gated=act != "srelu")
    got = run_grouped_mlp_fwd_mx(inp, act)
    assert int(got["err"].item()) == 0
    base = offsets.base_offsets(inp["splits"])
    ref = grouped.grouped_mlp_fwd_mxfp8(inp["x"], inp["w1"], inp["w2"], inp["p"], base, act)

    # quantized operands: bit-exact against the oracle's MXFP8
    for key, src in (("qx", inp["x"]), ("qw1", inp["w1"].reshape(-1, hidden)),
                     ("qw2", inp["w2"].reshape(G * hidden, ffn))):
        q, s = quant.mxfp8_rowwise(src)
        assert np.array_equal(host_u8(got[key]["q_row"]), q), key
        assert np.array_equal(host_u8(got[key]["s_row"]), s), key

    # fused activation + group quantize == the oracle's MXFP8 of the same launch's bf16 activation
    assert_oracle_mx_rowwise(host_bits(got["y"]), host_u8(got["yq"]), host_u8(got["ys"]), what="y (fused MXFP8)")
    # and == the standalone quantizer on it
    assert np.array_equal(host_u8(got["yq"]), host_u8(got["y_unfused"]["q_row"]))
    assert np.array_equal(host_u8(got["ys"]), host_u8(got["y_unfused"]["s_row"]))
    # the token-blocked y from the same epilogue == the oracle's blocking of that bf16 y
    c, pad = quant.mx_group_layout(base, T)
    P = int(pad[-1])
    q, s = quant.mxfp8_colwise_grouped(host_bits(got["y"]), c, pad, got["q_y"]["ld"])
    assert np.array_equal(host_u8(got["q_y"]["q_colT"])[:, :P], q[:, :P])
    assert np.array_equal(host_u8(got["q_y"]["s_colT"])[:, :P // 32], s[:, :P // 32])

    assert_close(host_f64(got["h"]), ref["h"], TAU_FP8, what="h", **KW)
    assert_close(host_f64(got["y"]), ref["y"], TAU_FP8, what="y", **KW)
    # the MXFP8 activation against the oracle's MXFP8 of its own activation (the shared
    # exponent saturates a block's largest element at 448 * 2^X: compare like with like)
    y_deq = mx_dequantize(host_u8(got["yq"]), host_u8(got["ys"]))
    assert_mx_dequant_close(y_deq, mx_dequantize(ref["y_q"], ref["y_s"]), what="y (MXFP8)")
    assert_close(host_f64(got["out"]), ref["out"], TAU_FP8, what="out", **KW)


COLT_CASES = {
    # groups of whole tiles, one 129 rows long (its aligned range ends 127 rows into its
    # second tile), an empty one, and one ending 128 rows into an aligned 256
    "tile_multiples": ([512, 256, 129, 0, 383], 128, 384),
    "ragged_with_empty_groups": ([300, 0, 211, 9, 0, 40], 256, 128),
    "many_small_groups": ([7, 0, 128, 33, 1, 256, 0, 90, 12, 5, 64, 31, 2, 0, 19, 40], 128, 128),
}


@pytest.mark.parametrize("act", ["swiglu", "srelu", CLAMPED], ids=["swiglu", "srelu", "clamped_swiglu"])
@pytest.mark.parametrize("case", list(COLT_CASES))
def test_mxfp8_grouped_fwd_token_blocked_output(case, act):
    """fc1's token-blocked activation output: bit-exact against the oracle's token blocking of
    the same launch's bf16 output and against the standalone token-blocked quantizer, padding
    included; nothing written past the last group's range; the same bytes without the bf16
    output."""
    splits, hidden, ffn = COLT_CASES[case]
    T, G = sum(splits), len(splits)
    print(f"case mxfp8 grouped fwd token-blocked {case} {act} T={T} G={G} hidden={hidden} ffn={ffn}", flush=True)
    inp = synth.grouped(T, G, hidden, ffn, seed=33, splits=splits, gated=act != "srelu")
    X, W1 = dev_bf16(inp["x"]), dev_bf16(inp["w1"])
    P = torch.from_numpy(inp["p"]).cuda()
    _, N1, H = W1.shape
    width, fwd_epi, _ = _act_epilogues(act)
    F = width(N1)
    base_h = offsets.base_offsets(splits)
    base = dev(base_h)
    lay = mx_layout(base, T)
    ld = sge.mx_token_capacity(T, G)
    qx = quant_mx(X, col=False)
    qw1 = quant_mx(W1.reshape(G * N1, H), col=False)
    y = torch.empty(T, F, dtype=torch.bfloat16, device="cuda")

    def call(out, fill):
        qT = torch.full((F, ld), fill, dtype=torch.uint8, device="cuda")
        sT = torch.full((F, ld // 32), fill, dtype=torch.uint8, device="cuda")
        sge.grouped_linear_fwd_mxfp8(qx["q_row"], qx["s_row"], qw1["q_row"].reshape(G, N1, H),
                                     qw1["s_row"].reshape(G, N1, H // 32), base, out=out, epilogue=fwd_epi, probs=P,
                                     act=_act_params(act), layout=lay, out_colT_q=qT, out_colT_s=sT)
        return host_u8(qT), host_u8(sT)

    gq, gs = call(y, 0xAB)
    aq, as_ = call(None, 0x5C)
    std = quant_mx_grouped(y, lay)
    torch.cuda.synchronize()
    c, pad = quant.mx_group_layout(base_h, T)
    Pn = int(pad[-1])
    q, s = quant.mxfp8_colwise_grouped(host_bits(y), c, pad, ld)
    assert np.array_equal(gq[:, :Pn], q[:, :Pn]) and np.array_equal(gs[:, :Pn // 32], s[:, :Pn // 32])
    assert np.all(gq[:, Pn:] == 0xAB) and np.all(gs[:, Pn // 32:] == 0xAB)
    assert np.array_equal(gq[:, :Pn], host_u8(std["q_colT"])[:, :Pn])
    assert np.array_equal(gs[:, :Pn // 32], host_u8(std["s_colT"])[:, :Pn // 32])
    assert np.array_equal(aq[:, :Pn], gq[:, :Pn]) and np.array_equal(as_[:, :Pn // 32], gs[:, :Pn // 32])
    assert np.all(aq[:, Pn:] == 0x5C) and np.all(as_[:, Pn // 32:] == 0x5C)

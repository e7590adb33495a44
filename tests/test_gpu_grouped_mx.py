"""MXFP8 grouped MLP forward with the fused activation + group quantize, against the oracle.

The fused MXFP8 output of fc1 must equal, byte for byte, the oracle's MXFP8 quantization of the
same launch's bf16 output (the fusion of the activation and the group quantize; the standalone
quantizer on that output writes the same bytes); every
value is compared with the oracle's own pipeline from the same seeded inputs within the FP8 bar.
"""

import numpy as np
import pytest

import synth
from oracle import grouped, offsets, quant
from oracle.quant import mx_dequantize

from .gpu_paths import run_grouped_mlp_fwd_mx
from .helpers import (TAU_FP8, assert_close, assert_mx_dequant_close, assert_oracle_mx_rowwise, host_bits, host_f64,
                      host_u8)

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

    assert_close(host_f64(got["h"]), ref["h"], TAU_FP8, what="h", **KW)
    assert_close(host_f64(got["y"]), ref["y"], TAU_FP8, what="y", **KW)
    # the MXFP8 activation against the oracle's MXFP8 of its own activation (the shared
    # exponent saturates a block's largest element at 448 * 2^X: compare like with like)
    y_deq = mx_dequantize(host_u8(got["yq"]), host_u8(got["ys"]))
    assert_mx_dequant_close(y_deq, mx_dequantize(ref["y_q"], ref["y_s"]), what="y (MXFP8)")
    assert_close(host_f64(got["out"]), ref["out"], TAU_FP8, what="out", **KW)

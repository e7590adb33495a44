"""The no-allocation FP8 current-scaling quantizer (partials in the library's per-GPU scratch
array) against the workspace entry point and the oracle, on two calls in a row, the second on a
smaller tensor (the array keeps the first call's partials)."""

import numpy as np
import pytest
import torch

import scaled_gemm_epilogues_amd as sge
import synth
from oracle import quant

from .gpu_paths import quant_fp8
from .helpers import dev_bf16, host_u8

pytestmark = pytest.mark.gpu


def _f32_bits(t):
    return t.detach().cpu().numpy().astype(np.float32).view(np.uint32)


@pytest.mark.parametrize("order", ["large_then_small"])
def test_quantize_fp8_amax_noalloc(order):
    r = synth.streams(41)
    # the large tensor asks for all 1024 partials; the smaller one for fewer (its amax is far
    # below the first one's, so a stale partial would change the scale)
    shapes = [((4096, 2048), 1.0), ((512, 272), 1e-3)]
    for (R, C), std in shapes:
        print(f"case noalloc fp8 {R}x{C} std={std}", flush=True)
        bits = synth.normal_bf16(r["x"], (R, C), std)
        X = dev_bf16(bits)
        ref = quant_fp8(X)
        u8, f32 = dict(dtype=torch.uint8, device="cuda"), dict(dtype=torch.float32, device="cuda")
        q, qt = torch.empty(R, C, **u8), torch.empty(C, R, **u8)
        amax, scale, sinv = torch.empty(1, **f32), torch.empty(1, **f32), torch.empty(1, **f32)
        sge.quantize_fp8_amax_noalloc(X, q, qt, amax, scale, sinv)
        torch.cuda.synchronize()
        assert np.array_equal(host_u8(q), host_u8(ref["q"]))
        assert np.array_equal(host_u8(qt), host_u8(ref["q_t"]))
        for got, want in ((amax, ref["amax"]), (scale, ref["scale"]), (sinv, ref["scale_inv"])):
            assert np.array_equal(_f32_bits(got), _f32_bits(want))
        o = quant.fp8_current_scaling(bits)
        assert _f32_bits(scale)[0] == np.float32(o["scale"]).view(np.uint32)
        assert np.array_equal(host_u8(q), o["q"])

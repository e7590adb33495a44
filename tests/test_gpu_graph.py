"""Every libsge call is capture-safe: a step captured in a HIP graph and replayed several times
(with eager work and synchronizations between replays) gives the eager result on every replay."""

import numpy as np
import pytest
import torch

import scaled_gemm_epilogues_amd as sge
import synth

from .gpu_paths import quant_fp8
from .helpers import dev_bf16

pytestmark = pytest.mark.gpu


def _capture(fn):
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _bits(t):
    return t.view(torch.int16).cpu().numpy().copy() if t.dtype == torch.bfloat16 else t.cpu().numpy().copy()


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_dense_step_graph_replays_match_eager(fmt):
    d = synth.dense(512, 512, 256, seed=31)
    X, W, DY = dev_bf16(d["x"]), dev_bf16(d["w"]), dev_bf16(d["dy"])
    R0 = dev_bf16(d["residual"])
    R = R0.clone()
    dg = torch.empty(512, 256, dtype=torch.bfloat16, device="cuda")
    wg = torch.empty(512, 256, dtype=torch.bfloat16, device="cuda")
    if fmt == "bf16":
        def step():
            sge.linear_scale_add_fwd(sge.Operand.bf16(X), sge.Operand.bf16(W), R, 0.5)
            sge.linear_scale_bwd(sge.Operand.bf16(DY), sge.Operand.bf16(W, transposed=True),
                                 sge.Operand.bf16(DY, transposed=True), sge.Operand.bf16(X, transposed=True),
                                 dg, wg, 0.5, 0.5)
    else:
        qx, qw, qd = quant_fp8(X), quant_fp8(W), quant_fp8(DY)

        def step():
            for src, b in ((X, qx), (W, qw), (DY, qd)):
                ws = b.setdefault("ws", torch.empty(sge.quantize_fp8_amax_workspace_size(*src.shape),
                                                    dtype=torch.uint8, device="cuda"))
                sge.quantize_fp8_amax(src, b["q"], b["q_t"], b["amax"], b["scale"], b["scale_inv"], ws)
            sge.linear_scale_add_fwd(sge.Operand.e4m3(qx["q"], qx["scale_inv"]),
                                     sge.Operand.e4m3(qw["q"], qw["scale_inv"]), R, 0.5)
            sge.linear_scale_bwd(sge.Operand.e4m3(qd["q"], qd["scale_inv"]), sge.Operand.e4m3(qw["q_t"], qw["scale_inv"]),
                                 sge.Operand.e4m3(qd["q_t"], qd["scale_inv"]), sge.Operand.e4m3(qx["q_t"], qx["scale_inv"]),
                                 dg, wg, 0.5, 0.5)
    step()
    torch.cuda.synchronize()
    want = [_bits(R), _bits(dg), _bits(wg)]
    g = _capture(step)
    for _ in range(3):
        R.copy_(R0)
        dg.fill_(float("nan"))
        wg.fill_(float("nan"))
        torch.cuda.synchronize()
        _ = torch.randn(64, 64, device="cuda") @ torch.randn(64, 64, device="cuda")   # eager work between
        g.replay()
        torch.cuda.synchronize()
        got = [_bits(R), _bits(dg), _bits(wg)]
        for a, b in zip(got, want):
            assert np.array_equal(a, b)


def test_grouped_step_graph_replays_match_eager():
    inp = synth.grouped(700, 4, 256, 256, seed=32)
    X, W1, W2, DOUT = dev_bf16(inp["x"]), dev_bf16(inp["w1"]), dev_bf16(inp["w2"]), dev_bf16(inp["dout"])
    P = torch.from_numpy(inp["p"]).cuda()
    splits = torch.from_numpy(inp["splits"]).cuda()
    T, G, F = 700, 4, 256
    offs = torch.empty(1, G + 1, dtype=torch.int64, device="cuda")
    bf = dict(dtype=torch.bfloat16, device="cuda")
    h, y, out = torch.empty(T, 2 * F, **bf), torch.empty(T, F, **bf), torch.empty(T, 256, **bf)
    dh, dp = torch.empty(T, 2 * F, **bf), torch.empty(T, dtype=torch.float32, device="cuda")
    dw2, dx, dw1 = torch.empty(G, 256, F, **bf), torch.empty(T, 256, **bf), torch.empty(G, 2 * F, 256, **bf)
    ws = torch.empty(sge.grouped_linear_bwd_workspace_size(T, F, G, sge.EPI_DSCALED_SWIGLU), dtype=torch.uint8,
                     device="cuda")
    outs = [offs, h, y, out, dh, dp, dw2, dx, dw1]

    def step():
        sge.splits_to_offsets(splits, [1], offs)
        base = offs[0]
        sge.grouped_linear_fwd(X, W1, base, y, epilogue=sge.EPI_SCALED_SWIGLU, probs=P, preact=h)
        sge.grouped_linear_fwd(y, W2, base, out)
        sge.grouped_linear_bwd(DOUT, y, W2, base, epilogue=sge.EPI_DSCALED_SWIGLU, preact=h, probs=P, dact=dh,
                               dprobs=dp, dw=dw2, workspace=ws)
        sge.grouped_linear_bwd(dh, X, W1, base, dx=dx, dw=dw1)
    step()
    torch.cuda.synchronize()
    want = [_bits(t) for t in outs]
    g = _capture(step)
    for _ in range(3):
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, w in zip(outs, want):
            assert np.array_equal(_bits(t), w)

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


def _replays_match(step, outs):
    """Run ``step`` eagerly, capture it, replay three times (poisoning the outputs, with eager
    work between) and compare every output bitwise with the eager run. Outputs are poisoned
    before the eager run too: regions a call leaves unwritten (past the last group of a
    token-blocked copy) must stay as they were."""
    for t in outs:
        t.fill_(float("nan") if t.is_floating_point() else 0xAB)
    step()
    torch.cuda.synchronize()
    want = [_bits(t) for t in outs]
    g = _capture(step)
    for _ in range(3):
        for t in outs:
            t.fill_(float("nan") if t.is_floating_point() else 0xAB)
        torch.cuda.synchronize()
        _ = torch.randn(64, 64, device="cuda") @ torch.randn(64, 64, device="cuda")
        g.replay()
        torch.cuda.synchronize()
        for t, w in zip(outs, want):
            assert np.array_equal(_bits(t), w)


def test_quantized_grouped_steps_graph_replays_match_eager():
    inp = synth.grouped(700, 4, 256, 256, seed=33)
    X, W1, DOUT = dev_bf16(inp["x"]), dev_bf16(inp["w1"]), dev_bf16(inp["dout"])
    P = torch.from_numpy(inp["p"]).cuda()
    T, H = X.shape
    G, N1, _ = W1.shape
    F = N1 // 2
    u8, f32, bf = (dict(dtype=d, device="cuda") for d in (torch.uint8, torch.float32, torch.bfloat16))
    offs = torch.empty(1, G + 1, dtype=torch.int64, device="cuda")
    splits = torch.from_numpy(inp["splits"]).cuda()
    lay = torch.empty(2, G + 1, dtype=torch.int64, device="cuda")
    ld = sge.mx_token_capacity(T, G)
    # FP8 per group: quantize x and W1 (with fused amax downstream), fc1 + SwiGLU, quantize y
    qws = torch.empty(16, **u8)
    fx = [torch.empty(T, H, **u8), torch.empty(H, ld, **u8)] + [torch.empty(G, **f32) for _ in range(3)]
    fw = [torch.empty(G * N1, H, **u8), torch.empty(H, G * N1, **u8)] + [torch.empty(G, **f32) for _ in range(3)]
    fy = [torch.empty(T, F, **u8), torch.empty(F, ld, **u8)] + [torch.empty(G, **f32) for _ in range(3)]
    h, y, amax_y = torch.empty(T, N1, **bf), torch.empty(T, F, **bf), torch.empty(G, **f32)
    # MXFP8: token-blocked dout, W2 columnwise, dgrad with dSwiGLU + MXFP8 dh, wgrad
    W2 = dev_bf16(inp["w2"])
    mdT, msT = torch.empty(H, ld, **u8), torch.empty(H, ld // 32, **u8)
    md, ms = torch.empty(T, H, **u8), torch.empty(T, H // 32, **u8)
    w2c, w2s = torch.empty(F, G * H, **u8), torch.empty(F, G * H // 32, **u8)
    myT, mysT = torch.empty(F, ld, **u8), torch.empty(F, ld // 32, **u8)
    dh, dp = torch.empty(T, N1, **bf), torch.empty(T, **f32)
    dhq, dhs = torch.empty(T, N1, **u8), torch.empty(T, N1 // 32, **u8)
    dw2 = torch.empty(G, H, F, **bf)
    ws = torch.empty(max(1, sge.grouped_linear_bwd_workspace_size(T, F, G, sge.EPI_DSCALED_SWIGLU)), **u8)
    # MXFP8 fc1 forward whose epilogue writes y rowwise and token-blocked (no bf16 y), and the
    # dgrad's token-blocked dh
    mx, mxs = torch.empty(T, H, **u8), torch.empty(T, H // 32, **u8)
    w1q, w1s = torch.empty(G * N1, H, **u8), torch.empty(G * N1, H // 32, **u8)
    h2, yq2, ys2 = torch.empty(T, N1, **bf), torch.empty(T, F, **u8), torch.empty(T, F // 32, **u8)
    yT2, ysT2 = torch.empty(F, ld, **u8), torch.empty(F, ld // 32, **u8)
    dhT, dhsT = torch.empty(N1, ld, **u8), torch.empty(N1, ld // 32, **u8)

    def step():
        sge.splits_to_offsets(splits, [1], offs)
        base = offs[0]
        sge.mx_group_layout(base, T, lay)
        sge.quantize_fp8_grouped(X, G, *fx[2:], qws, layout=lay, q=fx[0], q_t=fx[1])
        sge.quantize_fp8_grouped(W1.reshape(G * N1, H), G, *fw[2:], qws, q=fw[0], q_t=fw[1])
        sge.grouped_linear_fwd_fp8(fx[0], fx[4], fw[0].view(G, N1, H), fw[4], base, y,
                                   epilogue=sge.EPI_SCALED_SWIGLU, probs=P, preact=h, out_amax=amax_y)
        sge.quantize_fp8_grouped(y, G, *fy[2:], layout=lay, q=fy[0], q_t=fy[1], amax_in=amax_y)
        sge.quantize_mxfp8_grouped(DOUT, lay, mdT, msT, q_row=md, s_row=ms)
        sge.quantize_mxfp8(W2.reshape(G * H, F), q_colT=w2c, s_colT=w2s)
        sge.quantize_mxfp8_grouped(y, lay, myT, mysT)
        sge.grouped_linear_dgrad_mxfp8(md, ms, w2c, w2s, base, epilogue=sge.EPI_DSCALED_SWIGLU, preact=h, probs=P,
                                       dact=dh, dprobs=dp, dact_q=dhq, dact_s=dhs, workspace=ws, layout=lay,
                                       dact_colT_q=dhT, dact_colT_s=dhsT)
        sge.grouped_linear_wgrad_mxfp8(mdT, msT, myT, mysT, lay, dw2)
        sge.quantize_mxfp8(X, q_row=mx, s_row=mxs)
        sge.quantize_mxfp8(W1.reshape(G * N1, H), q_row=w1q, s_row=w1s)
        sge.grouped_linear_fwd_mxfp8(mx, mxs, w1q.view(G, N1, H), w1s.view(G, N1, H // 32), base, out=None,
                                     epilogue=sge.EPI_SCALED_SWIGLU, probs=P, preact=h2, out_q=yq2, out_s=ys2,
                                     layout=lay, out_colT_q=yT2, out_colT_s=ysT2)

    _replays_match(step, [lay, fx[0], fx[1], fx[4], fw[1], y, amax_y, fy[0], fy[4], md, mdT, w2c, dh, dp, dhq,
                          dhs, dw2, dhT, dhsT, mx, w1q, h2, yq2, ys2, yT2, ysT2])


@pytest.mark.parametrize("kind", [sge.NORM_RMS, sge.NORM_LAYER])
def test_norm_steps_graph_replays_match_eager(kind):
    R, C = 256, 1024
    r = synth.streams(34)
    X = dev_bf16(synth.normal_bf16(r["x"], (R, C), 1.0))
    DZ = dev_bf16(synth.normal_bf16(r["dy"], (R, C), 1.0))
    gam, bet = dev_bf16(synth.norm_gamma(C, seed=34)), dev_bf16(synth.normal_bf16(r["residual"], (C,), 0.1))
    u8, f32, bf = (dict(dtype=d, device="cuda") for d in (torch.uint8, torch.float32, torch.bfloat16))
    Y, RS, MU = torch.empty(R, C, **bf), torch.empty(R, **f32), torch.empty(R, **f32)
    f8 = {"q": torch.empty(R, C, **u8), "q_t": torch.empty(C, R, **u8), "amax": torch.empty(1, **f32),
          "scale": torch.empty(1, **f32), "scale_inv": torch.empty(1, **f32)}
    mr = (torch.empty(R, C, **u8), torch.empty(R, C // 32, **u8))
    mc = (torch.empty(C, R, **u8), torch.empty(C, R // 32, **u8))
    wsf = torch.empty(sge.norm_fwd_workspace_size(R, C), **u8)
    DX, DG, DB = torch.empty(R, C, **bf), torch.empty(C, **bf), torch.empty(C, **bf)
    wsb = torch.empty(sge.norm_bwd_workspace_size(R, C), **u8)
    ln = kind == sge.NORM_LAYER

    def step():
        sge.norm_fwd(kind, X, gam, Y, RS, beta=bet if ln else None, mu=MU if ln else None, fp8=f8, mx_row=mr,
                     mx_col=mc, workspace=wsf)
        sge.norm_bwd(kind, DZ, X, RS, gam, DX, DG, wsb, mu=MU if ln else None, dbeta=DB if ln else None)

    _replays_match(step, [Y, RS, f8["q"], f8["q_t"], f8["scale_inv"], mr[0], mr[1], mc[0], mc[1], DX, DG] +
                   ([MU, DB] if ln else []))


@pytest.mark.parametrize("act", ["swiglu", "clamped_swiglu"])
def test_grouped_mlp_module_graph_replays_match_eager(act):
    """The whole grouped MLP calls (offsets, fc1 + activation, fc2, and the backward) captured
    together in one graph."""
    epi, params = ((sge.EPI_SCALED_SWIGLU, None) if act == "swiglu"
                   else (sge.EPI_SCALED_CLAMPED_SWIGLU, (0.25, 1.702)))
    inp = synth.grouped(700, 5, 256, 256, seed=34, splits=[0, 300, 1, 390, 9])
    X, W1, W2, DOUT = dev_bf16(inp["x"]), dev_bf16(inp["w1"]), dev_bf16(inp["w2"]), dev_bf16(inp["dout"])
    P = torch.from_numpy(inp["p"]).cuda()
    splits = torch.from_numpy(inp["splits"]).cuda()
    T, G, H, F = 700, 5, 256, 256
    bf = dict(dtype=torch.bfloat16, device="cuda")
    offs = torch.empty(G + 1, dtype=torch.int64, device="cuda")
    err = torch.empty(1, dtype=torch.int32, device="cuda")
    h, y, out = torch.empty(T, 2 * F, **bf), torch.empty(T, F, **bf), torch.empty(T, H, **bf)
    dh, dp = torch.empty(T, 2 * F, **bf), torch.empty(T, dtype=torch.float32, device="cuda")
    dx, dw1, dw2 = torch.empty(T, H, **bf), torch.empty(G, 2 * F, H, **bf), torch.empty(G, H, F, **bf)
    ws = torch.empty(sge.grouped_mlp_bwd_workspace_size(T, F, G, epi), dtype=torch.uint8, device="cuda")
    outs = [offs, err, h, y, out, dh, dp, dx, dw1, dw2]

    def step():
        sge.grouped_mlp_fwd(X, W1, W2, splits, offs, P, h, y, out, activation=epi, act=params, err_flag=err)
        sge.grouped_mlp_bwd(DOUT, X, W1, W2, offs, P, h, y, dh, dp, dx=dx, dw1=dw1, dw2=dw2, workspace=ws,
                            activation=epi, act=params)
    step()
    torch.cuda.synchronize()
    want = [_bits(t) for t in outs]
    g = _capture(step)
    for _ in range(3):
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        _ = torch.randn(64, 64, device="cuda") @ torch.randn(64, 64, device="cuda")   # eager work between
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip([_bits(t) for t in outs], want):
            assert np.array_equal(a, b)

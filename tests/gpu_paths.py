"""Drives the HIP path through the Python binding of the C ABI for the GPU tests and the bench.

Argument marshalling and buffer allocation only; every number comes from libsge kernels.
"""

import torch

import scaled_gemm_epilogues_amd as sge

from .helpers import dev_bf16


def quant_fp8(t, want_q=True, want_qt=True):
    R, C = t.shape
    q = torch.empty(R, C, dtype=torch.uint8, device=t.device) if want_q else None
    qt = torch.empty(C, R, dtype=torch.uint8, device=t.device) if want_qt else None
    amax, scale, sinv = (torch.empty(1, dtype=torch.float32, device=t.device) for _ in range(3))
    ws = torch.empty(max(1, sge.quantize_fp8_amax_workspace_size(R, C)), dtype=torch.uint8, device=t.device)
    sge.quantize_fp8_amax(t, q, qt, amax, scale, sinv, ws)
    return {"q": q, "q_t": qt, "amax": amax, "scale": scale, "scale_inv": sinv}


def quant_mx(t, row=True, col=True):
    R, C = t.shape
    out = {}
    kw = {}
    if row:
        out["q_row"] = torch.empty(R, C, dtype=torch.uint8, device=t.device)
        out["s_row"] = torch.empty(R, C // 32, dtype=torch.uint8, device=t.device)
        kw.update(q_row=out["q_row"], s_row=out["s_row"])
    if col:
        out["q_colT"] = torch.empty(C, R, dtype=torch.uint8, device=t.device)
        out["s_colT"] = torch.empty(C, R // 32, dtype=torch.uint8, device=t.device)
        kw.update(q_colT=out["q_colT"], s_colT=out["s_colT"])
    sge.quantize_mxfp8(t, **kw)
    return out


def dense_operands(fmt, X, W, DY=None):
    """GEMM operands of fwd / dgrad / wgrad for device bf16 tensors X [M,K], W [N,K], DY [M,N]."""
    o = {"quant": {}}
    if fmt == "bf16":
        o["fwd"] = (sge.Operand.bf16(X), sge.Operand.bf16(W))
        if DY is not None:
            o["dgrad"] = (sge.Operand.bf16(DY), sge.Operand.bf16(W, transposed=True))
            o["wgrad"] = (sge.Operand.bf16(DY, transposed=True), sge.Operand.bf16(X, transposed=True))
        return o
    if fmt == "fp8":
        qx, qw = quant_fp8(X), quant_fp8(W)
        o["quant"].update(x=qx, w=qw)
        o["fwd"] = (sge.Operand.e4m3(qx["q"], qx["scale_inv"]), sge.Operand.e4m3(qw["q"], qw["scale_inv"]))
        if DY is not None:
            qd = quant_fp8(DY)
            o["quant"]["dy"] = qd
            o["dgrad"] = (sge.Operand.e4m3(qd["q"], qd["scale_inv"]), sge.Operand.e4m3(qw["q_t"], qw["scale_inv"]))
            o["wgrad"] = (sge.Operand.e4m3(qd["q_t"], qd["scale_inv"]), sge.Operand.e4m3(qx["q_t"], qx["scale_inv"]))
        return o
    if fmt == "mxfp8":
        mx, mw = quant_mx(X, row=True, col=DY is not None), quant_mx(W, row=True, col=DY is not None)
        o["quant"].update(x=mx, w=mw)
        o["fwd"] = (sge.Operand.mxfp8(mx["q_row"], mx["s_row"]), sge.Operand.mxfp8(mw["q_row"], mw["s_row"]))
        if DY is not None:
            md = quant_mx(DY)
            o["quant"]["dy"] = md
            o["dgrad"] = (sge.Operand.mxfp8(md["q_row"], md["s_row"]), sge.Operand.mxfp8(mw["q_colT"], mw["s_colT"]))
            o["wgrad"] = (sge.Operand.mxfp8(md["q_colT"], md["s_colT"]),
                          sge.Operand.mxfp8(mx["q_colT"], mx["s_colT"]))
        return o
    raise ValueError(fmt)


def run_dense(fmt, inputs, alpha, passes=("fwd", "dgrad", "wgrad")):
    """Runs the dense path on seeded host inputs; returns device outputs and quantizer outputs."""
    X, W = dev_bf16(inputs["x"]), dev_bf16(inputs["w"])
    DY = dev_bf16(inputs["dy"]) if "dgrad" in passes or "wgrad" in passes else None
    ops = dense_operands(fmt, X, W, DY)
    out = {"quant": ops["quant"]}
    if "fwd" in passes:
        R = dev_bf16(inputs["residual"])
        sge.linear_scale_add_fwd(*ops["fwd"], R, alpha)
        out["fwd"] = R
    M, K = X.shape
    N = W.shape[0]
    dgrad = torch.empty(M, K, dtype=torch.bfloat16, device="cuda") if "dgrad" in passes else None
    wgrad = torch.empty(N, K, dtype=torch.bfloat16, device="cuda") if "wgrad" in passes else None
    if dgrad is not None or wgrad is not None:
        dg = ops["dgrad"] if dgrad is not None else (None, None)
        wg = ops["wgrad"] if wgrad is not None else (None, None)
        sge.linear_scale_bwd(dg[0], dg[1], wg[0], wg[1], dgrad, wgrad, alpha, alpha)
        out["dgrad"], out["wgrad"] = dgrad, wgrad
    torch.cuda.synchronize()
    return out


def run_grouped_mlp(inp, with_backward=True):
    """Grouped MLP on device: offsets, fc1 + scaled SwiGLU, fc2, and the backward of both layers."""
    X, W1, W2 = dev_bf16(inp["x"]), dev_bf16(inp["w1"]), dev_bf16(inp["w2"])
    P = torch.from_numpy(inp["p"]).cuda()
    splits = torch.from_numpy(inp["splits"]).cuda()
    T, H = X.shape
    G, N1, _ = W1.shape
    F = N1 // 2
    offs = torch.empty(1, G + 1, dtype=torch.int64, device="cuda")
    err = torch.empty(1, dtype=torch.int32, device="cuda")
    sge.splits_to_offsets(splits, [1], offs, expected_total=T, err_flag=err)
    base = offs[0]
    h = torch.empty(T, N1, dtype=torch.bfloat16, device="cuda")
    y = torch.empty(T, F, dtype=torch.bfloat16, device="cuda")
    out = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
    sge.grouped_linear_fwd(X, W1, base, y, epilogue=sge.EPI_SCALED_SWIGLU, probs=P, preact=h)
    sge.grouped_linear_fwd(y, W2, base, out)
    res = {"offsets": offs, "err": err, "h": h, "y": y, "out": out}
    if with_backward:
        DOUT = dev_bf16(inp["dout"])
        dh = torch.empty(T, N1, dtype=torch.bfloat16, device="cuda")
        dp = torch.empty(T, dtype=torch.float32, device="cuda")
        dw2 = torch.empty(G, H, F, dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(max(1, sge.grouped_linear_bwd_workspace_size(T, F, G, sge.EPI_DSCALED_SWIGLU)),
                         dtype=torch.uint8, device="cuda")
        sge.grouped_linear_bwd(DOUT, y, W2, base, epilogue=sge.EPI_DSCALED_SWIGLU, preact=h, probs=P, dact=dh,
                               dprobs=dp, dw=dw2, workspace=ws)
        dx = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
        dw1 = torch.empty(G, N1, H, dtype=torch.bfloat16, device="cuda")
        sge.grouped_linear_bwd(dh, X, W1, base, dx=dx, dw=dw1)
        res.update(dh=dh, dp=dp, dw2=dw2, dx=dx, dw1=dw1)
    torch.cuda.synchronize()
    return res


def run_grouped_mlp_fwd_mx(inp):
    """MXFP8 grouped MLP forward: quantize x, W1, W2 rowwise; fc1 + scaled SwiGLU emitting y as
    bf16 and as MXFP8 rowwise; fc2 on the MXFP8 y."""
    X, W1, W2 = dev_bf16(inp["x"]), dev_bf16(inp["w1"]), dev_bf16(inp["w2"])
    P = torch.from_numpy(inp["p"]).cuda()
    T, H = X.shape
    G, N1, _ = W1.shape
    F = N1 // 2
    offs = torch.empty(1, G + 1, dtype=torch.int64, device="cuda")
    err = torch.empty(1, dtype=torch.int32, device="cuda")
    sge.splits_to_offsets(torch.from_numpy(inp["splits"]).cuda(), [1], offs, expected_total=T, err_flag=err)
    base = offs[0]
    qx = quant_mx(X, col=False)
    qw1 = quant_mx(W1.reshape(G * N1, H), col=False)
    qw2 = quant_mx(W2.reshape(G * H, F), col=False)
    h = torch.empty(T, N1, dtype=torch.bfloat16, device="cuda")
    y = torch.empty(T, F, dtype=torch.bfloat16, device="cuda")
    yq = torch.empty(T, F, dtype=torch.uint8, device="cuda")
    ys = torch.empty(T, F // 32, dtype=torch.uint8, device="cuda")
    out = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
    sge.grouped_linear_fwd_mxfp8(qx["q_row"], qx["s_row"], qw1["q_row"].reshape(G, N1, H),
                                 qw1["s_row"].reshape(G, N1, H // 32), base, out=y, epilogue=sge.EPI_SCALED_SWIGLU,
                                 probs=P, preact=h, out_q=yq, out_s=ys)
    sge.grouped_linear_fwd_mxfp8(yq, ys, qw2["q_row"].reshape(G, H, F), qw2["s_row"].reshape(G, H, F // 32), base,
                                 out=out)
    y_unfused = quant_mx(y, col=False)                    # the standalone quantizer on the bf16 y
    torch.cuda.synchronize()
    return {"err": err, "qx": qx, "qw1": qw1, "qw2": qw2, "h": h, "y": y, "yq": yq, "ys": ys, "out": out,
            "y_unfused": y_unfused}

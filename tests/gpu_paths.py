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


def run_grouped_mlp(inp, with_backward=True, act="swiglu"):
    """Grouped MLP on device: offsets, fc1 + scaled SwiGLU (or scaled SReLU), fc2, and the
    backward of both layers."""
    X, W1, W2 = dev_bf16(inp["x"]), dev_bf16(inp["w1"]), dev_bf16(inp["w2"])
    P = torch.from_numpy(inp["p"]).cuda()
    splits = torch.from_numpy(inp["splits"]).cuda()
    T, H = X.shape
    G, N1, _ = W1.shape
    width, fwd_epi, bwd_epi = _act_epilogues(act)
    F = width(N1)
    ap = _act_params(act)
    offs = torch.empty(1, G + 1, dtype=torch.int64, device="cuda")
    err = torch.empty(1, dtype=torch.int32, device="cuda")
    sge.splits_to_offsets(splits, [1], offs, expected_total=T, err_flag=err)
    base = offs[0]
    h = torch.empty(T, N1, dtype=torch.bfloat16, device="cuda")
    y = torch.empty(T, F, dtype=torch.bfloat16, device="cuda")
    out = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
    sge.grouped_linear_fwd(X, W1, base, y, epilogue=fwd_epi, probs=P, preact=h, act=ap)
    sge.grouped_linear_fwd(y, W2, base, out)
    res = {"offsets": offs, "err": err, "h": h, "y": y, "out": out}
    if with_backward:
        DOUT = dev_bf16(inp["dout"])
        dh = torch.empty(T, N1, dtype=torch.bfloat16, device="cuda")
        dp = torch.empty(T, dtype=torch.float32, device="cuda")
        dw2 = torch.empty(G, H, F, dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(max(1, sge.grouped_linear_bwd_workspace_size(T, F, G, bwd_epi)),
                         dtype=torch.uint8, device="cuda")
        sge.grouped_linear_bwd(DOUT, y, W2, base, epilogue=bwd_epi, preact=h, probs=P, dact=dh,
                               dprobs=dp, dw=dw2, workspace=ws, act=ap)
        dx = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
        dw1 = torch.empty(G, N1, H, dtype=torch.bfloat16, device="cuda")
        sge.grouped_linear_bwd(dh, X, W1, base, dx=dx, dw=dw1)
        res.update(dh=dh, dp=dp, dw2=dw2, dx=dx, dw1=dw1)
    torch.cuda.synchronize()
    return res


def _act_epilogues(act):
    """(fc1 width from W1's rows, forward epilogue, backward epilogue) of an activation:
    "swiglu", "srelu", or ("clamped_swiglu", limit, alpha) as the oracle names them."""
    if act == "swiglu":
        return (lambda n1: n1 // 2), sge.EPI_SCALED_SWIGLU, sge.EPI_DSCALED_SWIGLU
    if act == "srelu":
        return (lambda n1: n1), sge.EPI_SCALED_SRELU, sge.EPI_DSCALED_SRELU
    if isinstance(act, tuple) and act[0] == "clamped_swiglu":
        return (lambda n1: n1 // 2), sge.EPI_SCALED_CLAMPED_SWIGLU, sge.EPI_DSCALED_CLAMPED_SWIGLU
    raise ValueError(act)


def _act_params(act):
    """(limit, alpha) of a clamped activation, else None."""
    return tuple(act[1:]) if isinstance(act, tuple) else None


def run_grouped_mlp_fwd_mx(inp, act="swiglu"):
    """MXFP8 grouped MLP forward: quantize x, W1, W2 rowwise; fc1 + the scaled activation
    emitting y as bf16, as MXFP8 rowwise and token-blocked (the fc2 wgrad operand); fc2 on the
    MXFP8 y."""
    X, W1, W2 = dev_bf16(inp["x"]), dev_bf16(inp["w1"]), dev_bf16(inp["w2"])
    P = torch.from_numpy(inp["p"]).cuda()
    T, H = X.shape
    G, N1, _ = W1.shape
    width, fwd_epi, _ = _act_epilogues(act)
    F = width(N1)
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
    lay = mx_layout(base, T)
    ld = sge.mx_token_capacity(T, G)
    q_y = {"q_colT": torch.empty(F, ld, dtype=torch.uint8, device="cuda"),
           "s_colT": torch.empty(F, ld // 32, dtype=torch.uint8, device="cuda"), "ld": ld}
    sge.grouped_linear_fwd_mxfp8(qx["q_row"], qx["s_row"], qw1["q_row"].reshape(G, N1, H),
                                 qw1["s_row"].reshape(G, N1, H // 32), base, out=y, epilogue=fwd_epi,
                                 probs=P, preact=h, out_q=yq, out_s=ys, act=_act_params(act), layout=lay,
                                 out_colT_q=q_y["q_colT"], out_colT_s=q_y["s_colT"])
    sge.grouped_linear_fwd_mxfp8(yq, ys, qw2["q_row"].reshape(G, H, F), qw2["s_row"].reshape(G, H, F // 32), base,
                                 out=out)
    y_unfused = quant_mx(y, col=False)                    # the standalone quantizer on the bf16 y
    torch.cuda.synchronize()
    return {"err": err, "qx": qx, "qw1": qw1, "qw2": qw2, "h": h, "y": y, "yq": yq, "ys": ys, "out": out,
            "y_unfused": y_unfused, "base": base, "act": act, "lay": lay, "q_y": q_y}


# ------------------------------------------------------- MXFP8 grouped backward
def mx_layout(base, T):
    """[2, G+1] device layout (clamped offsets, 128-aligned starts) of device offsets ``base``."""
    lay = torch.empty(2, base.numel(), dtype=torch.int64, device="cuda")
    sge.mx_group_layout(base, T, lay)
    return lay


def quant_mx_grouped(t, lay, row=False, fill=None):
    """Token-blocked MXFP8 of device bf16 ``t`` [T, C] (+ the rowwise copy when ``row``).
    ``fill``: byte value the transposed outputs start with (to see what is left unwritten)."""
    T, C = t.shape
    G = lay.shape[1] - 1
    ld = sge.mx_token_capacity(T, G)
    mk = (lambda *s: torch.full(s, fill, dtype=torch.uint8, device="cuda")) if fill is not None else \
        (lambda *s: torch.empty(*s, dtype=torch.uint8, device="cuda"))
    out = {"q_colT": mk(C, ld), "s_colT": mk(C, ld // 32), "ld": ld}
    kw = {}
    if row:
        out["q_row"] = torch.empty(T, C, dtype=torch.uint8, device="cuda")
        out["s_row"] = torch.empty(T, C // 32, dtype=torch.uint8, device="cuda")
        kw.update(q_row=out["q_row"], s_row=out["s_row"])
    sge.quantize_mxfp8_grouped(t, lay, out["q_colT"], out["s_colT"], **kw)
    return out


def grouped_dgrad_mx(q_dy, w_colT, base, alpha=1.0, preact=None, probs=None, want_q=False, act="swiglu",
                     lay=None, want_bf16=True, fill=0xAB):
    """MXFP8 grouped dgrad from a rowwise-quantized dy and W's columnwise copy [K, G*N].
    With ``preact`` the scaled activation's backward runs in the epilogue (dact, dprobs, and
    the MXFP8 dact when ``want_q``; with the layout ``lay`` also the token-blocked dact, whose
    buffers start filled with ``fill``; ``want_bf16=False`` skips the bf16 dact); otherwise
    dx [T, K] is returned."""
    T, N = q_dy["q_row"].shape
    K = w_colT["q_colT"].shape[0]
    G = base.numel() - 1
    out = {}
    if preact is None:
        out["dx"] = torch.empty(T, K, dtype=torch.bfloat16, device="cuda")
        sge.grouped_linear_dgrad_mxfp8(q_dy["q_row"], q_dy["s_row"], w_colT["q_colT"], w_colT["s_colT"], base,
                                       alpha=alpha, dx=out["dx"])
        return out
    _, _, epi = _act_epilogues(act)
    hw = K if act == "srelu" else 2 * K                  # gated activations: two halves
    ws = torch.empty(max(1, sge.grouped_linear_bwd_workspace_size(T, K, G, epi)), dtype=torch.uint8, device="cuda")
    if want_bf16:
        out["dact"] = torch.empty(T, hw, dtype=torch.bfloat16, device="cuda")
    out["dprobs"] = torch.empty(T, dtype=torch.float32, device="cuda")
    if want_q:
        out["dact_q"] = torch.empty(T, hw, dtype=torch.uint8, device="cuda")
        out["dact_s"] = torch.empty(T, hw // 32, dtype=torch.uint8, device="cuda")
    if lay is not None:
        ld = sge.mx_token_capacity(T, G)
        out["ld"] = ld
        out["q_colT"] = torch.full((hw, ld), fill, dtype=torch.uint8, device="cuda")
        out["s_colT"] = torch.full((hw, ld // 32), fill, dtype=torch.uint8, device="cuda")
    sge.grouped_linear_dgrad_mxfp8(q_dy["q_row"], q_dy["s_row"], w_colT["q_colT"], w_colT["s_colT"], base,
                                   alpha=alpha, epilogue=epi, preact=preact, probs=probs,
                                   dact=out.get("dact"), dprobs=out["dprobs"], dact_q=out.get("dact_q"),
                                   dact_s=out.get("dact_s"), workspace=ws, act=_act_params(act), layout=lay,
                                   dact_colT_q=out.get("q_colT"), dact_colT_s=out.get("s_colT"))
    return out


def grouped_wgrad_mx(qa, qb, lay, G, alpha=1.0):
    """dW [G, N, K] from the token-blocked operands of dy (qa) and x (qb)."""
    N, K = qa["q_colT"].shape[0], qb["q_colT"].shape[0]
    dw = torch.empty(G, N, K, dtype=torch.bfloat16, device="cuda")
    sge.grouped_linear_wgrad_mxfp8(qa["q_colT"], qa["s_colT"], qb["q_colT"], qb["s_colT"], lay, dw, alpha=alpha)
    return dw


def run_grouped_mlp_bwd_mx(inp, fwd):
    """MXFP8 grouped MLP backward after ``run_grouped_mlp_fwd_mx``: fc2 dgrad with the fused
    backward of the scaled activation and group quantize of dh (rowwise and token-blocked),
    fc2 wgrad, fc1 dgrad on the MXFP8 dh, fc1 wgrad; every wgrad operand token-blocked per
    group (y's and dh's by the producing epilogues)."""
    X, W1, W2 = dev_bf16(inp["x"]), dev_bf16(inp["w1"]), dev_bf16(inp["w2"])
    DOUT = dev_bf16(inp["dout"])
    P = torch.from_numpy(inp["p"]).cuda()
    T, H = X.shape
    G, N1, _ = W1.shape
    act = fwd["act"]
    F = _act_epilogues(act)[0](N1)
    base = fwd["base"]
    lay = fwd["lay"]
    q_dout = quant_mx_grouped(DOUT, lay, row=True)
    w2c = quant_mx(W2.reshape(G * H, F), row=False, col=True)        # [F, G*H]
    w1c = quant_mx(W1.reshape(G * N1, H), row=False, col=True)       # [H, G*N1]
    d2 = grouped_dgrad_mx(q_dout, w2c, base, preact=fwd["h"], probs=P, want_q=True, act=act, lay=lay)
    q_y = fwd["q_y"]
    dw2 = grouped_wgrad_mx(q_dout, q_y, lay, G)
    d1 = grouped_dgrad_mx({"q_row": d2["dact_q"], "s_row": d2["dact_s"]}, w1c, base)
    q_dh = {"q_colT": d2["q_colT"], "s_colT": d2["s_colT"], "ld": d2["ld"]}
    q_x = quant_mx_grouped(X, lay)
    dw1 = grouped_wgrad_mx(q_dh, q_x, lay, G)
    dh_unfused = quant_mx(d2["dact"], col=False)                     # the standalone quantizer on dh
    torch.cuda.synchronize()
    return {"lay": lay, "q_dout": q_dout, "w2c": w2c, "w1c": w1c, "dh": d2["dact"], "dp": d2["dprobs"],
            "dhq": d2["dact_q"], "dhs": d2["dact_s"], "dh_unfused": dh_unfused, "dw2": dw2, "dx": d1["dx"],
            "dw1": dw1, "q_y": q_y, "q_dh": q_dh, "q_x": q_x}


# ------------------------------------------- FP8 current scaling per group
def quant_fp8_grouped(t, G, lay=None, row=True, col=True, fill=None, amax_in=None):
    """Per-group FP8 current scaling of device bf16 ``t`` [rows, C]: groups from ``lay`` or G
    equal runs of rows (``amax_in``: the groups' amax from the producing epilogue). Returns
    q [rows, C], q_t [C, ld] and the per-group amax / scale / scale_inv."""
    rows, C = t.shape
    ld = sge.mx_token_capacity(rows, G) if lay is not None else rows
    f32 = dict(dtype=torch.float32, device="cuda")
    out = {"amax": torch.empty(G, **f32), "scale": torch.empty(G, **f32), "scale_inv": torch.empty(G, **f32),
           "ld": ld}
    mk = (lambda *s: torch.full(s, fill, dtype=torch.uint8, device="cuda")) if fill is not None else \
        (lambda *s: torch.empty(*s, dtype=torch.uint8, device="cuda"))
    out["q"] = mk(rows, C) if row else None
    out["q_t"] = mk(C, ld) if col else None
    ws = torch.empty(max(16, sge.quantize_fp8_grouped_workspace_size(G)), dtype=torch.uint8, device="cuda")
    sge.quantize_fp8_grouped(t, G, out["amax"], out["scale"], out["scale_inv"], ws, layout=lay, q=out["q"],
                             q_t=out["q_t"], amax_in=amax_in)
    return out


def run_grouped_mlp_fp8(inp, act="swiglu"):
    """Grouped MLP forward + backward on E4M3 operands with current scaling per group: every
    operand quantized per group (x, y, dout, dh per token group; W1, W2 per expert), rowwise for
    the forward and the dgrads, transposed for the dgrads' weights and the wgrads' operands."""
    X, W1, W2, DOUT = dev_bf16(inp["x"]), dev_bf16(inp["w1"]), dev_bf16(inp["w2"]), dev_bf16(inp["dout"])
    P = torch.from_numpy(inp["p"]).cuda()
    T, H = X.shape
    G, N1, _ = W1.shape
    width, fwd_epi, bwd_epi = _act_epilogues(act)
    F = width(N1)
    offs = torch.empty(1, G + 1, dtype=torch.int64, device="cuda")
    sge.splits_to_offsets(torch.from_numpy(inp["splits"]).cuda(), [1], offs)
    base = offs[0]
    lay = mx_layout(base, T)
    bf = dict(dtype=torch.bfloat16, device="cuda")
    qx = quant_fp8_grouped(X, G, lay)
    qw1 = quant_fp8_grouped(W1.reshape(G * N1, H), G)
    qw2 = quant_fp8_grouped(W2.reshape(G * H, F), G)
    h, y, out = torch.empty(T, N1, **bf), torch.empty(T, F, **bf), torch.empty(T, H, **bf)
    amax_y = torch.empty(G, dtype=torch.float32, device="cuda")
    sge.grouped_linear_fwd_fp8(qx["q"], qx["scale_inv"], qw1["q"].view(G, N1, H), qw1["scale_inv"], base, y,
                               epilogue=fwd_epi, probs=P, preact=h, out_amax=amax_y, act=_act_params(act))
    qy = quant_fp8_grouped(y, G, lay, amax_in=amax_y)            # the amax fused into fc1's epilogue
    sge.grouped_linear_fwd_fp8(qy["q"], qy["scale_inv"], qw2["q"].view(G, H, F), qw2["scale_inv"], base, out)
    qd = quant_fp8_grouped(DOUT, G, lay)
    dh, dp = torch.empty(T, N1, **bf), torch.empty(T, dtype=torch.float32, device="cuda")
    amax_dh = torch.empty(G, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, sge.grouped_linear_bwd_workspace_size(T, F, G, bwd_epi)),
                     dtype=torch.uint8, device="cuda")
    sge.grouped_linear_dgrad_fp8(qd["q"], qd["scale_inv"], qw2["q_t"], qw2["scale_inv"], base,
                                 epilogue=bwd_epi, preact=h, probs=P, dact=dh, dprobs=dp,
                                 dact_amax=amax_dh, workspace=ws, act=_act_params(act))
    dw2 = torch.empty(G, H, F, **bf)
    sge.grouped_linear_wgrad_fp8(qd["q_t"], qd["scale_inv"], qy["q_t"], qy["scale_inv"], lay, dw2)
    qdh = quant_fp8_grouped(dh, G, lay, amax_in=amax_dh)        # the amax fused into fc2's dgrad epilogue
    dx, dw1 = torch.empty(T, H, **bf), torch.empty(G, N1, H, **bf)
    sge.grouped_linear_dgrad_fp8(qdh["q"], qdh["scale_inv"], qw1["q_t"], qw1["scale_inv"], base, dx=dx)
    sge.grouped_linear_wgrad_fp8(qdh["q_t"], qdh["scale_inv"], qx["q_t"], qx["scale_inv"], lay, dw1)
    # the standalone quantizer (its own amax pass) on the same bf16 y and dh
    qy_alone, qdh_alone = quant_fp8_grouped(y, G, lay), quant_fp8_grouped(dh, G, lay)
    torch.cuda.synchronize()
    return {"base": base, "lay": lay, "qx": qx, "qw1": qw1, "qw2": qw2, "qy": qy, "qd": qd, "qdh": qdh, "h": h,
            "y": y, "out": out, "dh": dh, "dp": dp, "dw2": dw2, "dx": dx, "dw1": dw1, "qy_alone": qy_alone,
            "qdh_alone": qdh_alone}

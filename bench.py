#!/usr/bin/env python3
"""Benchmark of the fused scaled linear on one MI355X.

One step is one pass of the hot path over one batch of seeded synthetic
inputs already resident in HBM:

* dense workloads: quantize the operands (FP8 / MXFP8 only), forward GEMM with
  the in-place residual add, dgrad and wgrad with alpha folded in;
* grouped workload: split offsets, fc1 + scaled SwiGLU, fc2, and the backward
  of both layers.

Prints ONE JSON line on stdout. The default workload is the bf16 forward +
backward at M = N = K = 4096 (alpha 0.125); the FP8 (8192 x 14336 x 4096), MXFP8
(16384 x 8192 x 8192) and grouped SwiGLU MLP (65,536 tokens, 8 experts) workloads
are timed the same way in the same run and reported under ``configs``, each
with its own oracle sample. Before the ``--warmup`` steps the
step runs untimed for ``--ramp-seconds`` (the GPU raises its clocks over the
first ~100 ms of load). The timed region is ``--steps``
eager steps between HIP events; ``ms_per_step_graph`` replays the same step
captured as one HIP graph (every libsge call is capture-safe), for
comparison. Per-kernel durations come from a graph of repeated
launches of that one call, timed with HIP events on the stream they run on;
``roofline`` reports the kernel with the largest share of the step, and its
``traffic`` comes from the committed rocprofv3 counter summary when that was
taken on the current kernel source. ``cpu_baseline`` times the CPU oracle on a
bounded sample of the same workload.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# published MI355X peaks
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "mxfp8": 5000.0}
PEAK_HBM_GBS = 8000.0
METRIC = "scaled-linear fwd+bwd TFLOP/s & % of MFMA peak (bf16/FP8/MXFP8), 1 MI355X"
DEFAULT_WORKLOAD = "bf16_fwdbwd_4096"
# timed in the same run as the default workload: the FP8 and MXFP8 dense configurations the metric
# names, and the grouped MLP
DEFAULT_CONFIGS = ("fp8_tensor_fwdbwd_8192x14336x4096", "mxfp8_fwdbwd_16384x8192x8192",
                   "grouped_swiglu_mlp_T65536_G8")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--ramp-seconds", type=float, default=0.3,
                    help="untimed steps run for this long before the warm-up steps (the GPU's clock ramp)")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--configs", default="auto",
                    help="comma-separated workloads timed in the same run after --workload and reported under "
                         "'configs' (auto: the FP8, MXFP8 and grouped workloads when --workload is the default; "
                         "none: no others)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--cpu-seconds-configs", type=float, default=4.0,
                    help="target CPU time of the oracle sample of each of the other --configs workloads")
    # measurement helpers (rocprofv3 targets and summaries); none of them prints the bench line
    ap.add_argument("--profile-launch", metavar="KEY",
                    help="one warm-up step, then --profile-reps launches of this call only (a --pmc target)")
    ap.add_argument("--profile-reps", type=int, default=5, help="keep the default for --summarize-traffic")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="one 1 GiB device-to-device copy (calibrates FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--summarize-mfma", metavar="PMC_DIR",
                    help="write profiles/mfma_util.md from rocprofv3 --pmc runs of the MFMA counters")
    ap.add_argument("--summarize-traffic", metavar="PMC_DIR",
                    help="write profiles/traffic.json and its summary from rocprofv3 --pmc CSV output")
    ap.add_argument("--summarize-trace", nargs=4, metavar=("TRACE_DIR", "BENCH_JSON", "OUT_MD", "COMMAND"),
                    help="write a kernel-trace summary from rocprofv3 --kernel-trace --stats CSV output")
    return ap.parse_args()


# --------------------------------------------------------------- GPU path
def capture(torch, fns):
    """A HIP graph of the given launches (every libsge call is capture-safe: no allocation, no sync)."""
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for f in fns:
            f()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for f in fns:
            f()
    torch.cuda.synchronize()
    return g


def time_ms(torch, fn, reps):
    """HIP events on the current stream around `reps` calls of fn; returns ms per call."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def build_dense(torch, sge, wl, inp):
    fmt = wl["fmt"]

    def dev_bf16(bits):
        import numpy as np
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

    bwd = "dgrad" in wl["passes"]
    X, W = dev_bf16(inp["x"]), dev_bf16(inp["w"])
    DY = dev_bf16(inp["dy"]) if bwd else torch.zeros(X.shape[0], W.shape[0], dtype=torch.bfloat16,
                                                       device="cuda")
    R = dev_bf16(inp["residual"])
    M, K = X.shape
    N = W.shape[0]
    alpha = wl["alpha"]
    dgrad = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
    wgrad = torch.empty(N, K, dtype=torch.bfloat16, device="cuda")
    u8 = dict(dtype=torch.uint8, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    flops = {"gemm_fwd": 2 * M * N * K}
    if bwd:
        flops.update(gemm_dgrad=2 * M * N * K, gemm_wgrad=2 * M * N * K)
    hbm = {}

    if fmt == "bf16":
        fwd = (sge.Operand.bf16(X), sge.Operand.bf16(W))
        dg = (sge.Operand.bf16(DY), sge.Operand.bf16(W, transposed=True))
        wg = (sge.Operand.bf16(DY, transposed=True), sge.Operand.bf16(X, transposed=True))

        def quantize_launches():
            return []
    elif fmt == "fp8":
        bufs = {}
        for name, t in (("x", X), ("w", W), ("dy", DY)):
            r, c = t.shape
            bufs[name] = {"q": torch.empty(r, c, **u8), "q_t": torch.empty(c, r, **u8),
                          "amax": torch.empty(1, **f32), "scale": torch.empty(1, **f32),
                          "scale_inv": torch.empty(1, **f32),
                          "ws": torch.empty(sge.quantize_fp8_amax_workspace_size(r, c), **u8), "src": t}
            hbm[f"quant_{name}"] = r * c * (2 + 2 + 1 + 1)      # amax read, quantize read, q and q_t written
        bx, bw, bd = bufs["x"], bufs["w"], bufs["dy"]
        fwd = (sge.Operand.e4m3(bx["q"], bx["scale_inv"]), sge.Operand.e4m3(bw["q"], bw["scale_inv"]))
        dg = (sge.Operand.e4m3(bd["q"], bd["scale_inv"]), sge.Operand.e4m3(bw["q_t"], bw["scale_inv"]))
        wg = (sge.Operand.e4m3(bd["q_t"], bd["scale_inv"]), sge.Operand.e4m3(bx["q_t"], bx["scale_inv"]))

        def quantize_launches():
            return [(f"quant_{name}", (lambda b=b: sge.quantize_fp8_amax(b["src"], b["q"], b["q_t"], b["amax"],
                                                                          b["scale"], b["scale_inv"], b["ws"])))
                    for name, b in bufs.items()]
    else:
        bufs = {}
        for name, t in (("x", X), ("w", W), ("dy", DY)):
            r, c = t.shape
            bufs[name] = {"q_row": torch.empty(r, c, **u8), "s_row": torch.empty(r, c // 32, **u8),
                          "q_colT": torch.empty(c, r, **u8), "s_colT": torch.empty(c, r // 32, **u8), "src": t}
            hbm[f"quant_{name}"] = r * c * (2 + 1 + 1) + 2 * (r * c // 32)
        bx, bw, bd = bufs["x"], bufs["w"], bufs["dy"]
        fwd = (sge.Operand.mxfp8(bx["q_row"], bx["s_row"]), sge.Operand.mxfp8(bw["q_row"], bw["s_row"]))
        dg = (sge.Operand.mxfp8(bd["q_row"], bd["s_row"]), sge.Operand.mxfp8(bw["q_colT"], bw["s_colT"]))
        wg = (sge.Operand.mxfp8(bd["q_colT"], bd["s_colT"]), sge.Operand.mxfp8(bx["q_colT"], bx["s_colT"]))

        def quantize_launches():
            return [(f"quant_{name}", (lambda b=b: sge.quantize_mxfp8(b["src"], b["q_row"], b["s_row"], b["q_colT"],
                                                                       b["s_colT"])))
                    for name, b in bufs.items()]

    launches = list(quantize_launches())
    if wl.get("norm"):
        # the linear's input is RMSNorm(x): the norm kernel writes the MXFP8 operands (rowwise
        # from registers, columnwise by a pass over its bf16 output) in place of quant_x, and
        # the norm's backward takes the dgrad as its incoming gradient
        assert fmt == "mxfp8" and wl["norm"] == "rms"
        gam = dev_bf16(inp["gamma"])
        Y = torch.empty_like(X)
        RS = torch.empty(M, **f32)
        DX = torch.empty_like(X)
        DG = torch.empty(K, dtype=torch.bfloat16, device="cuda")
        nws = torch.empty(sge.norm_bwd_workspace_size(M, K), **u8)
        launches = [(n, f) for n, f in launches if n != "quant_x"]
        launches.insert(0, ("norm_fwd", lambda: sge.norm_fwd(sge.NORM_RMS, X, gam, Y, RS, eps=wl["eps"],
                                                              mx_row=(bx["q_row"], bx["s_row"]),
                                                              mx_col=(bx["q_colT"], bx["s_colT"]))))
        hbm.pop("quant_x")
        # x read, y written, its two MXFP8 copies written, y read back for the columnwise copy
        hbm["norm_fwd"] = M * K * (2 + 2 + 1 + 2 + 1) + 2 * (M * K // 32)
        hbm["norm_bwd"] = M * K * (2 + 2 + 2)                    # dz and x read, dx written
    launches.append(("gemm_fwd", lambda: sge.linear_scale_add_fwd(*fwd, R, alpha)))
    if bwd:
        launches.append(("gemm_dgrad", lambda: sge.linear_scale_bwd(*dg, None, None, dgrad, None, alpha, alpha)))
        launches.append(("gemm_wgrad", lambda: sge.linear_scale_bwd(None, None, *wg, None, wgrad, alpha, alpha)))
    if wl.get("norm"):
        launches.append(("norm_bwd", lambda: sge.norm_bwd(sge.NORM_RMS, dgrad, X, RS, gam, DX, DG, nws)))
    return launches, flops, hbm


def act_config(sge, wl):
    """(gated, forward epilogue, backward epilogue, name of the fc2 dgrad launch, clamp parameters)
    of a grouped workload's activation: "swiglu", "srelu" or ("clamped_swiglu", limit, alpha)."""
    act = wl.get("act", "swiglu")
    if act == "srelu":
        return False, sge.EPI_SCALED_SRELU, sge.EPI_DSCALED_SRELU, "fc2_dgrad_dsrelu", None
    if act == "swiglu":
        return True, sge.EPI_SCALED_SWIGLU, sge.EPI_DSCALED_SWIGLU, "fc2_dgrad_dswiglu", None
    return (True, sge.EPI_SCALED_CLAMPED_SWIGLU, sge.EPI_DSCALED_CLAMPED_SWIGLU, "fc2_dgrad_dclamped_swiglu",
            tuple(act[1:]))


def build_grouped(torch, sge, wl, inp):
    import numpy as np

    def dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

    X, W1, W2, DOUT = dev_bf16(inp["x"]), dev_bf16(inp["w1"]), dev_bf16(inp["w2"]), dev_bf16(inp["dout"])
    P = torch.from_numpy(inp["p"]).cuda()
    splits = torch.from_numpy(inp["splits"]).cuda()
    T, H = X.shape
    G, N1, _ = W1.shape
    gated, fwd_epi, bwd_epi, dact, ap = act_config(sge, wl)
    F = N1 // 2 if gated else N1
    bf = dict(dtype=torch.bfloat16, device="cuda")
    offs = torch.empty(2, G + 1, dtype=torch.int64, device="cuda")
    h, y, out = torch.empty(T, N1, **bf), torch.empty(T, F, **bf), torch.empty(T, H, **bf)
    dh, dp = torch.empty(T, N1, **bf), torch.empty(T, dtype=torch.float32, device="cuda")
    dw2, dx, dw1 = torch.empty(G, H, F, **bf), torch.empty(T, H, **bf), torch.empty(G, N1, H, **bf)
    ws = torch.empty(max(1, sge.grouped_linear_bwd_workspace_size(T, F, G, bwd_epi)),
                     dtype=torch.uint8, device="cuda")
    flops = {"fc1_fwd": 2 * T * N1 * H, "fc2_fwd": 2 * T * H * F, dact: 2 * T * H * F,
             "fc2_wgrad": 2 * T * H * F, "fc1_dgrad": 2 * T * N1 * H, "fc1_wgrad": 2 * T * N1 * H}

    base = offs[0]
    if wl["fmt"] == "bf16":
        # each layer's backward is one call: its dgrad (with the activation's backward for fc2)
        # and its weight gradient share one launch
        flops = {"fc1_fwd": 2 * T * N1 * H, "fc2_fwd": 2 * T * H * F, "fc2_bwd": 4 * T * H * F,
                 "fc1_bwd": 4 * T * N1 * H}
    if wl["fmt"] == "mxfp8":
        return build_grouped_mx(torch, sge, wl, X, W1, W2, DOUT, P, splits, offs, h, out, dh, dp, dw2, dx, dw1, ws)
    if wl["fmt"] == "fp8":
        return build_grouped_fp8(torch, sge, wl, X, W1, W2, DOUT, P, splits, offs, h, out, dh, dp, dw2, dx, dw1,
                                 ws, flops)
    launches = [
        ("offsets", lambda: sge.splits_to_offsets(splits, [1, H], offs)),
        ("fc1_fwd", lambda: sge.grouped_linear_fwd(X, W1, base, y, epilogue=fwd_epi, probs=P, preact=h,
                                                   act=ap)),
        ("fc2_fwd", lambda: sge.grouped_linear_fwd(y, W2, base, out)),
        ("fc2_bwd", lambda: sge.grouped_linear_bwd(DOUT, y, W2, base, epilogue=bwd_epi, preact=h, probs=P,
                                                   dact=dh, dprobs=dp, dw=dw2, workspace=ws, act=ap)),
        ("fc1_bwd", lambda: sge.grouped_linear_bwd(dh, X, W1, base, dx=dx, dw=dw1)),
    ]
    return launches, flops, {}


def build_grouped_mx(torch, sge, wl, X, W1, W2, DOUT, P, splits, offs, h, out, dh, dp, dw2, dx, dw1, ws):
    """The grouped MLP on MXFP8 operands: every GEMM operand quantized each step, blocked along
    that GEMM's contraction (rowwise for the forward and the dgrads, W's columnwise copy for
    the dgrads, per-group token blocks for the wgrads). fc1's scaled activation emits its output
    as MXFP8 for fc2's forward and token-blocked for fc2's wgrad, and fc2's dgrad emits dh the
    same two ways for fc1's dgrad and wgrad (neither is written in bf16)."""
    T, H = X.shape
    G, N1, _ = W1.shape
    swiglu, fwd_epi, bwd_epi, dact, ap = act_config(sge, wl)   # swiglu: a gated activation
    F = N1 // 2 if swiglu else N1
    bwd = "bwd" in wl["passes"]
    u8 = dict(dtype=torch.uint8, device="cuda")
    base = offs[0]
    qx, sx = torch.empty(T, H, **u8), torch.empty(T, H // 32, **u8)
    qw1, sw1 = torch.empty(G * N1, H, **u8), torch.empty(G * N1, H // 32, **u8)
    qw2, sw2 = torch.empty(G * H, F, **u8), torch.empty(G * H, F // 32, **u8)
    qy, sy = torch.empty(T, F, **u8), torch.empty(T, F // 32, **u8)
    W1f, W2f = W1.reshape(G * N1, H), W2.reshape(G * H, F)
    flops = {"fc1_fwd": 2 * T * N1 * H, "fc2_fwd": 2 * T * H * F}
    if not bwd:
        hbm = {"quant_x": T * H * 3 + T * H // 32, "quant_w1": G * N1 * H * 3 + G * N1 * H // 32,
               "quant_w2": G * H * F * 3 + G * H * F // 32}
        return [
            ("offsets", lambda: sge.splits_to_offsets(splits, [1, H], offs)),
            ("quant_x", lambda: sge.quantize_mxfp8(X, q_row=qx, s_row=sx)),
            ("quant_w1", lambda: sge.quantize_mxfp8(W1f, q_row=qw1, s_row=sw1)),
            ("quant_w2", lambda: sge.quantize_mxfp8(W2f, q_row=qw2, s_row=sw2)),
            ("fc1_fwd", lambda: sge.grouped_linear_fwd_mxfp8(
                qx, sx, qw1.view(G, N1, H), sw1.view(G, N1, H // 32), base, out=None,
                epilogue=fwd_epi, probs=P, preact=h, out_q=qy, out_s=sy, act=ap)),
            ("fc2_fwd", lambda: sge.grouped_linear_fwd_mxfp8(qy, sy, qw2.view(G, H, F), sw2.view(G, H, F // 32),
                                                             base, out=out)),
        ], flops, hbm
    ld = sge.mx_token_capacity(T, G)
    lay = torch.empty(2, G + 1, dtype=torch.int64, device="cuda")
    qxT, sxT = torch.empty(H, ld, **u8), torch.empty(H, ld // 32, **u8)
    qw1T, sw1T = torch.empty(H, G * N1, **u8), torch.empty(H, G * N1 // 32, **u8)
    qw2T, sw2T = torch.empty(F, G * H, **u8), torch.empty(F, G * H // 32, **u8)
    qyT, syT = torch.empty(F, ld, **u8), torch.empty(F, ld // 32, **u8)
    qd, sd = torch.empty(T, H, **u8), torch.empty(T, H // 32, **u8)
    qdT, sdT = torch.empty(H, ld, **u8), torch.empty(H, ld // 32, **u8)
    qdh, sdh = torch.empty(T, N1, **u8), torch.empty(T, N1 // 32, **u8)
    qdhT, sdhT = torch.empty(N1, ld, **u8), torch.empty(N1, ld // 32, **u8)
    flops.update({dact: 2 * T * H * F, "fc2_wgrad": 2 * T * H * F, "fc1_dgrad": 2 * T * N1 * H,
                  "fc1_wgrad": 2 * T * N1 * H})
    # algorithmic bytes: bf16 read, E4M3 written per copy, one E8M0 byte per 32 (padding not counted)
    hbm = {"quant_x": T * H * 4 + T * H // 16, "quant_w1": G * N1 * H * 4 + G * N1 * H // 16,
           "quant_w2": G * H * F * 4 + G * H * F // 16, "quant_dout": T * H * 4 + T * H // 16}
    launches = [
        ("offsets", lambda: sge.splits_to_offsets(splits, [1, H], offs)),
        ("mx_layout", lambda: sge.mx_group_layout(base, T, lay)),
        ("quant_x", lambda: sge.quantize_mxfp8_grouped(X, lay, qxT, sxT, q_row=qx, s_row=sx)),
        ("quant_w1", lambda: sge.quantize_mxfp8(W1f, q_row=qw1, s_row=sw1, q_colT=qw1T, s_colT=sw1T)),
        ("quant_w2", lambda: sge.quantize_mxfp8(W2f, q_row=qw2, s_row=sw2, q_colT=qw2T, s_colT=sw2T)),
        ("fc1_fwd", lambda: sge.grouped_linear_fwd_mxfp8(
            qx, sx, qw1.view(G, N1, H), sw1.view(G, N1, H // 32), base, out=None,
            epilogue=fwd_epi, probs=P, preact=h, out_q=qy, out_s=sy, act=ap, layout=lay,
            out_colT_q=qyT, out_colT_s=syT)),
        ("fc2_fwd", lambda: sge.grouped_linear_fwd_mxfp8(qy, sy, qw2.view(G, H, F), sw2.view(G, H, F // 32),
                                                         base, out=out)),
        ("quant_dout", lambda: sge.quantize_mxfp8_grouped(DOUT, lay, qdT, sdT, q_row=qd, s_row=sd)),
        (dact, lambda: sge.grouped_linear_dgrad_mxfp8(
            qd, sd, qw2T, sw2T, base, epilogue=bwd_epi, preact=h, probs=P, dact=None, dprobs=dp, act=ap,
            dact_q=qdh, dact_s=sdh, workspace=ws, layout=lay, dact_colT_q=qdhT, dact_colT_s=sdhT)),
        ("fc2_wgrad", lambda: sge.grouped_linear_wgrad_mxfp8(qdT, sdT, qyT, syT, lay, dw2)),
        ("fc1_dgrad", lambda: sge.grouped_linear_dgrad_mxfp8(qdh, sdh, qw1T, sw1T, base, dx=dx)),
        ("fc1_wgrad", lambda: sge.grouped_linear_wgrad_mxfp8(qdhT, sdhT, qxT, sxT, lay, dw1)),
    ]
    return launches, flops, hbm


def build_grouped_fp8(torch, sge, wl, X, W1, W2, DOUT, P, splits, offs, h, out, dh, dp, dw2, dx, dw1, ws, flops):
    """The grouped MLP on E4M3 operands with current scaling per group: each step quantizes x,
    y, dout and dh per token group and W1, W2 per expert (an amax pass, then one pass writing
    the rowwise bytes and the transposed copy), and runs the six grouped GEMMs with per-group
    scales."""
    T, H = X.shape
    G, N1, _ = W1.shape
    swiglu, fwd_epi, bwd_epi, dact, ap = act_config(sge, wl)   # swiglu: a gated activation
    F = N1 // 2 if swiglu else N1
    base = offs[0]
    u8 = dict(dtype=torch.uint8, device="cuda")
    ld = sge.mx_token_capacity(T, G)
    lay = torch.empty(2, G + 1, dtype=torch.int64, device="cuda")
    y = torch.empty(T, F, dtype=torch.bfloat16, device="cuda")
    qws = torch.empty(max(16, sge.quantize_fp8_grouped_workspace_size(G)), **u8)

    def qbuf(rows, cols, lcols):
        return {"q": torch.empty(rows, cols, **u8), "q_t": torch.empty(cols, lcols, **u8),
                "s": [torch.empty(G, dtype=torch.float32, device="cuda") for _ in range(3)]}

    qx, qy, qd, qdh = qbuf(T, H, ld), qbuf(T, F, ld), qbuf(T, H, ld), qbuf(T, N1, ld)
    qw1, qw2 = qbuf(G * N1, H, G * N1), qbuf(G * H, F, G * H)
    W1f, W2f = W1.reshape(G * N1, H), W2.reshape(G * H, F)

    amax_y = torch.empty(G, dtype=torch.float32, device="cuda")
    amax_dh = torch.empty(G, dtype=torch.float32, device="cuda")

    def quant(src, b, layout, amax_in=None):
        return lambda: sge.quantize_fp8_grouped(src, G, *b["s"], qws, layout=layout, q=b["q"], q_t=b["q_t"],
                                                amax_in=amax_in)

    sinv = lambda b: b["s"][2]   # noqa: E731
    # amax pass 2 B + quantize pass 2 B read, q and q_t 1 + 1 B written; y's and dh's amax come
    # from fc1's and fc2's epilogues, so their quantize pass alone (4 B)
    hbm = {"quant_x": T * H * 6, "quant_w1": G * N1 * H * 6, "quant_w2": G * H * F * 6, "quant_y": T * F * 4,
           "quant_dout": T * H * 6, "quant_dh": T * N1 * 4}
    launches = [
        ("offsets", lambda: sge.splits_to_offsets(splits, [1, H], offs)),
        ("layout", lambda: sge.mx_group_layout(base, T, lay)),
        ("quant_x", quant(X, qx, lay)),
        ("quant_w1", quant(W1f, qw1, None)),
        ("quant_w2", quant(W2f, qw2, None)),
        ("fc1_fwd", lambda: sge.grouped_linear_fwd_fp8(qx["q"], sinv(qx), qw1["q"].view(G, N1, H), sinv(qw1), base,
                                                       y, epilogue=fwd_epi, probs=P, preact=h, act=ap,
                                                       out_amax=amax_y)),
        ("quant_y", quant(y, qy, lay, amax_y)),
        ("fc2_fwd", lambda: sge.grouped_linear_fwd_fp8(qy["q"], sinv(qy), qw2["q"].view(G, H, F), sinv(qw2), base,
                                                       out)),
        ("quant_dout", quant(DOUT, qd, lay)),
        (dact, lambda: sge.grouped_linear_dgrad_fp8(
            qd["q"], sinv(qd), qw2["q_t"], sinv(qw2), base, epilogue=bwd_epi, preact=h, probs=P, act=ap,
            dact=dh, dprobs=dp, dact_amax=amax_dh, workspace=ws)),
        ("fc2_wgrad", lambda: sge.grouped_linear_wgrad_fp8(qd["q_t"], sinv(qd), qy["q_t"], sinv(qy), lay, dw2)),
        ("quant_dh", quant(dh, qdh, lay, amax_dh)),
        ("fc1_dgrad", lambda: sge.grouped_linear_dgrad_fp8(qdh["q"], sinv(qdh), qw1["q_t"], sinv(qw1), base, dx=dx)),
        ("fc1_wgrad", lambda: sge.grouped_linear_wgrad_fp8(qdh["q_t"], sinv(qdh), qx["q_t"], sinv(qx), lay, dw1)),
    ]
    return launches, flops, hbm


# ----------------------------------------------------------- CPU baseline
def cpu_baseline(wl, inp, target_s):
    """The oracle, as it stands, on a bounded sample of the same workload (rows of the token dim)."""
    import numpy as np
    try:                                                       # the threads the BLAS pool runs with
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:                                          # pragma: no cover
        cores = cpu_threads()
    from oracle import grouped, linear, norm, offsets
    from oracle.codecs import bf16_to_f64, f64_to_bf16

    if wl["kind"] == "dense":
        M = inp["x"].shape[0]
        N, K = inp["w"].shape
        rows = 64
        bwd = "dgrad" in wl["passes"]

        def run(rows):
            xin = inp["x"][:rows]
            if wl.get("norm"):
                nf = norm.norm_fwd(wl["norm"], xin, inp["gamma"], None, wl["eps"])
                xin = nf["y_bits"]
            ops = linear.operands(wl["fmt"], xin, inp["w"], inp["dy"][:rows] if bwd else None)
            linear.linear_scale_add_fwd(*ops["fwd"], bf16_to_f64(inp["residual"][:rows]), wl["alpha"])
            if bwd:
                dz = linear.linear_scale_dgrad(*ops["dgrad"], wl["alpha"])
                linear.linear_scale_wgrad(*ops["wgrad"], wl["alpha"])
                if wl.get("norm"):
                    norm.norm_bwd(wl["norm"], f64_to_bf16(dz), inp["x"][:rows], nf["mu"], nf["rsigma"],
                                  inp["gamma"])

        while True:
            t0 = time.perf_counter()
            run(rows)
            dt = time.perf_counter() - t0
            if dt >= target_s / 4 or rows >= M:
                break
            rows = min(M, rows * 4)
        reps = 1
        if dt < target_s / 4:                                   # the whole workload is quick: repeat it
            reps = max(1, int(target_s / max(dt, 1e-3)))        # for about target_s of CPU time
            t0 = time.perf_counter()
            for _ in range(reps):
                run(rows)
            dt = (time.perf_counter() - t0) / reps
        flops = (3 if bwd else 1) * 2 * rows * N * K
        sample = (f"first {rows} of {M} token rows through {'/'.join(wl['passes'])} (quantizers included)"
                  + (f", mean of {reps} runs" if reps > 1 else ""))
    elif wl["fmt"] == "fp8":
        T = inp["x"].shape[0]
        tok = 256
        act = wl.get("act", "swiglu")
        while True:
            t0 = time.perf_counter()
            # first `tok` tokens, all routed to expert 0 (its weights only are quantized)
            b1 = np.array([0, tok], np.int64)
            f = grouped.grouped_mlp_fwd_fp8(inp["x"][:tok], inp["w1"][:1], inp["w2"][:1], inp["p"][:tok], b1, act)
            grouped.grouped_mlp_bwd_fp8(inp["x"][:tok], inp["w1"][:1], inp["w2"][:1], inp["p"][:tok], b1,
                                        inp["dout"][:tok], fwd=f, act=act)
            dt = time.perf_counter() - t0
            if dt >= target_s / 4 or tok >= T:
                break
            tok = min(T, tok * 4)
        H = inp["x"].shape[1]
        N1 = inp["w1"].shape[1]
        flops = 3 * (2 * tok * N1 * H + 2 * tok * H * (N1 if act == "srelu" else N1 // 2))
        sample = (f"first {tok} of {T} tokens through the FP8 (per-group current scaling) grouped MLP forward + "
                  "backward with one expert (quantization of that expert's weights included)")
    elif wl["fmt"] == "mxfp8":
        T = inp["x"].shape[0]
        tok = 256
        bwd = "bwd" in wl["passes"]
        act = wl.get("act", "swiglu")
        while True:
            t0 = time.perf_counter()
            # first `tok` tokens, all routed to expert 0 (its weights only are quantized)
            b1 = np.array([0, tok], np.int64)
            f = grouped.grouped_mlp_fwd_mxfp8(inp["x"][:tok], inp["w1"][:1], inp["w2"][:1], inp["p"][:tok], b1,
                                              act)
            if bwd:
                grouped.grouped_mlp_bwd_mxfp8(inp["x"][:tok], inp["w1"][:1], inp["w2"][:1], inp["p"][:tok], b1,
                                              inp["dout"][:tok], fwd=f, act=act)
            dt = time.perf_counter() - t0
            if dt >= target_s / 4 or tok >= T:
                break
            tok = min(T, tok * 4)
        H = inp["x"].shape[1]
        N1 = inp["w1"].shape[1]
        flops = (3 if bwd else 1) * (2 * tok * N1 * H + 2 * tok * H * (N1 if act == "srelu" else N1 // 2))
        sample = (f"first {tok} of {T} tokens through the MXFP8 grouped MLP {'forward + backward' if bwd else 'forward'}"
                  " with one expert (quantization of that expert's weights included)")
    else:
        T = inp["x"].shape[0]
        tok = 256
        while True:
            t0 = time.perf_counter()
            G = len(inp["splits"])
            splits = np.zeros(G, np.int64)
            splits[0] = tok                                     # first `tok` tokens, all in group 0's weights
            base = offsets.base_offsets(splits)
            x = bf16_to_f64(inp["x"][:tok])
            w1, w2 = bf16_to_f64(inp["w1"]), bf16_to_f64(inp["w2"])
            p = inp["p"][:tok].astype(np.float64)
            act = wl.get("act", "swiglu")
            f = grouped.grouped_mlp_fwd(x, w1, w2, p, base, act=act)
            grouped.grouped_mlp_bwd(bf16_to_f64(inp["dout"][:tok]), x, w1, w2, p, base, h=f["h"], y=f["y"], act=act)
            dt = time.perf_counter() - t0
            if dt >= target_s / 4 or tok >= T:
                break
            tok = min(T, tok * 4)
        H = inp["x"].shape[1]
        N1 = inp["w1"].shape[1]
        F = N1 if wl.get("act", "swiglu") == "srelu" else N1 // 2
        flops = 3 * (2 * tok * N1 * H + 2 * tok * H * F)
        sample = f"first {tok} of {T} tokens through the grouped MLP forward and backward"
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": sample, "seconds": round(dt, 3)}


# ---------------------------------------------------------------- traffic
def traffic_for(kernel_key):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if its kernel source is current."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    src = os.path.join(ROOT, "scaled_gemm_epilogues_amd", "csrc", t.get("source", "gemm.hip"))
    if not os.path.exists(src) or hashlib.sha256(open(src, "rb").read()).hexdigest() != t.get("source_sha256"):
        return None
    return t.get("bytes_per_launch", {}).get(kernel_key)


# ------------------------------------------------------ profile summaries
COPY_BYTES = 1 << 30
PROFILE_REPS_KEY = "profile_reps"
PROFILE_REPS = 5


def copy_calibration():
    """Two plain copies of COPY_BYTES: the runtime's device-to-device copy (its blit kernel), then
    an elementwise kernel (out = in * 1, 16-byte vector loads and stores per thread, the access
    size of the GEMM tile copies), each reading and writing COPY_BYTES once."""
    import torch
    a = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    torch.mul(a, 1.0, out=b)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES}), flush=True)


def _pmc_rows(path):
    """Counter value summed over the rows of each dispatch: {dispatch_id: (kernel, value)}."""
    import csv
    out = {}
    for r in csv.DictReader(open(path)):
        d = int(r["Dispatch_Id"])
        k, v = out.get(d, (r["Kernel_Name"], 0.0))
        out[d] = (k, v + float(r["Counter_Value"]))
    return out


def summarize_traffic(pmc_dir, out_dir=None):
    """profiles/traffic.json: HBM bytes per launch of each profiled kernel.

    Expects rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE runs named ``copy_<COUNTER>`` (of
    ``bench.py --copy-calibration``) and ``<workload>__<key>_<COUNTER>`` (of ``bench.py
    --workload <workload> --profile-launch <key>``). A launch's traffic is the mean over its
    last profile-reps dispatches (all of one kernel), each counter scaled by the bytes a plain
    copy moves per unit of that counter."""
    import glob
    cal, blit = {}, {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        rows = _pmc_rows(os.path.join(pmc_dir, f"copy_{c}_counter_collection.csv"))
        blits = [v for k, v in rows.values() if "copyBuffer" in k]
        elem = [v for k, v in rows.values() if "elementwise" in k and "Fill" not in k]   # not the inputs' fill
        if blits:
            blit[c] = COPY_BYTES / (blits[-1] * 1024.0)        # counters count KiB
        # the scale factor comes from the elementwise copy (16-byte accesses, like the GEMMs'
        # tile copies) when it was profiled, else from the blit
        cal[c] = COPY_BYTES / ((elem or blits)[-1] * 1024.0)
    kind = "elementwise copy" if cal != blit else "device-to-device copy (blit kernel)"
    src = os.path.join(ROOT, "scaled_gemm_epilogues_amd", "csrc", "gemm.hip")
    out = {"source": "gemm.hip", "source_sha256": hashlib.sha256(open(src, "rb").read()).hexdigest(),
           "calibration": {"copy_bytes": COPY_BYTES, "kernel": kind, "fetch_factor": cal["FETCH_SIZE"],
                           "write_factor": cal["WRITE_SIZE"], "blit_fetch_factor": blit.get("FETCH_SIZE"),
                           "blit_write_factor": blit.get("WRITE_SIZE")},
           "bytes_per_launch": {}, "raw_kib_per_launch": {}}
    blit_note = (f" (the runtime's device-to-device blit of the same size reads as fetch factor "
                 f"{blit['FETCH_SIZE']:.3f}, write factor {blit['WRITE_SIZE']:.3f})") if blit and cal != blit else ""
    md = ["# Traffic between the L2s and the fabric per launch (GEMMs and quantizers)", "",
          "Two rocprofv3 counter runs per launch (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each",
          f"scaled by what the same counter reads for a 1 GiB {kind}",
          f"(fetch factor {cal['FETCH_SIZE']:.3f}, write factor {cal['WRITE_SIZE']:.3f}){blit_note}.",
          "Commands, from /tmp:", "",
          "```",
          "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o copy_FETCH_SIZE -- python3 bench.py --copy-calibration",
          "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o <workload>__<key>_FETCH_SIZE -- \\",
          "    python3 bench.py --workload <workload> --profile-launch <key> --no-cpu-baseline",
          "(the same with WRITE_SIZE), then: python3 bench.py --summarize-traffic <dir>",
          "```", "",
          "FETCH_SIZE counts the bytes each XCD's L2 fetches on a miss, from HBM or from the Infinity",
          "Cache: operand panels that several XCDs' L2s each need count once per XCD, and only the",
          "first of them comes from HBM. So these are L2 fill bytes, an upper bound of the HBM bytes.", "",
          "| workload | launch | kernels | FETCH_SIZE MiB | WRITE_SIZE MiB | traffic MB (scaled) |", "|---|---|---|---|---|---|"]
    for f in sorted(glob.glob(os.path.join(pmc_dir, "*__*_FETCH_SIZE_counter_collection.csv"))):
        tag = os.path.basename(f)[: -len("_FETCH_SIZE_counter_collection.csv")]
        wl, key = tag.split("__", 1)
        per_kernel = {}
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            rows = _pmc_rows(os.path.join(pmc_dir, f"{tag}_{c}_counter_collection.csv"))
            seq = [rows[d] for d in sorted(rows)]
            # the repeated launch is the last k * profile-reps dispatches, k its kernel count:
            # the smallest period of the kernel-name sequence there
            k = next(k for k in range(1, 9) if all(seq[-k * PROFILE_REPS + i][0] == seq[-k * PROFILE_REPS + i + k][0]
                                                  for i in range(k * PROFILE_REPS - k)))
            for name, v in seq[-k * PROFILE_REPS:]:
                per_kernel.setdefault(name, {}).setdefault(c, 0.0)
                per_kernel[name][c] += v * 1024.0 / PROFILE_REPS
        per_kernel = {k: v for k, v in per_kernel.items() if len(v) == 2}
        fetch = sum(v["FETCH_SIZE"] for v in per_kernel.values())
        write = sum(v["WRITE_SIZE"] for v in per_kernel.values())
        t = fetch * cal["FETCH_SIZE"] + write * cal["WRITE_SIZE"]
        out["bytes_per_launch"][f"{wl}:{key}"] = int(t)
        out["raw_kib_per_launch"][f"{wl}:{key}"] = {"FETCH_SIZE": fetch / 1024.0, "WRITE_SIZE": write / 1024.0}
        kern = " + ".join(f"`{k.split('(')[0].replace('void ', '')[:60]}`" for k in per_kernel)
        md.append(f"| {wl} | {key} | {kern} | {fetch / 2**20:.1f} | {write / 2**20:.1f} | {t / 1e6:.1f} |")
    out_dir = out_dir or os.path.join(ROOT, "profiles")
    with open(os.path.join(out_dir, "traffic.json"), "w") as fh:
        json.dump(out, fh, indent=1)
    with open(os.path.join(out_dir, "traffic_per_launch.md"), "w") as fh:
        fh.write("\n".join(md) + "\n")
    print("\n".join(md))


MFMA_COUNTERS = "SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F8"


def summarize_mfma(pmc_dir, out_dir=None):
    """profiles/mfma_util.md and .json: MFMA utilisation of each profiled GEMM launch.

    Expects one rocprofv3 --pmc run of MFMA_COUNTERS per launch, named
    ``<workload>__<key>_MFMA`` (of ``bench.py --workload <workload> --profile-launch <key>``).
    Per launch, over its last profile-reps GEMM dispatches: the MFMA pipe's busy fraction
    (SQ_VALU_MFMA_BUSY_CYCLES summed over the SIMDs / (GRBM_GUI_ACTIVE of one XCD x SIMDs));
    the clock the GPU ran at (GRBM_GUI_ACTIVE of one XCD / dispatch duration); the MFMA FLOPs
    the counters saw (MOPS x 512); and the rate against the dense peak at 2.4 GHz, which is
    the busy fraction times the clock's share of 2.4 GHz."""
    import csv
    import glob
    agent = None
    out = {}
    md = ["# MFMA utilisation per GEMM launch", "",
          "One rocprofv3 counter run per launch, from /tmp:", "", "```",
          f"rocprofv3 --pmc {MFMA_COUNTERS} --output-format csv -d <dir> -o <workload>__<key>_MFMA -- \\",
          "    python3 bench.py --workload <workload> --profile-launch <key> --no-cpu-baseline",
          "then: python3 bench.py --summarize-mfma <dir>", "```", "",
          "busy = SQ_VALU_MFMA_BUSY_CYCLES (all SIMDs) / (GRBM_GUI_ACTIVE of one XCD x SIMDs); clock =",
          "GRBM_GUI_ACTIVE of one XCD / dispatch time; MFMA TFLOP = (MOPS_BF16 + MOPS_F8) x 512 per",
          "dispatch; of peak = busy x clock / 2.4 GHz (the fraction of the dense MFMA peak, 2.5 PFLOP/s",
          "bf16 or 5.0 PFLOP/s FP8, reached inside the counted dispatch).", "",
          "| workload | launch | kernel | MFMA busy | clock GHz | MFMA TFLOP / dispatch | dispatch us | of peak |",
          "|---|---|---|---|---|---|---|---|"]
    for f in sorted(glob.glob(os.path.join(pmc_dir, "*__*_MFMA_counter_collection.csv"))):
        tag = os.path.basename(f)[: -len("_MFMA_counter_collection.csv")]
        wl, key = tag.split("__", 1)
        if agent is None:
            for a in csv.DictReader(open(f.replace("_counter_collection.csv", "_agent_info.csv"))):
                if a.get("Name", "").startswith("gfx"):
                    agent = {"xcc": int(a["Num_Xcc"]), "simd": int(a["Simd_Count"])}
        disp = {}
        for r in csv.DictReader(open(f)):
            if "gemm_kernel" not in r["Kernel_Name"] and "gemm_pair_kernel" not in r["Kernel_Name"]:
                continue
            d = disp.setdefault(int(r["Dispatch_Id"]), {"kernel": r["Kernel_Name"], "ns": int(r["End_Timestamp"]) -
                                                         int(r["Start_Timestamp"])})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        last = [disp[k] for k in sorted(disp)][-PROFILE_REPS:]
        n = len(last)
        gui = sum(d["GRBM_GUI_ACTIVE"] for d in last) / n / agent["xcc"]
        busy = sum(d["SQ_VALU_MFMA_BUSY_CYCLES"] for d in last) / n / (gui * agent["simd"])
        ns = sum(d["ns"] for d in last) / n
        clk = gui / ns
        tflop = sum(d["SQ_INSTS_VALU_MFMA_MOPS_BF16"] + d["SQ_INSTS_VALU_MFMA_MOPS_F8"] for d in last) / n * 512 / 1e12
        out[f"{wl}:{key}"] = {"mfma_busy": busy, "clock_ghz": clk, "mfma_tflop_per_dispatch": tflop,
                              "dispatch_us": ns / 1e3, "frac_of_peak": busy * clk / 2.4}
        kern = last[0]["kernel"].split("(")[0].replace("void ", "")
        md.append(f"| {wl} | {key} | `{kern}` | {busy:.3f} | {clk:.2f} | {tflop:.3f} | {ns / 1e3:.1f} | "
                  f"{busy * clk / 2.4:.3f} |")
    out_dir = out_dir or os.path.join(ROOT, "profiles")
    with open(os.path.join(out_dir, "mfma_util.json"), "w") as fh:
        json.dump(out, fh, indent=1)
    with open(os.path.join(out_dir, "mfma_util.md"), "w") as fh:
        fh.write("\n".join(md) + "\n")
    print("\n".join(md))


def summarize_trace(trace_dir, bench_json, out_md, command):
    """Markdown summary of a rocprofv3 --kernel-trace --stats CSV run of bench.py."""
    import csv
    import collections
    rows = list(csv.DictReader(open(os.path.join(trace_dir, "trace_kernel_trace.csv"))))
    stats = list(csv.DictReader(open(os.path.join(trace_dir, "trace_kernel_stats.csv"))))
    with open(bench_json) as fh:
        b = json.loads([ln for ln in fh.read().splitlines() if ln.startswith("{")][-1])
    per = collections.defaultdict(list)
    for r in rows:
        per[r["Kernel_Name"]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    L = [f"# Kernel trace: {b['config']['workload']}", "", "Produced by (from /tmp):", "", "```", command, "```", "",
         "## rocprofv3 kernel statistics (every dispatch of the run)", "",
         "| kernel | calls | avg us | median us | min us | max us | % time |", "|---|---|---|---|---|---|---|"]
    for st in stats:
        d = sorted(per.get(st["Name"], []))
        med = d[len(d) // 2] if d else 0.0
        L.append(f"| `{st['Name'][:110]}` | {st['Calls']} | {float(st['AverageNs']) / 1e3:.1f} | {med:.1f} | "
                 f"{float(st['MinNs']) / 1e3:.1f} | {float(st['MaxNs']) / 1e3:.1f} | {float(st['Percentage']):.1f} |")
    L += ["", "## bench.py line of the same run", "",
          f"value {b['value']} {b['unit']}, ms_per_step {b['ms_per_step']} (graph {b.get('ms_per_step_graph')})", "",
          "| launch | ms | rate |", "|---|---|---|"]
    for k, v in b["kernels"].items():
        rate = f"{v['tflops']} TFLOP/s" if "tflops" in v else (f"{v['gbs']} GB/s" if "gbs" in v else "")
        L.append(f"| {k} | {v['ms']} | {rate} |")
    L += ["", f"roofline: `{json.dumps(b['roofline'])}`", ""]
    with open(out_md, "w") as fh:
        fh.write("\n".join(L) + "\n")


def host_info():
    """Host CPUs visible to this process, their model and the BLAS library numpy calls."""
    info = {"host_cpus": len(os.sched_getaffinity(0)), "cpu_model": None, "blas": None}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:                                            # pragma: no cover
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if blas:
            info["blas"] = f"{blas[0].get('internal_api')} {blas[0].get('version')}"
    except Exception:                                          # pragma: no cover
        pass
    return info


def cpu_threads():
    """Threads the oracle's BLAS runs with: every CPU this process may use, capped by
    OMP_NUM_THREADS when the host sets it (the share of the machine this job holds)."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS")
    if cap and cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return n


def ramp(torch, step, seconds):
    """Untimed steps for ``seconds`` (the GPU raises its clocks over ~100 ms of load)."""
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(8):
            step()
        torch.cuda.synchronize()


def measure(torch, sge, synth, args, name, cpu_seconds):
    """Times one workload: ``args.steps`` eager steps after the clock ramp and ``args.warmup``
    steps, per-kernel graph timings, cold HBM-bound launches, the roofline of the kernel with the
    largest share of the step, and (cpu_seconds > 0) the oracle on a bounded sample of it."""
    wl = synth.WORKLOADS[name]
    inp = synth.workload_inputs(name, seed=0)
    builder = build_dense if wl["kind"] == "dense" else build_grouped
    launches, flops, hbm = builder(torch, sge, wl, inp)
    step_flops = sum(flops.values())

    def eager_step():
        for _, f in launches:
            f()

    # Clock ramp: under sustained load MI355X raises its clocks over the first ~50-100 ms (the
    # 4096^3 bf16 step falls from 0.50 to 0.33 ms over its first ~150 steps, and is back near
    # 0.40 ms after 2 s idle), so the step runs untimed for ramp_seconds before the `warmup`
    # steps, and the timed steps measure the steady state a training loop runs at.
    ramp(torch, eager_step, args.ramp_seconds)
    for _ in range(args.warmup):
        eager_step()
    torch.cuda.synchronize()
    # The timed region: exactly `steps` eager steps between HIP events, synchronized on both sides.
    ms_per_step = time_ms(torch, eager_step, args.steps)
    # The same step as one HIP graph (reported for comparison; not the timed value), and per
    # kernel a graph of `reps` back-to-back launches of one call. Capturing leaves the GPU idle
    # for milliseconds, long enough for its clocks to drop, so every graph is captured first,
    # the step runs untimed again for half the ramp time, and only then are the graphs timed
    # with HIP events around their replays (on the replay stream the events mark).
    reps = 8
    step_graph = capture(torch, [f for _, f in launches])
    graphs = {k: capture(torch, [f] * reps) for k, f in launches}
    ramp(torch, eager_step, args.ramp_seconds / 2)
    ms_graph = time_ms(torch, step_graph.replay, max(1, min(args.steps, 10)))
    per = {}
    for k, g in graphs.items():
        g.replay()
        per[k] = time_ms(torch, g.replay, 3) / reps
    del step_graph, graphs
    # HBM-bound launches (quantizers, norms) are timed cold as well: before each timed launch a
    # 512 MiB write evicts the 256 MB Infinity Cache, so their inputs come from HBM; the median
    # of 10 such launches is their duration (the in-step figure is kept as ms_warm).
    cold = {}
    if any(k in hbm for k in per):
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        for k, f in launches:
            if k not in hbm:
                continue
            ts = []
            for _ in range(10):
                flush.zero_()
                ev[0].record()
                f()
                ev[1].record()
                torch.cuda.synchronize()
                ts.append(ev[0].elapsed_time(ev[1]))
            cold[k] = sorted(ts)[len(ts) // 2]
        del flush

    fmt = wl["fmt"]
    peak = PEAK_TFLOPS[fmt]
    kernels = {}
    for k, ms in per.items():
        if k in flops:
            kernels[k] = {"ms": round(ms, 4), "tflops": round(flops[k] / ms / 1e9, 1),
                          "frac_peak": round(flops[k] / ms / 1e9 / peak, 4)}
        elif k in hbm:
            c = cold[k]
            kernels[k] = {"ms": round(c, 4), "gbs": round(hbm[k] / c / 1e6, 1),
                          "frac_hbm": round(hbm[k] / c / 1e6 / PEAK_HBM_GBS, 4), "ms_warm": round(ms, 4)}
        else:
            kernels[k] = {"ms": round(ms, 4)}
    dom = max((k for k in per if k in flops), key=lambda k: per[k])
    achieved = flops[dom] / per[dom] / 1e9
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": traffic_for(f"{name}:{dom}"),
                "kernel": dom, "flops_per_launch": flops[dom], "avg_launch_ms": round(per[dom], 4)}
    gemm_ms = sum(per[k] for k in per if k in flops)
    value = step_flops / (ms_per_step * 1e9)
    cfg = {"workload": name}
    cfg.update({k: wl[k] for k in ("M", "N", "K", "T", "G", "hidden", "ffn", "alpha") if k in wl})
    res = {"value": round(value, 2), "unit": "TFLOP/s", "ms_per_step": round(ms_per_step, 4),
           "ms_per_step_graph": round(ms_graph, 4), "dtype": fmt, "config": cfg,
           "frac_of_peak": round(value / peak, 4),
           "gemm_tflops": round(step_flops / (gemm_ms * 1e9), 1),
           "gemm_frac_of_peak": round(step_flops / (gemm_ms * 1e9) / peak, 4),
           "kernels": kernels, "roofline": roofline}
    del launches
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if cpu_seconds > 0:
        res["cpu_baseline"] = cpu_baseline(wl, inp, cpu_seconds)
    return res


def main():
    args = parse()
    if args.summarize_traffic:
        summarize_traffic(args.summarize_traffic)
        return 0
    if args.summarize_mfma:
        summarize_mfma(args.summarize_mfma)
        return 0
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return 0
    if args.copy_calibration:
        copy_calibration()
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (this path has no "
              "multi-GPU sharding).", file=sys.stderr)
        return 2
    import torch
    import numpy as np  # noqa: F401
    import scaled_gemm_epilogues_amd as sge
    import synth

    if args.profile_launch:
        wl = synth.WORKLOADS[args.workload]
        inp = synth.workload_inputs(args.workload, seed=0)
        builder = build_dense if wl["kind"] == "dense" else build_grouped
        launches, _, _ = builder(torch, sge, wl, inp)
        fns = dict(launches)
        if args.profile_launch not in fns:
            print(f"unknown launch {args.profile_launch}; this workload has {list(fns)}", file=sys.stderr)
            return 2

        def eager_step():
            for _, f in launches:
                f()

        eager_step()
        torch.cuda.synchronize()
        ramp(torch, eager_step, args.ramp_seconds)             # the clock ramp, as for the timed steps
        for _ in range(args.profile_reps):
            fns[args.profile_launch]()
        torch.cuda.synchronize()
        print(json.dumps({"profile_launch": args.profile_launch, PROFILE_REPS_KEY: args.profile_reps}), flush=True)
        return 0

    if args.configs == "auto":
        extra = list(DEFAULT_CONFIGS) if args.workload == DEFAULT_WORKLOAD else []
    elif args.configs in ("", "none"):
        extra = []
    else:
        extra = [c for c in args.configs.split(",") if c and c != args.workload]
    for c in [args.workload] + extra:
        if c not in synth.WORKLOADS:
            print(f"unknown workload {c}", file=sys.stderr)
            return 2
    want_cpu = not args.no_cpu_baseline
    if want_cpu:
        # the oracle's BLAS threads, fixed before its first call
        try:
            from threadpoolctl import threadpool_limits
            threadpool_limits(limits=cpu_threads(), user_api="blas")
        except Exception:                                      # pragma: no cover
            pass
    head = measure(torch, sge, synth, args, args.workload, args.cpu_seconds if want_cpu else 0)
    print(f"# {args.workload}: {head['value']} TFLOP/s, {head['ms_per_step']} ms/step", file=sys.stderr, flush=True)
    configs = {}
    for c in extra:
        r = measure(torch, sge, synth, args, c, args.cpu_seconds_configs if want_cpu else 0)
        configs[c] = r
        print(f"# {c}: {r['value']} TFLOP/s, {r['ms_per_step']} ms/step", file=sys.stderr, flush=True)

    line = {
        "metric": METRIC, "value": head["value"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "warmup_ramp_s": args.ramp_seconds, "ms_per_step": head["ms_per_step"],
        "ms_per_step_graph": head["ms_per_step_graph"],
        "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": head["dtype"], "data": "synthetic (seeded; see synth/)",
        "config": head["config"], "frac_of_peak": head["frac_of_peak"], "gemm_tflops": head["gemm_tflops"],
        "gemm_frac_of_peak": head["gemm_frac_of_peak"], "kernels": head["kernels"], "roofline": head["roofline"],
    }
    if "cpu_baseline" in head:
        line["cpu_baseline"] = head["cpu_baseline"]
    if configs:
        line["configs"] = configs
    if want_cpu:
        line["host"] = host_info()
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

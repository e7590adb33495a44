"""The whole grouped MLP in one call each way: bit-identical to the layer-by-layer grouped calls
(which the other grouped tests hold to the oracle), and within the oracle's bar itself."""

import numpy as np
import pytest
import torch

import scaled_gemm_epilogues_amd as sge
import synth
from oracle import grouped, offsets
from oracle.codecs import bf16_to_f64

from .gpu_paths import run_grouped_mlp
from .helpers import TAU_BF16, assert_close, host_f64

pytestmark = pytest.mark.gpu

ACTS = {"swiglu": (sge.EPI_SCALED_SWIGLU, None, "swiglu"),
        "srelu": (sge.EPI_SCALED_SRELU, None, "srelu"),
        "clamped_swiglu": (sge.EPI_SCALED_CLAMPED_SWIGLU, (0.25, 1.702), ("clamped_swiglu", 0.25, 1.702))}


def _module(inp, epi, params):
    X, W1, W2 = (torch.from_numpy(np.ascontiguousarray(inp[k]).view(np.int16)).view(torch.bfloat16).cuda()
                 for k in ("x", "w1", "w2"))
    DOUT = torch.from_numpy(np.ascontiguousarray(inp["dout"]).view(np.int16)).view(torch.bfloat16).cuda()
    P = torch.from_numpy(inp["p"]).cuda()
    S = torch.from_numpy(inp["splits"]).cuda()
    T, H = X.shape
    G, N1, _ = W1.shape
    F = W2.shape[2]
    bf = dict(dtype=torch.bfloat16, device="cuda")
    r = {"offsets": torch.empty(G + 1, dtype=torch.int64, device="cuda"),
         "err": torch.full((1,), 7, dtype=torch.int32, device="cuda"),
         "h": torch.empty(T, N1, **bf), "y": torch.empty(T, F, **bf), "out": torch.empty(T, H, **bf),
         "dh": torch.empty(T, N1, **bf), "dp": torch.empty(T, dtype=torch.float32, device="cuda"),
         "dx": torch.empty(T, H, **bf), "dw1": torch.empty(G, N1, H, **bf), "dw2": torch.empty(G, H, F, **bf)}
    sge.grouped_mlp_fwd(X, W1, W2, S, r["offsets"], P, r["h"], r["y"], r["out"], activation=epi, act=params,
                        err_flag=r["err"])
    ws = torch.empty(max(1, sge.grouped_mlp_bwd_workspace_size(T, F, G, epi)), dtype=torch.uint8, device="cuda")
    sge.grouped_mlp_bwd(DOUT, X, W1, W2, r["offsets"], P, r["h"], r["y"], r["dh"], r["dp"], dx=r["dx"], dw1=r["dw1"],
                        dw2=r["dw2"], workspace=ws, activation=epi, act=params)
    torch.cuda.synchronize()
    return r


@pytest.mark.parametrize("act", list(ACTS))
def test_grouped_mlp_module_equals_layer_calls(act):
    epi, params, oact = ACTS[act]
    print(f"case grouped mlp module {act}", flush=True)
    inp = synth.grouped(700, 6, 256, 256, seed=41, splits=[0, 1, 300, 0, 391, 8], gated=act != "srelu")
    got = _module(inp, epi, params)
    ref = run_grouped_mlp(inp, act=oact)
    assert int(got["err"].item()) == 0
    assert torch.equal(got["offsets"], ref["offsets"][0])
    for k in ("h", "y", "out", "dh", "dx", "dw1", "dw2"):
        assert torch.equal(got[k].view(torch.int16), ref[k].view(torch.int16)), k
    assert torch.equal(got["dp"], ref["dp"])


def test_grouped_mlp_module_parity_and_skips():
    """The oracle's bar on a Dirichlet split; the backward with dx, dw1 and dw2 skipped (NULL) gives
    the same activation gradients."""
    inp = synth.grouped(520, 5, 256, 256, seed=42)
    got = _module(inp, sge.EPI_SCALED_SWIGLU, None)
    base = offsets.base_offsets(inp["splits"])
    x, w1, w2 = bf16_to_f64(inp["x"]), bf16_to_f64(inp["w1"]), bf16_to_f64(inp["w2"])
    p = inp["p"].astype(np.float64)
    f = grouped.grouped_mlp_fwd(x, w1, w2, p, base)
    b = grouped.grouped_mlp_bwd(bf16_to_f64(inp["dout"]), x, w1, w2, p, base, h=f["h"], y=f["y"])
    kw = dict(rel_tight=2.0 ** -7, abs_tight=5e-2)
    for k, ref in (("out", f["out"]), ("dh", b["dh"]), ("dp", b["dp"]), ("dx", b["dx"]), ("dw1", b["dw1"]),
                   ("dw2", b["dw2"])):
        assert_close(host_f64(got[k]), ref, TAU_BF16, what=k, **kw)
    # the backward with only the activation's gradients requested
    T = inp["x"].shape[0]
    dh = torch.empty_like(got["dh"])
    dp = torch.empty_like(got["dp"])
    W1 = torch.from_numpy(np.ascontiguousarray(inp["w1"]).view(np.int16)).view(torch.bfloat16).cuda()
    W2 = torch.from_numpy(np.ascontiguousarray(inp["w2"]).view(np.int16)).view(torch.bfloat16).cuda()
    X = torch.from_numpy(np.ascontiguousarray(inp["x"]).view(np.int16)).view(torch.bfloat16).cuda()
    DOUT = torch.from_numpy(np.ascontiguousarray(inp["dout"]).view(np.int16)).view(torch.bfloat16).cuda()
    P = torch.from_numpy(inp["p"]).cuda()
    G, F = W2.shape[0], W2.shape[2]
    ws = torch.empty(sge.grouped_mlp_bwd_workspace_size(T, F, G, sge.EPI_SCALED_SWIGLU), dtype=torch.uint8,
                     device="cuda")
    sge.grouped_mlp_bwd(DOUT, X, W1, W2, got["offsets"], P, got["h"], got["y"], dh, dp, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(dh.view(torch.int16), got["dh"].view(torch.int16)) and torch.equal(dp, got["dp"])


def test_grouped_mlp_module_flags_bad_splits():
    inp = synth.grouped(300, 3, 256, 256, seed=43, splits=[100, 100, 99])    # sums to 299, not T = 300
    got = _module(inp, sge.EPI_SCALED_SWIGLU, None)
    assert int(got["err"].item()) == 1


def test_grouped_mlp_module_edge_cases():
    """No tokens (offsets still written, nothing else launched), one group, every token in one
    group of several."""
    # T = 0
    G, H, F = 3, 256, 128
    bf = dict(dtype=torch.bfloat16, device="cuda")
    W1 = torch.zeros(G, 2 * F, H, **bf)
    W2 = torch.zeros(G, H, F, **bf)
    X = torch.zeros(0, H, **bf)
    S = torch.zeros(G, dtype=torch.int64, device="cuda")
    offs = torch.full((G + 1,), -1, dtype=torch.int64, device="cuda")
    err = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    empty = torch.zeros(0, 2 * F, **bf)
    sge.grouped_mlp_fwd(X, W1, W2, S, offs, torch.zeros(0, device="cuda"), empty, torch.zeros(0, F, **bf),
                        torch.zeros(0, H, **bf), err_flag=err)
    torch.cuda.synchronize()
    assert torch.equal(offs.cpu(), torch.zeros(G + 1, dtype=torch.int64)) and int(err.item()) == 0
    dw1, dw2 = torch.ones(G, 2 * F, H, **bf), torch.ones(G, H, F, **bf)
    sge.grouped_mlp_bwd(torch.zeros(0, H, **bf), X, W1, W2, offs, torch.zeros(0, device="cuda"), empty,
                        torch.zeros(0, F, **bf), torch.zeros(0, 2 * F, **bf), torch.zeros(0, device="cuda"),
                        dx=torch.zeros(0, H, **bf), dw1=dw1, dw2=dw2)
    torch.cuda.synchronize()
    assert torch.all(dw1 == 0) and torch.all(dw2 == 0)                 # empty sums
    # one group, and all tokens in the middle group of three
    for splits, G in (([300], 1), ([0, 300, 0], 3)):
        inp = synth.grouped(300, G, 256, 128, seed=44, splits=splits)
        got = _module(inp, sge.EPI_SCALED_SWIGLU, None)
        ref = run_grouped_mlp(inp)
        for k in ("h", "y", "out", "dh", "dx", "dw1", "dw2"):
            assert torch.equal(got[k].view(torch.int16), ref[k].view(torch.int16)), (splits, k)
        if G == 3:
            assert torch.all(got["dw1"][0] == 0) and torch.all(got["dw2"][2] == 0)

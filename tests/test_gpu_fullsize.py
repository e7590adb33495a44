"""Full-size parity: each workload at its own size, run through the same calls as bench.py, checked
on sampled outputs that the oracle computes row by row / column by column.

Per-tensor FP8 scales come from the oracle's amax over the whole tensor; MXFP8 blocks are local to
a row (rowwise) or a column (columnwise), so sampled rows and columns quantize on their own."""

import numpy as np
import pytest
import torch

import synth
from oracle import grouped, linear, offsets, quant
from oracle.codecs import bf16_to_f64, f64_to_bf16

from .gpu_paths import (quant_mx_grouped, run_dense, run_grouped_mlp, run_grouped_mlp_bwd_mx, run_grouped_mlp_fp8,
                        run_grouped_mlp_fwd_mx)
from .helpers import (TAU_BF16, TAU_FP8, assert_close, assert_mx_dequant_close, assert_oracle_mx_rowwise, host_bits,
                      host_f64, host_u8)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _pick(n, k, rng):
    idx = set(rng.choice(n, size=min(k, n), replace=False).tolist()) | {0, n - 1}
    return np.array(sorted(idx))


def _small_and_largest(sizes):
    """The two smallest non-empty groups and the largest one."""
    small = [int(v) for v in np.argsort(np.where(sizes > 0, sizes, 1 << 62))[:2]]
    return sorted(set(small) | {int(np.argmax(sizes))})


def _boundary_and_sampled_rows(base, rng, k):
    """k sampled token rows plus every non-empty group's first and last row."""
    T = int(base[-1])
    rows = set(rng.choice(T, size=min(k, T), replace=False).tolist())
    for g in range(len(base) - 1):
        if base[g + 1] > base[g]:
            rows |= {int(base[g]), int(base[g + 1]) - 1}
    return np.array(sorted(rows))


def _assert_fused_mx_rows(y, yq, ys, base, rng, what):
    """Fused MXFP8 rows of a bf16 tensor == the oracle's rowwise MXFP8 of those bf16 rows."""
    rows = _boundary_and_sampled_rows(base, rng, 2048)
    rr = torch.from_numpy(rows).cuda()
    assert_oracle_mx_rowwise(host_bits(y[rr]), host_u8(yq[rr]), host_u8(ys[rr]), what=what)


def _assert_fused_token_blocked(out, qT, lay, base, rng, what, ncols=6):
    """An epilogue's token-blocked MXFP8 copy of its bf16 output: the whole tensor against the
    standalone token-blocked quantizer on the same launch's bf16 output (compared on the GPU), and
    sampled columns over all tokens against the oracle's token blocking of those bf16 columns."""
    T = out.shape[0]
    c, pad = quant.mx_group_layout(base, T)
    P = int(pad[-1])
    std = quant_mx_grouped(out, lay)
    assert torch.equal(qT["q_colT"][:, :P], std["q_colT"][:, :P]), what
    assert torch.equal(qT["s_colT"][:, :P // 32], std["s_colT"][:, :P // 32]), what
    cols = _pick(out.shape[1], ncols, rng)
    cc = torch.from_numpy(cols).cuda()
    q, s = quant.mxfp8_colwise_grouped(host_bits(out[:, cc]), c, pad, qT["ld"])
    assert np.array_equal(host_u8(qT["q_colT"][cc])[:, :P], q[:, :P]), what
    assert np.array_equal(host_u8(qT["s_colT"][cc])[:, :P // 32], s[:, :P // 32]), what


def _fp8_rows(bits, rows, scale):
    """Oracle E4M3 codes of the given rows with the whole tensor's scale, and their values."""
    q = quant.fp8_quantize_with_scale(bits[rows], scale)
    return q, quant.fp8_dequantize(q, quant.fp8_scale_inv(scale))


@pytest.mark.parametrize("name", ["bf16_fwdbwd_4096", "fp8_tensor_fwdbwd_8192x14336x4096",
                                  "mxfp8_fwdbwd_16384x8192x8192"])
def test_dense_workload_full_size_sampled(name):
    w = synth.WORKLOADS[name]
    print(f"case full-size {name}", flush=True)
    d = synth.workload_inputs(name, seed=0)
    fmt, alpha = w["fmt"], w["alpha"]
    got = run_dense(fmt, d, alpha)
    M, N, K = w["M"], w["N"], w["K"]
    rng = np.random.default_rng(123)
    R, C = _pick(M, 24, rng), _pick(N, 48, rng)          # sampled rows of x/dy, rows of W (= out columns)
    Ck = _pick(K, 48, rng)                               # sampled contraction columns (dgrad/wgrad columns)
    tau = TAU_BF16 if fmt == "bf16" else TAU_FP8
    x, W, dy = d["x"], d["w"], d["dy"]
    xT, WT, dyT = (np.ascontiguousarray(a.T) for a in (x, W, dy))

    if fmt == "bf16":
        xr, Wc, dyr = bf16_to_f64(x[R]), bf16_to_f64(W[C]), bf16_to_f64(dy[R])
        Wk, dyn_, xk = bf16_to_f64(WT[Ck]), bf16_to_f64(dyT[C]), bf16_to_f64(xT[Ck])
    elif fmt == "fp8":
        sx, sw, sd = (quant.fp8_scale(quant.amax(a)) for a in (x, W, dy))
        qg = got["quant"]
        for src, g, s in ((x, qg["x"], sx), (W, qg["w"], sw), (dy, qg["dy"], sd)):
            assert float(g["scale"].item()) == float(s)
            assert float(g["amax"].item()) == float(quant.amax(src))
        qx, xr = _fp8_rows(x, R, sx)
        qw, Wc = _fp8_rows(W, C, sw)
        qd, dyr = _fp8_rows(dy, R, sd)
        assert np.array_equal(host_u8(qg["x"]["q"][torch.from_numpy(R).cuda()]), qx)
        assert np.array_equal(host_u8(qg["w"]["q"][torch.from_numpy(C).cuda()]), qw)
        qwt, Wk = _fp8_rows(WT, Ck, sw)                  # rows of W^T = columns of W
        qdt, dyn_ = _fp8_rows(dyT, C, sd)
        qxt, xk = _fp8_rows(xT, Ck, sx)
        assert np.array_equal(host_u8(qg["x"]["q_t"][torch.from_numpy(Ck).cuda()]), qxt)
        assert np.array_equal(host_u8(qg["dy"]["q_t"][torch.from_numpy(C).cuda()]), qdt)
    else:
        qg = got["quant"]
        qxr, sxr = quant.mxfp8_rowwise(x[R])
        qwr, swr = quant.mxfp8_rowwise(W[C])
        qdr, sdr = quant.mxfp8_rowwise(dy[R])
        rr, cc = torch.from_numpy(R).cuda(), torch.from_numpy(C).cuda()
        assert np.array_equal(host_u8(qg["x"]["q_row"][rr]), qxr) and np.array_equal(host_u8(qg["x"]["s_row"][rr]), sxr)
        assert np.array_equal(host_u8(qg["w"]["q_row"][cc]), qwr) and np.array_equal(host_u8(qg["w"]["s_row"][cc]), swr)
        xr, Wc, dyr = quant.mx_dequantize(qxr, sxr), quant.mx_dequantize(qwr, swr), quant.mx_dequantize(qdr, sdr)
        # columnwise copies: blocks run down a column, so a column quantizes on its own
        qwc, swc = quant.mxfp8_rowwise(WT[Ck])
        qdc, sdc = quant.mxfp8_rowwise(dyT[C])
        qxc, sxc = quant.mxfp8_rowwise(xT[Ck])
        kk = torch.from_numpy(Ck).cuda()
        assert np.array_equal(host_u8(qg["x"]["q_colT"][kk]), qxc) and np.array_equal(host_u8(qg["x"]["s_colT"][kk]), sxc)
        assert np.array_equal(host_u8(qg["dy"]["q_colT"][cc]), qdc)
        Wk, dyn_, xk = quant.mx_dequantize(qwc, swc), quant.mx_dequantize(qdc, sdc), quant.mx_dequantize(qxc, sxc)

    # forward: sampled rows x sampled output columns
    ref_f = linear.linear_scale_add_fwd(xr, Wc, bf16_to_f64(d["residual"][np.ix_(R, C)]), alpha)
    assert_close(host_f64(got["fwd"][torch.from_numpy(R).cuda()][:, torch.from_numpy(C).cuda()]), ref_f, tau,
                 what=f"{name} fwd")
    # dgrad[R, Ck] = alpha * dy[R, :] @ W[:, Ck]  (W columns Ck as rows of W^T)
    ref_d = linear.linear_scale_dgrad(dyr, Wk.T, alpha)
    assert_close(host_f64(got["dgrad"][torch.from_numpy(R).cuda()][:, torch.from_numpy(Ck).cuda()]), ref_d, tau,
                 what=f"{name} dgrad")
    # wgrad[C, Ck] = alpha * dy[:, C]^T @ x[:, Ck]
    ref_w = linear.linear_scale_wgrad(dyn_.T, xk.T, alpha)
    assert_close(host_f64(got["wgrad"][torch.from_numpy(C).cuda()][:, torch.from_numpy(Ck).cuda()]), ref_w, tau,
                 what=f"{name} wgrad")


def _gated_act(act):
    """(forward, backward) of a gated activation of the oracle: SwiGLU or the clamped SwiGLU."""
    if act == "swiglu":
        return grouped.scaled_swiglu_fwd, grouped.scaled_swiglu_bwd
    _, limit, alpha = act
    return (lambda h, p: grouped.scaled_clamped_swiglu_fwd(h, p, limit, alpha),
            lambda gy, h, p: grouped.scaled_clamped_swiglu_bwd(gy, h, p, limit, alpha))


@pytest.mark.parametrize("name", ["grouped_swiglu_mlp_T65536_G8", "grouped_clamped_swiglu_mlp_T65536_G8"])
def test_grouped_workload_full_size_sampled(name):
    w = synth.WORKLOADS[name]
    act = w.get("act", "swiglu")
    act_fwd, act_bwd = _gated_act(act)
    print(f"case full-size {name}", flush=True)
    inp = synth.workload_inputs(name, seed=0)
    got = run_grouped_mlp(inp, act=act)
    assert int(got["err"].item()) == 0
    base = offsets.base_offsets(inp["splits"])
    assert np.array_equal(got["offsets"][0].cpu().numpy(), base)
    T, F, G = w["T"], w["ffn"], w["G"]
    rng = np.random.default_rng(7)
    x = inp["x"]
    W1, W2 = bf16_to_f64(inp["w1"]), bf16_to_f64(inp["w2"])
    p = inp["p"].astype(np.float64)
    dout = inp["dout"]
    cols = _pick(F, 6, rng)
    for g in range(G):
        lo, hi = int(base[g]), int(base[g + 1])
        if hi == lo:
            continue
        toks = np.array(sorted({lo, hi - 1} | set(rng.integers(lo, hi, size=min(6, hi - lo)).tolist())))
        one = np.array([0, len(toks)])
        xs = bf16_to_f64(x[toks])
        f = grouped.grouped_mlp_fwd(xs, W1[g:g + 1], W2[g:g + 1], p[toks], one, act=act)
        b = grouped.grouped_mlp_bwd(bf16_to_f64(dout[toks]), xs, W1[g:g + 1], W2[g:g + 1], p[toks], one,
                                    h=f["h"], y=f["y"], act=act)
        tt = torch.from_numpy(toks).cuda()
        kw = dict(rel_tight=2.0 ** -7, abs_tight=5e-2)
        assert_close(host_f64(got["out"][tt]), f["out"], TAU_BF16, what=f"out g{g}", **kw)
        assert_close(host_f64(got["h"][tt]), f["h"], TAU_BF16, what=f"h g{g}", **kw)
        assert_close(host_f64(got["dh"][tt]), b["dh"], TAU_BF16, what=f"dh g{g}", **kw)
        assert_close(host_f64(got["dp"][tt]), b["dp"], TAU_BF16, what=f"dp g{g}", **kw)
        assert_close(host_f64(got["dx"][tt]), b["dx"], TAU_BF16, what=f"dx g{g}", **kw)
        # weight gradients at sampled columns: every token of the group, column-local quantities
        xg = bf16_to_f64(x[lo:hi])
        hk = xg @ W1[g][np.concatenate([cols, F + cols])].T          # h[:, k] and h[:, F+k]
        yk = act_fwd(hk, p[lo:hi])                                    # y[:, cols]
        dg = bf16_to_f64(dout[lo:hi])
        ref_dw2 = dg.T @ yk                                           # dW2_g[:, cols]
        assert_close(host_f64(got["dw2"][g][:, torch.from_numpy(cols).cuda()]), ref_dw2, TAU_BF16,
                     what=f"dw2 g{g}", **kw)
        gk = dg @ W2[g][:, cols]                                      # g[:, cols]
        dhk, _ = act_bwd(gk, hk, p[lo:hi])                            # dh[:, cols] and dh[:, F+cols]
        rows1 = np.concatenate([cols, F + cols])
        ref_dw1 = dhk.T @ xg                                          # dW1_g[rows1, :]
        assert_close(host_f64(got["dw1"][g][torch.from_numpy(rows1).cuda()]), ref_dw1, TAU_BF16,
                     what=f"dw1 g{g}", **kw)


def test_grouped_mxfp8_forward_full_size_sampled():
    name = "mxfp8_grouped_swiglu_mlp_fwd_T65536_G8"
    print(f"case full-size {name}", flush=True)
    inp = synth.workload_inputs(name, seed=0)
    got = run_grouped_mlp_fwd_mx(inp)
    assert int(got["err"].item()) == 0
    # the fused activation + group quantize equals the standalone quantizer, over the whole tensor
    assert np.array_equal(host_u8(got["yq"]), host_u8(got["y_unfused"]["q_row"]))
    assert np.array_equal(host_u8(got["ys"]), host_u8(got["y_unfused"]["s_row"]))
    base = offsets.base_offsets(inp["splits"])
    # and the oracle's MXFP8 of the launch's bf16 y (rowwise blocks are row-local): sampled rows
    # and every group's first and last row
    _assert_fused_mx_rows(got["y"], got["yq"], got["ys"], base, np.random.default_rng(21), "y (fused MXFP8)")
    # the token-blocked y written by the same epilogue
    _assert_fused_token_blocked(got["y"], got["q_y"], got["lay"], base, np.random.default_rng(23),
                                "y (fused token-blocked MXFP8)")
    sizes = np.diff(base)
    nonempty = [g for g in range(len(sizes)) if sizes[g] > 0]
    rng = np.random.default_rng(11)
    # the oracle quantizes a group's whole weights; three groups keep it to seconds
    for g in sorted({nonempty[0], int(np.argmax(sizes)), nonempty[-1]}):
        lo, hi = int(base[g]), int(base[g + 1])
        toks = np.array(sorted({lo, hi - 1} | set(rng.integers(lo, hi, size=min(6, hi - lo)).tolist())))
        ref = grouped.grouped_mlp_fwd_mxfp8(inp["x"][toks], inp["w1"][g:g + 1], inp["w2"][g:g + 1], inp["p"][toks],
                                            np.array([0, len(toks)]))
        tt = torch.from_numpy(toks).cuda()
        kw = dict(rel_tight=2.0 ** -3, abs_tight=0.1)
        assert_close(host_f64(got["h"][tt]), ref["h"], TAU_FP8, what=f"h g{g}", **kw)
        assert_close(host_f64(got["y"][tt]), ref["y"], TAU_FP8, what=f"y g{g}", **kw)
        y_deq = quant.mx_dequantize(host_u8(got["yq"][tt]), host_u8(got["ys"][tt]))
        assert_mx_dequant_close(y_deq, quant.mx_dequantize(ref["y_q"], ref["y_s"]), what=f"y (MXFP8) g{g}")
        assert_close(host_f64(got["out"][tt]), ref["out"], TAU_FP8, what=f"out g{g}", **kw)



def test_grouped_mxfp8_backward_full_size_sampled():
    name = "mxfp8_grouped_swiglu_mlp_T65536_G8"
    print(f"case full-size {name}", flush=True)
    inp = synth.workload_inputs(name, seed=0)
    fwd = run_grouped_mlp_fwd_mx(inp)
    assert int(fwd["err"].item()) == 0
    got = run_grouped_mlp_bwd_mx(inp, fwd)
    # the fused activation backward + group quantize equals the standalone quantizer, whole tensor
    assert np.array_equal(host_u8(got["dhq"]), host_u8(got["dh_unfused"]["q_row"]))
    assert np.array_equal(host_u8(got["dhs"]), host_u8(got["dh_unfused"]["s_row"]))
    base = offsets.base_offsets(inp["splits"])
    # and the oracle's MXFP8 of the launch's bf16 dh, on sampled rows and the group boundaries
    _assert_fused_mx_rows(got["dh"], got["dhq"], got["dhs"], base, np.random.default_rng(22), "dh (fused MXFP8)")
    # the token-blocked dh written by the dgrad epilogue
    _assert_fused_token_blocked(got["dh"], got["q_dh"], got["lay"], base, np.random.default_rng(24),
                                "dh (fused token-blocked MXFP8)")
    sizes = np.diff(base)
    F = inp["w2"].shape[2]
    rng = np.random.default_rng(12)
    kw = dict(rel_tight=2.0 ** -3, abs_tight=0.1)
    # the two smallest non-empty groups and the largest one (its wgrad tiles have the longest
    # contraction); the wgrad samples take sampled columns over all of a group's tokens
    for g in _small_and_largest(sizes):
        lo, hi = int(base[g]), int(base[g + 1])
        Tg = hi - lo
        # per-token outputs at sampled tokens (the per-token oracle on those tokens alone)
        toks = np.array(sorted({lo, hi - 1} | set(rng.integers(lo, hi, size=6).tolist())))
        ref = grouped.grouped_mlp_bwd_mxfp8(inp["x"][toks], inp["w1"][g:g + 1], inp["w2"][g:g + 1],
                                            inp["p"][toks], np.array([0, len(toks)]), inp["dout"][toks])
        tt = torch.from_numpy(toks).cuda()
        assert_close(host_f64(got["dh"][tt]), ref["dh"], TAU_FP8, what=f"dh g{g}", **kw)
        assert_close(host_f64(got["dp"][tt]), ref["dp"], TAU_FP8, what=f"dprobs g{g}", **kw)
        assert_close(host_f64(got["dx"][tt]), ref["dx"], TAU_FP8, what=f"dx g{g}", **kw)
        # weight-gradient entries: sampled columns of the group's activations, over all its tokens
        fs = _pick(F, 6, rng)
        hs = _pick(inp["x"].shape[1], 6, rng)
        xg, doutg, pg = inp["x"][lo:hi], inp["dout"][lo:hi], inp["p"][lo:hi]
        x_hat = quant.mx_dequantize(*quant.mxfp8_rowwise(xg))
        rows1 = np.concatenate([fs, F + fs])                          # gate rows fs and up rows F + fs
        w1_hat = quant.mx_dequantize(*quant.mxfp8_rowwise(inp["w1"][g][rows1]))
        h_sub = x_hat @ w1_hat.T                                      # [Tg, 2k]: a | b of the sampled columns
        y_bits = f64_to_bf16(grouped.scaled_swiglu_fwd(h_sub, pg))
        one = np.array([0, Tg])
        ref_dw2 = grouped.grouped_linear_wgrad_mxfp8(doutg[:, hs], y_bits, one)[0]
        assert_close(host_f64(got["dw2"][g][torch.from_numpy(hs).cuda()][:, torch.from_numpy(fs).cuda()]),
                     ref_dw2, TAU_FP8, what=f"dw2 g{g}", **kw)
        dout_hat = quant.mx_dequantize(*quant.mxfp8_rowwise(doutg))
        w2c_hat = quant.mx_dequantize(*quant.mxfp8_colwise(inp["w2"][g][:, fs]))    # [k, H] blocked along H
        gy = dout_hat @ w2c_hat.T                                     # [Tg, k]
        dh_sub, _ = grouped.scaled_swiglu_bwd(gy, bf16_to_f64(f64_to_bf16(h_sub)), pg)
        ref_dw1 = grouped.grouped_linear_wgrad_mxfp8(f64_to_bf16(dh_sub), xg[:, hs], one)[0]
        assert_close(host_f64(got["dw1"][g][torch.from_numpy(rows1).cuda()][:, torch.from_numpy(hs).cuda()]),
                     ref_dw1, TAU_FP8, what=f"dw1 g{g}", **kw)


def test_grouped_fp8_full_size_sampled():
    name = "fp8_grouped_swiglu_mlp_T65536_G8"
    print(f"case full-size {name}", flush=True)
    inp = synth.workload_inputs(name, seed=0)
    got = run_grouped_mlp_fp8(inp)
    base = offsets.base_offsets(inp["splits"])
    sizes = np.diff(base)
    rng = np.random.default_rng(13)
    kw = dict(rel_tight=2.0 ** -3, abs_tight=0.1)
    # the fused amax of y and dh, and the codes quantized with it: the oracle's per-group current
    # scaling of the launch's bf16 tensors (amax and scales over each whole group; codes of
    # sampled rows and the group boundaries)
    for key, q in (("y", "qy"), ("dh", "qdh")):
        bits = host_bits(got[key])
        rows = _boundary_and_sampled_rows(base, np.random.default_rng(23), 2048)
        rr = torch.from_numpy(rows).cuda()
        qrows = host_u8(got[q]["q"][rr])
        for g in range(len(sizes)):
            lo, hi = int(base[g]), int(base[g + 1])
            a = quant.amax(bits[lo:hi])
            s_ = quant.fp8_scale(a)
            for k, ref in (("amax", a), ("scale", s_), ("scale_inv", quant.fp8_scale_inv(s_))):
                gv = np.float32(got[q][k][g].item())
                assert gv.view(np.uint32) == np.float32(ref).view(np.uint32), (key, g, k, gv, ref)
            sel = (rows >= lo) & (rows < hi)
            assert np.array_equal(qrows[sel], quant.fp8_quantize_with_scale(bits[rows[sel]], s_)), (key, g)
    # per-group scales depend on a whole group: the oracle reruns the two smallest groups and the
    # largest one whole
    for g in _small_and_largest(sizes):
        lo, hi = int(base[g]), int(base[g + 1])
        one = np.array([0, hi - lo])
        args = (inp["x"][lo:hi], inp["w1"][g:g + 1], inp["w2"][g:g + 1], inp["p"][lo:hi], one)
        fwd = grouped.grouped_mlp_fwd_fp8(*args)
        bwd = grouped.grouped_mlp_bwd_fp8(*args, inp["dout"][lo:hi], fwd=fwd)
        rows = _pick(hi - lo, 8, rng)
        tt = torch.from_numpy(rows + lo).cuda()
        for key, ref in (("h", fwd["h"]), ("y", fwd["y"]), ("out", fwd["out"]), ("dh", bwd["dh"]),
                         ("dx", bwd["dx"])):
            assert_close(host_f64(got[key][tt]), ref[rows], TAU_FP8, what=f"{key} g{g}", **kw)
        assert_close(host_f64(got["dp"][tt]), bwd["dp"][rows], TAU_FP8, what=f"dprobs g{g}", **kw)
        for key in ("dw1", "dw2"):
            r_, c_ = _pick(bwd[key].shape[1], 8, rng), _pick(bwd[key].shape[2], 8, rng)
            sub = got[key][g][torch.from_numpy(r_).cuda()][:, torch.from_numpy(c_).cuda()]
            assert_close(host_f64(sub), bwd[key][0][np.ix_(r_, c_)], TAU_FP8, what=f"{key} g{g}", **kw)


def test_rmsnorm_full_size_sampled():
    name = "rmsnorm_mxfp8_linear_fwdbwd_16384x8192x8192"
    w = synth.WORKLOADS[name]
    print(f"case full-size {name} (norm)", flush=True)
    import scaled_gemm_epilogues_amd as sge
    from oracle import norm
    from .gpu_paths import quant_mx
    from .helpers import dev_bf16
    d = synth.workload_inputs(name, seed=0)
    M, K = w["M"], w["K"]
    X, gam, DZ = dev_bf16(d["x"]), dev_bf16(d["gamma"]), dev_bf16(d["dy"][:, :K])
    u8 = dict(dtype=torch.uint8, device="cuda")
    Y, RS = torch.empty_like(X), torch.empty(M, dtype=torch.float32, device="cuda")
    mx_row = (torch.empty(M, K, **u8), torch.empty(M, K // 32, **u8))
    mx_col = (torch.empty(K, M, **u8), torch.empty(K, M // 32, **u8))
    sge.norm_fwd(sge.NORM_RMS, X, gam, Y, RS, eps=w["eps"], mx_row=mx_row, mx_col=mx_col)
    DX, DG = torch.empty_like(X), torch.empty(K, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(sge.norm_bwd_workspace_size(M, K), **u8)
    sge.norm_bwd(sge.NORM_RMS, DZ, X, RS, gam, DX, DG, ws)
    alone = quant_mx(Y)
    torch.cuda.synchronize()
    # the fused MXFP8 copies equal the standalone quantizer on the same bf16 output, whole tensor
    assert np.array_equal(host_u8(mx_row[0]), host_u8(alone["q_row"]))
    assert np.array_equal(host_u8(mx_row[1]), host_u8(alone["s_row"]))
    assert np.array_equal(host_u8(mx_col[0]), host_u8(alone["q_colT"]))
    assert np.array_equal(host_u8(mx_col[1]), host_u8(alone["s_colT"]))
    # and the oracle's MXFP8 of the launch's bf16 output: sampled rows (rowwise copy) and sampled
    # columns (columnwise copy, blocks down a column)
    rs_ = _pick(M, 256, np.random.default_rng(16))
    cs_ = _pick(K, 128, np.random.default_rng(17))
    rr, cc = torch.from_numpy(rs_).cuda(), torch.from_numpy(cs_).cuda()
    assert_oracle_mx_rowwise(host_bits(Y[rr]), host_u8(mx_row[0][rr]), host_u8(mx_row[1][rr]), what="norm MXFP8 row")
    assert_oracle_mx_rowwise(host_bits(Y[:, cc].t()), host_u8(mx_col[0][cc]), host_u8(mx_col[1][cc]),
                             what="norm MXFP8 col")
    rows = _pick(M, 8, np.random.default_rng(14))
    ref = norm.norm_fwd("rms", d["x"][rows], d["gamma"], None, w["eps"])
    tt = torch.from_numpy(rows).cuda()
    kw = dict(rel_tight=2.0 ** -7, abs_tight=1e-3)
    assert_close(host_f64(Y[tt]), ref["y"], TAU_BF16, what="y", **kw)
    refb = norm.norm_bwd("rms", d["dy"][rows, :K], d["x"][rows], ref["mu"], ref["rsigma"], d["gamma"])
    assert_close(host_f64(DX[tt]), refb["dx"], TAU_BF16, what="dx", **kw)
    # dgamma sums every row: the oracle's statistics of all rows, and (dgamma of a column needs
    # only that column given the statistics) the sampled columns over all rows
    mu, rs = norm.norm_stats("rms", d["x"], w["eps"])
    cs = _pick(K, 16, np.random.default_rng(15))
    refg = norm.norm_bwd("rms", d["dy"][:, cs], d["x"][:, cs], mu.astype(np.float32), rs.astype(np.float32),
                         d["gamma"][cs])
    assert_close(host_f64(DG)[cs], refg["dgamma"], TAU_BF16, what="dgamma", **kw)

"""Pins of the oracle's scaled linear: brute force, invariants, adjoint identities, torch autograd."""

import math

import numpy as np
import pytest
import torch

from oracle import linear
import synth

SHAPES = [(1, 1, 32), (2, 3, 32), (5, 17, 64), (17, 33, 32), (33, 5, 96)]


def _torch_e4m3(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double().numpy()


def _torch_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).double().numpy()


def _brute_operands(fmt, ops, x, w, dy):
    """Operand values rebuilt by hand from the quantizer outputs, with torch's decoders."""
    M, K = x.shape
    N = w.shape[0]
    if fmt == "bf16":
        X, W, D = _torch_bf16(x), _torch_bf16(w), _torch_bf16(dy)
        return {"fwd": (X, W), "dgrad": (D, W), "wgrad": (D, X)}
    q = ops["quant"]
    if fmt == "fp8":
        def deq(qq):
            return _torch_e4m3(qq["q"]) * float(qq["scale_inv"])
        X, W, D = deq(q["x"]), deq(q["w"]), deq(q["dy"])
        return {"fwd": (X, W), "dgrad": (D, W), "wgrad": (D, X)}

    def mx(qs, rows, cols):
        codes, sc = qs
        vals = _torch_e4m3(codes)
        out = np.empty((rows, cols))
        for i in range(rows):
            for j in range(cols):
                out[i, j] = vals[i, j] * math.ldexp(1.0, int(sc[i, j // 32]) - 127)
        return out
    Xr, Wr, Dr = mx(q["x_row"], M, K), mx(q["w_row"], N, K), mx(q["dy_row"], M, N)
    Wc, Dc, Xc = mx(q["w_col"], K, N), mx(q["dy_col"], N, M), mx(q["x_col"], K, M)
    return {"fwd": (Xr, Wr), "dgrad": (Dr, Wc.T), "wgrad": (Dc.T, Xc.T)}


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mxfp8"])
@pytest.mark.parametrize("shape", SHAPES)
def test_brute_force_fsum(fmt, shape):
    M, N, K = shape
    if fmt == "mxfp8" and M % 32:
        M = 32                       # the wgrad contraction (tokens) must be a multiple of 32
    if fmt == "mxfp8" and N % 32:
        N = 32 * (1 + N // 32)      # so must the dgrad contraction
    d = synth.dense(M, N, K, seed=M * 100 + N, outliers=(fmt == "mxfp8"))
    ops = linear.operands(fmt, d["x"], d["w"], d["dy"])
    bo = _brute_operands(fmt, ops, d["x"], d["w"], d["dy"])
    res = _torch_bf16(d["residual"])
    alpha = 0.375
    fwd = linear.linear_scale_add_fwd(*ops["fwd"], res, alpha)
    X, W = bo["fwd"]
    for m in range(M):
        for n in range(N):
            exact = res[m, n] + alpha * math.fsum(X[m, k] * W[n, k] for k in range(K))
            assert abs(fwd[m, n] - exact) <= 1e-12 * (1 + abs(exact))
    dg = linear.linear_scale_dgrad(*ops["dgrad"], alpha)
    D, W2 = bo["dgrad"]
    for m in range(M):
        for k in range(K):
            exact = alpha * math.fsum(D[m, n] * W2[n, k] for n in range(N))
            assert abs(dg[m, k] - exact) <= 1e-12 * (1 + abs(exact))
    wg = linear.linear_scale_wgrad(*ops["wgrad"], alpha)
    D2, X2 = bo["wgrad"]
    for n in range(N):
        for k in range(K):
            exact = alpha * math.fsum(D2[m, n] * X2[m, k] for m in range(M))
            assert abs(wg[n, k] - exact) <= 1e-12 * (1 + abs(exact))


def test_alpha_zero_returns_residual_bitwise():
    d = synth.dense(7, 9, 32, seed=3)
    res = _torch_bf16(d["residual"])
    res[0, 0] = -0.0
    x, w = linear.operands("bf16", d["x"], d["w"])["fwd"]
    x = x.copy()
    x[1, 1] = np.inf                              # a non-finite product must not leak in
    out = linear.linear_scale_add_fwd(x, w, res, 0.0)
    assert np.array_equal(out.view(np.uint64), res.view(np.uint64))
    dg = linear.linear_scale_dgrad(x, w.T, 0.0)
    assert np.all(dg == 0) and not np.any(np.signbit(dg))


def test_residual_zero_alpha_one_is_plain_gemm():
    d = synth.dense(6, 10, 40, seed=4)
    x, w = linear.operands("bf16", d["x"], d["w"])["fwd"]
    a = linear.linear_scale_add_fwd(x, w, np.zeros((6, 10)), 1.0)
    b = linear.linear_scale_add_fwd(x, w, None, 1.0, accumulate=False)
    brute = np.array([[math.fsum(x[m] * w[n]) for n in range(10)] for m in range(6)])
    assert np.array_equal(a, b)
    assert np.allclose(a, brute, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mxfp8"])
def test_gradients_linear_in_alpha(fmt):
    d = synth.dense(32, 64, 32, seed=5, outliers=(fmt == "mxfp8"))
    ops = linear.operands(fmt, d["x"], d["w"], d["dy"])
    g1 = linear.linear_scale_dgrad(*ops["dgrad"], 1.0)
    w1 = linear.linear_scale_wgrad(*ops["wgrad"], 1.0)
    for a in (0.125, 0.25, 0.5, 4.0):
        assert np.array_equal(linear.linear_scale_dgrad(*ops["dgrad"], a), a * g1)
        assert np.array_equal(linear.linear_scale_wgrad(*ops["wgrad"], a), a * w1)
    assert np.allclose(linear.linear_scale_dgrad(*ops["dgrad"], 0.3), 0.3 * g1, rtol=1e-14, atol=0)


def test_adjoint_identities_pin_backward_to_forward():
    """<dy, alpha*v W^T> = <alpha*dy W, v> and <dy, alpha*x V^T> = <alpha*dy^T x, V>."""
    rng = np.random.default_rng(9)
    M, N, K, alpha = 13, 11, 7, 0.625
    x, w = rng.standard_normal((M, K)), rng.standard_normal((N, K))
    v, V = rng.standard_normal((M, K)), rng.standard_normal((N, K))
    dy = rng.standard_normal((M, N))
    lhs1 = np.sum(dy * linear.linear_scale_add_fwd(v, w, None, alpha, accumulate=False))
    rhs1 = np.sum(linear.linear_scale_dgrad(dy, w, alpha) * v)
    lhs2 = np.sum(dy * linear.linear_scale_add_fwd(x, V, None, alpha, accumulate=False))
    rhs2 = np.sum(linear.linear_scale_wgrad(dy, x, alpha) * V)
    assert abs(lhs1 - rhs1) <= 1e-12 * (1 + abs(lhs1))
    assert abs(lhs2 - rhs2) <= 1e-12 * (1 + abs(lhs2))


def test_backward_vs_torch_autograd_fp64():
    rng = np.random.default_rng(10)
    M, N, K, alpha = 9, 6, 5, 0.125
    x = torch.tensor(rng.standard_normal((M, K)), requires_grad=True)
    w = torch.tensor(rng.standard_normal((N, K)), requires_grad=True)
    r = torch.tensor(rng.standard_normal((M, N)), requires_grad=True)
    dy = torch.tensor(rng.standard_normal((M, N)))
    out = r + alpha * (x @ w.T)
    out.backward(dy)
    ours = linear.linear_scale_add_fwd(x.detach().numpy(), w.detach().numpy(), r.detach().numpy(), alpha)
    assert np.allclose(ours, out.detach().numpy(), rtol=1e-13, atol=1e-14)
    assert np.allclose(linear.linear_scale_dgrad(dy.numpy(), w.detach().numpy(), alpha), x.grad.numpy(),
                       rtol=1e-13, atol=1e-14)
    assert np.allclose(linear.linear_scale_wgrad(dy.numpy(), x.detach().numpy(), alpha), w.grad.numpy(),
                       rtol=1e-13, atol=1e-14)
    assert np.array_equal(r.grad.numpy(), dy.numpy())      # the residual's gradient is dy itself


def test_mx_operands_use_the_gemm_contraction_dim():
    """dgrad's W operand is quantized in blocks along N, wgrad's along M: a block outlier only
    coarsens its own block, so swapping the orientations changes the dequantized values."""
    d = synth.dense(64, 64, 64, seed=11, outliers=True)
    ops = linear.operands("mxfp8", d["x"], d["w"], d["dy"])
    w_fwd = ops["fwd"][1]
    w_dg = ops["dgrad"][1]
    assert w_fwd.shape == w_dg.shape == (64, 64)
    assert not np.array_equal(w_fwd, w_dg)
    assert ops["quant"]["w_col"][0].shape == (64, 64) and ops["quant"]["w_col"][1].shape == (64, 2)

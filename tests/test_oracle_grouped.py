"""Pins of the oracle's split offsets, grouped linear and scaled SwiGLU."""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import grouped, linear, offsets
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_splits_to_offsets_golden():
    with open(os.path.join(GOLDEN, "splits_offsets.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        got = offsets.splits_to_offsets(c["splits"], c["multipliers"])
        assert got.dtype == np.int64
        assert got.tolist() == c["offsets"]
        assert offsets.split_points(c["splits"]).tolist() == c["split_points"]


def test_offsets_invariants_on_random_splits():
    rng = np.random.default_rng(0)
    for G, T in [(1, 5), (8, 65536), (64, 1000), (3, 0)]:
        s = synth.dirichlet_splits(rng, G, T)
        base = offsets.splits_to_offsets(s, [1])[0]
        assert base[0] == 0 and base[-1] == T
        assert np.array_equal(np.diff(base), s)
        assert np.all(np.diff(base) >= 0)


def _rand(shape, seed, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


@pytest.mark.parametrize("splits", [[5], [3, 0, 4], [1, 1, 1, 2], [0, 0, 6]])
def test_grouped_linear_vs_brute_force(splits):
    T, N, K = sum(splits), 5, 3
    base = offsets.base_offsets(splits)
    G = len(splits)
    x, w, dy = _rand((T, K), 1), _rand((G, N, K), 2), _rand((T, N), 3)
    fwd = grouped.grouped_linear_fwd(x, w, base, alpha=0.5)
    dg = grouped.grouped_linear_dgrad(dy, w, base, alpha=0.5)
    wg = grouped.grouped_linear_wgrad(dy, x, base, alpha=0.5)
    owner = [g for g, n in enumerate(splits) for _ in range(n)]
    for t in range(T):
        g = owner[t]
        for n in range(N):
            assert math.isclose(fwd[t, n], 0.5 * math.fsum(x[t, k] * w[g, n, k] for k in range(K)),
                                rel_tol=1e-13, abs_tol=1e-14)
        for k in range(K):
            assert math.isclose(dg[t, k], 0.5 * math.fsum(dy[t, n] * w[g, n, k] for n in range(N)),
                                rel_tol=1e-13, abs_tol=1e-14)
    for g in range(G):
        rows = [t for t in range(T) if owner[t] == g]
        for n in range(N):
            for k in range(K):
                exact = 0.5 * math.fsum(dy[t, n] * x[t, k] for t in rows)
                assert math.isclose(wg[g, n, k], exact, rel_tol=1e-13, abs_tol=1e-14)
        if not rows:
            assert np.all(wg[g] == 0)


def test_single_group_reduces_to_dense():
    T, N, K = 7, 6, 4
    x, w, dy = _rand((T, K), 4), _rand((1, N, K), 5), _rand((T, N), 6)
    base = offsets.base_offsets([T])
    assert np.allclose(grouped.grouped_linear_fwd(x, w, base),
                       linear.linear_scale_add_fwd(x, w[0], None, 1.0, accumulate=False), rtol=1e-14)
    assert np.allclose(grouped.grouped_linear_dgrad(dy, w, base), linear.linear_scale_dgrad(dy, w[0], 1.0))
    assert np.allclose(grouped.grouped_linear_wgrad(dy, x, base)[0], linear.linear_scale_wgrad(dy, x, 1.0))


def test_swiglu_closed_forms():
    h = np.array([[0.0, 2.0, 3.0, -1.5]])       # a = [0, 2], b = [3, -1.5]
    y = grouped.scaled_swiglu_fwd(h, np.array([0.5]))
    s2 = 1.0 / (1.0 + math.exp(-2.0))
    assert y[0, 0] == 0.0                                         # silu(0) = 0
    assert math.isclose(y[0, 1], 0.5 * 2.0 * s2 * -1.5, rel_tol=1e-15)
    dh, dp = grouped.scaled_swiglu_bwd(np.array([[1.0, 1.0]]), h, np.array([0.5]))
    assert math.isclose(dh[0, 0], 0.5 * 3.0 * 0.5, rel_tol=1e-15)  # silu'(0) = 1/2
    ones = grouped.scaled_swiglu_fwd(h, np.ones(1))
    assert np.allclose(ones, h[:, :2] / (1 + np.exp(-h[:, :2])) * h[:, 2:])
    z, zd = grouped.scaled_swiglu_fwd(h, np.zeros(1)), grouped.scaled_swiglu_bwd(np.ones((1, 2)), h, np.zeros(1))[0]
    assert np.all(z == 0) and np.all(zd == 0)


def test_swiglu_backward_central_differences():
    rng = np.random.default_rng(7)
    T, F = 3, 4
    h, p, gy = rng.standard_normal((T, 2 * F)) * 2, rng.random(T), rng.standard_normal((T, F))
    dh, dp = grouped.scaled_swiglu_bwd(gy, h, p)

    def loss(hh, pp):
        return np.sum(gy * grouped.scaled_swiglu_fwd(hh, pp))
    eps = 1e-6
    for t in range(T):
        for j in range(2 * F):
            e = np.zeros_like(h)
            e[t, j] = eps
            fd = (loss(h + e, p) - loss(h - e, p)) / (2 * eps)
            assert abs(fd - dh[t, j]) <= 1e-7 * (1 + abs(fd))
        e = np.zeros(T)
        e[t] = eps
        fd = (loss(h, p + e) - loss(h, p - e)) / (2 * eps)
        assert abs(fd - dp[t]) <= 1e-7 * (1 + abs(fd))


def test_grouped_mlp_backward_vs_torch_autograd():
    splits = [2, 0, 3, 1]
    T, H, F, G = 6, 4, 3, 4
    base = offsets.base_offsets(splits)
    rng = np.random.default_rng(8)
    x = rng.standard_normal((T, H))
    w1 = rng.standard_normal((G, 2 * F, H)) * 0.5
    w2 = rng.standard_normal((G, H, F)) * 0.5
    p = rng.random(T)
    dout = rng.standard_normal((T, H))
    ours_f = grouped.grouped_mlp_fwd(x, w1, w2, p, base)
    ours_b = grouped.grouped_mlp_bwd(dout, x, w1, w2, p, base)

    tx, tw1, tw2, tp = (torch.tensor(a, requires_grad=True) for a in (x, w1, w2, p))
    outs = []
    for g in range(G):
        lo, hi = base[g], base[g + 1]
        h = tx[lo:hi] @ tw1[g].T
        a, b = h[:, :F], h[:, F:]
        y = tp[lo:hi, None] * torch.nn.functional.silu(a) * b
        outs.append(y @ tw2[g].T)
    out = torch.cat(outs)
    out.backward(torch.tensor(dout))
    assert np.allclose(ours_f["out"], out.detach().numpy(), rtol=1e-12, atol=1e-13)
    assert np.allclose(ours_b["dx"], tx.grad.numpy(), rtol=1e-12, atol=1e-13)
    assert np.allclose(ours_b["dw1"], tw1.grad.numpy(), rtol=1e-12, atol=1e-13)
    assert np.allclose(ours_b["dw2"], tw2.grad.numpy(), rtol=1e-12, atol=1e-13)
    assert np.allclose(ours_b["dp"], tp.grad.numpy(), rtol=1e-12, atol=1e-13)
    assert np.all(ours_b["dw1"][1] == 0) and np.all(ours_b["dw2"][1] == 0)     # empty group


def test_grouped_inputs_recipe():
    d = synth.grouped(1000, 8, 64, 32, seed=0)
    assert d["splits"].sum() == 1000 and d["splits"].dtype == np.int64
    assert d["w1"].shape == (8, 64, 64) and d["w2"].shape == (8, 64, 32)
    assert d["p"].dtype == np.float32 and np.all((d["p"] >= 0) & (d["p"] < 1))
    again = synth.grouped(1000, 8, 64, 32, seed=0)
    assert all(np.array_equal(d[k], again[k]) for k in d)


def test_srelu_closed_forms():
    h = np.array([[-2.0, -0.0, 0.0, 0.5, 3.0]])
    p = np.array([0.25])
    y = grouped.scaled_srelu_fwd(h, p)
    assert y.tolist() == [[0.0, 0.0, 0.0, 0.0625, 2.25]]                   # 0.25 * max(h, 0)^2
    dh, dp = grouped.scaled_srelu_bwd(np.ones_like(h), h, p)
    assert dh.tolist() == [[0.0, 0.0, 0.0, 0.25, 1.5]]                    # 0.25 * 2 * max(h, 0)
    assert dp.tolist() == [0.25 + 9.0]


def test_grouped_srelu_mlp_backward_vs_torch_autograd():
    splits = [2, 0, 3, 1]
    T, H, F, G = 6, 4, 3, 4
    base = offsets.base_offsets(splits)
    rng = np.random.default_rng(9)
    x = rng.standard_normal((T, H))
    w1 = rng.standard_normal((G, F, H)) * 0.5
    w2 = rng.standard_normal((G, H, F)) * 0.5
    p = rng.random(T)
    dout = rng.standard_normal((T, H))
    ours_f = grouped.grouped_mlp_fwd(x, w1, w2, p, base, act="srelu")
    ours_b = grouped.grouped_mlp_bwd(dout, x, w1, w2, p, base, act="srelu")
    tx, tw1, tw2, tp = (torch.tensor(a, requires_grad=True) for a in (x, w1, w2, p))
    outs = []
    for g in range(G):
        lo, hi = base[g], base[g + 1]
        y = tp[lo:hi, None] * torch.relu(tx[lo:hi] @ tw1[g].T) ** 2
        outs.append(y @ tw2[g].T)
    out = torch.cat(outs)
    out.backward(torch.tensor(dout))
    assert np.allclose(ours_f["out"], out.detach().numpy(), rtol=1e-12, atol=1e-13)
    for k, t in (("dx", tx), ("dw1", tw1), ("dw2", tw2), ("dp", tp)):
        assert np.allclose(ours_b[k], t.grad.numpy(), rtol=1e-12, atol=1e-13), k


def test_clamped_swiglu_closed_forms():
    L = math.log(3.0)                                   # sigmoid(ln 3) = 3/4
    # gate: below, at and above the limit; linear half: inside, at +-limit, beyond both sides
    h = np.array([[0.0, L, 5.0, -1.0, 0.5, L, -L, 9.0, -9.0, 0.0]])
    p = np.array([0.5])
    y = grouped.scaled_clamped_swiglu_fwd(h, p, L, 1.0)
    s1 = 1.0 / (1.0 + math.exp(1.0))                      # sigmoid(-1)
    q = [0.0, 0.75 * L, 0.75 * L, -s1, 0.5 / (1.0 + math.exp(-0.5))]
    bp = [1.0 + L, 1.0 - L, 1.0 + L, 1.0 - L, 1.0]
    assert np.allclose(y[0], [0.5 * qi * bi for qi, bi in zip(q, bp)], rtol=1e-15, atol=0)
    dh, dp = grouped.scaled_clamped_swiglu_bwd(np.ones((1, 5)), h, p, L, 1.0)
    da, db = dh[0, :5], dh[0, 5:]
    assert da[2] == 0.0 and da[1] != 0.0                  # gate above the limit: no gradient; at it: passes
    assert db[2] == 0.0 and db[3] == 0.0 and db[1] != 0.0 and db[4] != 0.0   # beyond +-limit: none; at -limit: passes
    assert np.isclose(dp[0], sum(qi * bi for qi, bi in zip(q, bp)), rtol=1e-15)


def test_clamped_swiglu_reductions():
    rng = np.random.default_rng(3)
    h = rng.standard_normal((5, 16)) * 3
    p = rng.random(5)
    F = 8
    # no clamp (infinite limit) and alpha = 1: SwiGLU of (a, b + 1)
    shifted = h.copy()
    shifted[:, F:] += 1.0
    assert np.allclose(grouped.scaled_clamped_swiglu_fwd(h, p, np.inf, 1.0),
                       grouped.scaled_swiglu_fwd(shifted, p), rtol=1e-14, atol=0)
    # alpha = 2: a * sigmoid(2 a) = a * (1 + tanh a) / 2
    a = np.minimum(h[:, :F], 1.5)
    b = np.clip(h[:, F:], -1.5, 1.5)
    ref = p[:, None] * a * (1.0 + np.tanh(a)) / 2.0 * (b + 1.0)
    assert np.allclose(grouped.scaled_clamped_swiglu_fwd(h, p, 1.5, 2.0), ref, rtol=1e-13, atol=1e-15)


def test_clamped_swiglu_backward_central_differences():
    rng = np.random.default_rng(4)
    T, F, L, alpha = 3, 6, 1.25, 1.702
    h = rng.standard_normal((T, 2 * F)) * 1.5
    h[np.abs(np.abs(h) - L) < 1e-3] += 0.01             # keep every point off the clamps' kinks
    p = rng.random(T)
    gy = rng.standard_normal((T, F))
    dh, dp = grouped.scaled_clamped_swiglu_bwd(gy, h, p, L, alpha)
    loss = lambda hh, pp: float(np.sum(gy * grouped.scaled_clamped_swiglu_fwd(hh, pp, L, alpha)))  # noqa: E731
    eps = 1e-6
    for t in range(T):
        for j in range(2 * F):
            e = np.zeros_like(h)
            e[t, j] = eps
            num = (loss(h + e, p) - loss(h - e, p)) / (2 * eps)
            assert abs(num - dh[t, j]) <= 1e-7 * (1 + abs(num)), (t, j)
        e = np.zeros_like(p)
        e[t] = eps
        assert abs((loss(h, p + e) - loss(h, p - e)) / (2 * eps) - dp[t]) <= 1e-7 * (1 + abs(dp[t]))


def test_grouped_clamped_swiglu_mlp_backward_vs_torch_autograd():
    splits = [2, 0, 3, 1]
    T, H, F, G = 6, 4, 3, 4
    L, alpha = 0.75, 1.702
    base = offsets.base_offsets(splits)
    rng = np.random.default_rng(10)
    x = rng.standard_normal((T, H))
    w1 = rng.standard_normal((G, 2 * F, H)) * 0.7
    w2 = rng.standard_normal((G, H, F)) * 0.5
    p = rng.random(T)
    dout = rng.standard_normal((T, H))
    act = ("clamped_swiglu", L, alpha)
    ours_f = grouped.grouped_mlp_fwd(x, w1, w2, p, base, act=act)
    ours_b = grouped.grouped_mlp_bwd(dout, x, w1, w2, p, base, act=act)
    h = ours_f["h"]
    assert np.any(h[:, :F] > L) and np.any(np.abs(h[:, F:]) > L)    # both clamps engage
    tx, tw1, tw2, tp = (torch.tensor(a, requires_grad=True) for a in (x, w1, w2, p))
    outs = []
    for g in range(G):
        lo, hi = base[g], base[g + 1]
        hh = tx[lo:hi] @ tw1[g].T
        a = torch.clamp(hh[:, :F], max=L)
        b = torch.clamp(hh[:, F:], min=-L, max=L)
        y = tp[lo:hi, None] * a * torch.sigmoid(alpha * a) * (b + 1.0)
        outs.append(y @ tw2[g].T)
    out = torch.cat(outs)
    out.backward(torch.tensor(dout))
    assert np.allclose(ours_f["out"], out.detach().numpy(), rtol=1e-12, atol=1e-13)
    for k, t in (("dx", tx), ("dw1", tw1), ("dw2", tw2), ("dp", tp)):
        assert np.allclose(ours_b[k], t.grad.numpy(), rtol=1e-12, atol=1e-13), k

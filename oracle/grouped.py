"""Grouped (MoE) scaled linear and the per-token scaled SwiGLU.

Test infrastructure (see the package docstring): never used by the product path.

"Activation + GroupedLinear Fusion for MOE and other MOE optimizations"
(Description; Greptile Summary; Sequence Diagram) describes a grouped MLP:
fc1 as a GroupedLinear, a scaled SwiGLU whose scales are per-token
probabilities, fc2 as a GroupedLinear; in the backward the activation
gradient also returns the gradient of the scales ("grad_scales"). Rows of
group g are tokens ``base[g] .. base[g+1]-1`` (see ``offsets``).

Readings where the page is silent:

* The page names scaled SReLU beside scaled SwiGLU and clamped SwiGLU without formulas; SReLU
  is read as the squared ReLU, ``max(h, 0)^2``, applied elementwise (fc1 has F outputs, no
  gate half), scaled per token like SwiGLU: ``y = p * max(h, 0)^2``.

* fc1's output h [T, 2F] holds the SwiGLU gate in its first half and the
  linear ("up") part in its second half: ``a = h[:, :F]``, ``b = h[:, F:]``.
* ``y = p[:, None] * silu(a) * b`` with ``silu(a) = a * sigmoid(a)``.
* The grouped GEMMs take an alpha like the dense ones (1 for the MLP).
* A group with no token contributes an all-zero weight gradient.
"""

import numpy as np

from .codecs import bf16_to_f64, f64_to_bf16
from .quant import (MX_TOKEN_ALIGN, fp8_current_scaling_grouped, fp8_dequantize, mx_dequantize,
                    mx_group_layout, mxfp8_colwise, mxfp8_colwise_grouped, mxfp8_rowwise)


def _groups(base):
    base = np.asarray(base, dtype=np.int64)
    return [(g, int(base[g]), int(base[g + 1])) for g in range(len(base) - 1)]


def grouped_linear_fwd(x, w, base, alpha=1.0):
    """out[t] = alpha * x[t] @ W_g^T for t in group g. x [T, K], W [G, N, K] -> [T, N]."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    out = np.zeros((x.shape[0], w.shape[1]), np.float64)
    for g, lo, hi in _groups(base):
        out[lo:hi] = alpha * (x[lo:hi] @ w[g].T)
    return out


def grouped_linear_dgrad(dy, w, base, alpha=1.0):
    """dx[t] = alpha * dy[t] @ W_g. dy [T, N], W [G, N, K] -> [T, K]."""
    dy = np.asarray(dy, np.float64)
    w = np.asarray(w, np.float64)
    out = np.zeros((dy.shape[0], w.shape[2]), np.float64)
    for g, lo, hi in _groups(base):
        out[lo:hi] = alpha * (dy[lo:hi] @ w[g])
    return out


def grouped_linear_wgrad(dy, x, base, alpha=1.0):
    """dW_g = alpha * sum over t in g of dy[t]^T x[t]. -> [G, N, K] (zero for an empty group)."""
    dy = np.asarray(dy, np.float64)
    x = np.asarray(x, np.float64)
    G = len(base) - 1
    out = np.zeros((G, dy.shape[1], x.shape[1]), np.float64)
    for g, lo, hi in _groups(base):
        out[g] = alpha * (dy[lo:hi].T @ x[lo:hi])
    return out


def _sigmoid(a):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-a))


def scaled_swiglu_fwd(h, p):
    """y = p * silu(a) * b with a, b the two halves of h [T, 2F]; p [T]."""
    h = np.asarray(h, np.float64)
    F = h.shape[1] // 2
    a, b = h[:, :F], h[:, F:]
    return np.asarray(p, np.float64)[:, None] * (a * _sigmoid(a)) * b


def scaled_swiglu_bwd(gy, h, p):
    """Gradients of y = p * silu(a) * b given dL/dy.

    da = gy * p * b * silu'(a),  silu'(a) = s(a) * (1 + a * (1 - s(a)))
    db = gy * p * silu(a)
    dp = sum_j gy_j * silu(a_j) * b_j        (the per-token "grad_scales")
    Returns (dh [T, 2F] = [da, db], dp [T]).
    """
    gy = np.asarray(gy, np.float64)
    h = np.asarray(h, np.float64)
    p = np.asarray(p, np.float64)[:, None]
    F = h.shape[1] // 2
    a, b = h[:, :F], h[:, F:]
    s = _sigmoid(a)
    silu = a * s
    dsilu = s * (1.0 + a * (1.0 - s))
    da = gy * p * b * dsilu
    db = gy * p * silu
    dp = np.sum(gy * silu * b, axis=1)
    return np.concatenate([da, db], axis=1), dp


def scaled_srelu_fwd(h, p):
    """y = p * srelu(h), srelu(h) = max(h, 0)^2 (squared ReLU, elementwise: no gate half)."""
    h = np.asarray(h, np.float64)
    r = np.maximum(h, 0.0)
    return np.asarray(p, np.float64)[:, None] * r * r


def scaled_srelu_bwd(gy, h, p):
    """Gradients of y = p * max(h, 0)^2 given dL/dy: dh = gy * p * 2 max(h, 0), dp = sum_j gy_j * max(h_j, 0)^2."""
    gy = np.asarray(gy, np.float64)
    r = np.maximum(np.asarray(h, np.float64), 0.0)
    p = np.asarray(p, np.float64)[:, None]
    return gy * p * 2.0 * r, np.sum(gy * r * r, axis=1)


def scaled_clamped_swiglu_fwd(h, p, limit, alpha):
    """Clamped SwiGLU scaled per token: with a, b the two halves of h [T, 2F],
    a_c = min(a, limit), b_c = clamp(b, -limit, limit),
    y = p * a_c * sigmoid(alpha * a_c) * (b_c + 1).

    The PR page ("Activation + GroupedLinear Fusion for MOE ...", Description; Important Files
    Changed: ScaledClampedQGeGLU) names the clamped SwiGLU without its formula. Read as the
    published clamped form: the gate is clamped from above and passed through the quick-GELU
    shape a * sigmoid(alpha * a) (the "QGeGLU"), the linear half is clamped both ways and
    offset by one; limit and alpha are parameters.
    """
    h = np.asarray(h, np.float64)
    F = h.shape[1] // 2
    a = np.minimum(h[:, :F], limit)
    b = np.clip(h[:, F:], -limit, limit)
    return np.asarray(p, np.float64)[:, None] * (a * _sigmoid(alpha * a)) * (b + 1.0)


def scaled_clamped_swiglu_bwd(gy, h, p, limit, alpha):
    """Gradients of ``scaled_clamped_swiglu_fwd`` given dL/dy. A clamp passes the gradient
    where its input lies inside the closed interval (as torch.clamp does) and stops it
    outside: da = gy * p * (b_c + 1) * q'(a_c) where a <= limit, with
    q'(u) = s * (1 + alpha * u * (1 - s)), s = sigmoid(alpha * u); db = gy * p * q(a_c) where
    |b| <= limit; dp = sum_j gy_j * q(a_c,j) * (b_c,j + 1). Returns (dh [T, 2F], dp [T])."""
    gy = np.asarray(gy, np.float64)
    h = np.asarray(h, np.float64)
    p = np.asarray(p, np.float64)[:, None]
    F = h.shape[1] // 2
    a_raw, b_raw = h[:, :F], h[:, F:]
    a = np.minimum(a_raw, limit)
    b = np.clip(b_raw, -limit, limit)
    s = _sigmoid(alpha * a)
    q = a * s
    dq = s * (1.0 + alpha * a * (1.0 - s))
    da = np.where(a_raw <= limit, gy * p * (b + 1.0) * dq, 0.0)
    db = np.where(np.abs(b_raw) <= limit, gy * p * q, 0.0)
    dp = np.sum(gy * q * (b + 1.0), axis=1)
    return np.concatenate([da, db], axis=1), dp


_ACTS = {"swiglu": (scaled_swiglu_fwd, scaled_swiglu_bwd), "srelu": (scaled_srelu_fwd, scaled_srelu_bwd)}


def _act(act):
    """(forward, backward) of an activation: "swiglu", "srelu", or ("clamped_swiglu", limit, alpha)."""
    if isinstance(act, tuple):
        name, limit, alpha = act
        assert name == "clamped_swiglu", name
        return (lambda h, p: scaled_clamped_swiglu_fwd(h, p, limit, alpha),
                lambda gy, h, p: scaled_clamped_swiglu_bwd(gy, h, p, limit, alpha))
    return _ACTS[act]


def grouped_mlp_fwd(x, w1, w2, p, base, act="swiglu"):
    """fc1 -> scaled activation (SwiGLU, SReLU, or clamped SwiGLU as ("clamped_swiglu", limit,
    alpha)) -> fc2. Returns dict(h, y, out)."""
    h = grouped_linear_fwd(x, w1, base)
    y = _act(act)[0](h, p)
    out = grouped_linear_fwd(y, w2, base)
    return {"h": h, "y": y, "out": out}


def grouped_mlp_bwd(dout, x, w1, w2, p, base, h=None, y=None, act="swiglu"):
    """Backward of ``grouped_mlp_fwd`` given dL/dout.

    Returns dict(gy = dL/dy, dh, dp, dw2, dx, dw1). ``h`` and ``y`` are
    recomputed in fp64 when not given.
    """
    if h is None:
        h = grouped_linear_fwd(x, w1, base)
    if y is None:
        y = _act(act)[0](h, p)
    gy = grouped_linear_dgrad(dout, w2, base)
    dh, dp = _act(act)[1](gy, h, p)
    dw2 = grouped_linear_wgrad(dout, y, base)
    dx = grouped_linear_dgrad(dh, w1, base)
    dw1 = grouped_linear_wgrad(dh, x, base)
    return {"gy": gy, "dh": dh, "dp": dp, "dw2": dw2, "dx": dx, "dw1": dw1}


def grouped_mlp_fwd_mxfp8(x_bits, w1_bits, w2_bits, p, base, act="swiglu"):
    """Grouped MLP forward on MXFP8 operands, with the activation quantized for fc2.

    "Activation + GroupedLinear Fusion for MOE and other MOE optimizations" (Description:
    Activation + GroupQuantize Fusion; Sequence Diagram, forward): the scaled activation's
    output is group-quantized and reaches FC2 quantized. Every GEMM operand here is MXFP8
    with blocks of 32 along that GEMM's contraction dim (rowwise for the forward), and:

    1. x and each W1_g, W2_g are quantized rowwise (``mxfp8_rowwise``) and dequantized;
    2. h = x_hat @ W1_g^T per group, y = p * silu(a) * b (``scaled_swiglu_fwd``), in fp64;
    3. the activation is rounded to bf16 (the dtype the activation has when it is not
       quantized) and that bf16 tensor is quantized rowwise: (y_q, y_s);
    4. out = y_hat @ W2_g^T per group, y_hat the dequantized (y_q, y_s).

    x_bits [T, H], w1_bits [G, 2F, H], w2_bits [G, H, F] (bf16 bit patterns); p [T]; base [G+1].
    Returns h, y (fp64), y_bits (bf16), y_q, y_s and out (fp64).
    """
    x_bits = np.asarray(x_bits, np.uint16)
    w1_bits = np.asarray(w1_bits, np.uint16)
    w2_bits = np.asarray(w2_bits, np.uint16)
    G, N1, H = w1_bits.shape
    F = w2_bits.shape[2]
    x_hat = mx_dequantize(*mxfp8_rowwise(x_bits))
    w1_hat = mx_dequantize(*mxfp8_rowwise(w1_bits.reshape(G * N1, H))).reshape(G, N1, H)
    w2_hat = mx_dequantize(*mxfp8_rowwise(w2_bits.reshape(G * H, F))).reshape(G, H, F)
    h = grouped_linear_fwd(x_hat, w1_hat, base)
    y = _act(act)[0](h, p)
    y_bits = f64_to_bf16(y)
    y_q, y_s = mxfp8_rowwise(y_bits)
    out = grouped_linear_fwd(mx_dequantize(y_q, y_s), w2_hat, base)
    return {"h": h, "y": y, "y_bits": y_bits, "y_q": y_q, "y_s": y_s, "out": out,
            "y_value": bf16_to_f64(y_bits)}



def grouped_linear_dgrad_mxfp8(dy_bits, w_bits, base, alpha=1.0):
    """dgrad of a grouped linear on MXFP8 operands: g[t] = alpha * dy_hat[t] @ W_hat_g.

    The contraction runs over the layer's output features N, so both operands carry blocks
    of 32 along N: dy [T, N] is quantized rowwise, every W_g [N, K] columnwise (its copy
    blocked along N, ``mxfp8_colwise``). Blocks never cross experts (N % 32 == 0).
    dy_bits [T, N], w_bits [G, N, K] (bf16 bit patterns) -> [T, K] fp64.
    """
    w_bits = np.asarray(w_bits, np.uint16)
    dy_hat = mx_dequantize(*mxfp8_rowwise(dy_bits))
    w_hat = np.stack([mx_dequantize(*mxfp8_colwise(w_bits[g])).T for g in range(w_bits.shape[0])])
    return grouped_linear_dgrad(dy_hat, w_hat, base, alpha)


def grouped_linear_wgrad_mxfp8(dy_bits, x_bits, base, alpha=1.0, align=MX_TOKEN_ALIGN):
    """wgrad of a grouped linear on MXFP8 operands: dW_g = alpha * sum_{t in g} dy_hat[t]^T x_hat[t].

    The contraction runs over the tokens of each group, so dy [T, N] and x [T, K] are both
    quantized in blocks of 32 along the tokens of each group (``mxfp8_colwise_grouped``);
    the zero padding between groups adds nothing. Returns [G, N, K] fp64 (zero for an
    empty group).
    """
    dy_bits = np.asarray(dy_bits, np.uint16)
    T = dy_bits.shape[0]
    c, pad = mx_group_layout(base, T, align)
    ld = max(int(pad[-1]), align)
    a = mx_dequantize(*mxfp8_colwise_grouped(dy_bits, c, pad, ld))      # [N, ld]
    b = mx_dequantize(*mxfp8_colwise_grouped(x_bits, c, pad, ld))       # [K, ld]
    G = len(c) - 1
    out = np.zeros((G, a.shape[0], b.shape[0]), np.float64)
    for g in range(G):
        lo, hi = int(pad[g]), int(pad[g + 1])
        out[g] = alpha * (a[:, lo:hi] @ b[:, lo:hi].T)
    return out


def grouped_mlp_bwd_mxfp8(x_bits, w1_bits, w2_bits, p, base, dout_bits, fwd=None, act="swiglu"):
    """Backward of ``grouped_mlp_fwd_mxfp8`` on MXFP8 operands, given dL/dout (bf16 bits).

    "Activation + GroupedLinear Fusion for MOE and other MOE optimizations" (Sequence
    Diagram, backward): the activation backward returns the quantized activation gradient
    for FC1's dgrad, the same gradient unquantized for FC1's wgrad, and the gradient of the
    scales. Every GEMM operand is MXFP8 blocked along that GEMM's contraction dim:

    1. fc2 dgrad: gy = dout_hat @ W2_hat_g (``grouped_linear_dgrad_mxfp8``);
    2. dh, dp = ``scaled_swiglu_bwd(gy, h, p)`` with h the pre-activation as the forward
       saved it (bf16); dh is rounded to bf16, the dtype the gradient has unquantized;
    3. fc2 wgrad: dW2 from dout and the forward's bf16 activation y, token-blocked;
    4. fc1 dgrad: dx from the bf16 dh (rowwise) and W1 blocked along 2F;
    5. fc1 wgrad: dW1 from the bf16 dh and x, token-blocked.

    Returns gy, dh (fp64), dh_bits, dh_q, dh_s (the rowwise MXFP8 of dh_bits), dp, dw2, dx, dw1.
    """
    if fwd is None:
        fwd = grouped_mlp_fwd_mxfp8(x_bits, w1_bits, w2_bits, p, base, act)
    h_saved = bf16_to_f64(f64_to_bf16(fwd["h"]))
    gy = grouped_linear_dgrad_mxfp8(dout_bits, w2_bits, base)
    dh, dp = _act(act)[1](gy, h_saved, p)
    dh_bits = f64_to_bf16(dh)
    dh_q, dh_s = mxfp8_rowwise(dh_bits)
    dw2 = grouped_linear_wgrad_mxfp8(dout_bits, fwd["y_bits"], base)
    dx = grouped_linear_dgrad_mxfp8(dh_bits, w1_bits, base)
    dw1 = grouped_linear_wgrad_mxfp8(dh_bits, x_bits, base)
    return {"gy": gy, "dh": dh, "dh_bits": dh_bits, "dh_q": dh_q, "dh_s": dh_s, "dp": dp,
            "dw2": dw2, "dx": dx, "dw1": dw1}


# ------------------------------------------------ FP8 current scaling, grouped -----
def _fp8_groups_hat(bits, c):
    """Exact values of a per-group current-scaled tensor (rows c[g] .. c[g+1]-1 share a scale)."""
    r = fp8_current_scaling_grouped(bits, c, c)
    out = np.zeros(np.asarray(bits).shape, np.float64)
    for g in range(len(c) - 1):
        lo, hi = int(c[g]), int(c[g + 1])
        out[lo:hi] = fp8_dequantize(r["q"][lo:hi], r["scale_inv"][g])
    return out


def _fp8_experts_hat(w_bits):
    """Exact values of each expert's weight W_g [N, K] quantized as its own tensor."""
    w_bits = np.asarray(w_bits, np.uint16)
    G, N, K = w_bits.shape
    c = np.arange(G + 1, dtype=np.int64) * N
    return _fp8_groups_hat(w_bits.reshape(G * N, K), c).reshape(G, N, K)


def grouped_mlp_fwd_fp8(x_bits, w1_bits, w2_bits, p, base, act="swiglu"):
    """Grouped MLP forward on FP8 operands with per-group current scaling.

    Every GEMM operand is E4M3 with one scale per group ("Activation + GroupedLinear Fusion for
    MOE and other MOE optimizations", Description: group quantize; fp8_current_scaling in the
    grouped-MLP test matrix): x's slice of each group, each W1_g and W2_g, and fc1's
    activation, which is rounded to bf16 and then quantized per group for fc2. Per-tensor
    scales are orientation-free, so the same codes serve every GEMM of the backward.
    Returns h, y (fp64), y_bits (bf16) and out (fp64).
    """
    T = np.asarray(x_bits).shape[0]
    c, _ = mx_group_layout(base, T)
    h = grouped_linear_fwd(_fp8_groups_hat(x_bits, c), _fp8_experts_hat(w1_bits), base)
    y = _act(act)[0](h, p)
    y_bits = f64_to_bf16(y)
    out = grouped_linear_fwd(_fp8_groups_hat(y_bits, c), _fp8_experts_hat(w2_bits), base)
    return {"h": h, "y": y, "y_bits": y_bits, "out": out}


def grouped_mlp_bwd_fp8(x_bits, w1_bits, w2_bits, p, base, dout_bits, fwd=None, act="swiglu"):
    """Backward of ``grouped_mlp_fwd_fp8``: dout, dh, x, y and every W_g are E4M3 with one
    current-scaling scale per group; h is the forward's bf16 pre-activation and dh is rounded
    to bf16 before it is quantized. Returns gy, dh (fp64), dh_bits, dp, dw2, dx, dw1."""
    if fwd is None:
        fwd = grouped_mlp_fwd_fp8(x_bits, w1_bits, w2_bits, p, base, act)
    T = np.asarray(x_bits).shape[0]
    c, _ = mx_group_layout(base, T)
    dout_hat = _fp8_groups_hat(dout_bits, c)
    w1_hat, w2_hat = _fp8_experts_hat(w1_bits), _fp8_experts_hat(w2_bits)
    gy = grouped_linear_dgrad(dout_hat, w2_hat, base)
    dh, dp = _act(act)[1](gy, bf16_to_f64(f64_to_bf16(fwd["h"])), p)
    dh_bits = f64_to_bf16(dh)
    dh_hat = _fp8_groups_hat(dh_bits, c)
    dw2 = grouped_linear_wgrad(dout_hat, _fp8_groups_hat(fwd["y_bits"], c), base)
    dx = grouped_linear_dgrad(dh_hat, w1_hat, base)
    dw1 = grouped_linear_wgrad(dh_hat, _fp8_groups_hat(x_bits, c), base)
    return {"gy": gy, "dh": dh, "dh_bits": dh_bits, "dp": dp, "dw2": dw2, "dx": dx, "dw1": dw1}

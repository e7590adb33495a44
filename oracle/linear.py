"""The scaled linear: forward with in-place residual add, backward with alpha folded in.

Test infrastructure (see the package docstring): never used by the product path.

Forward ("NVIDIA TransformerEngine Ops Fused Forward Linear Scale Add",
Description and I/O Contract): the scale is the GEMM's alpha and the residual
buffer is the GEMM's output with accumulation on, so

    out = residual + alpha * (x @ W^T)          x [M, K], W [N, K], out [M, N]

Backward ("NVIDIA TransformerEngine Ops Fused Backward Linear Scale",
Description and I/O Contract): the same scale is the alpha of the dgrad and of
the wgrad GEMM,

    dgrad = alpha_d * (dy @ W)                  [M, K]
    wgrad = alpha_w * (dy^T @ x)                [N, K]

The gradient reaching the residual is dy itself; no kernel computes it.

Operands are the exact fp64 values the GEMM consumes: a bf16 operand is its
own value; an FP8 operand is ``e4m3(q) * scale_inv``; an MXFP8 operand is
``e4m3(q) * 2^(s-127)`` with blocks of 32 along that GEMM's contraction
dimension (``operands`` below builds them with this package's quantizers).
Products of such values are exact in fp64 and the sums use BLAS dgemm, so
the result is the exact real-number result up to fp64 summation error.

Readings where the pages are silent:

* alpha == 0 returns the residual unchanged (no product is formed, so even a
  non-finite product leaves it untouched); in the backward it gives +0.
* dgrad and wgrad overwrite their outputs (no accumulation).
"""

import numpy as np

from .codecs import bf16_to_f64
from . import quant


def linear_scale_add_fwd(x_hat, w_hat, residual, alpha, accumulate=True):
    """residual + alpha * (x_hat @ w_hat^T) in fp64; alpha == 0 returns the residual.

    With ``accumulate=False`` the residual is not read and the result is the
    plain scaled GEMM ``alpha * (x_hat @ w_hat^T)``.
    """
    res = np.asarray(residual, dtype=np.float64)
    if not accumulate:
        res = np.zeros((x_hat.shape[0], w_hat.shape[0]), np.float64)
    if alpha == 0:
        return res.copy()
    return res + np.float64(alpha) * (np.asarray(x_hat, np.float64) @ np.asarray(w_hat, np.float64).T)


def linear_scale_dgrad(dy_hat, w_hat, alpha):
    """alpha * (dy_hat @ w_hat): dy [M, N], W [N, K] -> [M, K]; alpha == 0 gives +0."""
    if alpha == 0:
        return np.zeros((dy_hat.shape[0], w_hat.shape[1]), np.float64)
    return np.float64(alpha) * (np.asarray(dy_hat, np.float64) @ np.asarray(w_hat, np.float64))


def linear_scale_wgrad(dy_hat, x_hat, alpha):
    """alpha * (dy_hat^T @ x_hat): dy [M, N], x [M, K] -> [N, K]; alpha == 0 gives +0."""
    if alpha == 0:
        return np.zeros((dy_hat.shape[1], x_hat.shape[1]), np.float64)
    return np.float64(alpha) * (np.asarray(dy_hat, np.float64).T @ np.asarray(x_hat, np.float64))


def operands(fmt, x_bits, w_bits, dy_bits=None):
    """Exact fp64 operands of the three GEMMs for one operand format.

    fmt: "bf16", "fp8" (per-tensor current scaling) or "mxfp8".
    Returns a dict with ``fwd`` = (x, W), ``dgrad`` = (dy, W), ``wgrad`` =
    (dy, x), each a pair of fp64 arrays in the logical shapes of the module
    docstring, plus the quantizer outputs under ``quant``.

    MXFP8 blocks run along each GEMM's own contraction dimension:
    forward contracts K (x and W rowwise), dgrad contracts N (dy rowwise, W
    columnwise), wgrad contracts M (dy and x columnwise). Each re-quantization
    starts again from the bf16 tensor.
    """
    out = {"quant": {}}
    if fmt == "bf16":
        x, w = bf16_to_f64(x_bits), bf16_to_f64(w_bits)
        dy = None if dy_bits is None else bf16_to_f64(dy_bits)
        out["fwd"] = (x, w)
        if dy is not None:
            out["dgrad"] = (dy, w)
            out["wgrad"] = (dy, x)
        return out
    if fmt == "fp8":
        qx = quant.fp8_current_scaling(x_bits)
        qw = quant.fp8_current_scaling(w_bits)
        out["quant"].update(x=qx, w=qw)
        x = quant.fp8_dequantize(qx["q"], qx["scale_inv"])
        w = quant.fp8_dequantize(qw["q"], qw["scale_inv"])
        out["fwd"] = (x, w)
        if dy_bits is not None:
            qd = quant.fp8_current_scaling(dy_bits)
            out["quant"]["dy"] = qd
            dy = quant.fp8_dequantize(qd["q"], qd["scale_inv"])
            out["dgrad"] = (dy, w)
            out["wgrad"] = (dy, x)
        return out
    if fmt == "mxfp8":
        xr = quant.mxfp8_rowwise(x_bits)
        wr = quant.mxfp8_rowwise(w_bits)
        out["quant"].update(x_row=xr, w_row=wr)
        out["fwd"] = (quant.mx_dequantize(*xr), quant.mx_dequantize(*wr))
        if dy_bits is not None:
            dyr = quant.mxfp8_rowwise(dy_bits)
            wc = quant.mxfp8_colwise(w_bits)          # [K, N], blocks along N
            dyc = quant.mxfp8_colwise(dy_bits)        # [N, M], blocks along M
            xc = quant.mxfp8_colwise(x_bits)          # [K, M], blocks along M
            out["quant"].update(dy_row=dyr, w_col=wc, dy_col=dyc, x_col=xc)
            out["dgrad"] = (quant.mx_dequantize(*dyr), quant.mx_dequantize(*wc).T)
            out["wgrad"] = (quant.mx_dequantize(*dyc).T, quant.mx_dequantize(*xc).T)
        return out
    raise ValueError(f"unknown operand format {fmt!r}")

"""RMSNorm and LayerNorm, forward and backward, with the quantized outputs they can feed a linear.

Test infrastructure (see the package docstring): never used by the product path.

"NVIDIA TransformerEngine PyTorch Ext Normalization" (Description, I/O Contract): the forward
takes the input, the weight gamma, LayerNorm's bias beta, eps and a zero-centered-gamma flag,
and returns the normalized (optionally quantized) output plus the statistics saved for the
backward (LayerNorm's mean, the reciprocal standard deviation); the backward returns dx, dgamma
and (LayerNorm) dbeta. Quantized outputs come from the norm fused with the quantization: for
current scaling the norm and its amax first, then the quantize pass; for MXFP8 one kernel.
The page gives no formulas; the readings taken are the textbook definitions:

* RMSNorm: ``rsigma = 1 / sqrt(mean(x^2) + eps)``, ``y = x * rsigma * g``.
* LayerNorm: ``mu = mean(x)``, ``rsigma = 1 / sqrt(mean((x - mu)^2) + eps)`` (biased variance,
  eps inside the root), ``y = (x - mu) * rsigma * g + beta``.
* ``g = gamma``, or ``1 + gamma`` with zero-centered gamma.
* The saved statistics are fp32; the backward uses them as saved.
* Backward with ``xhat = (x - mu) * rsigma`` (mu = 0 for RMSNorm) and ``d = dz * g``:
  ``dx = rsigma * (d - mean(d) - xhat * mean(d * xhat))`` (RMSNorm drops ``mean(d)``),
  ``dgamma = sum_rows dz * xhat``, ``dbeta = sum_rows dz``.
* The output is bf16 (the input's dtype). A quantized output is the quantization of that
  bf16 output (FP8 current scaling over the whole tensor, or MXFP8 rowwise / columnwise), i.e.
  the bytes the unfused "norm, then quantize" sequence produces: fusing changes no byte.
"""

import numpy as np

from .codecs import bf16_to_f64, f64_to_bf16
from .quant import fp8_current_scaling, mxfp8_colwise, mxfp8_rowwise


def _g(gamma_bits, zero_centered):
    g = bf16_to_f64(gamma_bits)
    return g + 1.0 if zero_centered else g


def norm_stats(kind, x_bits, eps):
    """Per-row statistics in fp64: mu (zeros for RMS) and rsigma."""
    x = bf16_to_f64(x_bits)
    mu = np.mean(x, axis=1) if kind == "ln" else np.zeros(x.shape[0])
    xc = x - mu[:, None]
    return mu, 1.0 / np.sqrt(np.mean(xc * xc, axis=1) + eps)


def norm_fwd(kind, x_bits, gamma_bits, beta_bits, eps, zero_centered=False):
    """kind 'rms' or 'ln'. Returns y (fp64), y_bits (bf16), mu (fp32 [R]; zeros for RMS),
    rsigma (fp32 [R])."""
    x = bf16_to_f64(x_bits)
    g = _g(gamma_bits, zero_centered)
    mu, rsigma = norm_stats(kind, x_bits, eps)
    xc = x - mu[:, None]
    y = xc * rsigma[:, None] * g
    if kind == "ln":
        y = y + bf16_to_f64(beta_bits)
    return {"y": y, "y_bits": f64_to_bf16(y), "mu": mu.astype(np.float32), "rsigma": rsigma.astype(np.float32)}


def norm_fwd_quantized(kind, x_bits, gamma_bits, beta_bits, eps, zero_centered=False):
    """The forward plus its quantized outputs: FP8 current scaling and MXFP8 (both copies) of
    the bf16 output."""
    r = norm_fwd(kind, x_bits, gamma_bits, beta_bits, eps, zero_centered)
    r["fp8"] = fp8_current_scaling(r["y_bits"])
    r["mx_row"] = mxfp8_rowwise(r["y_bits"])
    r["mx_col"] = mxfp8_colwise(r["y_bits"])
    return r


def norm_bwd(kind, dz_bits, x_bits, mu, rsigma, gamma_bits, zero_centered=False):
    """Returns dx (fp64 [R, C]), dgamma and dbeta (fp64 [C]; dbeta zeros for RMS)."""
    dz = bf16_to_f64(dz_bits)
    x = bf16_to_f64(x_bits)
    g = _g(gamma_bits, zero_centered)
    mu = np.asarray(mu, np.float64) if kind == "ln" else np.zeros(x.shape[0])
    rs = np.asarray(rsigma, np.float64)[:, None]
    xhat = (x - mu[:, None]) * rs
    d = dz * g
    inner = d - xhat * np.mean(d * xhat, axis=1, keepdims=True)
    if kind == "ln":
        inner = inner - np.mean(d, axis=1, keepdims=True)
    dx = rs * inner
    dgamma = np.sum(dz * xhat, axis=0)
    dbeta = np.sum(dz, axis=0) if kind == "ln" else np.zeros(x.shape[1])
    return {"dx": dx, "dgamma": dgamma, "dbeta": dbeta}

"""Seeded synthetic inputs for the scaled linear, shared by the tests, the bench and the smoke check.

This module only draws random numbers and stores them in the dtypes the
library consumes. It holds none of the method's arithmetic, so the CPU oracle
and the HIP path can both be fed from it without sharing code.

Recipe (every workload):

* One ``numpy.random.Generator`` per tensor, spawned from
  ``SeedSequence(seed)`` in a fixed order, so a tensor's values do not depend
  on which other tensors are drawn.
* Normal values are drawn in float32 as ``std * standard_normal`` and rounded
  to bf16 with round-to-nearest-even (torch's CPU cast); bf16 tensors are
  returned as uint16 bit patterns.
* "1% outliers x50": an independent Bernoulli(0.01) mask multiplies the
  selected float32 values by 50 before the bf16 rounding.
* Probabilities are float32 U(0, 1).
* Group split sizes are Dirichlet(alpha=1) shares of the token count turned
  into integers by largest remainder: floor every share, then add one token to
  the groups with the largest fractional parts (ties to the lower group index)
  until the sizes sum to the token count.
"""

import numpy as np
import torch

# Stream order within a workload; fixed so every consumer sees the same values.
STREAMS = ("x", "w", "residual", "dy", "p", "splits", "outliers_x", "outliers_w",
           "outliers_dy", "w2", "dout", "gamma")


def streams(seed):
    """Dict name -> Generator, one independent stream per tensor."""
    kids = np.random.SeedSequence(seed).spawn(len(STREAMS))
    return {n: np.random.default_rng(k) for n, k in zip(STREAMS, kids)}


def f32_to_bf16_bits(a):
    """Round float32 values to bf16 (nearest-even) and return the uint16 bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def normal_bf16(rng, shape, std, outlier_rng=None, outlier_rate=0.01, outlier_mult=50.0):
    """bf16 bits of std * N(0, 1), optionally with Bernoulli(outlier_rate) values times outlier_mult."""
    a = rng.standard_normal(size=shape, dtype=np.float32)
    a *= np.float32(std)
    if outlier_rng is not None:
        mask = outlier_rng.random(size=shape, dtype=np.float32) < np.float32(outlier_rate)
        a[mask] *= np.float32(outlier_mult)
    return f32_to_bf16_bits(a)


def dirichlet_splits(rng, groups, tokens):
    """int64 [groups] split sizes summing to ``tokens`` (Dirichlet(1) + largest remainder)."""
    share = rng.dirichlet(np.ones(groups)) * tokens
    base = np.floor(share).astype(np.int64)
    frac = share - base
    short = int(tokens - base.sum())
    order = sorted(range(groups), key=lambda g: (-frac[g], g))
    for g in order[:short]:
        base[g] += 1
    return base


def dense(M, N, K, *, x_std=1.0, w_std=0.02, res_std=1.0, dy_std=1e-2, outliers=False,
          seed=0, with_dy=True, with_residual=True):
    """Inputs of one dense scaled linear: x [M, K], W [N, K], residual [M, N], dy [M, N] (bf16 bits)."""
    r = streams(seed)
    out = {
        "x": normal_bf16(r["x"], (M, K), x_std, r["outliers_x"] if outliers else None),
        "w": normal_bf16(r["w"], (N, K), w_std, r["outliers_w"] if outliers else None),
    }
    if with_residual:
        out["residual"] = normal_bf16(r["residual"], (M, N), res_std)
    if with_dy:
        out["dy"] = normal_bf16(r["dy"], (M, N), dy_std, r["outliers_dy"] if outliers else None)
    return out


def norm_gamma(C, seed=0, std=0.1):
    """bf16 bits of a normalization weight gamma [C] = 1 + std * N(0, 1) (drawn in float32)."""
    a = streams(seed)["gamma"].standard_normal(size=C, dtype=np.float32) * np.float32(std) + np.float32(1.0)
    return f32_to_bf16_bits(a)


def grouped(T, G, hidden, ffn, *, seed=0, x_std=1.0, w_std=0.02, dout_std=1e-2, splits=None, gated=True):
    """Inputs of the grouped MLP: x [T, hidden], W1 [G, 2*ffn, hidden] (gated activation; [G, ffn,
    hidden] otherwise), W2 [G, hidden, ffn], p [T] float32 U(0,1), dout [T, hidden], splits [G] int64."""
    r = streams(seed)
    if splits is None:
        splits = dirichlet_splits(r["splits"], G, T)
    return {
        "x": normal_bf16(r["x"], (T, hidden), x_std),
        "w1": normal_bf16(r["w"], (G, (2 if gated else 1) * ffn, hidden), w_std),
        "w2": normal_bf16(r["w2"], (G, hidden, ffn), w_std),
        "p": r["p"].random(size=T, dtype=np.float32),
        "dout": normal_bf16(r["dout"], (T, hidden), dout_std),
        "splits": np.asarray(splits, dtype=np.int64),
    }


# The workloads (sizes, distributions, alpha) of the fused scaled linear.
WORKLOADS = {
    "bf16_fwd_256x512x512": dict(kind="dense", fmt="bf16", M=256, N=512, K=512, alpha=0.5,
                                 passes=("fwd",)),
    "bf16_fwdbwd_4096": dict(kind="dense", fmt="bf16", M=4096, N=4096, K=4096, alpha=0.125,
                             passes=("fwd", "dgrad", "wgrad")),
    "fp8_tensor_fwdbwd_8192x14336x4096": dict(kind="dense", fmt="fp8", M=8192, N=14336, K=4096,
                                              alpha=0.5, passes=("fwd", "dgrad", "wgrad")),
    "mxfp8_fwdbwd_16384x8192x8192": dict(kind="dense", fmt="mxfp8", M=16384, N=8192, K=8192,
                                         alpha=0.25, outliers=True, w_std=1.0, dy_std=1.0,
                                         passes=("fwd", "dgrad", "wgrad")),
    "grouped_swiglu_mlp_T65536_G8": dict(kind="grouped", fmt="bf16", T=65536, G=8, hidden=2048,
                                         ffn=2048, alpha=1.0),
    # the same grouped MLP on MXFP8 operands, fc1's activation quantized for fc2 (forward only,
    # and forward + backward)
    "mxfp8_grouped_swiglu_mlp_fwd_T65536_G8": dict(kind="grouped", fmt="mxfp8", T=65536, G=8, hidden=2048,
                                                   ffn=2048, alpha=1.0, passes=("fwd",)),
    "mxfp8_grouped_swiglu_mlp_T65536_G8": dict(kind="grouped", fmt="mxfp8", T=65536, G=8, hidden=2048,
                                               ffn=2048, alpha=1.0, passes=("fwd", "bwd")),
    # and on FP8 E4M3 operands with current scaling per group (forward + backward)
    "fp8_grouped_swiglu_mlp_T65536_G8": dict(kind="grouped", fmt="fp8", T=65536, G=8, hidden=2048, ffn=2048,
                                             alpha=1.0, passes=("fwd", "bwd")),
    # the bf16 grouped MLP with the scaled squared-ReLU activation (fc1 has ffn outputs, no gate)
    "grouped_srelu_mlp_T65536_G8": dict(kind="grouped", fmt="bf16", T=65536, G=8, hidden=2048, ffn=2048,
                                        alpha=1.0, act="srelu"),
    # and on MXFP8 / FP8 (per-group current scaling) operands (forward + backward)
    "mxfp8_grouped_srelu_mlp_T65536_G8": dict(kind="grouped", fmt="mxfp8", T=65536, G=8, hidden=2048, ffn=2048,
                                              alpha=1.0, act="srelu", passes=("fwd", "bwd")),
    "fp8_grouped_srelu_mlp_T65536_G8": dict(kind="grouped", fmt="fp8", T=65536, G=8, hidden=2048, ffn=2048,
                                            alpha=1.0, act="srelu", passes=("fwd", "bwd")),
    # the bf16 grouped MLP with the clamped SwiGLU (gate clamped above at 7 through u * sigmoid(1.702 u), up
    # half clamped to [-7, 7] and offset by one)
    "grouped_clamped_swiglu_mlp_T65536_G8": dict(kind="grouped", fmt="bf16", T=65536, G=8, hidden=2048,
                                                 ffn=2048, alpha=1.0, act=("clamped_swiglu", 7.0, 1.702)),
    # the MXFP8 linear fed by an RMSNorm whose kernel writes the MXFP8 operand (forward + backward,
    # the norm's backward included); x, W, dy as in the MXFP8 linear above, gamma = 1 + 0.1 N(0,1)
    "rmsnorm_mxfp8_linear_fwdbwd_16384x8192x8192": dict(kind="dense", fmt="mxfp8", M=16384, N=8192, K=8192,
                                                        alpha=0.25, outliers=True, w_std=1.0, dy_std=1.0,
                                                        norm="rms", eps=1e-5, passes=("fwd", "dgrad", "wgrad")),
}


def workload_inputs(name, seed=0):
    """Inputs of one named workload at its full size."""
    w = WORKLOADS[name]
    if w["kind"] == "dense":
        d = dense(w["M"], w["N"], w["K"], w_std=w.get("w_std", 0.02),
                  dy_std=w.get("dy_std", 1e-2), outliers=w.get("outliers", False), seed=seed,
                  with_dy="dgrad" in w["passes"])
        if w.get("norm"):
            d["gamma"] = norm_gamma(w["K"], seed=seed)
        return d
    return grouped(w["T"], w["G"], w["hidden"], w["ffn"], seed=seed, gated=w.get("act", "swiglu") != "srelu")

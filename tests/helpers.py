"""Test helpers: moving seeded inputs to the device and comparing against the oracle."""

import numpy as np
import torch

# Parity bars: |gpu - ref| <= tau * (|ref| + 1) per element.
TAU_BF16 = 2e-2
TAU_FP8 = 6e-2


def dev_bf16(bits):
    """uint16 bf16 bit patterns (numpy) -> torch bf16 tensor on cuda:0."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host_f64(t):
    """Any device tensor -> numpy float64 (bf16 decoded by torch)."""
    return t.detach().to("cpu").double().numpy()


def host_u8(t):
    return t.detach().to("cpu").contiguous().view(torch.uint8).numpy()


def host_bits(t):
    """bf16 tensor -> uint16 bit patterns."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def assert_close(gpu, ref, tau, what="", rel_tight=2.0 ** -8, abs_tight=1e-2):
    """Both the parity bar and a tighter bar scaled by the output's RMS.

    The tight bar allows one bf16 rounding of the output (2^-8 relative) plus
    ``abs_tight`` of the RMS for accumulation-order and intermediate roundings;
    it fails e.g. an all-zero output, which the parity bar alone would
    accept for outputs much smaller than 1.
    """
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite output"
    err = np.abs(gpu - ref)
    bound = tau * (np.abs(ref) + 1.0)
    if not np.all(err <= bound):
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: parity bar broken at {i}: gpu={gpu[i]} ref={ref[i]}")
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    tight = rel_tight * np.abs(ref) + abs_tight * rms
    if not np.all(err <= tight):
        i = np.unravel_index(np.argmax(err - tight), err.shape)
        raise AssertionError(f"{what}: tight bar broken at {i}: gpu={gpu[i]} ref={ref[i]} rms={rms}")
    return float(np.max(err / (np.abs(ref) + 1.0))) if ref.size else 0.0


def assert_close_requantized(gpu, ref, tau, what="", rel_tight=2.0 ** -3, abs_tight=0.1, max_frac=1e-4,
                             flip_rms=0.5):
    """A GEMM output whose operand is a bf16 intermediate quantized to E4M3 on each side (the
    GPU's and the oracle's intermediates agree to bf16 rounding, each quantized on its own).
    An element of the two intermediates one bf16 step apart may straddle an E4M3 rounding
    boundary; the two sides then take neighbouring codes (one step is 2^-3 of the element's
    binade), which moves every output that the element feeds by that step times the other
    operand. So: the parity bar on every element, the tight bar of ``assert_close`` on all
    but ``max_frac`` of them, and those within ``flip_rms`` of the output's RMS."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite output"
    err = np.abs(gpu - ref)
    bound = tau * (np.abs(ref) + 1.0)
    if not np.all(err <= bound):
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: parity bar broken at {i}: gpu={gpu[i]} ref={ref[i]}")
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    bad = err > rel_tight * np.abs(ref) + abs_tight * rms
    assert bad.sum() <= max_frac * bad.size, f"{what}: {bad.sum()} of {bad.size} outside the tight bar"
    assert np.all(err[bad] <= flip_rms * rms), f"{what}: beyond one rounding flip ({err.max()} vs rms {rms})"


def assert_mx_dequant_close(gpu, ref, what=""):
    """Dequantized MXFP8 values of two activations that agree to rounding (the GPU's and the
    oracle's), each quantized on its own: within the FP8 bar element by element, except in a
    block whose maximum sits on a power of two in one and just below it in the other. Such a
    block takes shared exponents one apart (and the larger element of the lower one may
    saturate at 448), so its values may differ by up to one E4M3 step of the larger exponent;
    at most 1 in 1000 elements may do so."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    err = np.abs(gpu - ref)
    bad = err > TAU_FP8 * (np.abs(ref) + 1.0)
    assert bad.mean() <= 1e-3, f"{what}: {bad.sum()} of {bad.size} outside the FP8 bar"
    assert np.all(err[bad] <= 0.25 * np.abs(ref[bad]) + 0.05), f"{what}: beyond one shared-exponent step"



def clamp_settled_h(gpu_dh, dh, gy, h, p, act, delta=2.0 ** -16):
    """The oracle's pre-activation for a clamped SwiGLU backward, with its ambiguous pass-through
    decisions settled the way the kernel took them.

    Both sides decide on the saved bf16 pre-activation (the oracle on its fp64 h rounded to
    bf16, the kernel on its fp32 h rounded to bf16). Where the fp64 h lies within ``delta`` of
    the bf16 rounding midpoint just above the limit (the gate, a) or its magnitude does (the up
    half, b), an fp32 accumulation may round to the other side, and both decisions are correct.
    For those elements only, h moves to the bf16 value on the other side of the decision when
    the oracle's gradient from there (``dh`` is the oracle's from ``h``, ``gy`` its incoming
    gradient) is the closer one to the kernel's ``gpu_dh``; the clamped values, and so the
    forward and dprobs, are the same on both sides. Returns (h, number of ambiguous elements);
    the caller reruns the oracle's backward from that h."""
    from oracle.codecs import bf16_to_f64, f64_to_bf16
    from oracle.grouped import scaled_clamped_swiglu_bwd
    _, limit, alpha = act
    u = 2.0 ** (np.floor(np.log2(limit)) - 7)                 # bf16 spacing at the limit
    mid = limit + u / 2
    F = h.shape[1] // 2
    hb = bf16_to_f64(f64_to_bf16(h))
    amb = np.concatenate([np.abs(h[:, :F] - mid) <= delta, np.abs(np.abs(h[:, F:]) - mid) <= delta], axis=1)
    other = np.where(np.abs(hb) <= limit, limit + u, limit) * np.where(h < 0, -1.0, 1.0)
    alt, _ = scaled_clamped_swiglu_bwd(gy, np.where(amb, other, hb), p, limit, alpha)
    gpu_dh = np.asarray(gpu_dh, np.float64)
    take = amb & (np.abs(gpu_dh - alt) < np.abs(gpu_dh - dh))
    return np.where(take, other, h), int(amb.sum())


def assert_oracle_mx_rowwise(bits, q, s, what=""):
    """MXFP8 bytes written by a fused epilogue equal the oracle's rowwise MXFP8 of the GPU's own
    bf16 tensor (``bits``, uint16): the quantization is a function of the bf16 values alone, so
    the codes and E8M0 scales must agree bit for bit."""
    from oracle import quant
    rq, rs = quant.mxfp8_rowwise(np.asarray(bits, np.uint16))
    q, s = np.asarray(q), np.asarray(s)
    assert q.shape == rq.shape and s.shape == rs.shape, (what, q.shape, rq.shape, s.shape, rs.shape)
    if not np.array_equal(s, rs):
        i = np.argwhere(s != rs)[0]
        raise AssertionError(f"{what}: E8M0 scale {tuple(i)} = {s[tuple(i)]}, oracle {rs[tuple(i)]}")
    if not np.array_equal(q, rq):
        i = np.argwhere(q != rq)[0]
        raise AssertionError(f"{what}: code {tuple(i)} = {q[tuple(i)]:#04x}, oracle {rq[tuple(i)]:#04x}")


def assert_oracle_fp8_grouped(bits, got, c, pad, what=""):
    """Per-group FP8 current scaling written by the GPU (``got``: amax, scale, scale_inv, q and,
    if present, q_t in the aligned token layout) equals the oracle's applied to the GPU's own
    bf16 tensor ``bits``: amax, scale and scale_inv as fp32 bit patterns, every code."""
    from oracle import quant
    ld = None if got.get("q_t") is None else got["q_t"].shape[1]
    ref = quant.fp8_current_scaling_grouped(np.asarray(bits, np.uint16), c, pad, ld)
    for k in ("amax", "scale", "scale_inv"):
        g = got[k].detach().cpu().numpy().astype(np.float32)
        assert np.array_equal(g.view(np.uint32), ref[k].astype(np.float32).view(np.uint32)), (what, k, g, ref[k])
    lo, hi = int(c[0]), int(c[-1])
    assert np.array_equal(host_u8(got["q"])[lo:hi], ref["q"][lo:hi]), f"{what}: codes differ from the oracle's"
    if ld is not None:
        P = int(pad[-1])
        assert np.array_equal(host_u8(got["q_t"])[:, :P], ref["q_t"][:, :P]), f"{what}: transposed codes differ"

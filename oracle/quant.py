"""Quantizers: FP8 E4M3 with per-tensor current scaling, and MXFP8.

Test infrastructure (see the package docstring): never used by the product path.

Per-tensor current scaling follows "NVIDIA TransformerEngine PyTorch Ext
Normalization", Description: for current scaling the amax of the tensor is
computed first, then the tensor is quantized with a scale derived from it.
The scale is 448/amax (448 is the E4M3 maximum). The pages give no formula
for the inverse scale or for degenerate amax values; the readings taken are:

* ``scale = fp32(448 / amax)`` with IEEE correctly rounded fp32 division;
  ``amax == 0`` gives ``scale = 1``; a quotient that overflows fp32 is clamped
  to the largest finite fp32 value.
* ``scale_inv = fp32(1 / scale)``.
* ``q = e4m3(fp32(x * scale))``: one fp32 multiply, rounded, then converted.

MXFP8 ("core.tensor_parallel.inference_layers", ``_apply_linear`` with an
MXFP8Tensor weight) stores E4M3 data with one E8M0 scale per 32 consecutive
elements along the contraction dimension. The pages give no rule for the
shared exponent; the plainest published one is OCP MX v1.0 section 6.3:
``X = floor(log2(max|v|)) - emax_elem`` with ``emax_elem = 8`` for E4M3,
clamped to the E8M0 range [-127, 127]; elements are ``e4m3(v / 2^X)`` with
saturation. An all-zero block takes X = -127 (the smallest scale).
"""

import numpy as np

from .codecs import bf16_to_f32, e4m3_encode, e4m3_decode, e8m0_decode, E4M3_MAX

MX_BLOCK = 32
E4M3_EMAX = 8          # floor(log2(448))
_FLT_MAX = np.float32(np.finfo(np.float32).max)


# ------------------------------------------------- per-tensor (current) -----
def amax(x_bits):
    """max_i |x_i| of a bf16 tensor, as float32 (exact: a max has no rounding)."""
    x = bf16_to_f32(x_bits)
    if x.size == 0:
        return np.float32(0.0)
    return np.float32(np.max(np.abs(x)))


def fp8_scale(amax_f32):
    """scale = fp32(448 / amax), with the degenerate readings of the module docstring."""
    a = np.float32(amax_f32)
    if a == 0:
        return np.float32(1.0)
    with np.errstate(over="ignore", divide="ignore"):
        s = np.float32(E4M3_MAX) / a             # numpy fp32 '/' is IEEE RN division
    if not np.isfinite(s):
        s = _FLT_MAX
    return np.float32(s)


def fp8_scale_inv(scale_f32):
    """scale_inv = fp32(1 / scale)."""
    return np.float32(np.float32(1.0) / np.float32(scale_f32))


def fp8_quantize_with_scale(x_bits, scale_f32):
    """E4M3 codes of fp32(x * scale) for every element of a bf16 tensor."""
    with np.errstate(over="ignore"):
        prod = bf16_to_f32(x_bits) * np.float32(scale_f32)   # fp32 multiply, RN
    return e4m3_encode(prod)


def fp8_current_scaling(x_bits):
    """Full per-tensor current scaling of a bf16 matrix [R, C].

    Returns a dict with ``amax``, ``scale``, ``scale_inv`` (float32 scalars),
    ``q`` (uint8 [R, C]) and ``q_t`` (uint8 [C, R], the transpose of ``q``;
    the scale is per tensor, so orientation changes no byte).
    """
    a = amax(x_bits)
    s = fp8_scale(a)
    q = fp8_quantize_with_scale(x_bits, s)
    return {"amax": a, "scale": s, "scale_inv": fp8_scale_inv(s), "q": q,
            "q_t": np.ascontiguousarray(q.T)}


def fp8_dequantize(q, scale_inv_f32):
    """Exact fp64 value each code stands for: e4m3(q) * scale_inv."""
    return e4m3_decode(q) * np.float64(np.float32(scale_inv_f32))


# ------------------------------------------------------------- MXFP8 --------
def mx_shared_exponent(block_amax_f32):
    """OCP MX v1.0 section 6.3 shared exponent of blocks with the given amax.

    X = floor(log2(amax)) - 8, clamped to [-127, 127]; amax == 0 gives -127.
    floor(log2(a)) of a positive float is read off frexp exactly.
    """
    a = np.asarray(block_amax_f32, dtype=np.float32).astype(np.float64)
    _, e2 = np.frexp(np.where(a > 0, a, 1.0))      # a = f * 2^e2, f in [0.5, 1)
    x = (e2.astype(np.int64) - 1) - E4M3_EMAX
    x = np.where(a > 0, x, -127)
    return np.clip(x, -127, 127)


def mxfp8_rowwise(x_bits):
    """MXFP8 with blocks of 32 along the last dim of a bf16 matrix [R, C].

    Returns (q uint8 [R, C], s uint8 [R, C/32]) with s the E8M0 byte X + 127.
    C must be a multiple of 32.
    """
    x = bf16_to_f32(x_bits)
    R, C = x.shape
    if C % MX_BLOCK:
        raise ValueError("MXFP8 needs the blocked dimension to be a multiple of 32")
    blocks = x.reshape(R, C // MX_BLOCK, MX_BLOCK)
    bamax = np.max(np.abs(blocks), axis=2) if x.size else np.zeros((R, 0), np.float32)
    X = mx_shared_exponent(bamax)                                   # [R, C/32]
    inv = np.ldexp(np.float32(1.0), -X).astype(np.float32)          # 2^-X, exact in fp32
    with np.errstate(over="ignore", under="ignore"):
        scaled = (blocks * inv[:, :, None]).astype(np.float32)      # exact power-of-two scaling
    q = e4m3_encode(scaled).reshape(R, C)
    return q, (X + 127).astype(np.uint8)


def mxfp8_colwise(x_bits):
    """MXFP8 with blocks of 32 along the first dim, stored transposed.

    Defined as the rowwise quantization of x^T: returns (q_colT uint8 [C, R],
    s_colT uint8 [C, R/32]). This is the operand a GEMM contracting over the
    rows of x consumes.
    """
    return mxfp8_rowwise(np.ascontiguousarray(np.asarray(x_bits, dtype=np.uint16).T))


def mx_dequantize(q, s):
    """Exact fp64 value: e4m3(q) * 2^(s-127), the scale repeated over each block of 32."""
    q = np.asarray(q)
    R, C = q.shape
    sc = np.repeat(e8m0_decode(s), MX_BLOCK, axis=1)[:, :C]
    return e4m3_decode(q) * sc


# ------------------------------------------- MXFP8 blocked along grouped tokens -----
# A wgrad contracts over the tokens of one group, so its MXFP8 operands carry blocks of 32
# along tokens. The pages quantize each group's slice of the grouped tensor as a tensor of
# its own ("Activation + GroupedLinear Fusion for MOE and other MOE optimizations",
# Description: the activation is followed by a group quantize; the split sizes travel with
# it). The reading taken here: a group's first block starts at the group's first token, a
# group whose length is not a multiple of 32 ends in a short block (its missing elements
# count as zeros, which leave the block's amax unchanged), and in the stored operand each
# group starts at a multiple of MX_TOKEN_ALIGN tokens, the space up to the next group
# holding zero codes under all-zero blocks (scale byte 0).
MX_TOKEN_ALIGN = 128


def mx_group_layout(offsets, T, align=MX_TOKEN_ALIGN):
    """Token ranges and aligned positions of the groups of a token-blocked MXFP8 operand.

    offsets [G+1] are first made a non-decreasing sequence inside [0, T], the way every
    grouped call reads them: ``c[0] = clip(offsets[0], 0, T)`` and
    ``c[g] = max(c[g-1], min(offsets[g], T))``. Group g owns tokens ``c[g] .. c[g+1]-1``.
    Its position in the stored operand is ``pad[g]``, with ``pad[0] = 0`` and
    ``pad[g+1] = pad[g] + ceil((c[g+1] - c[g]) / align) * align``.
    Returns (c, pad), int64 [G+1] each.
    """
    off = [int(v) for v in np.asarray(offsets, np.int64)]
    c, pad = [], [0]
    prev = 0
    for v in off:
        v = min(v, int(T))
        prev = max(prev, v)
        c.append(prev)
    for g in range(len(off) - 1):
        n = c[g + 1] - c[g]
        pad.append(pad[g] + -(-n // align) * align)
    return np.asarray(c, np.int64), np.asarray(pad, np.int64)


def mxfp8_colwise_grouped(x_bits, c, pad, ld):
    """MXFP8 of a bf16 matrix [T, C] with blocks of 32 along the tokens of each group.

    Each group's rows ``c[g] .. c[g+1]-1``, followed by zero rows up to its aligned length
    ``pad[g+1] - pad[g]``, are quantized columnwise on their own (``mxfp8_colwise``) and stored
    at columns ``pad[g] ..`` of the transposed operand. Returns (q [C, ld] uint8,
    s [C, ld/32] uint8); columns from pad[G] to ld are left zero.
    """
    x = np.asarray(x_bits, np.uint16)
    C = x.shape[1]
    if ld % MX_BLOCK or ld < pad[-1]:
        raise ValueError("ld must be a multiple of 32 and hold every group")
    q = np.zeros((C, ld), np.uint8)
    s = np.zeros((C, ld // MX_BLOCK), np.uint8)
    for g in range(len(c) - 1):
        n, L = int(c[g + 1] - c[g]), int(pad[g + 1] - pad[g])
        if L == 0:
            continue
        rows = np.zeros((L, C), np.uint16)                  # bf16 +0 beyond the group's tokens
        rows[:n] = x[c[g]:c[g + 1]]
        qg, sg = mxfp8_colwise(rows)
        q[:, pad[g]:pad[g] + L] = qg
        s[:, pad[g] // MX_BLOCK:(pad[g] + L) // MX_BLOCK] = sg
    return q, s


# ---------------------------------------- FP8 current scaling per group ------
# A group quantize hands each group's slice of a grouped tensor (and each expert's weight) a
# quantizer of its own ("Activation + GroupedLinear Fusion for MOE and other MOE
# optimizations", Description: grouped scaled activations followed by a group quantize; Greptile
# Summary: fp8_current_scaling in the grouped-MLP test matrix). With current scaling that
# means one amax, scale and scale_inv per group. The transposed copy a grouped wgrad reads uses
# the aligned layout of ``mx_group_layout`` (zero codes between groups).
def fp8_current_scaling_grouped(x_bits, c, pad, ld=None):
    """Per-group FP8 current scaling of a bf16 matrix [T, C] with group rows c[g] .. c[g+1]-1.

    Returns amax, scale, scale_inv (float32 [G]), q (uint8 [T, C]; rows outside every group
    are left 0) and, when ``ld`` is given, q_t (uint8 [C, ld]): group g's row t at column
    pad[g] + t - c[g], zeros elsewhere.
    """
    x = np.asarray(x_bits, np.uint16)
    T, C = x.shape
    G = len(c) - 1
    amax_g = np.zeros(G, np.float32)
    scale_g = np.zeros(G, np.float32)
    sinv_g = np.zeros(G, np.float32)
    q = np.zeros((T, C), np.uint8)
    q_t = None if ld is None else np.zeros((C, ld), np.uint8)
    for g in range(G):
        lo, hi = int(c[g]), int(c[g + 1])
        a = amax(x[lo:hi])
        s = fp8_scale(a)
        amax_g[g], scale_g[g], sinv_g[g] = a, s, fp8_scale_inv(s)
        qg = fp8_quantize_with_scale(x[lo:hi], s)
        q[lo:hi] = qg
        if q_t is not None:
            q_t[:, int(pad[g]):int(pad[g]) + (hi - lo)] = qg.T
    return {"amax": amax_g, "scale": scale_g, "scale_inv": sinv_g, "q": q, "q_t": q_t}

"""Python binding of libsge, the fused scaled linear for MI355X (gfx950).

Argument marshalling only: every step runs in the HIP kernels of
``libsge.so``. Tensors are torch tensors on the current HIP device; calls are
enqueued on ``torch.cuda.current_stream()`` unless a stream is given. The
library is loaded after torch so both share one HIP runtime. There is no CPU
fallback: importing this package fails loudly when the library is missing.

Names follow the C ABI in ``include/sge.h``.
"""

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsge.so")

if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is missing: build it with `python -m scaled_gemm_epilogues_amd.build`")

_lib = ctypes.CDLL(_LIB_PATH)

# status codes
OK, ERR_NULL, ERR_SHAPE, ERR_FORMAT, ERR_ALIGN, ERR_ALIAS, ERR_WORKSPACE, ERR_ARG, ERR_HIP = range(9)
# operand formats
FMT_BF16, FMT_E4M3, FMT_MXFP8 = 0, 1, 2
# grouped epilogues
EPI_NONE, EPI_SCALED_SWIGLU, EPI_DSCALED_SWIGLU, EPI_SCALED_SRELU, EPI_DSCALED_SRELU = 0, 1, 2, 3, 4
EPI_SCALED_CLAMPED_SWIGLU, EPI_DSCALED_CLAMPED_SWIGLU = 5, 6
# normalizations
NORM_RMS, NORM_LAYER = 0, 1

EXPORTED = (
    "sge_abi_version", "sge_status_string", "sge_last_error_message",
    "sge_linear_scale_add_fwd", "sge_linear_scale_bwd",
    "sge_quantize_fp8_amax_workspace_size", "sge_quantize_fp8_amax", "sge_quantize_fp8_amax_noalloc",
    "sge_quantize_mxfp8",
    "sge_splits_to_offsets", "sge_grouped_linear_fwd", "sge_grouped_linear_fwd_mxfp8",
    "sge_grouped_linear_bwd_workspace_size", "sge_grouped_linear_bwd",
    "sge_scaled_swiglu_fwd", "sge_scaled_swiglu_bwd",
    "sge_mx_token_capacity", "sge_mx_group_layout", "sge_quantize_mxfp8_grouped",
    "sge_grouped_linear_dgrad_mxfp8", "sge_grouped_linear_wgrad_mxfp8",
    "sge_quantize_fp8_grouped_workspace_size", "sge_quantize_fp8_grouped", "sge_grouped_linear_fwd_fp8",
    "sge_grouped_linear_dgrad_fp8", "sge_grouped_linear_wgrad_fp8",
    "sge_norm_fwd_workspace_size", "sge_norm_fwd", "sge_norm_bwd_workspace_size", "sge_norm_bwd",
    "sge_grouped_mlp_fwd", "sge_grouped_mlp_bwd_workspace_size", "sge_grouped_mlp_bwd",
)


class SgeOperand(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p), ("outer", ctypes.c_int64), ("inner", ctypes.c_int64),
        ("ld", ctypes.c_int64), ("inner_contiguous", ctypes.c_int32), ("format", ctypes.c_int32),
        ("scale_inv", ctypes.c_void_p), ("mx_scale", ctypes.c_void_p), ("mx_ld", ctypes.c_int64),
    ]


class SgeActParams(ctypes.Structure):
    """Clamped SwiGLU parameters: limit (the clamp bound) and alpha (the gate's sigmoid slope)."""
    _fields_ = [("limit", ctypes.c_float), ("alpha", ctypes.c_float)]


def _act(act):
    """(limit, alpha) -> a pointer to SgeActParams (None -> NULL)."""
    if act is None:
        return None
    limit, alpha = act
    return ctypes.pointer(SgeActParams(float(limit), float(alpha)))


class SgeError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{_lib.sge_status_string(status).decode()}: {message}")
        self.status = status


_vp, _i64, _i32, _f32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
_OP = ctypes.POINTER(SgeOperand)
_ACT = ctypes.POINTER(SgeActParams)
_SIGS = {
    "sge_abi_version": ([], ctypes.c_int),
    "sge_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "sge_last_error_message": ([], ctypes.c_char_p),
    "sge_linear_scale_add_fwd": ([_OP, _OP, _vp, _i64, _f32, _i32, _vp], ctypes.c_int),
    "sge_linear_scale_bwd": ([_OP, _OP, _OP, _OP, _vp, _i64, _vp, _i64, _f32, _f32, _vp], ctypes.c_int),
    "sge_quantize_fp8_amax_workspace_size": ([_i64, _i64], _sz),
    "sge_quantize_fp8_amax": ([_vp, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "sge_quantize_fp8_amax_noalloc": ([_vp, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp], ctypes.c_int),
    "sge_quantize_mxfp8": ([_vp, _i64, _i64, _vp, _vp, _vp, _vp, _vp], ctypes.c_int),
    "sge_splits_to_offsets": ([_vp, _i32, ctypes.POINTER(_i64), _i32, _i64, _vp, _vp, _vp], ctypes.c_int),
    "sge_grouped_linear_fwd": ([_vp, _vp, _i32, _i64, _i64, _i64, _vp, _f32, _i32, _ACT, _vp, _vp, _vp, _vp],
                               ctypes.c_int),
    "sge_grouped_linear_fwd_mxfp8": ([_vp, _vp, _vp, _vp, _i32, _i64, _i64, _i64, _vp, _f32, _i32, _ACT, _vp, _vp, _vp,
                                      _vp, _vp, _vp, _i64, _vp, _vp, _vp], ctypes.c_int),
    "sge_grouped_linear_bwd_workspace_size": ([_i64, _i64, _i32, _i32], _sz),
    "sge_grouped_linear_bwd": ([_vp, _vp, _vp, _i32, _i64, _i64, _i64, _vp, _f32, _i32, _ACT, _vp, _vp, _vp, _vp,
                                _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "sge_scaled_swiglu_fwd": ([_vp, _vp, _vp, _i64, _i64, _vp], ctypes.c_int),
    "sge_scaled_swiglu_bwd": ([_vp, _vp, _vp, _vp, _vp, _i64, _i64, _vp], ctypes.c_int),
    "sge_mx_token_capacity": ([_i64, _i32], _i64),
    "sge_mx_group_layout": ([_vp, _i32, _i64, _vp, _vp], ctypes.c_int),
    "sge_quantize_mxfp8_grouped": ([_vp, _i64, _i64, _i32, _vp, _i64, _vp, _vp, _vp, _vp, _vp], ctypes.c_int),
    "sge_grouped_linear_dgrad_mxfp8": ([_vp, _vp, _vp, _vp, _i32, _i64, _i64, _i64, _vp, _f32, _i32, _ACT, _vp, _vp,
                                        _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "sge_grouped_linear_wgrad_mxfp8": ([_vp, _vp, _vp, _vp, _i32, _i64, _i64, _vp, _i64, _f32, _vp, _vp],
                                       ctypes.c_int),
    "sge_quantize_fp8_grouped_workspace_size": ([_i32], _sz),
    "sge_quantize_fp8_grouped": ([_vp, _i64, _i64, _i32, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
                                 ctypes.c_int),
    "sge_grouped_linear_fwd_fp8": ([_vp, _vp, _vp, _vp, _i32, _i64, _i64, _i64, _vp, _f32, _i32, _ACT, _vp, _vp, _vp,
                                    _vp, _vp], ctypes.c_int),
    "sge_grouped_linear_dgrad_fp8": ([_vp, _vp, _vp, _vp, _i32, _i64, _i64, _i64, _vp, _f32, _i32, _ACT, _vp, _vp, _vp,
                                      _vp, _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "sge_grouped_linear_wgrad_fp8": ([_vp, _vp, _vp, _vp, _i32, _i64, _i64, _vp, _i64, _f32, _vp, _vp],
                                     ctypes.c_int),
    "sge_norm_fwd_workspace_size": ([_i64, _i64], _sz),
    "sge_norm_fwd": ([_i32, _vp, _vp, _vp, _i64, _i64, _f32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                      _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "sge_norm_bwd_workspace_size": ([_i64, _i64], _sz),
    "sge_grouped_mlp_fwd": ([_vp, _vp, _vp, _i32, _i64, _i64, _i64, _vp, _vp, _vp, _i32, _ACT, _vp, _vp, _vp, _vp, _vp],
                            ctypes.c_int),
    "sge_grouped_mlp_bwd_workspace_size": ([_i64, _i64, _i32, _i32], _sz),
    "sge_grouped_mlp_bwd": ([_vp, _vp, _vp, _vp, _i32, _i64, _i64, _i64, _vp, _i32, _ACT, _vp, _vp, _vp, _vp, _vp, _vp,
                             _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "sge_norm_bwd": ([_i32, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i32, _vp, _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
}
for _name, (_args, _res) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res


def library_path():
    return _LIB_PATH


def abi_version():
    return _lib.sge_abi_version()


def _check(status):
    if status != OK:
        raise SgeError(status, _lib.sge_last_error_message().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


# ----------------------------------------------------------------- operands
class Operand:
    """A GEMM operand: logical [outer, inner] with inner the contraction dim.

    Build with ``Operand.bf16``, ``Operand.e4m3`` or ``Operand.mxfp8``; the
    tensors are kept alive by the object.
    """

    def __init__(self, data, outer, inner, ld, inner_contiguous, fmt, scale_inv=None, mx_scale=None,
                 mx_ld=0):
        self.keep = (data, scale_inv, mx_scale)
        self.c = SgeOperand(data.data_ptr() if data is not None else None, outer, inner, ld,
                            1 if inner_contiguous else 0, fmt,
                            scale_inv.data_ptr() if scale_inv is not None else None,
                            mx_scale.data_ptr() if mx_scale is not None else None, mx_ld)

    @classmethod
    def bf16(cls, t, transposed=False):
        """``t`` stored [outer, inner]; with ``transposed=True`` it is stored [inner, outer]."""
        assert t.dtype == torch.bfloat16 and t.dim() == 2 and t.stride(1) == 1
        if transposed:
            return cls(t, t.shape[1], t.shape[0], t.stride(0), False, FMT_BF16)
        return cls(t, t.shape[0], t.shape[1], t.stride(0), True, FMT_BF16)

    @classmethod
    def e4m3(cls, q, scale_inv):
        """E4M3 bytes ``q`` [outer, inner] (uint8 or float8_e4m3fn) with device fp32[1] scale_inv."""
        assert q.dim() == 2 and q.stride(1) == 1 and q.element_size() == 1
        return cls(q, q.shape[0], q.shape[1], q.stride(0), True, FMT_E4M3, scale_inv=scale_inv)

    @classmethod
    def mxfp8(cls, q, s):
        """E4M3 bytes ``q`` [outer, inner] with E8M0 scales ``s`` [outer, inner/32] (uint8)."""
        assert q.dim() == 2 and q.stride(1) == 1 and s.dim() == 2 and s.stride(1) == 1
        return cls(q, q.shape[0], q.shape[1], q.stride(0), True, FMT_MXFP8, mx_scale=s, mx_ld=s.stride(0))


def _op(o):
    return None if o is None else ctypes.byref(o.c)


# -------------------------------------------------------------- dense path
def linear_scale_add_fwd(x, w, residual, alpha, accumulate=True, stream=None):
    """residual <- residual + alpha * x @ w^T in place (bf16 [M, N]); x, w are Operands."""
    _check(_lib.sge_linear_scale_add_fwd(_op(x), _op(w), _ptr(residual), residual.stride(0), float(alpha),
                                         1 if accumulate else 0, _stream(stream)))
    return residual


def linear_scale_bwd(dg_a, dg_b, wg_a, wg_b, dgrad, wgrad, dgrad_alpha, wgrad_alpha, stream=None):
    """dgrad = a_d * dy @ W and wgrad = a_w * dy^T @ x (operands in GEMM form, see sge.h)."""
    _check(_lib.sge_linear_scale_bwd(_op(dg_a), _op(dg_b), _op(wg_a), _op(wg_b), _ptr(dgrad),
                                     dgrad.stride(0) if dgrad is not None else 0, _ptr(wgrad),
                                     wgrad.stride(0) if wgrad is not None else 0, float(dgrad_alpha),
                                     float(wgrad_alpha), _stream(stream)))


def quantize_fp8_amax_workspace_size(rows, cols):
    return int(_lib.sge_quantize_fp8_amax_workspace_size(rows, cols))


def quantize_fp8_amax(src, q, q_t, amax, scale, scale_inv, workspace, stream=None):
    """Per-tensor current scaling of bf16 ``src`` [rows, cols] into E4M3 ``q`` and/or ``q_t``."""
    rows, cols = src.shape
    _check(_lib.sge_quantize_fp8_amax(_ptr(src), rows, cols, _ptr(q), _ptr(q_t), _ptr(amax), _ptr(scale),
                                      _ptr(scale_inv), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(), _stream(stream)))


def quantize_fp8_amax_noalloc(src, q, q_t, amax, scale, scale_inv, stream=None):
    """``quantize_fp8_amax`` with the amax partials in the library's per-GPU scratch array (no
    workspace; calls overlapping on one GPU race on that array)."""
    rows, cols = src.shape
    _check(_lib.sge_quantize_fp8_amax_noalloc(_ptr(src), rows, cols, _ptr(q), _ptr(q_t), _ptr(amax), _ptr(scale),
                                              _ptr(scale_inv), _stream(stream)))


def quantize_mxfp8(src, q_row=None, s_row=None, q_colT=None, s_colT=None, stream=None):
    """MXFP8 rowwise and/or columnwise (transposed) quantization of bf16 ``src`` [rows, cols]."""
    rows, cols = src.shape
    _check(_lib.sge_quantize_mxfp8(_ptr(src), rows, cols, _ptr(q_row), _ptr(s_row), _ptr(q_colT), _ptr(s_colT),
                                   _stream(stream)))


# ------------------------------------------------------------ grouped path
def splits_to_offsets(splits, multipliers, offsets, expected_total=-1, err_flag=None, stream=None):
    """offsets [n, G+1] int64 = exclusive prefix sum of device ``splits`` [G] times each multiplier."""
    m = (ctypes.c_int64 * len(multipliers))(*[int(v) for v in multipliers])
    _check(_lib.sge_splits_to_offsets(_ptr(splits), splits.numel(), m, len(multipliers), int(expected_total),
                                      _ptr(offsets), _ptr(err_flag), _stream(stream)))


def grouped_linear_fwd(x, w, offsets, out, alpha=1.0, epilogue=EPI_NONE, probs=None, preact=None, act=None,
                       stream=None):
    """Grouped forward: x [T, K], w [G, N, K], offsets [G+1] (device) -> out (and preact for SwiGLU).
    ``act``: (limit, alpha) of the clamped SwiGLU epilogues."""
    G, N, K = w.shape
    T = x.shape[0]
    _check(_lib.sge_grouped_linear_fwd(_ptr(x), _ptr(w), G, T, N, K, _ptr(offsets), float(alpha), epilogue,
                                       _act(act), _ptr(probs), _ptr(out), _ptr(preact), _stream(stream)))


def grouped_linear_fwd_mxfp8(x_q, x_s, w_q, w_s, offsets, out=None, alpha=1.0, epilogue=EPI_NONE, probs=None,
                             preact=None, out_q=None, out_s=None, act=None, layout=None, out_colT_q=None,
                             out_colT_s=None, stream=None):
    """Grouped forward with MXFP8 operands: x_q [T, K] u8 + x_s [T, K/32] u8, w_q [G, N, K] u8 +
    w_s [G, N, K/32] u8 (rowwise). SwiGLU may also emit out_q [T, N/2] + out_s [T, N/64], and
    the token-blocked out_colT_q [N/2, ld] + out_colT_s [N/2, ld/32] with ``layout``."""
    G, N, K = w_q.shape
    T = x_q.shape[0]
    ld_t = 0 if out_colT_q is None else out_colT_q.shape[1]
    _check(_lib.sge_grouped_linear_fwd_mxfp8(_ptr(x_q), _ptr(x_s), _ptr(w_q), _ptr(w_s), G, T, N, K, _ptr(offsets),
                                             float(alpha), epilogue, _act(act), _ptr(probs), _ptr(out), _ptr(preact),
                                             _ptr(out_q), _ptr(out_s), _ptr(layout), ld_t, _ptr(out_colT_q),
                                             _ptr(out_colT_s), _stream(stream)))


def grouped_linear_bwd_workspace_size(T, K, G, epilogue):
    return int(_lib.sge_grouped_linear_bwd_workspace_size(T, K, G, epilogue))


def grouped_linear_bwd(dy, x, w, offsets, alpha=1.0, epilogue=EPI_NONE, preact=None, probs=None, dact=None,
                       dprobs=None, dx=None, dw=None, workspace=None, act=None, stream=None):
    """Grouped backward of one layer (see sge.h): dgrad (optionally through dSwiGLU) and wgrad."""
    G, N, K = w.shape
    T = dy.shape[0]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.sge_grouped_linear_bwd(_ptr(dy), _ptr(x), _ptr(w), G, T, N, K, _ptr(offsets), float(alpha),
                                       epilogue, _act(act), _ptr(preact), _ptr(probs), _ptr(dact), _ptr(dprobs),
                                       _ptr(dx), _ptr(dw), _ptr(workspace), ws_bytes, _stream(stream)))


# ------------------------------------------------ the whole grouped MLP
def grouped_mlp_fwd(x, w1, w2, splits, offsets, probs, preact, act_out, out, activation=EPI_SCALED_SWIGLU,
                    act=None, err_flag=None, stream=None):
    """fc1 -> scaled activation -> fc2 in one call: x [T, H], w1 [G, N1, H], w2 [G, H, F], splits [G]
    (device int64) -> offsets [G+1], preact [T, N1], act_out [T, F], out [T, H]."""
    G, H, F = w2.shape
    T = x.shape[0]
    _check(_lib.sge_grouped_mlp_fwd(_ptr(x), _ptr(w1), _ptr(w2), G, T, H, F, _ptr(splits), _ptr(offsets),
                                    _ptr(err_flag), activation, _act(act), _ptr(probs), _ptr(preact), _ptr(act_out),
                                    _ptr(out), _stream(stream)))


def grouped_mlp_bwd_workspace_size(T, F, G, activation):
    return int(_lib.sge_grouped_mlp_bwd_workspace_size(T, F, G, activation))


def grouped_mlp_bwd(dout, x, w1, w2, offsets, probs, preact, act_out, dpreact, dprobs, dx=None, dw1=None, dw2=None,
                    workspace=None, activation=EPI_SCALED_SWIGLU, act=None, stream=None):
    """Backward of ``grouped_mlp_fwd`` from dout [T, H] with the forward's offsets, preact and act_out."""
    G, H, F = w2.shape
    T = dout.shape[0]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.sge_grouped_mlp_bwd(_ptr(dout), _ptr(x), _ptr(w1), _ptr(w2), G, T, H, F, _ptr(offsets), activation,
                                    _act(act), _ptr(probs), _ptr(preact), _ptr(act_out), _ptr(dpreact), _ptr(dprobs),
                                    _ptr(dx), _ptr(dw1), _ptr(dw2), _ptr(workspace), ws_bytes, _stream(stream)))


# ------------------------------------------------ MXFP8 grouped backward
MX_TOKEN_ALIGN = 128


def mx_token_capacity(T, G):
    """Smallest leading dimension of a token-blocked MXFP8 operand of T tokens in G groups."""
    return int(_lib.sge_mx_token_capacity(int(T), int(G)))


def mx_group_layout(offsets, T, layout, stream=None):
    """layout [2, G+1] int64 (device): clamped offsets and 128-aligned group starts."""
    G = offsets.numel() - 1
    _check(_lib.sge_mx_group_layout(_ptr(offsets), G, int(T), _ptr(layout), _stream(stream)))


def quantize_mxfp8_grouped(src, layout, q_colT, s_colT, q_row=None, s_row=None, stream=None):
    """Token-blocked MXFP8 of bf16 ``src`` [T, cols]: q_colT [cols, ld] + s_colT [cols, ld/32],
    optionally the rowwise copy q_row [T, cols] + s_row [T, cols/32]."""
    T, cols = src.shape
    G = layout.numel() // 2 - 1
    _check(_lib.sge_quantize_mxfp8_grouped(_ptr(src), T, cols, G, _ptr(layout), q_colT.shape[1], _ptr(q_row),
                                           _ptr(s_row), _ptr(q_colT), _ptr(s_colT), _stream(stream)))


def grouped_linear_dgrad_mxfp8(dy_q, dy_s, w_q, w_s, offsets, alpha=1.0, epilogue=EPI_NONE, preact=None,
                               probs=None, dx=None, dact=None, dprobs=None, dact_q=None, dact_s=None,
                               workspace=None, act=None, layout=None, dact_colT_q=None, dact_colT_s=None,
                               stream=None):
    """MXFP8 grouped dgrad: dy_q [T, N] + dy_s [T, N/32] (rowwise), w_q [K, G*N] + w_s [K, G*N/32]
    (W viewed [G*N, K], quantized columnwise). SwiGLU backward writes dact / dact_q+dact_s and dprobs,
    and the token-blocked dact_colT_q [2K, ld] + dact_colT_s [2K, ld/32] with ``layout``."""
    T, N = dy_q.shape
    K = w_q.shape[0]
    G = offsets.numel() - 1
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    ld_t = 0 if dact_colT_q is None else dact_colT_q.shape[1]
    _check(_lib.sge_grouped_linear_dgrad_mxfp8(_ptr(dy_q), _ptr(dy_s), _ptr(w_q), _ptr(w_s), G, T, N, K,
                                               _ptr(offsets), float(alpha), epilogue, _act(act), _ptr(preact),
                                               _ptr(probs), _ptr(dx), _ptr(dact), _ptr(dprobs), _ptr(dact_q),
                                               _ptr(dact_s), _ptr(layout), ld_t, _ptr(dact_colT_q),
                                               _ptr(dact_colT_s), _ptr(workspace), ws_bytes, _stream(stream)))


def grouped_linear_wgrad_mxfp8(dyT_q, dyT_s, xT_q, xT_s, layout, dw, alpha=1.0, stream=None):
    """MXFP8 grouped wgrad from token-blocked operands: dyT [N, ld], xT [K, ld] -> dw [G, N, K] bf16."""
    N, ld = dyT_q.shape
    K = xT_q.shape[0]
    G = layout.numel() // 2 - 1
    _check(_lib.sge_grouped_linear_wgrad_mxfp8(_ptr(dyT_q), _ptr(dyT_s), _ptr(xT_q), _ptr(xT_s), G, N, K,
                                               _ptr(layout), ld, float(alpha), _ptr(dw), _stream(stream)))


# ------------------------------------ FP8 current scaling per group (grouped)
def quantize_fp8_grouped_workspace_size(G):
    return int(_lib.sge_quantize_fp8_grouped_workspace_size(int(G)))


def quantize_fp8_grouped(src, G, amax, scale, scale_inv, workspace=None, layout=None, q=None, q_t=None,
                         amax_in=None, stream=None):
    """Per-group FP8 current scaling of bf16 ``src`` [rows, cols]: groups from ``layout`` [2, G+1]
    or, without one, G equal runs of rows. q [rows, cols] and/or q_t [cols, ld_t]. ``amax_in``: the
    groups' amax reduced by the producing epilogue (skips the amax pass)."""
    rows, cols = src.shape
    ld_t = 0 if q_t is None else q_t.shape[1]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.sge_quantize_fp8_grouped(_ptr(src), rows, cols, int(G), _ptr(layout), ld_t, _ptr(q), _ptr(q_t),
                                         _ptr(amax), _ptr(scale), _ptr(scale_inv), _ptr(amax_in), _ptr(workspace),
                                         ws_bytes, _stream(stream)))


def grouped_linear_fwd_fp8(x_q, x_sinv, w_q, w_sinv, offsets, out, alpha=1.0, epilogue=EPI_NONE, probs=None,
                           preact=None, out_amax=None, act=None, stream=None):
    """Grouped forward on E4M3 operands with one scale_inv per group: x_q [T, K], w_q [G, N, K]."""
    G, N, K = w_q.shape
    T = x_q.shape[0]
    _check(_lib.sge_grouped_linear_fwd_fp8(_ptr(x_q), _ptr(x_sinv), _ptr(w_q), _ptr(w_sinv), G, T, N, K,
                                           _ptr(offsets), float(alpha), epilogue, _act(act), _ptr(probs), _ptr(out),
                                           _ptr(preact), _ptr(out_amax), _stream(stream)))


def grouped_linear_dgrad_fp8(dy_q, dy_sinv, w_qT, w_sinv, offsets, alpha=1.0, epilogue=EPI_NONE, preact=None,
                             probs=None, dx=None, dact=None, dprobs=None, dact_amax=None, workspace=None,
                             act=None, stream=None):
    """E4M3 grouped dgrad: dy_q [T, N], w_qT [K, G*N] (transpose of W viewed [G*N, K])."""
    T, N = dy_q.shape
    K = w_qT.shape[0]
    G = offsets.numel() - 1
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.sge_grouped_linear_dgrad_fp8(_ptr(dy_q), _ptr(dy_sinv), _ptr(w_qT), _ptr(w_sinv), G, T, N, K,
                                             _ptr(offsets), float(alpha), epilogue, _act(act), _ptr(preact),
                                             _ptr(probs), _ptr(dx), _ptr(dact), _ptr(dprobs), _ptr(dact_amax),
                                             _ptr(workspace), ws_bytes, _stream(stream)))


def grouped_linear_wgrad_fp8(dyT_q, dy_sinv, xT_q, x_sinv, layout, dw, alpha=1.0, stream=None):
    """E4M3 grouped wgrad from the transposed copies dyT [N, ld], xT [K, ld] -> dw [G, N, K]."""
    N, ld = dyT_q.shape
    K = xT_q.shape[0]
    G = layout.numel() // 2 - 1
    _check(_lib.sge_grouped_linear_wgrad_fp8(_ptr(dyT_q), _ptr(dy_sinv), _ptr(xT_q), _ptr(x_sinv), G, N, K,
                                             _ptr(layout), ld, float(alpha), _ptr(dw), _stream(stream)))


# ---------------------------------------------------------- normalization
def norm_fwd_workspace_size(rows, cols):
    return int(_lib.sge_norm_fwd_workspace_size(int(rows), int(cols)))


def norm_fwd(kind, x, gamma, y, rsigma, beta=None, mu=None, eps=1e-5, zero_centered=False, fp8=None, mx_row=None,
             mx_col=None, workspace=None, stream=None):
    """RMSNorm / LayerNorm of bf16 ``x`` [rows, cols] into bf16 ``y`` (+ mu, rsigma). ``fp8``: dict of q, q_t,
    amax, scale, scale_inv; ``mx_row`` / ``mx_col``: (q, s) pairs of the MXFP8 copies of y."""
    rows, cols = x.shape
    f = fp8 or {}
    qr, sr = mx_row if mx_row is not None else (None, None)
    qc, sc = mx_col if mx_col is not None else (None, None)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.sge_norm_fwd(int(kind), _ptr(x), _ptr(gamma), _ptr(beta), rows, cols, float(eps), int(zero_centered),
                             _ptr(y), _ptr(mu), _ptr(rsigma), _ptr(f.get("q")), _ptr(f.get("q_t")), _ptr(f.get("amax")),
                             _ptr(f.get("scale")), _ptr(f.get("scale_inv")), _ptr(qr), _ptr(sr), _ptr(qc), _ptr(sc),
                             _ptr(workspace), ws_bytes, _stream(stream)))


def norm_bwd_workspace_size(rows, cols):
    return int(_lib.sge_norm_bwd_workspace_size(int(rows), int(cols)))


def norm_bwd(kind, dz, x, rsigma, gamma, dx, dgamma, workspace, mu=None, dbeta=None, zero_centered=False,
             stream=None):
    """Backward of ``norm_fwd``: dx [rows, cols], dgamma (and LayerNorm dbeta) [cols], all bf16."""
    rows, cols = x.shape
    _check(_lib.sge_norm_bwd(int(kind), _ptr(dz), _ptr(x), _ptr(mu), _ptr(rsigma), _ptr(gamma), rows, cols,
                             int(zero_centered), _ptr(dx), _ptr(dgamma), _ptr(dbeta), _ptr(workspace),
                             workspace.numel() * workspace.element_size(), _stream(stream)))


def scaled_swiglu_fwd(h, probs, y, stream=None):
    T, F2 = h.shape
    _check(_lib.sge_scaled_swiglu_fwd(_ptr(h), _ptr(probs), _ptr(y), T, F2 // 2, _stream(stream)))


def scaled_swiglu_bwd(gy, h, probs, dh, dprobs, stream=None):
    T, F2 = h.shape
    _check(_lib.sge_scaled_swiglu_bwd(_ptr(gy), _ptr(h), _ptr(probs), _ptr(dh), _ptr(dprobs), T, F2 // 2,
                                      _stream(stream)))

"""The C ABI on the host: the library loads, exports what include/sge.h declares, and rejects
bad arguments before touching the GPU (no compute call is made here)."""

import ctypes
import os
import re

import pytest
import torch  # noqa: F401  (loads the HIP runtime libsge links against)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sge.h")


@pytest.fixture(scope="module")
def sge():
    import scaled_gemm_epilogues_amd as m
    return m


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(sge_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_abi(sge):
    assert set(_declared()) == set(sge.EXPORTED)


def test_library_exports_every_declared_symbol(sge):
    lib = ctypes.CDLL(sge.library_path())
    for name in _declared():
        assert hasattr(lib, name), name
    assert sge.abi_version() == 7


def test_status_strings(sge):
    lib = sge._lib
    assert lib.sge_status_string(0) == b"SGE_OK"
    assert lib.sge_status_string(sge.ERR_ALIAS) == b"SGE_ERR_ALIAS"


FAKE = 0x10000            # never dereferenced: every call below fails validation first


def _act_after(fn, epi_index, act=None):
    """Calls ``fn`` with the activation-parameter pointer (``act``, default NULL) inserted right
    after its epilogue argument at ``epi_index``; the remaining arguments keep their positions."""
    return lambda *a: fn(*a[:epi_index + 1], act, *a[epi_index + 1:])



def _op(sge, outer, inner, ld=None, contig=1, fmt=0, data=FAKE, sinv=None, mx=None, mx_ld=0):
    return sge.SgeOperand(data, outer, inner, ld if ld is not None else (inner if contig else outer), contig, fmt,
                          sinv, mx, mx_ld)


def _fwd(sge, x, w, res=FAKE * 64, ld_res=None, alpha=0.5):
    lib = sge._lib
    st = lib.sge_linear_scale_add_fwd(ctypes.byref(x), ctypes.byref(w), res,
                                      ld_res if ld_res is not None else w.outer, alpha, 1, None)
    return st, lib.sge_last_error_message().decode()


def test_forward_validation_errors(sge):
    ok_x, ok_w = _op(sge, 64, 128), _op(sge, 64, 128, data=FAKE * 2)
    st, msg = _fwd(sge, _op(sge, 64, 128, data=None), ok_w)
    assert st == sge.ERR_NULL, msg
    st, msg = _fwd(sge, ok_x, _op(sge, 64, 96, data=FAKE * 2))
    assert st == sge.ERR_SHAPE and "contraction" in msg
    st, _ = _fwd(sge, _op(sge, 64, 100), _op(sge, 64, 100, data=FAKE * 2))
    assert st == sge.ERR_SHAPE                       # bf16 K % 8
    st, _ = _fwd(sge, ok_x, _op(sge, 60, 128, data=FAKE * 2))
    assert st == sge.ERR_SHAPE                       # N % 8
    st, _ = _fwd(sge, _op(sge, 64, 128, data=FAKE + 2), ok_w)
    assert st == sge.ERR_ALIGN
    st, _ = _fwd(sge, ok_x, _op(sge, 64, 128, fmt=1, data=FAKE * 2, sinv=FAKE))
    assert st == sge.ERR_FORMAT                      # mixed formats
    st, _ = _fwd(sge, _op(sge, 64, 128, fmt=1, sinv=None), _op(sge, 64, 128, fmt=1, data=FAKE * 2, sinv=FAKE))
    assert st == sge.ERR_NULL                        # E4M3 needs scale_inv
    st, _ = _fwd(sge, _op(sge, 64, 128, contig=0, fmt=1, sinv=FAKE), _op(sge, 64, 128, fmt=1, data=FAKE * 2,
                                                                        sinv=FAKE))
    assert st == sge.ERR_FORMAT                      # E4M3 must be inner-contiguous
    st, _ = _fwd(sge, _op(sge, 64, 48, fmt=2, mx=FAKE, mx_ld=1), _op(sge, 64, 48, fmt=2, data=FAKE * 2, mx=FAKE,
                                                                       mx_ld=1))
    assert st == sge.ERR_SHAPE                       # MX needs K % 32
    st, _ = _fwd(sge, ok_x, ok_w, res=FAKE)          # residual over x
    assert st == sge.ERR_ALIAS
    st, _ = _fwd(sge, ok_x, ok_w, res=FAKE * 64 + 8)
    assert st == sge.ERR_ALIGN


def test_forward_shape_zero_is_a_noop(sge):
    st, msg = _fwd(sge, _op(sge, 0, 128), _op(sge, 64, 128, data=FAKE * 2))
    assert st == 0, msg


def test_backward_validation_errors(sge):
    lib = sge._lib
    M, N, K = 64, 32, 16
    dy = _op(sge, M, N, data=FAKE)
    wT = _op(sge, K, N, contig=0, data=FAKE * 4)          # W [N, K] read as [K, N]
    dyT = _op(sge, N, M, contig=0, data=FAKE)
    xT = _op(sge, K, M + 8, contig=0, data=FAKE * 8)      # wrong: contraction M+8
    st = lib.sge_linear_scale_bwd(ctypes.byref(dy), ctypes.byref(wT), ctypes.byref(dyT), ctypes.byref(xT),
                                  FAKE * 16, K, FAKE * 32, K, 1.0, 1.0, None)
    assert st == sge.ERR_SHAPE
    xT = _op(sge, K, M, contig=0, data=FAKE * 8)
    st = lib.sge_linear_scale_bwd(ctypes.byref(dy), ctypes.byref(wT), ctypes.byref(dyT), ctypes.byref(xT),
                                  FAKE * 16, K, FAKE, K, 1.0, 1.0, None)          # wgrad over dy
    assert st == sge.ERR_ALIAS


def test_quantizer_validation_errors(sge):
    lib = sge._lib
    assert lib.sge_quantize_fp8_amax_workspace_size(1024, 1024) > 0
    st = lib.sge_quantize_fp8_amax(FAKE, 64, 64, FAKE * 8, None, FAKE * 16, FAKE * 17, FAKE * 18, FAKE * 32, 0, None)
    assert st == sge.ERR_WORKSPACE
    st = lib.sge_quantize_fp8_amax(FAKE, 60, 64, FAKE * 8, None, FAKE * 16, FAKE * 17, FAKE * 18, FAKE * 32, 1 << 20,
                                   None)
    assert st == sge.ERR_SHAPE
    st = lib.sge_quantize_fp8_amax(FAKE, 64, 64, FAKE, None, FAKE * 16, FAKE * 17, FAKE * 18, FAKE * 32, 1 << 20, None)
    assert st == sge.ERR_ALIAS
    st = lib.sge_quantize_mxfp8(FAKE, 64, 48, FAKE * 8, FAKE * 9, None, None, None)
    assert st == sge.ERR_SHAPE
    st = lib.sge_quantize_mxfp8(FAKE, 48, 64, None, None, FAKE * 8, FAKE * 9, None)
    assert st == sge.ERR_SHAPE                       # columnwise needs rows % 32
    st = lib.sge_quantize_mxfp8(FAKE, 64, 64, FAKE * 8, None, None, None, None)
    assert st == sge.ERR_NULL
    st = lib.sge_quantize_mxfp8(FAKE, 64, 64, None, None, None, None, None)
    assert st == sge.ERR_NULL


def test_grouped_validation_errors(sge):
    lib = sge._lib
    m = (ctypes.c_int64 * 1)(1)
    assert lib.sge_splits_to_offsets(FAKE, 0, m, 1, -1, FAKE * 2, None, None) == sge.ERR_ARG
    assert lib.sge_splits_to_offsets(FAKE, 8, m, 9, -1, FAKE * 2, None, None) == sge.ERR_ARG
    assert lib.sge_splits_to_offsets(None, 8, m, 1, -1, FAKE * 2, None, None) == sge.ERR_NULL
    fwd, bwd = _act_after(lib.sge_grouped_linear_fwd, 8), _act_after(lib.sge_grouped_linear_bwd, 9)
    st = fwd(FAKE, FAKE * 64, 8, 100, 136, 64, FAKE * 1024, 1.0, 1, FAKE * 4096, FAKE * 8192, None, None)
    assert st == sge.ERR_SHAPE                       # SwiGLU needs N % 256
    st = fwd(FAKE, FAKE * 64, 8, 100, 256, 64, FAKE * 1024, 1.0, 1, None, FAKE * 8192, None, None)
    assert st == sge.ERR_NULL                        # SwiGLU needs probs
    st = fwd(FAKE, FAKE * 64, 8, 100, 256, 64, FAKE * 1024, 1.0, 7, None, FAKE * 8192, None, None)
    assert st == sge.ERR_ARG
    ws = lib.sge_grouped_linear_bwd_workspace_size(1000, 2048, 8, 2)
    assert ws > 0 and ws % (1000 * 4) == 0
    st = bwd(FAKE, FAKE * 8, FAKE * 64, 8, 1000, 256, 2048, FAKE * 1024, 1.0, 2,
             FAKE * 2048, FAKE * 4096, FAKE * 8192, FAKE * 9000, None, None, None, 0, None)
    assert st == sge.ERR_WORKSPACE


def test_grouped_mxfp8_validation_errors(sge):
    f = _act_after(sge._lib.sge_grouped_linear_fwd_mxfp8, 10)
    G, T, N, K = 4, 100, 512, 256
    x_q, x_s, w_q, w_s, offs, probs = FAKE, FAKE * 64, FAKE * 128, FAKE * 4096, FAKE * 8192, FAKE * 8300
    y, h, yq, ys = FAKE * 10000, FAKE * 20000, FAKE * 30000, FAKE * 40000
    swiglu = sge.EPI_SCALED_SWIGLU
    lay, yT, yTs = FAKE * 50000, FAKE * 60000, FAKE * 70000
    ld_t = sge.mx_token_capacity(T, G)
    ok_args = (x_q, x_s, w_q, w_s, G, T, N, K, offs, 1.0, swiglu, probs, y, h, yq, ys, lay, ld_t, yT, yTs, None)
    assert f(*((None,) + ok_args[1:])) == sge.ERR_NULL                  # x_q
    args = list(ok_args); args[14] = None
    assert f(*args) == sge.ERR_NULL                                       # out_q without out_s
    args = list(ok_args); args[12] = None; args[14] = None; args[15] = None; args[18] = None; args[19] = None
    assert f(*args) == sge.ERR_NULL                                       # no output at all
    args = list(ok_args); args[11] = None
    assert f(*args) == sge.ERR_NULL                                       # SwiGLU needs probs
    args = list(ok_args); args[7] = 160
    assert f(*args) == sge.ERR_SHAPE                                      # K % 128
    args = list(ok_args); args[6] = 136
    assert f(*args) == sge.ERR_SHAPE                                      # SwiGLU needs N % 256
    args = list(ok_args); args[10] = sge.EPI_NONE
    assert f(*args) == sge.ERR_ARG                                        # quantized output needs SwiGLU
    args = list(ok_args); args[12] = FAKE + 8
    assert f(*args) == sge.ERR_ALIGN
    args = list(ok_args); args[14] = x_q
    assert f(*args) == sge.ERR_ALIAS                                      # out_q over x_q
    args = list(ok_args); args[15] = y
    assert f(*args) == sge.ERR_ALIAS                                      # out_s over out
    # the token-blocked output
    args = list(ok_args); args[19] = None
    assert f(*args) == sge.ERR_NULL                                       # out_colT_q without out_colT_s
    args = list(ok_args); args[16] = None
    assert f(*args) == sge.ERR_NULL                                       # needs the layout
    args = list(ok_args); args[17] = ld_t - 128
    assert f(*args) == sge.ERR_SHAPE                                      # ld_t below capacity
    args = list(ok_args); args[17] = ld_t + 64
    assert f(*args) == sge.ERR_SHAPE                                      # ld_t % 128
    args = list(ok_args); args[10] = sge.EPI_NONE; args[14] = None; args[15] = None
    assert f(*args) == sge.ERR_ARG                                        # needs an activation epilogue
    args = list(ok_args); args[18] = FAKE * 60000 + 8
    assert f(*args) == sge.ERR_ALIGN
    args = list(ok_args); args[19] = FAKE * 70000 + 4
    assert f(*args) == sge.ERR_ALIGN                                      # out_colT_s too (word stores)
    args = list(ok_args); args[18] = x_q
    assert f(*args) == sge.ERR_ALIAS                                      # out_colT_q over x_q
    args = list(ok_args); args[19] = lay
    assert f(*args) == sge.ERR_ALIAS                                      # out_colT_s over the layout
    args = list(ok_args); args[18] = y
    assert f(*args) == sge.ERR_ALIAS                                      # out_colT_q over out



def test_mx_token_capacity(sge):
    assert sge.mx_token_capacity(65536, 8) == 65536 + 8 * 128
    assert sge.mx_token_capacity(560, 6) == 640 + 6 * 128
    assert sge.mx_token_capacity(0, 1) == 128
    assert sge.mx_token_capacity(-1, 1) == -1 and sge.mx_token_capacity(10, 0) == -1


def test_mxfp8_grouped_backward_validation_errors(sge):
    def B(k):                      # far-apart fake addresses (no accidental overlaps)
        return FAKE * 8 * k

    lay = sge._lib.sge_mx_group_layout
    assert lay(None, 4, 100, FAKE, None) == sge.ERR_NULL
    assert lay(FAKE, 0, 100, B(2), None) == sge.ERR_ARG
    assert lay(FAKE, 4097, 100, B(2), None) == sge.ERR_ARG
    assert lay(FAKE, 4, -1, B(2), None) == sge.ERR_SHAPE
    assert lay(FAKE, 4, 100, FAKE + 16, None) == sge.ERR_ALIAS           # layout over offsets

    q = sge._lib.sge_quantize_mxfp8_grouped
    T, C, G = 100, 64, 4
    ld = sge.mx_token_capacity(T, G)
    ok = [B(1), T, C, G, B(3), ld, B(5), B(7), B(9), B(11), None]
    a = list(ok); a[8] = None
    assert q(*a) == sge.ERR_NULL                                          # q_colT required
    a = list(ok); a[7] = None
    assert q(*a) == sge.ERR_NULL                                          # q_row without s_row
    a = list(ok); a[2] = 48
    assert q(*a) == sge.ERR_SHAPE                                         # cols % 32
    a = list(ok); a[5] = ld - 128
    assert q(*a) == sge.ERR_SHAPE                                         # ld below capacity
    a = list(ok); a[5] = ld + 64
    assert q(*a) == sge.ERR_SHAPE                                         # ld % 128
    a = list(ok); a[8] = B(9) + 8
    assert q(*a) == sge.ERR_ALIGN
    a = list(ok); a[8] = B(1)
    assert q(*a) == sge.ERR_ALIAS                                         # q_colT over src
    a = list(ok); a[9] = B(3)
    assert q(*a) == sge.ERR_ALIAS                                         # s_colT over layout

    d = _act_after(sge._lib.sge_grouped_linear_dgrad_mxfp8, 10)
    G, T, N, K = 4, 100, 256, 512
    sw = sge.EPI_DSCALED_SWIGLU
    ws = sge.grouped_linear_bwd_workspace_size(T, K, G, sw)
    ld_t = sge.mx_token_capacity(T, G)
    ok = [B(1), B(2), B(3), B(4), G, T, N, K, B(5), 1.0, sw, B(6), B(7), None,
          B(8), B(9), B(10), B(11), B(16), ld_t, B(14), B(20), B(12), ws, None]
    a = list(ok); a[11] = None
    assert d(*a) == sge.ERR_NULL                                          # SwiGLU needs preact
    a = list(ok); a[14] = None; a[16] = None; a[17] = None; a[20] = None; a[21] = None
    assert d(*a) == sge.ERR_NULL                                          # no output
    a = list(ok); a[17] = None
    assert d(*a) == sge.ERR_NULL                                          # dact_q without dact_s
    a = list(ok); a[10] = sge.EPI_NONE; a[13] = B(13)
    assert d(*a) == sge.ERR_ARG                                           # quantized output needs SwiGLU
    a = list(ok); a[6] = 96
    assert d(*a) == sge.ERR_SHAPE                                         # N % 128
    a = list(ok); a[7] = 520
    assert d(*a) == sge.ERR_SHAPE                                         # SwiGLU K % 32
    a = list(ok); a[16] = B(10) + 4
    assert d(*a) == sge.ERR_ALIGN
    a = list(ok); a[14] = B(6)
    assert d(*a) == sge.ERR_ALIAS                                         # dact over preact
    a = list(ok); a[16] = B(8)
    assert d(*a) == sge.ERR_ALIAS                                         # dact_q over dact
    a = list(ok); a[23] = ws - 4
    assert d(*a) == sge.ERR_WORKSPACE
    a = list(ok); a[21] = None
    assert d(*a) == sge.ERR_NULL                                          # dact_colT_q without dact_colT_s
    a = list(ok); a[18] = None
    assert d(*a) == sge.ERR_NULL                                          # needs the layout
    a = list(ok); a[19] = ld_t - 128
    assert d(*a) == sge.ERR_SHAPE                                         # ld_t below capacity
    a = list(ok); a[10] = sge.EPI_NONE; a[13] = B(15); a[16] = None; a[17] = None
    assert d(*a) == sge.ERR_ARG                                           # token-blocked output needs SwiGLU
    a = list(ok); a[20] = B(14) + 8
    assert d(*a) == sge.ERR_ALIGN
    a = list(ok); a[20] = B(6)
    assert d(*a) == sge.ERR_ALIAS                                         # dact_colT_q over preact
    a = list(ok); a[21] = B(8)
    assert d(*a) == sge.ERR_ALIAS                                         # dact_colT_s over dact

    w = sge._lib.sge_grouped_linear_wgrad_mxfp8
    ok = [B(1), B(2), B(3), B(4), G, N, K, B(5), 640, 1.0, B(6), None]
    a = list(ok); a[10] = None
    assert w(*a) == sge.ERR_NULL
    a = list(ok); a[8] = 600
    assert w(*a) == sge.ERR_SHAPE                                         # ld % 128
    a = list(ok); a[4] = 0
    assert w(*a) == sge.ERR_SHAPE
    a = list(ok); a[10] = B(6) + 2
    assert w(*a) == sge.ERR_ALIGN
    a = list(ok); a[10] = B(3)
    assert w(*a) == sge.ERR_ALIAS                                         # dw over xT_q


def test_fp8_grouped_validation_errors(sge):
    def B(k):                      # far-apart fake addresses (no accidental overlaps)
        return FAKE * 8 * k

    assert sge.quantize_fp8_grouped_workspace_size(8) == 32
    q = sge._lib.sge_quantize_fp8_grouped
    rows, C, G = 100, 64, 4
    ld = sge.mx_token_capacity(rows, G)
    ws = sge.quantize_fp8_grouped_workspace_size(G)
    ok = [B(1), rows, C, G, B(2), ld, B(3), B(4), B(5), B(6), B(7), None, B(8), ws, None]
    a = list(ok); a[8] = None
    assert q(*a) == sge.ERR_NULL                                          # amax required
    a = list(ok); a[6] = None; a[7] = None
    assert q(*a) == sge.ERR_NULL                                          # no output
    a = list(ok); a[2] = 40
    assert q(*a) == sge.ERR_SHAPE                                         # cols % 16
    a = list(ok); a[5] = ld - 128
    assert q(*a) == sge.ERR_SHAPE                                         # ld below capacity
    a = list(ok); a[4] = None
    assert q(*a) == sge.ERR_SHAPE                                         # equal runs need rows/G % 128
    a = list(ok); a[4] = None; a[1] = 4 * 256; a[5] = 1000
    assert q(*a) == sge.ERR_SHAPE                                         # ld_t % 16 without a layout
    a = list(ok); a[6] = B(6) + 4
    assert q(*a) == sge.ERR_ALIGN
    a = list(ok); a[13] = ws - 1
    assert q(*a) == sge.ERR_WORKSPACE
    a = list(ok); a[11] = B(9); a[12] = None; a[13] = 0; a[2] = 40
    assert q(*a) == sge.ERR_SHAPE                                         # no workspace needed with amax_in
    a = list(ok); a[7] = B(1)
    assert q(*a) == sge.ERR_ALIAS                                         # q_t over src
    a = list(ok); a[10] = B(6)
    assert q(*a) == sge.ERR_ALIAS                                         # scale_inv over scale
    a = list(ok); a[11] = B(9); a[8] = B(9)
    assert q(*a) == sge.ERR_ALIAS                                         # amax output over amax_in

    f = _act_after(sge._lib.sge_grouped_linear_fwd_fp8, 10)
    G, T, N, K = 4, 100, 512, 256
    ok = [B(1), B(2), B(3), B(4), G, T, N, K, B(5), 1.0, sge.EPI_SCALED_SWIGLU, B(6), B(7), B(8), None, None]
    a = list(ok); a[1] = None
    assert f(*a) == sge.ERR_NULL                                          # x_sinv
    a = list(ok); a[11] = None
    assert f(*a) == sge.ERR_NULL                                          # SwiGLU needs probs
    a = list(ok); a[7] = 200
    assert f(*a) == sge.ERR_SHAPE                                         # K % 16
    a = list(ok); a[6] = 264
    assert f(*a) == sge.ERR_SHAPE                                         # SwiGLU N % 256
    a = list(ok); a[12] = B(1)
    assert f(*a) == sge.ERR_ALIAS                                         # out over x_q
    a = list(ok); a[10] = sge.EPI_NONE; a[14] = B(9)
    assert f(*a) == sge.ERR_ARG                                           # out_amax needs SwiGLU
    a = list(ok); a[14] = B(7)
    assert f(*a) == sge.ERR_ALIAS                                         # out_amax over out

    d = _act_after(sge._lib.sge_grouped_linear_dgrad_fp8, 10)
    sw = sge.EPI_DSCALED_SWIGLU
    wsb = sge.grouped_linear_bwd_workspace_size(T, K, G, sw)
    ok = [B(1), B(2), B(3), B(4), G, T, N, K, B(5), 1.0, sw, B(6), B(7), None, B(8), B(9), None, B(10), wsb, None]
    a = list(ok); a[14] = None
    assert d(*a) == sge.ERR_NULL                                          # SwiGLU needs dact
    a = list(ok); a[10] = sge.EPI_NONE
    assert d(*a) == sge.ERR_NULL                                          # dx required without SwiGLU
    a = list(ok); a[6] = 200
    assert d(*a) == sge.ERR_SHAPE                                         # N % 16
    a = list(ok); a[14] = B(6)
    assert d(*a) == sge.ERR_ALIAS                                         # dact over preact
    a = list(ok); a[18] = wsb - 4
    assert d(*a) == sge.ERR_WORKSPACE
    a = list(ok); a[10] = sge.EPI_NONE; a[13] = B(11); a[16] = B(12)
    assert d(*a) == sge.ERR_ARG                                           # dact_amax needs the SwiGLU backward

    w = sge._lib.sge_grouped_linear_wgrad_fp8
    ok = [B(1), B(2), B(3), B(4), G, N, K, B(5), 640, 1.0, B(6), None]
    a = list(ok); a[1] = None
    assert w(*a) == sge.ERR_NULL
    a = list(ok); a[8] = 600
    assert w(*a) == sge.ERR_SHAPE
    a = list(ok); a[10] = B(3)
    assert w(*a) == sge.ERR_ALIAS


def test_norm_validation_errors(sge):
    def B(k):
        return FAKE * 8 * k

    f = sge._lib.sge_norm_fwd
    R, C = 64, 96
    ws = sge.norm_fwd_workspace_size(R, C)
    ok = [sge.NORM_LAYER, B(1), B(2), B(3), R, C, 1e-5, 0, B(4), B(5), B(6), B(7), B(8), B(9), B(10), B(11),
          B(12), B(13), B(14), B(15), B(16), ws, None]
    a = list(ok); a[0] = 5
    assert f(*a) == sge.ERR_ARG
    a = list(ok); a[3] = None
    assert f(*a) == sge.ERR_NULL                                          # LayerNorm needs beta
    a = list(ok); a[13] = None
    assert f(*a) == sge.ERR_NULL                                          # FP8 output needs amax
    a = list(ok); a[17] = None
    assert f(*a) == sge.ERR_NULL                                          # q_row without s_row
    a = list(ok); a[5] = 16392
    assert f(*a) == sge.ERR_SHAPE                                         # cols <= 16384
    a = list(ok); a[5] = 72
    assert f(*a) == sge.ERR_SHAPE                                         # MXFP8 needs cols % 32
    a = list(ok); a[4] = 48
    assert f(*a) == sge.ERR_SHAPE                                         # MXFP8 columnwise needs rows % 32
    a = list(ok); a[8] = B(4) + 2
    assert f(*a) == sge.ERR_ALIGN
    a = list(ok); a[8] = B(1)
    assert f(*a) == sge.ERR_ALIAS                                         # y over x
    a = list(ok); a[21] = 0
    assert f(*a) == sge.ERR_WORKSPACE
    b = sge._lib.sge_norm_bwd
    wsb = sge.norm_bwd_workspace_size(R, C)
    ok = [sge.NORM_RMS, B(1), B(2), None, B(3), B(4), R, C, 0, B(5), B(6), None, B(7), wsb, None]
    a = list(ok); a[10] = None
    assert b(*a) == sge.ERR_NULL                                          # dgamma
    a = list(ok); a[0] = sge.NORM_LAYER
    assert b(*a) == sge.ERR_NULL                                          # LayerNorm needs mu and dbeta
    a = list(ok); a[7] = 100
    assert b(*a) == sge.ERR_SHAPE
    a = list(ok); a[9] = B(2)
    assert b(*a) == sge.ERR_ALIAS                                         # dx over x
    a = list(ok); a[13] = wsb - 4
    assert b(*a) == sge.ERR_WORKSPACE


def test_srelu_epilogue_validation(sge):
    def B(k):
        return FAKE * 8 * k

    f = _act_after(sge._lib.sge_grouped_linear_fwd, 8)
    # bf16 grouped forward: SReLU needs probs
    assert f(B(1), B(2), 4, 100, 264, 256, B(3), 1.0, sge.EPI_SCALED_SRELU, None, B(4), B(5), None) == sge.ERR_NULL
    fm = _act_after(sge._lib.sge_grouped_linear_fwd_mxfp8, 10)
    assert fm(B(1), B(2), B(3), B(4), 4, 100, 256, 256, B(5), 1.0, sge.EPI_SCALED_SRELU, None, B(7), B(8),
              None, None, None, 0, None, None, None) == sge.ERR_NULL       # MXFP8 SReLU needs probs
    assert fm(B(1), B(2), B(3), B(4), 4, 100, 264, 256, B(5), 1.0, sge.EPI_SCALED_SRELU, B(6), B(7), B(8),
              B(9), B(10), None, 0, None, None, None) == sge.ERR_SHAPE     # MXFP8 output: N % 32
    assert fm(B(1), B(2), B(3), B(4), 4, 100, 256, 256, B(5), 1.0, sge.EPI_NONE, None, B(7), None,
              B(9), B(10), None, 0, None, None, None) == sge.ERR_ARG       # MXFP8 output needs an activation
    dm = _act_after(sge._lib.sge_grouped_linear_dgrad_mxfp8, 10)
    assert dm(B(1), B(2), B(3), B(4), 4, 100, 256, 256, B(5), 1.0, sge.EPI_DSCALED_SRELU, None, B(6), None, B(7),
              B(8), None, None, None, 0, None, None, B(9), 1 << 20, None) == sge.ERR_NULL   # needs preact
    ff = _act_after(sge._lib.sge_grouped_linear_fwd_fp8, 10)
    assert ff(B(1), B(2), B(3), B(4), 4, 100, 256, 256, B(5), 1.0, sge.EPI_NONE, None, B(7), None, B(8),
              None) == sge.ERR_ARG                                         # a fused amax needs an activation
    df = _act_after(sge._lib.sge_grouped_linear_dgrad_fp8, 10)
    assert df(B(1), B(2), B(3), B(4), 4, 100, 256, 256, B(5), 1.0, sge.EPI_DSCALED_SRELU, B(6), B(7), None, None,
              B(8), None, B(9), 1 << 20, None) == sge.ERR_NULL              # the backward needs dact
    b = _act_after(sge._lib.sge_grouped_linear_bwd, 9)
    assert b(B(1), None, B(2), 4, 100, 256, 264, B(3), 1.0, sge.EPI_DSCALED_SRELU, B(4), B(5), None, B(6), None,
              None, B(7), 0, None) == sge.ERR_NULL                        # SReLU backward needs dact
    assert sge.grouped_linear_bwd_workspace_size(100, 264, 4, sge.EPI_DSCALED_SRELU) == 2 * 100 * 4


def test_clamped_swiglu_epilogue_validation(sge):
    """The clamped SwiGLU epilogues need their (limit, alpha): NULL is ERR_NULL, a limit that is
    not finite and positive or a non-finite alpha is ERR_ARG; the workspace query and the shape
    rules are those of the SwiGLU epilogues."""
    def B(k):
        return FAKE * 8 * k

    cf, cb = sge.EPI_SCALED_CLAMPED_SWIGLU, sge.EPI_DSCALED_CLAMPED_SWIGLU
    good = sge._act((7.0, 1.702))
    fwd = sge._lib.sge_grouped_linear_fwd

    def f(act, n=256):
        return _act_after(fwd, 8, act)(B(1), B(2), 4, 100, n, 256, B(3), 1.0, cf, B(4), B(5), B(6), None)

    assert f(None) == sge.ERR_NULL
    for bad in ((0.0, 1.0), (-1.0, 1.0), (float("inf"), 1.0), (float("nan"), 1.0), (7.0, float("nan"))):
        assert f(sge._act(bad)) == sge.ERR_ARG, bad
    assert f(good, n=264) == sge.ERR_SHAPE                                # gated: N % 256
    assert sge.grouped_linear_bwd_workspace_size(100, 264, 4, cb) == sge.grouped_linear_bwd_workspace_size(
        100, 264, 4, sge.EPI_DSCALED_SWIGLU) > 0
    b = _act_after(sge._lib.sge_grouped_linear_bwd, 9)
    assert b(B(1), None, B(2), 4, 100, 256, 264, B(3), 1.0, cb, B(4), B(5), B(6), B(7), None,
             None, B(8), 1 << 20, None) == sge.ERR_NULL                  # act missing
    b = _act_after(sge._lib.sge_grouped_linear_bwd, 9, good)
    assert b(B(1), None, B(2), 4, 100, 256, 264, B(3), 1.0, cb, B(4), B(5), B(6), B(7), None,
             None, B(8), 16, None) == sge.ERR_WORKSPACE
    fm = _act_after(sge._lib.sge_grouped_linear_fwd_mxfp8, 10)
    assert fm(B(1), B(2), B(3), B(4), 4, 100, 256, 256, B(5), 1.0, cf, B(6), B(7), B(8),
              None, None, None, 0, None, None, None) == sge.ERR_NULL       # MXFP8: act missing
    dm = _act_after(sge._lib.sge_grouped_linear_dgrad_mxfp8, 10, sge._act((0.0, 1.0)))
    assert dm(B(1), B(2), B(3), B(4), 4, 100, 256, 256, B(5), 1.0, cb, B(6), B(7), None, B(8),
              B(9), None, None, None, 0, None, None, B(10), 1 << 20, None) == sge.ERR_ARG   # bad limit
    ff = _act_after(sge._lib.sge_grouped_linear_fwd_fp8, 10)
    assert ff(B(1), B(2), B(3), B(4), 4, 100, 256, 256, B(5), 1.0, cf, B(6), B(7), B(8), None,
              None) == sge.ERR_NULL                                        # FP8: act missing
    df = _act_after(sge._lib.sge_grouped_linear_dgrad_fp8, 10)
    assert df(B(1), B(2), B(3), B(4), 4, 100, 256, 256, B(5), 1.0, cb, B(6), B(7), None, B(8),
              B(9), None, B(10), 1 << 20, None) == sge.ERR_NULL            # FP8 dgrad: act missing


def test_grouped_mlp_validation(sge):
    """The whole grouped MLP checks every argument before its first launch."""
    def B(k):
        return FAKE * 8 * k

    G, T, H, F = 4, 100, 256, 256
    sw = sge.EPI_SCALED_SWIGLU
    f = sge._lib.sge_grouped_mlp_fwd
    # x, w1, w2, G, T, H, F, splits, offsets, err, act, params, probs, preact, y, out, stream
    ok = [B(1), B(1000), B(3000), G, T, H, F, B(5000), B(5100), None, sw, None, B(5200), B(6000), B(20000),
          B(30000), None]
    a = list(ok); a[0] = None
    assert f(*a) == sge.ERR_NULL
    a = list(ok); a[10] = sge.EPI_DSCALED_SWIGLU
    assert f(*a) == sge.ERR_ARG                                           # a backward epilogue
    a = list(ok); a[10] = sge.EPI_SCALED_CLAMPED_SWIGLU
    assert f(*a) == sge.ERR_NULL                                          # clamped without its parameters
    a = list(ok); a[6] = 200
    assert f(*a) == sge.ERR_SHAPE                                         # gated: F % 128
    a = list(ok); a[6] = 200; a[10] = sge.EPI_SCALED_SRELU; a[15] = B(1)
    assert f(*a) == sge.ERR_ALIAS                                         # SReLU: F % 8 passes the shape check
    a = list(ok); a[13] = B(6000) + 8
    assert f(*a) == sge.ERR_ALIGN
    a = list(ok); a[8] = B(5000) + 4
    assert f(*a) == sge.ERR_ALIGN                                         # offsets: 8-byte aligned
    a = list(ok); a[15] = B(1)
    assert f(*a) == sge.ERR_ALIAS                                         # out over x
    a = list(ok); a[14] = B(6000)
    assert f(*a) == sge.ERR_ALIAS                                         # act_out over preact
    a = list(ok); a[9] = B(5100)
    assert f(*a) == sge.ERR_ALIAS                                         # err_flag over offsets
    b = sge._lib.sge_grouped_mlp_bwd
    ws = sge.grouped_mlp_bwd_workspace_size(T, F, G, sw)
    assert ws == sge.grouped_linear_bwd_workspace_size(T, F, G, sge.EPI_DSCALED_SWIGLU) > 0
    assert sge.grouped_mlp_bwd_workspace_size(T, F, G, sge.EPI_NONE) == 0
    # dout, x, w1, w2, G, T, H, F, offsets, act, params, probs, preact, y, dpreact, dprobs, dx, dw1, dw2, ws, bytes
    okb = [B(1), B(1000), B(2000), B(4000), G, T, H, F, B(5000), sw, None, B(5100), B(6000), B(20000), B(30000),
           B(40000), B(50000), B(60000), B(80000), B(90000), ws, None]
    assert b(*okb[:14], None, *okb[15:]) == sge.ERR_NULL                  # dpreact required
    a = list(okb); a[19] = None
    assert b(*a) == sge.ERR_WORKSPACE
    a = list(okb); a[20] = ws - 4
    assert b(*a) == sge.ERR_WORKSPACE
    a = list(okb); a[19] = B(1000)
    assert b(*a) == sge.ERR_ALIAS                                         # workspace over x
    a = list(okb); a[16] = B(30000)
    assert b(*a) == sge.ERR_ALIAS                                         # dx over dpreact


def test_shapes_beyond_32bit_tile_addressing_are_refused(sge):
    """Row strides whose 256-row tile span (or arrays addressed whole, such as MXFP8 scales and a
    gated weight's two halves) would not fit the kernels' 32-bit buffer offsets give
    SGE_ERR_SHAPE instead of reading zeros."""
    big = 1 << 23                                         # bf16 elements: 16 MiB per row
    st, msg = _fwd(sge, _op(sge, 64, 128, ld=big), _op(sge, 64, 128, data=FAKE * 2))
    assert st == sge.ERR_SHAPE and "32-bit" in msg, msg
    st, msg = _fwd(sge, _op(sge, 64, 128), _op(sge, 64, 128, data=FAKE * 2), ld_res=big)
    assert st == sge.ERR_SHAPE and "32-bit" in msg, msg
    # an MXFP8 scale array of 2^31 bytes (rows x mx_ld)
    st, msg = _fwd(sge, _op(sge, 1 << 21, 128, fmt=2, mx=FAKE, mx_ld=1 << 10),
                   _op(sge, 64, 128, fmt=2, data=FAKE * 2, mx=FAKE, mx_ld=4))
    assert st == sge.ERR_SHAPE and "32-bit" in msg, msg
    # one stride below the limit passes the check (and then fails later on the fake aliasing)
    st, msg = _fwd(sge, _op(sge, 64, 128, ld=1 << 21), _op(sge, 64, 128, data=FAKE * 2))
    assert "32-bit" not in msg, msg
    lib = sge._lib
    fwd = _act_after(lib.sge_grouped_linear_fwd, 8)
    # grouped: a contraction of 2^23 bf16 per row
    st = fwd(FAKE, FAKE * 64, 8, 100, 256, big, FAKE * 1024, 1.0, 0, None, FAKE * 8192, None, None)
    assert st == sge.ERR_SHAPE and "32-bit" in lib.sge_last_error_message().decode()
    # gated fc1: both halves of one expert's weight are addressed from one base (2^31 bytes here)
    st = fwd(FAKE, FAKE * 64, 8, 100, 1 << 20, 2048, FAKE * 1024, 1.0, 1, FAKE * 4096, FAKE * 8192, None, None)
    assert st == sge.ERR_SHAPE and "32-bit" in lib.sge_last_error_message().decode()
    # the same weight without the gate is only addressed tile by tile
    st = fwd(FAKE, FAKE * 64, 8, 100, 1 << 20, 2048, FAKE * 1024, 1.0, 0, None, FAKE * 8192, None, None)
    assert "32-bit" not in lib.sge_last_error_message().decode()


def test_quantizers_refuse_rows_beyond_32bit_tile_addressing(sge):
    """The quantizers address a tile of 128 rows through one buffer resource with 32-bit byte
    offsets: a row longer than that allows gives SGE_ERR_SHAPE (before any HIP call); one within
    it passes that check and fails a later one (the fake pointers overlap), so nothing launches."""
    lib = sge._lib
    big, fits = 1 << 23, 1 << 21                          # bf16 elements per row
    ld = sge.mx_token_capacity(100, 4)
    for cols, refused in ((big, True), (fits, False)):
        calls = (
            lambda: lib.sge_quantize_fp8_amax(FAKE, 16, cols, FAKE * 8, None, FAKE * 16, FAKE * 17, FAKE * 18,
                                              FAKE * 32, 1 << 20, None),
            lambda: lib.sge_quantize_fp8_amax_noalloc(FAKE, 16, cols, FAKE * 8, None, FAKE * 16, FAKE * 17,
                                                      FAKE * 18, None),
            lambda: lib.sge_quantize_mxfp8(FAKE, 32, cols, FAKE * 8, FAKE * 9, None, None, None),
            lambda: lib.sge_quantize_mxfp8_grouped(FAKE, 100, cols, 4, FAKE * 64, ld, None, None, FAKE * 80,
                                                   FAKE * 96, None),
            lambda: lib.sge_quantize_fp8_grouped(FAKE, 100, cols, 4, FAKE * 64, ld, FAKE * 72, None, FAKE * 88,
                                                 FAKE * 89, FAKE * 90, None, FAKE * 91, 64, None),
        )
        for call in calls:
            st = call()
            msg = lib.sge_last_error_message().decode()
            assert st != sge.OK, msg
            assert (st == sge.ERR_SHAPE and "32-bit" in msg) == refused, (st, msg)


def test_quantize_fp8_amax_noalloc_validation_errors(sge):
    """The no-allocation quantizer validates like the workspace call, before any HIP call."""
    lib = sge._lib
    f = lib.sge_quantize_fp8_amax_noalloc
    assert f(FAKE, 60, 64, FAKE * 8, None, FAKE * 16, FAKE * 17, FAKE * 18, None) == sge.ERR_SHAPE
    assert f(FAKE, 64, 64, FAKE * 8, None, None, FAKE * 17, FAKE * 18, None) == sge.ERR_NULL
    assert f(FAKE + 8, 64, 64, FAKE * 8, None, FAKE * 16, FAKE * 17, FAKE * 18, None) == sge.ERR_ALIGN
    assert f(FAKE, 64, 64, FAKE + 1024, None, FAKE * 16, FAKE * 17, FAKE * 18, None) == sge.ERR_ALIAS

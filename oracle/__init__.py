"""CPU oracle for the MXFP4 W4A8 linear layer -- TEST INFRASTRUCTURE ONLY.

Only tests/, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
bench.py may import this package.  The library (``w4a8_gemm_amd``) never does.

Thin numpy wrappers over liboracle.so (plain C, see oracle.c for the
algorithms, their page citations and the readings of open points).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

OCP, NOCLIP, MSE = 0, 1, 2
MODES = {"ocp": OCP, "noclip": NOCLIP, "mse": MSE}

_u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
_u16p = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(np.int64, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p


def lib():
    """Load liboracle.so, building it with gcc only if it is not there."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        L.orc_set_threads.argtypes = [ctypes.c_int]
        L.orc_set_threads.restype = None
        L.orc_max_threads.argtypes = []
        L.orc_max_threads.restype = ctypes.c_int
        L.orc_e2m1_value.argtypes = [ctypes.c_int]
        L.orc_e2m1_value.restype = ctypes.c_float
        L.orc_e4m3_value.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_value.restype = ctypes.c_double
        L.orc_bf16_value.argtypes = [ctypes.c_uint16]
        L.orc_bf16_value.restype = ctypes.c_float
        L.orc_f16_value.argtypes = [ctypes.c_uint16]
        L.orc_f16_value.restype = ctypes.c_double
        L.orc_e4m3_encode.argtypes = [ctypes.c_float]
        L.orc_e4m3_encode.restype = ctypes.c_uint8
        L.orc_e2m1_index.argtypes = [ctypes.c_float]
        L.orc_e2m1_index.restype = ctypes.c_int
        L.orc_block_exponent.argtypes = [ctypes.c_float, ctypes.c_int]
        L.orc_block_exponent.restype = ctypes.c_int
        L.orc_encode_block.argtypes = [_f32p, ctypes.c_int, _u8p]
        L.orc_encode_block.restype = ctypes.c_float
        L.orc_quant_block.argtypes = [_f32p, ctypes.c_int, _u8p, ctypes.POINTER(ctypes.c_float)]
        L.orc_quant_block.restype = ctypes.c_int
        L.orc_quant_mxfp4.argtypes = [_f32p, _i64, _i64, ctypes.c_int, _u8p, _u8p, _vp,
                                      ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
        L.orc_quant_mxfp4.restype = None
        L.orc_dequant_mxfp4.argtypes = [_u8p, _u8p, _i64, _i64, _f32p]
        L.orc_dequant_mxfp4.restype = None
        L.orc_dequant_nvfp4.argtypes = [_u8p, _u8p, _i64, _i64, ctypes.c_float, _f32p]
        L.orc_dequant_nvfp4.restype = None
        L.orc_requant_nvfp4_to_mxfp4.argtypes = [_u8p, _u8p, _i64p, _f32p, ctypes.c_int, _i64,
                                                 ctypes.c_int, _i64, _u8p, _u8p, _f64p]
        L.orc_requant_nvfp4_to_mxfp4.restype = ctypes.c_int
        L.orc_quant_bf16_to_mxfp4.argtypes = [_u16p, _i64, _i64, ctypes.c_int, _u8p, _u8p, _f64p]
        L.orc_quant_bf16_to_mxfp4.restype = ctypes.c_int
        L.orc_quant_fp8ch_to_mxfp4.argtypes = [_u8p, _f32p, _i64, _i64, ctypes.c_int, _u8p, _u8p, _f64p]
        L.orc_quant_fp8ch_to_mxfp4.restype = ctypes.c_int
        L.orc_quant_act_fp8.argtypes = [_u16p, _i64, _i64, _i64, _u8p, _f32p]
        L.orc_quant_act_fp8.restype = ctypes.c_int
        L.orc_mxfp4_gemm.argtypes = [_u8p, _f32p, _u8p, _u8p, _i64, _i64, _i64, _vp, _vp, _i64, _f64p]
        L.orc_mxfp4_gemm.restype = None
        L.orc_w4a4_gemm.argtypes = [_u8p, _u8p, _u8p, _u8p, _i64, _i64, _i64, _vp, _vp, _i64, _f64p]
        L.orc_w4a4_gemm.restype = None
        L.orc_int4_prepare.argtypes = [_i32p, _i32p, _i64, _i64, _i32p]
        L.orc_int4_prepare.restype = ctypes.c_int
        L.orc_int4_gemm.argtypes = [_u8p, _f32p, _i32p, _u16p, _i64, _i64, _i64, _vp, _vp, _i64, _f64p]
        L.orc_int4_gemm.restype = None
        L.orc_int4_zp_gemm.argtypes = [_u8p, _f32p, _i32p, _i32p, _u16p, _i64, _i64, _i64, _vp, _vp, _i64,
                                       _f64p]
        L.orc_int4_zp_gemm.restype = None
        L.orc_int5_gemm.argtypes = [_u8p, _f32p, _i32p, _i32p, _u8p, _u16p, _i64, _i64, _i64, _vp, _vp, _i64,
                                    _f64p]
        L.orc_int5_gemm.restype = None
        L.orc_e2m1_index_array.argtypes = [_f32p, _i64, _u8p]
        L.orc_e2m1_index_array.restype = None
        L.orc_block_exponent_array.argtypes = [_f32p, _i64, ctypes.c_int, _i32p]
        L.orc_block_exponent_array.restype = None
        L.orc_e4m3_encode_array.argtypes = [_f32p, _i64, _u8p]
        L.orc_e4m3_encode_array.restype = None
        _lib = L
    return _lib


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


# --- scalar format helpers -------------------------------------------------

def e2m1_value(code: int) -> float:
    return lib().orc_e2m1_value(int(code))


def e4m3_value(b: int) -> float:
    return lib().orc_e4m3_value(int(b))


def bf16_value(h: int) -> float:
    return lib().orc_bf16_value(int(h))


def f16_value(h: int) -> float:
    return lib().orc_f16_value(int(h))


def e4m3_encode(y: float) -> int:
    return lib().orc_e4m3_encode(float(y))


def e2m1_index(a: float) -> int:
    return lib().orc_e2m1_index(float(a))


def block_exponent(amax: float, mode) -> int:
    return lib().orc_block_exponent(float(amax), MODES.get(mode, mode))


def e2m1_index_array(a):
    a = _c(a, np.float32).ravel()
    out = np.zeros(a.size, np.uint8)
    lib().orc_e2m1_index_array(a, a.size, out)
    return out


def block_exponent_array(amax, mode):
    a = _c(amax, np.float32).ravel()
    out = np.zeros(a.size, np.int32)
    lib().orc_block_exponent_array(a, a.size, MODES.get(mode, mode), out)
    return out


def e4m3_encode_array(y):
    y = _c(y, np.float32).ravel()
    out = np.zeros(y.size, np.uint8)
    lib().orc_e4m3_encode_array(y, y.size, out)
    return out


# --- blocks and rows ------------------------------------------------------------

def encode_block(w32, e: int):
    """-> (idx uint8[32], fp32 error)."""
    w = _c(w32, np.float32)
    idx = np.zeros(32, np.uint8)
    err = lib().orc_encode_block(w, int(e), idx)
    return idx, np.float32(err)


def quant_block(w32, mode):
    """-> (exponent, codes uint8[32], fp32 error)."""
    w = _c(w32, np.float32)
    code = np.zeros(32, np.uint8)
    err = ctypes.c_float()
    e = lib().orc_quant_block(w, MODES.get(mode, mode), code, ctypes.byref(err))
    return e, code, np.float32(err.value)


def quant_mxfp4(w, mode="mse", with_block_err=False):
    """[rows, K] fp32 -> (packed [rows,K/2] u8, e8m0 [rows,K/32] u8, err_sum, ssq[, block_err])."""
    w = _c(w, np.float32)
    rows, K = w.shape
    assert K % 32 == 0
    packed = np.zeros((rows, K // 2), np.uint8)
    e8m0 = np.zeros((rows, K // 32), np.uint8)
    be = np.zeros((rows, K // 32), np.float32) if with_block_err else None
    es, ss = ctypes.c_double(), ctypes.c_double()
    lib().orc_quant_mxfp4(w, rows, K, MODES.get(mode, mode), packed, e8m0,
                          be.ctypes.data if be is not None else None,
                          ctypes.byref(es), ctypes.byref(ss))
    out = (packed, e8m0, es.value, ss.value)
    return out + (be,) if with_block_err else out


def dequant_mxfp4(packed, e8m0):
    packed = _c(packed, np.uint8)
    e8m0 = _c(e8m0, np.uint8)
    rows, half = packed.shape
    w = np.zeros((rows, half * 2), np.float32)
    lib().orc_dequant_mxfp4(packed, e8m0, rows, half * 2, w)
    return w


def set_threads(n):
    """Threads of the oracle's OpenMP loops (timing only; results do not change)."""
    lib().orc_set_threads(int(n))


def max_threads():
    return int(lib().orc_max_threads())


def dequant_nvfp4(packed, scale, divisor):
    packed = _c(packed, np.uint8)
    scale = _c(scale, np.uint8)
    rows, half = packed.shape
    w = np.zeros((rows, half * 2), np.float32)
    lib().orc_dequant_nvfp4(packed, scale, rows, half * 2, float(np.float32(divisor)), w)
    return w


def requant_nvfp4_to_mxfp4(nv_packed, nv_scale, part_rows, part_divisor, mode="mse", row_chunk=0):
    """-> (mx_packed, mx_e8m0, stats [n_parts, 2] = {sum err, sum w^2})."""
    nv_packed = _c(nv_packed, np.uint8)
    nv_scale = _c(nv_scale, np.uint8)
    pr = _c(part_rows, np.int64)
    pd = _c(part_divisor, np.float32)
    rows, half = nv_packed.shape
    K = half * 2
    mp = np.zeros((rows, K // 2), np.uint8)
    me = np.zeros((rows, K // 32), np.uint8)
    st = np.zeros(2 * len(pr), np.float64)
    rc = lib().orc_requant_nvfp4_to_mxfp4(nv_packed, nv_scale, pr, pd, len(pr), K,
                                          MODES.get(mode, mode), int(row_chunk), mp, me, st)
    if rc != 0:
        raise ValueError("oracle requant rejected its arguments")
    return mp, me, st.reshape(-1, 2)


def quant_bf16_to_mxfp4(w_bf16_bits, mode="mse"):
    """bf16 bits [rows, K] (uint16) -> (packed [rows,K/2], e8m0 [rows,K/32], stats {err, w^2})."""
    w = _c(w_bf16_bits, np.uint16)
    rows, K = w.shape
    mp = np.zeros((rows, K // 2), np.uint8)
    me = np.zeros((rows, K // 32), np.uint8)
    st = np.zeros(2, np.float64)
    if lib().orc_quant_bf16_to_mxfp4(w, rows, K, MODES.get(mode, mode), mp, me, st) != 0:
        raise ValueError("oracle bf16 quant rejected its arguments")
    return mp, me, st


def quant_fp8ch_to_mxfp4(w_e4m3, row_scale, mode="mse"):
    """e4m3 codes [rows, K] (uint8) + fp32 scale per row -> (packed, e8m0, stats {err, w^2})."""
    w = _c(w_e4m3, np.uint8)
    s = _c(row_scale, np.float32)
    rows, K = w.shape
    assert s.shape == (rows,)
    mp = np.zeros((rows, K // 2), np.uint8)
    me = np.zeros((rows, K // 32), np.uint8)
    st = np.zeros(2, np.float64)
    if lib().orc_quant_fp8ch_to_mxfp4(w, s, rows, K, MODES.get(mode, mode), mp, me, st) != 0:
        raise ValueError("oracle fp8 quant rejected its arguments")
    return mp, me, st


def quant_act_fp8(x_bf16_bits, K=None, ldx=None):
    """bf16 bits [M, ldx] (uint16) -> (x8 [M,K] u8, scale [M] f32)."""
    x = _c(x_bf16_bits, np.uint16)
    M, L = x.shape
    K = L if K is None else K
    ldx = L if ldx is None else ldx
    x8 = np.zeros((M, K), np.uint8)
    s = np.zeros(M, np.float32)
    if lib().orc_quant_act_fp8(x, M, K, ldx, x8, s) != 0:
        raise ValueError("non-finite activation")
    return x8, s


def mxfp4_gemm(x8, x_scale, w_packed, w_e8m0, mi=None, ni=None):
    """fp64 reference; full [M,N] or values at (mi[i], ni[i])."""
    x8 = _c(x8, np.uint8)
    xs = _c(x_scale, np.float32)
    wp = _c(w_packed, np.uint8)
    we = _c(w_e8m0, np.uint8)
    M, K = x8.shape
    N = wp.shape[0]
    if mi is None:
        ref = np.zeros((M, N), np.float64)
        lib().orc_mxfp4_gemm(x8, xs, wp, we, M, N, K, None, None, 0, ref)
        return ref
    mi = _c(mi, np.int64)
    ni = _c(ni, np.int64)
    ref = np.zeros(len(mi), np.float64)
    lib().orc_mxfp4_gemm(x8, xs, wp, we, M, N, K, mi.ctypes.data, ni.ctypes.data, len(mi), ref)
    return ref


def quant_act_mxfp4(x_bf16_bits):
    """MXFP4 activations (W4A4): each token row quantized per 32-block by the
    OCP rule -- the page's "ocp" exponent, nearest-even codes, saturation at 6.
    -> (packed [M, K/2], e8m0 [M, K/32])."""
    p, e, _ = quant_bf16_to_mxfp4(x_bf16_bits, "ocp")
    return p, e


def w4a4_gemm(x_packed, x_e8m0, w_packed, w_e8m0, mi=None, ni=None):
    """fp64 reference of the MXFP4 x MXFP4 GEMM; full [M,N] or values at (mi[i], ni[i])."""
    xp = _c(x_packed, np.uint8)
    xe = _c(x_e8m0, np.uint8)
    wp = _c(w_packed, np.uint8)
    we = _c(w_e8m0, np.uint8)
    M, K = xp.shape[0], 2 * xp.shape[1]
    N = wp.shape[0]
    if mi is None:
        ref = np.zeros((M, N), np.float64)
        lib().orc_w4a4_gemm(xp, xe, wp, we, M, N, K, None, None, 0, ref)
        return ref
    mi = _c(mi, np.int64)
    ni = _c(ni, np.int64)
    ref = np.zeros(len(mi), np.float64)
    lib().orc_w4a4_gemm(xp, xe, wp, we, M, N, K, mi.ctypes.data, ni.ctypes.data, len(mi), ref)
    return ref


def int4_prepare(qweight_kn, qzeros, N, K):
    """-> (qweight_nk [N, K/8] int32 or None, number of bad qzeros words)."""
    qw = _c(qweight_kn, np.int32)
    qz = _c(qzeros, np.int32)
    out = np.zeros((N, K // 8), np.int32)
    bad = lib().orc_int4_prepare(qw, qz, N, K, out)
    return (out if bad == 0 else None), bad


def int4_gemm(x8, x_scale, qweight_nk, scales_f16_bits, mi=None, ni=None):
    x8 = _c(x8, np.uint8)
    xs = _c(x_scale, np.float32)
    qw = _c(qweight_nk, np.int32)
    sc = _c(scales_f16_bits, np.uint16)
    M, K = x8.shape
    N = qw.shape[0]
    if mi is None:
        ref = np.zeros((M, N), np.float64)
        lib().orc_int4_gemm(x8, xs, qw, sc, M, N, K, None, None, 0, ref)
        return ref
    mi = _c(mi, np.int64)
    ni = _c(ni, np.int64)
    ref = np.zeros(len(mi), np.float64)
    lib().orc_int4_gemm(x8, xs, qw, sc, M, N, K, mi.ctypes.data, ni.ctypes.data, len(mi), ref)
    return ref


def int4_zp_gemm(x8, x_scale, qweight_kn, qzeros, scales_f16_bits, mi=None, ni=None):
    """int4 g128 with a zero point per group and column, from the checkpoint
    layout (qweight [K/8, N], qzeros [K/128, N/8] holding z - 1, scales
    [K/128, N] fp16 bits): fp64 reference, full [M, N] or values at (mi, ni)."""
    x8 = _c(x8, np.uint8)
    xs = _c(x_scale, np.float32)
    qw = _c(qweight_kn, np.int32)
    qz = _c(qzeros, np.int32)
    sc = _c(scales_f16_bits, np.uint16)
    M, K = x8.shape
    N = qw.shape[1]
    if mi is None:
        ref = np.zeros((M, N), np.float64)
        lib().orc_int4_zp_gemm(x8, xs, qw, qz, sc, M, N, K, None, None, 0, ref)
        return ref
    mi = _c(mi, np.int64)
    ni = _c(ni, np.int64)
    ref = np.zeros(len(mi), np.float64)
    lib().orc_int4_zp_gemm(x8, xs, qw, qz, sc, M, N, K, mi.ctypes.data, ni.ctypes.data, len(mi), ref)
    return ref


def int5_gemm(x8, x_scale, qweight_kn, qweight_hi, qzeros_u8, scales_f16_bits, mi=None, ni=None):
    """int5 g128 (W5A8): low four bits [K/8, N] int32, fifth bits [K/32, N]
    int32, zero points minus one [K/128, N] uint8, scales [K/128, N] fp16 bits:
    fp64 reference, full [M, N] or values at (mi, ni)."""
    x8 = _c(x8, np.uint8)
    xs = _c(x_scale, np.float32)
    qw = _c(qweight_kn, np.int32)
    qh = _c(qweight_hi, np.int32)
    qz = _c(qzeros_u8, np.uint8)
    sc = _c(scales_f16_bits, np.uint16)
    M, K = x8.shape
    N = qw.shape[1]
    if mi is None:
        ref = np.zeros((M, N), np.float64)
        lib().orc_int5_gemm(x8, xs, qw, qh, qz, sc, M, N, K, None, None, 0, ref)
        return ref
    mi = _c(mi, np.int64)
    ni = _c(ni, np.int64)
    ref = np.zeros(len(mi), np.float64)
    lib().orc_int5_gemm(x8, xs, qw, qh, qz, sc, M, N, K, mi.ctypes.data, ni.ctypes.data, len(mi), ref)
    return ref


def linear_bf16(x_bf16_bits, w_packed, w_e8m0, mi=None, ni=None):
    """The W4A8 linear on bf16 activations as one operation -- the fp8
    activation stream that the W4A8 kernel plugin serves ("radiance_nvfp4.py",
    module docstring; "vllm-radiance (MXFP4)", NVFP4 checkpoints: online
    requantization to MXFP4): per-token e4m3 quantization of the activations,
    then the block-scaled GEMM.  The two references above composed, nothing
    else.  -> fp64 [M, N], or the values at (mi[i], ni[i])."""
    x8, s = quant_act_fp8(x_bf16_bits)
    return mxfp4_gemm(x8, s, w_packed, w_e8m0, mi, ni)

"""ctypes binding of libw4a8.so (C ABI in include/w4a8.h).

Argument marshalling only: torch tensors become device pointers and sizes, the
current torch stream becomes the HIP stream, and status codes become
exceptions (ValueError for argument, shape and format errors, RuntimeError for
HIP errors).  Every computation runs in the library's HIP kernels; if the
library cannot be loaded, every call raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "LIB_PATH", "lib", "version", "status_string", "EXP_MODES", "W4A8Error",
    "requant_nvfp4_to_mxfp4", "quant_act_fp8_per_token", "gemm_workspace_bytes",
    "Workspace", "mxfp4_gemm", "int4g128_prepare", "int4g128_gemm", "w4a8_linear",
    "decode_with_plan", "PreparedMXFP4", "mxfp4_prepare", "mxfp4_gemm_prepared",
    "PreparedInt4", "int4g128_prepare_fragments", "int4g128_gemm_prepared",
    "quant_bf16_to_mxfp4", "quant_fp8ch_to_mxfp4", "quant_act_mxfp4", "w4a4_gemm_prepared",
    "mxfp4_linear_prepared", "int4g128_linear_prepared",
    "PreparedInt4ZP", "int4g128_zp_prepare_fragments", "int4g128_zp_gemm_prepared",
    "PreparedInt5", "int5g128_prepare_fragments", "int5g128_gemm_prepared",
    "mxfp4_gemm_prepared_noalloc", "requant_nvfp4_to_mxfp4_prepared", "quant_bf16_to_mxfp4_prepared",
    "quant_fp8ch_to_mxfp4_prepared",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libw4a8.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED_SHAPE, ERR_WORKSPACE, ERR_ASYMMETRIC, ERR_HIP = range(6)
EXP_MODES = {"ocp": 0, "noclip": 1, "mse": 2}
WEIGHT_MXFP4, WEIGHT_INT4G128, WEIGHT_MXFP4_PREPARED, WEIGHT_INT4G128_PREPARED, W4A4_PREPARED = 0, 1, 2, 3, 4
WEIGHT_INT4G128_ZP_PREPARED, WEIGHT_INT5G128_PREPARED = 5, 6
_KINDS = {"mxfp4": WEIGHT_MXFP4, "int4": WEIGHT_INT4G128, "prepared": WEIGHT_MXFP4_PREPARED,
          "int4_prepared": WEIGHT_INT4G128_PREPARED, "w4a4": W4A4_PREPARED,
          "int4_zp_prepared": WEIGHT_INT4G128_ZP_PREPARED, "int5_prepared": WEIGHT_INT5G128_PREPARED}

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int
_size = ctypes.c_size_t
_lib = None


class W4A8Error(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} (status {status})")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libw4a8.so (built by ``python -m w4a8_gemm_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libw4a8.so is not built ({LIB_PATH}); run "
                               "`python -m w4a8_gemm_amd.build` (there is no fallback path)")
        L = ctypes.CDLL(LIB_PATH)
        L.w4a8_requant_nvfp4_to_mxfp4.argtypes = [_vp, _vp, _vp, _vp, _int, _i64, _int, _i64,
                                                  _vp, _vp, _vp, _vp]
        L.w4a8_quant_act_fp8_per_token.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp, _vp]
        L.w4a8_quant_bf16_to_mxfp4.argtypes = [_vp, _i64, _i64, _int, _vp, _vp, _vp, _vp]
        L.w4a8_quant_bf16_to_mxfp4.restype = _int
        L.w4a8_quant_fp8ch_to_mxfp4.argtypes = [_vp, _vp, _i64, _i64, _int, _vp, _vp, _vp, _vp]
        L.w4a8_quant_fp8ch_to_mxfp4.restype = _int
        L.w4a8_requant_nvfp4_to_mxfp4_prepared.argtypes = [_vp, _vp, _vp, _vp, _int, _i64, _int, _vp, _vp, _vp]
        L.w4a8_requant_nvfp4_to_mxfp4_prepared.restype = _int
        L.w4a8_quant_bf16_to_mxfp4_prepared.argtypes = [_vp, _i64, _i64, _int, _vp, _vp, _vp]
        L.w4a8_quant_bf16_to_mxfp4_prepared.restype = _int
        L.w4a8_quant_fp8ch_to_mxfp4_prepared.argtypes = [_vp, _vp, _i64, _i64, _int, _vp, _vp, _vp]
        L.w4a8_quant_fp8ch_to_mxfp4_prepared.restype = _int
        L.w4a8_gemm_workspace_bytes.argtypes = [_i64, _i64, _i64, _int]
        L.w4a8_gemm_workspace_bytes.restype = _size
        L.w4a8_workspace_init.argtypes = [_vp, _size, _vp]
        L.w4a8_mxfp4_gemm.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _size, _vp]
        L.w4a8_int4g128_prepare.argtypes = [_vp, _vp, _i64, _i64, _vp, _vp]
        L.w4a8_int4g128_gemm.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _size, _vp]
        L.w4a8_decode_plan_workspace_bytes.argtypes = [_i64, _i64, _i64, _int, _int, _int]
        L.w4a8_decode_plan_workspace_bytes.restype = _size
        L.w4a8_decode_with_plan.argtypes = [_int, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _int,
                                            _int, _int, _vp, _size, _vp]
        L.w4a8_decode_with_plan.restype = _int
        L.w4a8_mxfp4_prepared_bytes.argtypes = [_i64, _i64, ctypes.POINTER(_size), ctypes.POINTER(_size)]
        L.w4a8_mxfp4_prepared_bytes.restype = _int
        L.w4a8_mxfp4_prepare.argtypes = [_vp, _vp, _i64, _i64, _vp, _vp, _vp]
        L.w4a8_mxfp4_prepare.restype = _int
        L.w4a8_mxfp4_gemm_prepared.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _size, _vp]
        L.w4a8_mxfp4_gemm_prepared.restype = _int
        L.w4a8_mxfp4_gemm_prepared_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp]
        L.w4a8_mxfp4_gemm_prepared_noalloc.restype = _int
        L.w4a8_mxfp4_gemm_prepared_noalloc_max_scratch.argtypes = []
        L.w4a8_mxfp4_gemm_prepared_noalloc_max_scratch.restype = _size
        for f in ("w4a8_mxfp4_linear_prepared", "w4a8_int4g128_linear_prepared"):
            getattr(L, f).argtypes = [_vp, _i64, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _size, _vp]
            getattr(L, f).restype = _int
        L.w4a8_w4a4_gemm_prepared.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _size, _vp]
        L.w4a8_w4a4_gemm_prepared.restype = _int
        L.w4a8_int4g128_prepared_bytes.argtypes = [_i64, _i64, ctypes.POINTER(_size),
                                                   ctypes.POINTER(_size)]
        L.w4a8_int4g128_prepared_bytes.restype = _int
        L.w4a8_int4g128_prepare_fragments.argtypes = [_vp, _vp, _vp, _i64, _i64, _vp, _vp, _vp]
        L.w4a8_int4g128_prepare_fragments.restype = _int
        L.w4a8_int4g128_zp_prepared_bytes.argtypes = [_i64, _i64, ctypes.POINTER(_size), ctypes.POINTER(_size)]
        L.w4a8_int4g128_zp_prepared_bytes.restype = _int
        L.w4a8_int4g128_zp_prepare_fragments.argtypes = [_vp, _vp, _vp, _i64, _i64, _vp, _vp, _vp]
        L.w4a8_int4g128_zp_prepare_fragments.restype = _int
        L.w4a8_int4g128_zp_gemm_prepared.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _size, _vp]
        L.w4a8_int4g128_zp_gemm_prepared.restype = _int
        L.w4a8_int5g128_prepared_bytes.argtypes = [_i64, _i64, ctypes.POINTER(_size), ctypes.POINTER(_size),
                                                   ctypes.POINTER(_size)]
        L.w4a8_int5g128_prepared_bytes.restype = _int
        L.w4a8_int5g128_prepare_fragments.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _vp, _vp, _vp, _vp]
        L.w4a8_int5g128_prepare_fragments.restype = _int
        L.w4a8_int5g128_gemm_prepared.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _size,
                                                  _vp]
        L.w4a8_int5g128_gemm_prepared.restype = _int
        L.w4a8_int4g128_gemm_prepared.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp,
                                                  _size, _vp]
        L.w4a8_int4g128_gemm_prepared.restype = _int
        L.w4a8_status_string.argtypes = [_int]
        L.w4a8_status_string.restype = ctypes.c_char_p
        L.w4a8_version.argtypes = []
        L.w4a8_version.restype = ctypes.c_char_p
        for name in ("w4a8_requant_nvfp4_to_mxfp4", "w4a8_quant_act_fp8_per_token",
                     "w4a8_workspace_init", "w4a8_mxfp4_gemm", "w4a8_int4g128_prepare",
                     "w4a8_int4g128_gemm"):
            getattr(L, name).restype = _int
        _lib = L
    return _lib


def version() -> str:
    return lib().w4a8_version().decode()


def status_string(status: int) -> str:
    return lib().w4a8_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status == OK:
        return
    if status == ERR_HIP:
        raise W4A8Error(status, what)
    raise ValueError(f"{what}: {status_string(status)} (status {status})")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


# ---------------------------------------------------------------------------
# load time: NVFP4 -> MXFP4
# ---------------------------------------------------------------------------

def requant_nvfp4_to_mxfp4(nv_packed: torch.Tensor, nv_scale: torch.Tensor, part_rows,
                           part_divisor, mode: str = "mse", row_chunk: int = 0,
                           out_packed: torch.Tensor | None = None,
                           out_e8m0: torch.Tensor | None = None, stats: bool = False):
    """NVFP4 [rows, K/2] u8 codes + [rows, K/16] u8 e4m3 scales -> MXFP4 codes
    [rows, K/2] u8 and e8m0 [rows, K/32] u8.  part_rows / part_divisor: row count
    and stored global divisor (6*448/amax) of each partition of a merged linear.
    With stats=True also returns a float64 [n_parts, 2] tensor of
    (sum of squared block errors, sum of w^2) per partition."""
    _need(nv_packed, "nv_packed", torch.uint8)
    _need(nv_scale, "nv_scale", torch.uint8, nv_packed.device)
    if nv_packed.dim() != 2 or nv_scale.dim() != 2:
        raise ValueError("nv_packed and nv_scale must be 2-D")
    rows, half = nv_packed.shape
    K = 2 * half
    if tuple(nv_scale.shape) != (rows, K // 16) or K % 16:
        raise ValueError("nv_scale must be [rows, K/16]")
    if not (nv_packed.is_contiguous() and nv_scale.is_contiguous()):
        raise ValueError("inputs must be contiguous")
    pr = (ctypes.c_int64 * len(part_rows))(*[int(r) for r in part_rows])
    pd = (ctypes.c_float * len(part_divisor))(*[float(d) for d in part_divisor])
    if len(part_rows) != len(part_divisor):
        raise ValueError("part_rows and part_divisor differ in length")
    if sum(int(r) for r in part_rows) != rows:
        raise ValueError(f"partition rows {list(part_rows)} do not add up to {rows}")
    dev = nv_packed.device
    if out_packed is None:
        out_packed = torch.empty((rows, half), dtype=torch.uint8, device=dev)
    if out_e8m0 is None:
        out_e8m0 = torch.empty((rows, max(K // 32, 0)), dtype=torch.uint8, device=dev)
    _need(out_packed, "out_packed", torch.uint8, dev)
    _need(out_e8m0, "out_e8m0", torch.uint8, dev)
    st = torch.empty((len(part_rows), 2), dtype=torch.float64, device=dev) if stats else None
    if mode not in EXP_MODES:
        raise ValueError(f"mode must be one of {sorted(EXP_MODES)}")
    status = lib().w4a8_requant_nvfp4_to_mxfp4(
        _ptr(nv_packed), _ptr(nv_scale), pr, pd, len(part_rows), K, EXP_MODES[mode],
        int(row_chunk), _ptr(out_packed), _ptr(out_e8m0), _ptr(st), _stream(nv_packed))
    _check(status, "w4a8_requant_nvfp4_to_mxfp4")
    return (out_packed, out_e8m0, st) if stats else (out_packed, out_e8m0)


def _load_outputs(rows, K, dev, out_packed, out_e8m0, stats, mode):
    if mode not in EXP_MODES:
        raise ValueError(f"mode must be one of {sorted(EXP_MODES)}")
    if out_packed is None:
        out_packed = torch.empty((rows, K // 2), dtype=torch.uint8, device=dev)
    if out_e8m0 is None:
        out_e8m0 = torch.empty((rows, K // 32), dtype=torch.uint8, device=dev)
    _need(out_packed, "out_packed", torch.uint8, dev)
    _need(out_e8m0, "out_e8m0", torch.uint8, dev)
    if tuple(out_packed.shape) != (rows, K // 2) or tuple(out_e8m0.shape) != (rows, K // 32):
        raise ValueError("outputs must be [rows, K/2] and [rows, K/32]")
    st = torch.empty(2, dtype=torch.float64, device=dev) if stats else None
    return out_packed, out_e8m0, st


def quant_bf16_to_mxfp4(w: torch.Tensor, mode: str = "mse", out_packed: torch.Tensor | None = None,
                        out_e8m0: torch.Tensor | None = None, stats: bool = False):
    """bf16 weight [rows, K] -> MXFP4 codes [rows, K/2] u8 and e8m0 [rows, K/32] u8
    (with stats=True also float64 [2]: sum of squared block errors, sum of w^2)."""
    _need(w, "w", torch.bfloat16)
    if w.dim() != 2 or not w.is_contiguous():
        raise ValueError("w must be a contiguous 2-D tensor")
    rows, K = w.shape
    out_packed, out_e8m0, st = _load_outputs(rows, K, w.device, out_packed, out_e8m0, stats, mode)
    status = lib().w4a8_quant_bf16_to_mxfp4(_ptr(w), rows, K, EXP_MODES[mode], _ptr(out_packed),
                                            _ptr(out_e8m0), _ptr(st), _stream(w))
    _check(status, "w4a8_quant_bf16_to_mxfp4")
    return (out_packed, out_e8m0, st) if stats else (out_packed, out_e8m0)


def quant_fp8ch_to_mxfp4(w8: torch.Tensor, row_scale: torch.Tensor, mode: str = "mse",
                         out_packed: torch.Tensor | None = None, out_e8m0: torch.Tensor | None = None,
                         stats: bool = False):
    """fp8 e4m3 weight [rows, K] (float8_e4m3fn or its uint8 codes) with one fp32
    scale per row ([rows] or [rows, 1]) -> MXFP4 as quant_bf16_to_mxfp4."""
    if isinstance(w8, torch.Tensor) and w8.dtype == torch.float8_e4m3fn:
        w8 = w8.view(torch.uint8)
    _need(w8, "w8", torch.uint8)
    if w8.dim() != 2 or not w8.is_contiguous():
        raise ValueError("w8 must be a contiguous 2-D tensor")
    rows, K = w8.shape
    _need(row_scale, "row_scale", torch.float32, w8.device)
    if row_scale.numel() != rows or not row_scale.is_contiguous():
        raise ValueError("row_scale must hold one contiguous fp32 scale per row")
    out_packed, out_e8m0, st = _load_outputs(rows, K, w8.device, out_packed, out_e8m0, stats, mode)
    status = lib().w4a8_quant_fp8ch_to_mxfp4(_ptr(w8), _ptr(row_scale), rows, K, EXP_MODES[mode],
                                             _ptr(out_packed), _ptr(out_e8m0), _ptr(st), _stream(w8))
    _check(status, "w4a8_quant_fp8ch_to_mxfp4")
    return (out_packed, out_e8m0, st) if stats else (out_packed, out_e8m0)


def _prepared_outputs(rows, K, dev, mode, out=None):
    if mode not in EXP_MODES:
        raise ValueError(f"mode must be one of {sorted(EXP_MODES)}")
    if K % 128:
        raise ValueError("the prepared layout needs K % 128 == 0")
    if out is not None:
        if (out.N, out.K) != (rows, K):
            raise ValueError(f"out holds a {out.N} x {out.K} weight, not {rows} x {K}")
        _check_weight_sizes("prepared", out.w, out.s, rows, K)
        return out.w, out.s
    wb, sb = _size(), _size()
    _check(lib().w4a8_mxfp4_prepared_bytes(rows, K, ctypes.byref(wb), ctypes.byref(sb)),
           "w4a8_mxfp4_prepared_bytes")
    return (torch.empty(wb.value, dtype=torch.uint8, device=dev),
            torch.empty(sb.value, dtype=torch.uint8, device=dev))


def requant_nvfp4_to_mxfp4_prepared(nv_packed: torch.Tensor, nv_scale: torch.Tensor, part_rows,
                                    part_divisor, mode: str = "mse", out=None) -> "PreparedMXFP4":
    """As requant_nvfp4_to_mxfp4, written straight into the GEMM's fragment
    order (the bytes mxfp4_prepare makes of the row-major result); `out`: a
    PreparedMXFP4 of the same shape to write into."""
    _need(nv_packed, "nv_packed", torch.uint8)
    _need(nv_scale, "nv_scale", torch.uint8, nv_packed.device)
    if nv_packed.dim() != 2 or nv_scale.dim() != 2:
        raise ValueError("nv_packed and nv_scale must be 2-D")
    rows, half = nv_packed.shape
    K = 2 * half
    if tuple(nv_scale.shape) != (rows, K // 16) or not (nv_packed.is_contiguous() and nv_scale.is_contiguous()):
        raise ValueError("nv_scale must be [rows, K/16], both contiguous")
    if len(part_rows) != len(part_divisor) or sum(int(r) for r in part_rows) != rows:
        raise ValueError("partition rows must add up to the rows, one divisor each")
    pr = (ctypes.c_int64 * len(part_rows))(*[int(r) for r in part_rows])
    pd = (ctypes.c_float * len(part_divisor))(*[float(d) for d in part_divisor])
    wt, st = _prepared_outputs(rows, K, nv_packed.device, mode, out)
    _check(lib().w4a8_requant_nvfp4_to_mxfp4_prepared(_ptr(nv_packed), _ptr(nv_scale), pr, pd, len(part_rows), K,
                                                       EXP_MODES[mode], _ptr(wt), _ptr(st), _stream(nv_packed)),
           "w4a8_requant_nvfp4_to_mxfp4_prepared")
    return PreparedMXFP4(wt, st, rows, K)


def quant_bf16_to_mxfp4_prepared(w: torch.Tensor, mode: str = "mse", out=None) -> "PreparedMXFP4":
    """As quant_bf16_to_mxfp4, written straight into fragment order."""
    _need(w, "w", torch.bfloat16)
    if w.dim() != 2 or not w.is_contiguous():
        raise ValueError("w must be a contiguous 2-D tensor")
    rows, K = w.shape
    wt, st = _prepared_outputs(rows, K, w.device, mode, out)
    _check(lib().w4a8_quant_bf16_to_mxfp4_prepared(_ptr(w), rows, K, EXP_MODES[mode], _ptr(wt), _ptr(st),
                                                    _stream(w)), "w4a8_quant_bf16_to_mxfp4_prepared")
    return PreparedMXFP4(wt, st, rows, K)


def quant_fp8ch_to_mxfp4_prepared(w8: torch.Tensor, row_scale: torch.Tensor, mode: str = "mse",
                                  out=None) -> "PreparedMXFP4":
    """As quant_fp8ch_to_mxfp4, written straight into fragment order."""
    if isinstance(w8, torch.Tensor) and w8.dtype == torch.float8_e4m3fn:
        w8 = w8.view(torch.uint8)
    _need(w8, "w8", torch.uint8)
    if w8.dim() != 2 or not w8.is_contiguous():
        raise ValueError("w8 must be a contiguous 2-D tensor")
    rows, K = w8.shape
    _need(row_scale, "row_scale", torch.float32, w8.device)
    if row_scale.numel() != rows or not row_scale.is_contiguous():
        raise ValueError("row_scale must hold one contiguous fp32 scale per row")
    wt, st = _prepared_outputs(rows, K, w8.device, mode, out)
    _check(lib().w4a8_quant_fp8ch_to_mxfp4_prepared(_ptr(w8), _ptr(row_scale), rows, K, EXP_MODES[mode], _ptr(wt),
                                                     _ptr(st), _stream(w8)), "w4a8_quant_fp8ch_to_mxfp4_prepared")
    return PreparedMXFP4(wt, st, rows, K)


# ---------------------------------------------------------------------------
# run time
# ---------------------------------------------------------------------------

def quant_act_fp8_per_token(x: torch.Tensor, out: torch.Tensor | None = None,
                            scale: torch.Tensor | None = None):
    """bf16 [M, K] (rows may be strided) -> (e4m3 codes u8 [M, K], fp32 scales [M])."""
    _need(x, "x", torch.bfloat16)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    M, K = x.shape
    dev = x.device
    if out is None:
        out = torch.empty((M, K), dtype=torch.uint8, device=dev)
    if scale is None:
        scale = torch.empty((M,), dtype=torch.float32, device=dev)
    _need(out, "out", torch.uint8, dev)
    _need(scale, "scale", torch.float32, dev)
    status = lib().w4a8_quant_act_fp8_per_token(_ptr(x), M, K, x.stride(0), _ptr(out),
                                                _ptr(scale), _stream(x))
    _check(status, "w4a8_quant_act_fp8_per_token")
    return out, scale


def gemm_workspace_bytes(M_max: int, N: int, K: int, kind: str = "mxfp4") -> int:
    return int(lib().w4a8_gemm_workspace_bytes(int(M_max), int(N), int(K), _KINDS[kind]))


class Workspace:
    """Caller-owned split-K workspace for GEMMs with M <= M_max on one (N, K).
    Allocated by torch and zeroed once; every GEMM leaves its counters at zero."""

    def __init__(self, M_max: int, N: int, K: int, kind: str = "mxfp4", device="cuda"):
        self.nbytes = gemm_workspace_bytes(M_max, N, K, kind)
        self.buf = None
        if self.nbytes:
            self.buf = torch.empty((self.nbytes + 255) // 256 * 256, dtype=torch.uint8,
                                   device=device)
            status = lib().w4a8_workspace_init(_ptr(self.buf), self.buf.numel(),
                                               _stream(self.buf))
            _check(status, "w4a8_workspace_init")

    def args(self):
        if self.buf is None:
            return None, 0
        return _ptr(self.buf), self.buf.numel()


def _ws_args(workspace, M, N, K, kind, device):
    if workspace is None:
        need = gemm_workspace_bytes(M, N, K, kind)
        if need == 0:
            return None, 0, None
        workspace = Workspace(M, N, K, kind, device)
    p, n = workspace.args()
    return p, n, workspace


def mxfp4_gemm(x_fp8: torch.Tensor, x_scale: torch.Tensor, w_packed: torch.Tensor,
               w_e8m0: torch.Tensor, out: torch.Tensor | None = None,
               workspace: Workspace | None = None) -> torch.Tensor:
    """out[M, N] bf16 = s_m * (e4m3 x) @ (e2m1 w * 2^(e8m0 - 127))^T."""
    _need(x_fp8, "x_fp8", torch.uint8)
    dev = x_fp8.device
    _need(x_scale, "x_scale", torch.float32, dev)
    _need(w_packed, "w_packed", torch.uint8, dev)
    _need(w_e8m0, "w_e8m0", torch.uint8, dev)
    M, K = x_fp8.shape
    N = w_packed.shape[0]
    if tuple(w_packed.shape) != (N, K // 2) or tuple(w_e8m0.shape) != (N, K // 32):
        raise ValueError("weight shapes must be [N, K/2] and [N, K/32]")
    if x_scale.numel() != M:
        raise ValueError("x_scale must hold M values")
    for t, n in ((x_fp8, "x_fp8"), (w_packed, "w_packed"), (w_e8m0, "w_e8m0"), (x_scale, "x_scale")):
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, dev)
    wp, wn, _keep = _ws_args(workspace, M, N, K, "mxfp4", dev)
    status = lib().w4a8_mxfp4_gemm(_ptr(x_fp8), _ptr(x_scale), _ptr(w_packed), _ptr(w_e8m0),
                                   _ptr(out), M, N, K, wp, wn, _stream(x_fp8))
    _check(status, "w4a8_mxfp4_gemm")
    return out


def int4g128_prepare(qweight_kn: torch.Tensor, qzeros: torch.Tensor) -> torch.Tensor:
    """AutoGPTQ qweight [K/8, N] int32 -> [N, K/8] int32 after checking that every
    qzeros word is 0x77777777 (synchronizes the stream; load time)."""
    _need(qweight_kn, "qweight", torch.int32)
    dev = qweight_kn.device
    _need(qzeros, "qzeros", torch.int32, dev)
    K8, N = qweight_kn.shape
    K = 8 * K8
    out = torch.empty((N, K8), dtype=torch.int32, device=dev)
    status = lib().w4a8_int4g128_prepare(_ptr(qweight_kn), _ptr(qzeros), N, K, _ptr(out),
                                         _stream(qweight_kn))
    _check(status, "w4a8_int4g128_prepare")
    return out


def int4g128_gemm(x_fp8: torch.Tensor, x_scale: torch.Tensor, qweight_nk: torch.Tensor,
                  scales: torch.Tensor, out: torch.Tensor | None = None,
                  workspace: Workspace | None = None) -> torch.Tensor:
    """out[M, N] bf16 = s_m * (e4m3 x) @ ((c - 8) * scale[k/128, n])^T."""
    _need(x_fp8, "x_fp8", torch.uint8)
    dev = x_fp8.device
    _need(x_scale, "x_scale", torch.float32, dev)
    _need(qweight_nk, "qweight_nk", torch.int32, dev)
    _need(scales, "scales", torch.float16, dev)
    M, K = x_fp8.shape
    N = qweight_nk.shape[0]
    if tuple(qweight_nk.shape) != (N, K // 8) or tuple(scales.shape) != (K // 128, N):
        raise ValueError("shapes must be qweight [N, K/8] and scales [K/128, N]")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, dev)
    wp, wn, _keep = _ws_args(workspace, M, N, K, "int4", dev)
    status = lib().w4a8_int4g128_gemm(_ptr(x_fp8), _ptr(x_scale), _ptr(qweight_nk), _ptr(scales),
                                      _ptr(out), M, N, K, wp, wn, _stream(x_fp8))
    _check(status, "w4a8_int4g128_gemm")
    return out


def _check_weight_sizes(kind, w, w_scale, N, K):
    """The C ABI takes raw pointers: make sure the tensors really hold [N, K] weights."""
    if kind == "mxfp4":
        ok = tuple(w.shape) == (N, K // 2) and tuple(w_scale.shape) == (N, K // 32)
    elif kind == "int4":
        ok = tuple(w.shape) == (N, K // 8) and tuple(w_scale.shape) == (K // 128, N)
    else:
        fn = {"prepared": "w4a8_mxfp4_prepared_bytes", "int4_prepared": "w4a8_int4g128_prepared_bytes",
              "int4_zp_prepared": "w4a8_int4g128_zp_prepared_bytes"}[kind]
        wb, sb = _size(), _size()
        _check(getattr(lib(), fn)(N, K, ctypes.byref(wb), ctypes.byref(sb)), fn)
        ok = (w.numel() * w.element_size() == wb.value and
              w_scale.numel() * w_scale.element_size() == sb.value)
    if not ok:
        raise ValueError(f"{kind} weight tensors do not match N={N}, K={K}")


def decode_with_plan(x_fp8, x_scale, w, w_scale, rt: int, u: int, ks: int, kind: str = "mxfp4",
                     out=None, workspace=None, N: int | None = None):
    """Decode-band GEMM (M <= 64) with an explicit plan (for tile sweeps): rt 16-row
    weight tiles per wave, u 128-wide K steps per chunk, ks requested K splits
    (kind "prepared": rt 0, u the prefetch depth, N required).  `workspace` is a
    uint8 cuda tensor of at least the plan's workspace bytes, zeroed before its
    first use (its split-K arrival counters)."""
    M, K = x_fp8.shape
    if N is None:
        if kind == "prepared":
            raise ValueError("prepared weights need N")
        N = w.shape[0]
    _check_weight_sizes(kind, w, w_scale, int(N), int(K))
    dev = x_fp8.device
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    need = int(lib().w4a8_decode_plan_workspace_bytes(M, N, K, rt, u, ks))
    if need and (workspace is None or workspace.numel() < need):
        # zeroed: the split-K arrival counters start at zero (and stay there between calls)
        workspace = torch.zeros((need + 255) // 256 * 256, dtype=torch.uint8, device=dev)
    status = lib().w4a8_decode_with_plan(_KINDS[kind], _ptr(x_fp8), _ptr(x_scale), _ptr(w), _ptr(w_scale),
                                         _ptr(out), M, N, K, rt, u, ks, _ptr(workspace),
                                         0 if workspace is None else workspace.numel(),
                                         _stream(x_fp8))
    _check(status, "w4a8_decode_with_plan")
    return out


class PreparedMXFP4:
    """MXFP4 weight of one linear in matrix-core fragment order (w4a8_mxfp4_prepare)."""

    def __init__(self, w: torch.Tensor, s: torch.Tensor, N: int, K: int):
        self.w, self.s, self.N, self.K = w, s, int(N), int(K)


def mxfp4_prepare(w_packed: torch.Tensor, w_e8m0: torch.Tensor, out: "PreparedMXFP4 | None" = None) -> PreparedMXFP4:
    """[N, K/2] codes + [N, K/32] e8m0 -> PreparedMXFP4 (K % 128 == 0); `out`:
    a PreparedMXFP4 of the same shape to write into."""
    _need(w_packed, "w_packed", torch.uint8)
    dev = w_packed.device
    _need(w_e8m0, "w_e8m0", torch.uint8, dev)
    N, K = w_packed.shape[0], 2 * w_packed.shape[1]
    if tuple(w_e8m0.shape) != (N, K // 32):
        raise ValueError("w_e8m0 must be [N, K/32]")
    if out is not None:
        if (out.N, out.K) != (N, K):
            raise ValueError(f"out holds a {out.N} x {out.K} weight, not {N} x {K}")
        _check_weight_sizes("prepared", out.w, out.s, N, K)
        wt, st = out.w, out.s
    else:
        wb, sb = _size(), _size()
        _check(lib().w4a8_mxfp4_prepared_bytes(N, K, ctypes.byref(wb), ctypes.byref(sb)),
               "w4a8_mxfp4_prepared_bytes")
        wt = torch.empty(wb.value, dtype=torch.uint8, device=dev)
        st = torch.empty(sb.value, dtype=torch.uint8, device=dev)
    _check(lib().w4a8_mxfp4_prepare(_ptr(w_packed), _ptr(w_e8m0), N, K, _ptr(wt), _ptr(st),
                                    _stream(w_packed)), "w4a8_mxfp4_prepare")
    return PreparedMXFP4(wt, st, N, K)


def mxfp4_gemm_prepared(x_fp8: torch.Tensor, x_scale: torch.Tensor, w: PreparedMXFP4,
                        out: torch.Tensor | None = None,
                        workspace: Workspace | None = None) -> torch.Tensor:
    """As mxfp4_gemm, on prepared weights (any M >= 1)."""
    _need(x_fp8, "x_fp8", torch.uint8)
    dev = x_fp8.device
    _need(x_scale, "x_scale", torch.float32, dev)
    M, K = x_fp8.shape
    if K != w.K:
        raise ValueError(f"activation K {K} != weight K {w.K}")
    _check_weight_sizes("prepared", w.w, w.s, w.N, w.K)
    if out is None:
        out = torch.empty((M, w.N), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, dev)
    wp, wn, _keep = _ws_args(workspace, M, w.N, K, "prepared", dev)
    status = lib().w4a8_mxfp4_gemm_prepared(_ptr(x_fp8), _ptr(x_scale), _ptr(w.w), _ptr(w.s),
                                            _ptr(out), M, w.N, K, wp, wn, _stream(x_fp8))
    _check(status, "w4a8_mxfp4_gemm_prepared")
    return out


def mxfp4_gemm_prepared_noalloc(x_fp8: torch.Tensor, x_scale: torch.Tensor, w: PreparedMXFP4,
                                out: torch.Tensor) -> torch.Tensor:
    """As mxfp4_gemm_prepared with the library's static split-K scratch (no
    workspace, nothing allocated by the call: `out` is required)."""
    _need(x_fp8, "x_fp8", torch.uint8)
    dev = x_fp8.device
    _need(x_scale, "x_scale", torch.float32, dev)
    M, K = x_fp8.shape
    if K != w.K:
        raise ValueError(f"activation K {K} != weight K {w.K}")
    _check_weight_sizes("prepared", w.w, w.s, w.N, w.K)
    _need(out, "out", torch.bfloat16, dev)
    if tuple(out.shape) != (M, w.N) or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous [{M}, {w.N}] tensor")
    status = lib().w4a8_mxfp4_gemm_prepared_noalloc(_ptr(x_fp8), _ptr(x_scale), _ptr(w.w), _ptr(w.s),
                                                    _ptr(out), M, w.N, K, _stream(x_fp8))
    _check(status, "w4a8_mxfp4_gemm_prepared_noalloc")
    return out


class PreparedInt4:
    """int4 g128 weight of one linear in matrix-core fragment order
    (w4a8_int4g128_prepare_fragments)."""

    def __init__(self, w: torch.Tensor, s: torch.Tensor, N: int, K: int):
        self.w, self.s, self.N, self.K = w, s, int(N), int(K)


def int4g128_prepare_fragments(qweight_kn: torch.Tensor, qzeros: torch.Tensor,
                               scales: torch.Tensor) -> PreparedInt4:
    """Checkpoint qweight [K/8, N] int32, qzeros [K/128, N/8] int32 (all 0x77777777),
    scales [K/128, N] fp16 -> PreparedInt4 (synchronizes the stream; load time)."""
    _need(qweight_kn, "qweight", torch.int32)
    dev = qweight_kn.device
    _need(qzeros, "qzeros", torch.int32, dev)
    _need(scales, "scales", torch.float16, dev)
    K8, N = qweight_kn.shape
    K = 8 * K8
    if tuple(qzeros.shape) != (K // 128, N // 8) or tuple(scales.shape) != (K // 128, N):
        raise ValueError("shapes must be qweight [K/8, N], qzeros [K/128, N/8], scales [K/128, N]")
    wb, sb = _size(), _size()
    _check(lib().w4a8_int4g128_prepared_bytes(N, K, ctypes.byref(wb), ctypes.byref(sb)),
           "w4a8_int4g128_prepared_bytes")
    wt = torch.empty(wb.value, dtype=torch.uint8, device=dev)
    st = torch.empty(sb.value, dtype=torch.uint8, device=dev)
    _check(lib().w4a8_int4g128_prepare_fragments(_ptr(qweight_kn), _ptr(qzeros), _ptr(scales), N, K,
                                                 _ptr(wt), _ptr(st), _stream(qweight_kn)),
           "w4a8_int4g128_prepare_fragments")
    return PreparedInt4(wt, st, N, K)


class PreparedInt4ZP(PreparedInt4):
    """int4 g128 weight with zero points, fragment order
    (w4a8_int4g128_zp_prepare_fragments)."""


def int4g128_zp_prepare_fragments(qweight_kn: torch.Tensor, qzeros: torch.Tensor,
                                  scales: torch.Tensor) -> PreparedInt4ZP:
    """Checkpoint qweight [K/8, N] int32, qzeros [K/128, N/8] int32 (any zero
    points, each stored minus one), scales [K/128, N] fp16 -> PreparedInt4ZP."""
    _need(qweight_kn, "qweight", torch.int32)
    dev = qweight_kn.device
    _need(qzeros, "qzeros", torch.int32, dev)
    _need(scales, "scales", torch.float16, dev)
    K8, N = qweight_kn.shape
    K = 8 * K8
    if tuple(qzeros.shape) != (K // 128, N // 8) or tuple(scales.shape) != (K // 128, N):
        raise ValueError("shapes must be qweight [K/8, N], qzeros [K/128, N/8], scales [K/128, N]")
    wb, sb = _size(), _size()
    _check(lib().w4a8_int4g128_zp_prepared_bytes(N, K, ctypes.byref(wb), ctypes.byref(sb)),
           "w4a8_int4g128_zp_prepared_bytes")
    wt = torch.empty(wb.value, dtype=torch.uint8, device=dev)
    st = torch.empty(sb.value, dtype=torch.uint8, device=dev)
    _check(lib().w4a8_int4g128_zp_prepare_fragments(_ptr(qweight_kn), _ptr(qzeros), _ptr(scales), N, K,
                                                    _ptr(wt), _ptr(st), _stream(qweight_kn)),
           "w4a8_int4g128_zp_prepare_fragments")
    return PreparedInt4ZP(wt, st, N, K)


def int4g128_zp_gemm_prepared(x_fp8: torch.Tensor, x_scale: torch.Tensor, w: PreparedInt4ZP,
                              out: torch.Tensor | None = None,
                              workspace: Workspace | None = None) -> torch.Tensor:
    """The asymmetric int4 g128 GEMM on prepared weights (any M >= 1)."""
    _need(x_fp8, "x_fp8", torch.uint8)
    dev = x_fp8.device
    _need(x_scale, "x_scale", torch.float32, dev)
    M, K = x_fp8.shape
    if K != w.K:
        raise ValueError(f"activation K {K} != weight K {w.K}")
    _check_weight_sizes("int4_zp_prepared", w.w, w.s, w.N, w.K)
    if out is None:
        out = torch.empty((M, w.N), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, dev)
    wp, wn, _keep = _ws_args(workspace, M, w.N, K, "int4_zp_prepared", dev)
    status = lib().w4a8_int4g128_zp_gemm_prepared(_ptr(x_fp8), _ptr(x_scale), _ptr(w.w), _ptr(w.s),
                                                  _ptr(out), M, w.N, K, wp, wn, _stream(x_fp8))
    _check(status, "w4a8_int4g128_zp_gemm_prepared")
    return out


class PreparedInt5:
    """int5 g128 weight in fragment order (w4a8_int5g128_prepare_fragments):
    codes' low bits, the fifth-bit plane, scale and zero records."""

    def __init__(self, w: torch.Tensor, w5: torch.Tensor, s: torch.Tensor, N: int, K: int):
        self.w, self.w5, self.s, self.N, self.K = w, w5, s, int(N), int(K)


def _int5_sizes(N, K):
    wb, w5b, sb = _size(), _size(), _size()
    _check(lib().w4a8_int5g128_prepared_bytes(N, K, ctypes.byref(wb), ctypes.byref(w5b), ctypes.byref(sb)),
           "w4a8_int5g128_prepared_bytes")
    return wb.value, w5b.value, sb.value


def int5g128_prepare_fragments(qweight_kn: torch.Tensor, qweight_hi: torch.Tensor, qzeros: torch.Tensor,
                               scales: torch.Tensor) -> PreparedInt5:
    """int5 g128: low bits qweight [K/8, N] int32, fifth bits qweight_hi [K/32, N]
    int32, zero points minus one qzeros [K/128, N] uint8, scales [K/128, N] fp16
    -> PreparedInt5."""
    _need(qweight_kn, "qweight", torch.int32)
    dev = qweight_kn.device
    _need(qweight_hi, "qweight_hi", torch.int32, dev)
    _need(qzeros, "qzeros", torch.uint8, dev)
    _need(scales, "scales", torch.float16, dev)
    K8, N = qweight_kn.shape
    K = 8 * K8
    if (tuple(qweight_hi.shape) != (K // 32, N) or tuple(qzeros.shape) != (K // 128, N)
            or tuple(scales.shape) != (K // 128, N)):
        raise ValueError("shapes must be qweight [K/8, N], qweight_hi [K/32, N], qzeros [K/128, N], "
                         "scales [K/128, N]")
    wb, w5b, sb = _int5_sizes(N, K)
    wt = torch.empty(wb, dtype=torch.uint8, device=dev)
    w5 = torch.empty(w5b, dtype=torch.uint8, device=dev)
    st = torch.empty(sb, dtype=torch.uint8, device=dev)
    _check(lib().w4a8_int5g128_prepare_fragments(_ptr(qweight_kn), _ptr(qweight_hi), _ptr(qzeros), _ptr(scales),
                                                 N, K, _ptr(wt), _ptr(w5), _ptr(st), _stream(qweight_kn)),
           "w4a8_int5g128_prepare_fragments")
    return PreparedInt5(wt, w5, st, N, K)


def int5g128_gemm_prepared(x_fp8: torch.Tensor, x_scale: torch.Tensor, w: PreparedInt5,
                           out: torch.Tensor | None = None,
                           workspace: Workspace | None = None) -> torch.Tensor:
    """The int5 g128 GEMM on prepared weights (any M >= 1)."""
    _need(x_fp8, "x_fp8", torch.uint8)
    dev = x_fp8.device
    _need(x_scale, "x_scale", torch.float32, dev)
    M, K = x_fp8.shape
    if K != w.K:
        raise ValueError(f"activation K {K} != weight K {w.K}")
    sizes = _int5_sizes(w.N, w.K)
    if tuple(t.numel() * t.element_size() for t in (w.w, w.w5, w.s)) != sizes:
        raise ValueError("prepared int5 buffers do not match N, K")
    if out is None:
        out = torch.empty((M, w.N), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, dev)
    wp, wn, _keep = _ws_args(workspace, M, w.N, K, "int5_prepared", dev)
    status = lib().w4a8_int5g128_gemm_prepared(_ptr(x_fp8), _ptr(x_scale), _ptr(w.w), _ptr(w.w5), _ptr(w.s),
                                               _ptr(out), M, w.N, K, wp, wn, _stream(x_fp8))
    _check(status, "w4a8_int5g128_gemm_prepared")
    return out


def int4g128_gemm_prepared(x_fp8: torch.Tensor, x_scale: torch.Tensor, w: PreparedInt4,
                           out: torch.Tensor | None = None,
                           workspace: Workspace | None = None) -> torch.Tensor:
    """As int4g128_gemm, on fragment-order weights (any M >= 1)."""
    _need(x_fp8, "x_fp8", torch.uint8)
    dev = x_fp8.device
    _need(x_scale, "x_scale", torch.float32, dev)
    M, K = x_fp8.shape
    if K != w.K:
        raise ValueError(f"activation K {K} != weight K {w.K}")
    _check_weight_sizes("int4_prepared", w.w, w.s, w.N, w.K)
    if out is None:
        out = torch.empty((M, w.N), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, dev)
    wp, wn, _keep = _ws_args(workspace, M, w.N, K, "int4_prepared", dev)
    status = lib().w4a8_int4g128_gemm_prepared(_ptr(x_fp8), _ptr(x_scale), _ptr(w.w), _ptr(w.s),
                                               _ptr(out), M, w.N, K, wp, wn, _stream(x_fp8))
    _check(status, "w4a8_int4g128_gemm_prepared")
    return out


def _linear_prepared(fn, kind, x, w, out, workspace, x8, xs):
    _need(x, "x", torch.bfloat16)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    dev = x.device
    M, K = x.shape
    if K != w.K:
        raise ValueError(f"activation K {K} != weight K {w.K}")
    _check_weight_sizes(kind, w.w, w.s, w.N, w.K)
    if out is None:
        out = torch.empty((M, w.N), dtype=torch.bfloat16, device=dev)
    if x8 is None:
        x8 = torch.empty((M, K), dtype=torch.uint8, device=dev)
    if xs is None:
        xs = torch.empty((M,), dtype=torch.float32, device=dev)
    _need(out, "out", torch.bfloat16, dev)
    _need(x8, "x8", torch.uint8, dev)
    _need(xs, "xs", torch.float32, dev)
    if tuple(x8.shape) != (M, K) or tuple(xs.shape) != (M,) or tuple(out.shape) != (M, w.N):
        raise ValueError("out [M, N], x8 [M, K], xs [M] expected")
    wp, wn, _keep = _ws_args(workspace, M, w.N, K, kind, dev)
    status = getattr(lib(), fn)(_ptr(x), x.stride(0), _ptr(w.w), _ptr(w.s), _ptr(out), M, w.N, K,
                                _ptr(x8), _ptr(xs), wp, wn, _stream(x))
    _check(status, fn)
    return out, x8, xs


def mxfp4_linear_prepared(x: torch.Tensor, w: PreparedMXFP4, out: torch.Tensor | None = None,
                          workspace: Workspace | None = None, x8: torch.Tensor | None = None,
                          xs: torch.Tensor | None = None):
    """The linear on bf16 activations [M, K] (rows may be strided): per-token fp8
    quantization fused with the GEMM on prepared MXFP4 weights ->
    (out bf16 [M, N], e4m3 codes [M, K], token scales [M])."""
    return _linear_prepared("w4a8_mxfp4_linear_prepared", "prepared", x, w, out, workspace, x8, xs)


def int4g128_linear_prepared(x: torch.Tensor, w: PreparedInt4, out: torch.Tensor | None = None,
                             workspace: Workspace | None = None, x8: torch.Tensor | None = None,
                             xs: torch.Tensor | None = None):
    """As mxfp4_linear_prepared, on fragment-order int4 g128 weights."""
    return _linear_prepared("w4a8_int4g128_linear_prepared", "int4_prepared", x, w, out, workspace, x8, xs)


def quant_act_mxfp4(x: torch.Tensor):
    """W4A4 activations: bf16 [M, K] -> (e2m1 codes [M, K/2] u8, e8m0 [M, K/32] u8),
    per token and 32-block by the OCP rule (quant_bf16_to_mxfp4, mode "ocp")."""
    return quant_bf16_to_mxfp4(x, mode="ocp")


def w4a4_gemm_prepared(x_fp4: torch.Tensor, x_e8m0: torch.Tensor, w: PreparedMXFP4,
                       out: torch.Tensor | None = None, workspace: Workspace | None = None) -> torch.Tensor:
    """out[M, N] bf16 = (e2m1 x * 2^(Ex-127)) @ (e2m1 w * 2^(Ew-127))^T on prepared MXFP4 weights."""
    _need(x_fp4, "x_fp4", torch.uint8)
    dev = x_fp4.device
    _need(x_e8m0, "x_e8m0", torch.uint8, dev)
    M, K = x_fp4.shape[0], 2 * x_fp4.shape[1]
    if K != w.K or tuple(x_e8m0.shape) != (M, K // 32):
        raise ValueError(f"activations [M, K/2] + [M, K/32] with K = {w.K} expected")
    if not (x_fp4.is_contiguous() and x_e8m0.is_contiguous()):
        raise ValueError("activations must be contiguous")
    _check_weight_sizes("prepared", w.w, w.s, w.N, w.K)
    if out is None:
        out = torch.empty((M, w.N), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, dev)
    wp, wn, _keep = _ws_args(workspace, M, w.N, K, "w4a4", dev)
    status = lib().w4a8_w4a4_gemm_prepared(_ptr(x_fp4), _ptr(x_e8m0), _ptr(w.w), _ptr(w.s), _ptr(out),
                                           M, w.N, K, wp, wn, _stream(x_fp4))
    _check(status, "w4a8_w4a4_gemm_prepared")
    return out


def w4a8_linear(x: torch.Tensor, w_packed: torch.Tensor, w_e8m0: torch.Tensor,
                workspace: Workspace | None = None) -> torch.Tensor:
    """The layer's run-time path: per-token fp8 quantization, then the MXFP4 GEMM."""
    x2 = x.reshape(-1, x.shape[-1])
    x8, s = quant_act_fp8_per_token(x2)
    out = mxfp4_gemm(x8, s, w_packed, w_e8m0, workspace=workspace)
    return out.reshape(*x.shape[:-1], w_packed.shape[0])

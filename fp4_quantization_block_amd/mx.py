"""ctypes binding of libmx.so (the C ABI in include/mx.h).

Argument marshalling only: every step of quantization, dequantization and
the GEMM runs in the HIP kernels of libmx.so.  PyTorch supplies device
memory and the current HIP stream.  If the library is not built, calls raise
immediately; there is no fallback implementation.
"""
import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmx.so")

MX_OK, MX_ERR_INVALID_ARG, MX_ERR_UNSUPPORTED, MX_ERR_ALIGNMENT, MX_ERR_HIP = range(5)
MX_SRC_F32, MX_SRC_BF16 = 0, 1
MX_E4M3, MX_E5M2, MX_E2M1 = 0, 1, 2
MX_SCALE_E8M0, MX_SCALE_E8M0_TENSOR_F32 = 0, 1
MX_TSCALE_COMPUTE, MX_TSCALE_PROVIDED = 0, 1
MX_RNE, MX_SR = 0, 1
MX_AXIS_ROW, MX_AXIS_COL = 0, 1
MX_OUT_F32, MX_OUT_BF16 = 0, 1

FMTS = {"e4m3": MX_E4M3, "e5m2": MX_E5M2, "e2m1": MX_E2M1}
EXPORTED = ("mx_quantize", "mx_quantize_dual_layout", "mx_gemm", "mx_dequantize",
            "mx_status_string", "mx_last_error_message",
            "mx_predict_tensor_scale", "mx_predict_workspace_bytes", "mx_gemm_quantized",
            "mx_predict_tensor_scale_noalloc", "mx_quantize_optstate", "mx_dequantize_optstate",
            "mx_quantize_nvfp", "mx_dequantize_nvfp", "mx_gemm_nvfp")
NV_PANEL = 32                      # stored rows per CTA-local nvfp scale domain


class MXError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_status_name(status)}: {message}")
        self.status = status


class mx_qconfig(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("block", ctypes.c_int32),
                ("scale_fmt", ctypes.c_int32), ("tscale", ctypes.c_int32),
                ("rounding", ctypes.c_int32), ("hadamard", ctypes.c_int32),
                ("seed", ctypes.c_uint64), ("offset", ctypes.c_uint32),
                ("reserved", ctypes.c_uint32)]


_lib = None
_vp, _i64, _i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32


def load() -> ctypes.CDLL:
    """Load libmx.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    L = ctypes.CDLL(LIB_PATH)
    L.mx_quantize.restype = _i32
    L.mx_quantize.argtypes = [_vp, _i32, _i64, _i64, _i64, _i32, ctypes.POINTER(mx_qconfig),
                              _vp, _vp, _vp, _vp]
    L.mx_quantize_dual_layout.restype = _i32
    L.mx_quantize_dual_layout.argtypes = [_vp, _i32, _i64, _i64, _i64,
                                          ctypes.POINTER(mx_qconfig), _vp, _vp, _vp, _vp, _vp,
                                          _vp]
    L.mx_gemm.restype = _i32
    L.mx_gemm.argtypes = [_vp, _vp, _vp, _i32, _vp, _vp, _vp, _i32, _i64, _i64, _i64,
                          ctypes.c_float, _i32, _vp, _i32, _i64, _vp]
    L.mx_dequantize.restype = _i32
    L.mx_dequantize.argtypes = [_vp, _vp, _vp, _i32, _i64, _i64, _i32, _i32, _vp, _i32, _vp]
    L.mx_gemm_quantized.restype = _i32
    L.mx_gemm_quantized.argtypes = [_vp, _vp, _vp, _i32, _vp, _vp, _vp, _i32, _i64, _i64, _i64,
                                    ctypes.c_float, _i32, _i32, _vp, _vp, _vp]
    L.mx_predict_tensor_scale.restype = _i32
    L.mx_predict_tensor_scale.argtypes = [_vp, _i64, _vp, _i64, _i32, _i64, _i64, ctypes.c_float, _i32,
                                          _vp, _i64, _vp, _vp]
    L.mx_predict_tensor_scale_noalloc.restype = _i32
    L.mx_predict_tensor_scale_noalloc.argtypes = [_vp, _i64, _vp, _i64, _i32, _i64, _i64, ctypes.c_float,
                                                  _i32, _vp, _vp]
    L.mx_quantize_optstate.restype = _i32
    L.mx_quantize_optstate.argtypes = [_vp, _i64, _i32, _i32, _vp, _vp, _vp, _vp]
    L.mx_dequantize_optstate.restype = _i32
    L.mx_dequantize_optstate.argtypes = [_vp, _vp, _vp, _i64, _i32, _i32, _vp, _vp]
    L.mx_quantize_nvfp.restype = _i32
    L.mx_quantize_nvfp.argtypes = [_vp, _i32, _i64, _i64, _i64, _i32, _i32, _vp, _vp, _vp, _vp]
    L.mx_dequantize_nvfp.restype = _i32
    L.mx_dequantize_nvfp.argtypes = [_vp, _vp, _vp, _i64, _i64, _i32, _i32, _vp, _i32, _vp]
    L.mx_gemm_nvfp.restype = _i32
    L.mx_gemm_nvfp.argtypes = [_vp, _vp, _vp, _i32, _vp, _vp, _vp, _i32, _i64, _i64, _i64, ctypes.c_float,
                               _vp, _i32, _i64, _vp]
    L.mx_predict_workspace_bytes.restype = _i64
    L.mx_predict_workspace_bytes.argtypes = []
    L.mx_status_string.restype = ctypes.c_char_p
    L.mx_status_string.argtypes = [_i32]
    L.mx_last_error_message.restype = ctypes.c_char_p
    L.mx_last_error_message.argtypes = []
    _lib = L
    return L


def _status_name(s: int) -> str:
    try:
        return load().mx_status_string(s).decode()
    except Exception:
        return f"status {s}"


def _check(status: int):
    if status != MX_OK:
        raise MXError(status, load().mx_last_error_message().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _fmt(f) -> int:
    return FMTS[f] if isinstance(f, str) else int(f)


def elem_bits(fmt) -> int:
    return 4 if _fmt(fmt) == MX_E2M1 else 8


def qconfig(fmt, two_level=False, tscale_provided=False, sr=False, hadamard=False, seed=0,
            offset=0, block=32) -> mx_qconfig:
    return mx_qconfig(fmt=_fmt(fmt), block=block,
                      scale_fmt=MX_SCALE_E8M0_TENSOR_F32 if two_level else MX_SCALE_E8M0,
                      tscale=MX_TSCALE_PROVIDED if tscale_provided else MX_TSCALE_COMPUTE,
                      rounding=MX_SR if sr else MX_RNE, hadamard=int(bool(hadamard)),
                      seed=seed & 0xFFFFFFFFFFFFFFFF, offset=offset & 0xFFFFFFFF, reserved=0)


def _src(x: torch.Tensor):
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D tensor with unit column stride")
    if x.dtype == torch.float32:
        return MX_SRC_F32
    if x.dtype == torch.bfloat16:
        return MX_SRC_BF16
    raise TypeError("x must be float32 or bfloat16")


def copy_shapes(rows: int, cols: int, axis: int, fmt):
    """(codes shape, scales shape) of a stored copy."""
    bits = elem_bits(fmt)
    if axis == MX_AXIS_ROW:
        return (rows, cols * bits // 8), (rows, cols // 32)
    return (cols, rows * bits // 8), (cols, rows // 32)


def mx_quantize(x: torch.Tensor, axis: int, cfg: mx_qconfig, q: Optional[torch.Tensor] = None,
                scales: Optional[torch.Tensor] = None,
                tensor_scale: Optional[torch.Tensor] = None, stream=None
                ) -> Tuple[torch.Tensor, torch.Tensor, Optional[torch.Tensor]]:
    src = _src(x)
    rows, cols = x.shape
    qs, ss = copy_shapes(rows, cols, axis, cfg.fmt)
    if q is None:
        q = torch.empty(qs, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(ss, dtype=torch.uint8, device=x.device)
    if tensor_scale is None and cfg.scale_fmt == MX_SCALE_E8M0_TENSOR_F32:
        tensor_scale = torch.empty(1, dtype=torch.float32, device=x.device)
    _check(load().mx_quantize(_ptr(x), src, rows, cols, x.stride(0), axis, ctypes.byref(cfg),
                              _ptr(q), _ptr(scales), _ptr(tensor_scale), _stream(stream)))
    return q, scales, tensor_scale


def mx_quantize_dual_layout(x: torch.Tensor, cfg: mx_qconfig, q_row=None, s_row=None,
                            q_col=None, s_col=None, tensor_scale=None, stream=None):
    src = _src(x)
    rows, cols = x.shape
    qrs, srs = copy_shapes(rows, cols, MX_AXIS_ROW, cfg.fmt)
    qcs, scs = copy_shapes(rows, cols, MX_AXIS_COL, cfg.fmt)
    dev = x.device
    q_row = torch.empty(qrs, dtype=torch.uint8, device=dev) if q_row is None else q_row
    s_row = torch.empty(srs, dtype=torch.uint8, device=dev) if s_row is None else s_row
    q_col = torch.empty(qcs, dtype=torch.uint8, device=dev) if q_col is None else q_col
    s_col = torch.empty(scs, dtype=torch.uint8, device=dev) if s_col is None else s_col
    if tensor_scale is None and cfg.scale_fmt == MX_SCALE_E8M0_TENSOR_F32:
        tensor_scale = torch.empty(1, dtype=torch.float32, device=dev)
    _check(load().mx_quantize_dual_layout(_ptr(x), src, rows, cols, x.stride(0),
                                          ctypes.byref(cfg), _ptr(q_row), _ptr(s_row),
                                          _ptr(q_col), _ptr(s_col), _ptr(tensor_scale),
                                          _stream(stream)))
    return q_row, s_row, q_col, s_col, tensor_scale


def mx_gemm(qa, sa, ta, fa, qb, sb, tb, fb, M: int, N: int, K: int, alpha: float = 1.0,
            hadamard_k: bool = False, out_dtype: int = MX_OUT_BF16, c=None, ldc=None,
            stream=None) -> torch.Tensor:
    if c is None:
        c = torch.empty((M, N), dtype=torch.float32 if out_dtype == MX_OUT_F32 else torch.bfloat16,
                        device=qa.device)
    ldc = c.stride(0) if ldc is None else ldc
    _check(load().mx_gemm(_ptr(qa), _ptr(sa), _ptr(ta), _fmt(fa), _ptr(qb), _ptr(sb), _ptr(tb),
                          _fmt(fb), M, N, K, float(alpha), int(bool(hadamard_k)), _ptr(c),
                          out_dtype, ldc, _stream(stream)))
    return c


def mx_gemm_quantized(qa, sa, ta, fa, qb, sb, tb, fb, M: int, N: int, K: int, out_fmt="e4m3",
                      alpha: float = 1.0, hadamard_k: bool = False, qc=None, sc=None, stream=None):
    """GEMM with the output written as MX codes [M][N] and E8M0 scales [M][N/32]."""
    if qc is None:
        qc = torch.empty((M, N), dtype=torch.uint8, device=qa.device)
    if sc is None:
        sc = torch.empty((M, N // 32), dtype=torch.uint8, device=qa.device)
    _check(load().mx_gemm_quantized(_ptr(qa), _ptr(sa), _ptr(ta), _fmt(fa), _ptr(qb), _ptr(sb), _ptr(tb),
                                    _fmt(fb), M, N, K, float(alpha), int(bool(hadamard_k)), _fmt(out_fmt),
                                    _ptr(qc), _ptr(sc), _stream(stream)))
    return qc, sc


def mx_predict_tensor_scale(w: torch.Tensor, g: torch.Tensor, lr: float, fmt,
                            work: Optional[torch.Tensor] = None, scale_out: Optional[torch.Tensor] = None,
                            stream=None) -> torch.Tensor:
    """Predicted per-tensor scale of the next step's weights (weight auto-scaling)."""
    src = _src(w)
    if _src(g) != src or tuple(g.shape) != tuple(w.shape):
        raise ValueError("w and g must have the same dtype and shape")
    rows, cols = w.shape
    nbytes = int(load().mx_predict_workspace_bytes())
    if work is None:
        work = torch.empty(nbytes, dtype=torch.uint8, device=w.device)
    if scale_out is None:
        scale_out = torch.empty(1, dtype=torch.float32, device=w.device)
    _check(load().mx_predict_tensor_scale(_ptr(w), w.stride(0), _ptr(g), g.stride(0), src, rows, cols,
                                          float(lr), _fmt(fmt), _ptr(work), work.numel() * work.element_size(),
                                          _ptr(scale_out), _stream(stream)))
    return scale_out


def mx_predict_tensor_scale_noalloc(w: torch.Tensor, g: torch.Tensor, lr: float, fmt,
                                    scale_out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """mx_predict_tensor_scale without a workspace: the library's per-GPU
    scratch holds the partial maxima (calls overlapping on one GPU race)."""
    src = _src(w)
    if _src(g) != src or tuple(g.shape) != tuple(w.shape):
        raise ValueError("w and g must have the same dtype and shape")
    rows, cols = w.shape
    if scale_out is None:
        scale_out = torch.empty(1, dtype=torch.float32, device=w.device)
    _check(load().mx_predict_tensor_scale_noalloc(_ptr(w), w.stride(0), _ptr(g), g.stride(0), src, rows, cols,
                                                  float(lr), _fmt(fmt), _ptr(scale_out), _stream(stream)))
    return scale_out


def mx_dequantize(q, scales, tensor_scale, fmt, rows: int, cols: int, axis: int,
                  hadamard: bool = False, out_dtype: int = MX_OUT_F32, out=None,
                  stream=None) -> torch.Tensor:
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.float32 if out_dtype == MX_OUT_F32 else torch.bfloat16,
                          device=q.device)
    _check(load().mx_dequantize(_ptr(q), _ptr(scales), _ptr(tensor_scale), _fmt(fmt), rows, cols,
                                axis, int(bool(hadamard)), _ptr(out), out_dtype, _stream(stream)))
    return out


def mx_quantize_optstate(x: torch.Tensor, fmt="e4m3", group: int = 128, q=None, amax=None, kexp=None,
                         stream=None):
    """FP8 codes of an fp32 optimizer state after the per-group dynamic
    range expansion; returns (q uint8 [n], amax fp32 [n/group], k fp32 [n/group])."""
    if x.dtype != torch.float32 or not x.is_contiguous():
        raise TypeError("x must be a contiguous float32 tensor")
    n = x.numel()
    dev = x.device
    q = torch.empty(n, dtype=torch.uint8, device=dev) if q is None else q
    amax = torch.empty(n // group, dtype=torch.float32, device=dev) if amax is None else amax
    kexp = torch.empty(n // group, dtype=torch.float32, device=dev) if kexp is None else kexp
    _check(load().mx_quantize_optstate(_ptr(x), n, group, _fmt(fmt), _ptr(q), _ptr(amax), _ptr(kexp),
                                       _stream(stream)))
    return q, amax, kexp


def mx_dequantize_optstate(q, amax, kexp, fmt="e4m3", group: int = 128, out=None, stream=None) -> torch.Tensor:
    n = q.numel()
    out = torch.empty(n, dtype=torch.float32, device=q.device) if out is None else out
    _check(load().mx_dequantize_optstate(_ptr(q), _ptr(amax), _ptr(kexp), n, group, _fmt(fmt), _ptr(out),
                                         _stream(stream)))
    return out


def nvfp_shapes(rows: int, cols: int, axis: int, local: bool):
    """(codes, block scales, second-level scales) shapes of an nvfp copy."""
    SR, L = (rows, cols) if axis == MX_AXIS_ROW else (cols, rows)
    return (SR, L // 2), (SR, L // 16), ((SR + NV_PANEL - 1) // NV_PANEL if local else 1,)


def mx_quantize_nvfp(x: torch.Tensor, axis: int = MX_AXIS_ROW, local: bool = False, q=None, scales=None,
                     tscale=None, stream=None):
    """NVFP4 copy of x with a global (local=False) or per-32-row-panel
    (local=True) second-level scale; returns (q, scales, tscale)."""
    src = _src(x)
    rows, cols = x.shape
    qs, ss, ts = nvfp_shapes(rows, cols, axis, local)
    dev = x.device
    q = torch.empty(qs, dtype=torch.uint8, device=dev) if q is None else q
    scales = torch.empty(ss, dtype=torch.uint8, device=dev) if scales is None else scales
    tscale = torch.empty(ts, dtype=torch.float32, device=dev) if tscale is None else tscale
    _check(load().mx_quantize_nvfp(_ptr(x), src, rows, cols, x.stride(0), axis, int(bool(local)), _ptr(q),
                                   _ptr(scales), _ptr(tscale), _stream(stream)))
    return q, scales, tscale


def mx_dequantize_nvfp(q, scales, tscale, rows: int, cols: int, axis: int = MX_AXIS_ROW, local: bool = False,
                       out_dtype: int = MX_OUT_F32, out=None, stream=None) -> torch.Tensor:
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.float32 if out_dtype == MX_OUT_F32 else torch.bfloat16,
                          device=q.device)
    _check(load().mx_dequantize_nvfp(_ptr(q), _ptr(scales), _ptr(tscale), rows, cols, axis, int(bool(local)),
                                     _ptr(out), out_dtype, _stream(stream)))
    return out


def mx_gemm_nvfp(qa, sa, ta, local_a: bool, qb, sb, tb, local_b: bool, M: int, N: int, K: int,
                 alpha: float = 1.0, out_dtype: int = MX_OUT_BF16, c=None, ldc=None, stream=None) -> torch.Tensor:
    if c is None:
        c = torch.empty((M, N), dtype=torch.float32 if out_dtype == MX_OUT_F32 else torch.bfloat16,
                        device=qa.device)
    ldc = c.stride(0) if ldc is None else ldc
    _check(load().mx_gemm_nvfp(_ptr(qa), _ptr(sa), _ptr(ta), int(bool(local_a)), _ptr(qb), _ptr(sb), _ptr(tb),
                               int(bool(local_b)), M, N, K, float(alpha), _ptr(c), out_dtype, ldc, _stream(stream)))
    return c

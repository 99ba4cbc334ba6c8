"""CPU oracle for MX quantization and the block-scaled GEMM (numpy front end).

TEST INFRASTRUCTURE.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
library (``fp4_quantization_block_amd``) never imports, links or calls it, and
the two share no code: the arithmetic lives in ``mx_oracle.c`` (plain scalar
C, see the citations there); this module only marshals numpy arrays.

Sources (web pages):
  [MOSS] "MOSS: 用微缩放和自动缩放实现无损 FP8 训练，OLMo-7B 加速 34%"
  [COAT] write-up of "COAT: Compressing Optimizer States and Activation for
         memory efficient FP8 Training"
  [FAF]  "格式感知融合:让FP4预训练提速两倍的工程实践"

Source tensors are numpy arrays: float32 (source dtype fp32) or uint16
holding bfloat16 bit patterns (source dtype bf16).
"""
import ctypes
import os

import numpy as np

E4M3, E5M2, E2M1 = 0, 1, 2
SRC_F32, SRC_BF16 = 0, 1
AXIS_ROW, AXIS_COL = 0, 1
FMT_NAMES = {"e4m3": E4M3, "e5m2": E5M2, "e2m1": E2M1}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle_mx.so")
_lib = None

_i64 = ctypes.c_int64
_vp = ctypes.c_void_p


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    L = ctypes.CDLL(_LIB_PATH)
    L.or_elem_bits.argtypes = [ctypes.c_int]
    L.or_decode.restype = ctypes.c_double
    L.or_decode.argtypes = [ctypes.c_int, ctypes.c_uint]
    L.or_decode_e8m0.restype = ctypes.c_double
    L.or_decode_e8m0.argtypes = [ctypes.c_uint]
    L.or_fmax.restype = ctypes.c_double
    L.or_fmax.argtypes = [ctypes.c_int]
    L.or_emax.argtypes = [ctypes.c_int]
    L.or_encode_rne.restype = ctypes.c_uint
    L.or_encode_rne.argtypes = [ctypes.c_int, ctypes.c_double]
    L.or_encode_sr.restype = ctypes.c_uint
    L.or_encode_sr.argtypes = [ctypes.c_int, ctypes.c_double, ctypes.c_uint32]
    L.or_block_exponent.argtypes = [ctypes.c_int, ctypes.c_double]
    L.or_encode_array.argtypes = [ctypes.c_int, ctypes.c_int, _vp, _vp, _i64, _vp]
    L.or_philox4x32_10.argtypes = [_vp, _vp, _vp]
    L.or_fwht32.argtypes = [_vp]
    L.or_tensor_amax.restype = ctypes.c_float
    L.or_tensor_amax.argtypes = [_vp, ctypes.c_int, _i64, _i64, _i64]
    L.or_tensor_scale.restype = ctypes.c_float
    L.or_tensor_scale.argtypes = [ctypes.c_int, ctypes.c_float]
    L.or_predict_max.restype = ctypes.c_float
    L.or_predict_max.argtypes = [_vp, _vp, ctypes.c_int, _i64, _i64, _i64, _i64, ctypes.c_float]
    L.or_predict_tensor_scale.restype = ctypes.c_float
    L.or_predict_tensor_scale.argtypes = [_vp, _vp, ctypes.c_int, _i64, _i64, _i64, _i64, ctypes.c_float,
                                          ctypes.c_int]
    L.or_round_bf16.restype = ctypes.c_double
    L.or_round_bf16.argtypes = [ctypes.c_double]
    L.or_quantize_block.restype = ctypes.c_uint
    L.or_quantize_block.argtypes = [ctypes.c_int, ctypes.c_int, _vp, _vp, _vp]
    L.or_quantize.argtypes = [_vp, ctypes.c_int, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int,
                              ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_uint64,
                              ctypes.c_uint32, _vp, _vp, _vp, ctypes.c_int]
    L.or_quantize_blocks.argtypes = [_vp, ctypes.c_int, _i64, _i64, _i64, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_uint64, ctypes.c_uint32, _vp, _vp,
                                     _i64, _vp, _vp]
    L.or_dequantize.argtypes = [_vp, _vp, _vp, ctypes.c_int, _i64, _i64, ctypes.c_int,
                                ctypes.c_int, _vp, ctypes.c_int]
    L.or_gemm.argtypes = [_vp, _vp, _vp, ctypes.c_int, _vp, _vp, _vp, ctypes.c_int, _i64, _i64,
                          _i64, ctypes.c_double, ctypes.c_int, _vp, _vp, ctypes.c_int]
    L.or_gemm_entries.argtypes = [_vp, _vp, _vp, ctypes.c_int, _vp, _vp, _vp, ctypes.c_int,
                                  _i64, _i64, _i64, ctypes.c_double, ctypes.c_int, _vp, _vp,
                                  _i64, _vp, _vp, ctypes.c_int]
    L.or_log2_fp32.restype = ctypes.c_float
    L.or_log2_fp32.argtypes = [ctypes.c_float]
    L.or_exp2_fp32.restype = ctypes.c_float
    L.or_exp2_fp32.argtypes = [ctypes.c_float]
    L.or_pow_fp32.restype = ctypes.c_float
    L.or_pow_fp32.argtypes = [ctypes.c_float, ctypes.c_float]
    L.or_optstate_quantize.argtypes = [_vp, _i64, _i64, ctypes.c_int, _vp, _vp, _vp, ctypes.c_int]
    L.or_optstate_dequantize.argtypes = [_vp, _vp, _vp, _i64, _i64, ctypes.c_int, _vp, ctypes.c_int]
    L.or_nvfp_quantize.argtypes = [_vp, ctypes.c_int, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int, _vp, _vp, _vp,
                                   ctypes.c_int]
    L.or_nvfp_dequantize.argtypes = [_vp, _vp, _vp, _i64, _i64, ctypes.c_int, ctypes.c_int, _vp]
    L.or_nvfp_gemm.argtypes = [_vp, _vp, _vp, ctypes.c_int, _vp, _vp, _vp, ctypes.c_int, _i64, _i64, _i64,
                               ctypes.c_double, _vp, _vp, ctypes.c_int]
    L.or_nvfp_gemm_entries.argtypes = [_vp, _vp, _vp, ctypes.c_int, _vp, _vp, _vp, ctypes.c_int, _i64, _i64,
                                       _i64, ctypes.c_double, _vp, _vp, _i64, _vp, _vp, ctypes.c_int]
    _lib = L
    return L


def default_threads() -> int:
    return os.cpu_count() or 1


def _ptr(a):
    return a.ctypes.data_as(_vp) if a is not None else None


def _fmt(fmt):
    return FMT_NAMES[fmt] if isinstance(fmt, str) else int(fmt)


def _src(x):
    if x.dtype == np.float32:
        return SRC_F32
    if x.dtype == np.uint16:
        return SRC_BF16
    raise TypeError("source must be float32 or uint16 (bfloat16 bits)")


# ---------------------------------------------------------------- formats
def elem_bits(fmt):
    return _load().or_elem_bits(_fmt(fmt))


def decode(fmt, code):
    return _load().or_decode(_fmt(fmt), int(code))


def decode_e8m0(byte):
    return _load().or_decode_e8m0(int(byte))


def fmax(fmt):
    return _load().or_fmax(_fmt(fmt))


def emax(fmt):
    return _load().or_emax(_fmt(fmt))


def encode_rne(fmt, y):
    return _load().or_encode_rne(_fmt(fmt), float(y))


def encode_sr(fmt, y, u):
    return _load().or_encode_sr(_fmt(fmt), float(y), int(u) & 0xFFFFFFFF)


def encode_array(fmt, y, u=None):
    """Element-wise codes of float32 values y (RNE, or SR with words u)."""
    y = np.ascontiguousarray(np.asarray(y, dtype=np.float32).ravel())
    out = np.zeros(y.size, dtype=np.uint8)
    if u is not None:
        u = np.ascontiguousarray(np.asarray(u, dtype=np.uint32).ravel())
        assert u.size == y.size
    _load().or_encode_array(_fmt(fmt), int(u is not None), _ptr(y), _ptr(u), y.size, _ptr(out))
    return out


def block_exponent(fmt, amax):
    return _load().or_block_exponent(_fmt(fmt), float(amax))


def philox4x32_10(ctr, key):
    c = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint32))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint32))
    out = np.zeros(4, dtype=np.uint32)
    _load().or_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def fwht32(v):
    a = np.array(v, dtype=np.float32).copy()
    assert a.shape == (32,)
    _load().or_fwht32(_ptr(a))
    return a


def tensor_amax(x):
    x = np.ascontiguousarray(x)
    return _load().or_tensor_amax(_ptr(x), _src(x), x.shape[0], x.shape[1], x.shape[1])


def tensor_scale(fmt, amax):
    return _load().or_tensor_scale(_fmt(fmt), float(amax))


def _pair(w, g):
    w, g = np.ascontiguousarray(w), np.ascontiguousarray(g)
    if w.shape != g.shape or w.dtype != g.dtype:
        raise ValueError("w and g must have the same shape and dtype")
    return w, g


def predict_max(w, g, lr):
    """[MOSS, "创新 2：权重自动缩放"]: max|W| + lr*max|g| in fp32 (product, then sum)."""
    w, g = _pair(w, g)
    return _load().or_predict_max(_ptr(w), _ptr(g), _src(w), w.shape[0], w.shape[1], w.shape[1],
                                  g.shape[1], float(lr))


def predict_tensor_scale(w, g, lr, fmt):
    """Predicted per-tensor scale of the next step's weights: predict_max / Fmax."""
    w, g = _pair(w, g)
    return _load().or_predict_tensor_scale(_ptr(w), _ptr(g), _src(w), w.shape[0], w.shape[1],
                                           w.shape[1], g.shape[1], float(lr), _fmt(fmt))


def round_bf16(x):
    return _load().or_round_bf16(float(x))


def quantize_block(fmt, sr, v, u=None):
    v = np.ascontiguousarray(np.asarray(v, dtype=np.float32))
    u = np.zeros(32, np.uint32) if u is None else np.ascontiguousarray(np.asarray(u, np.uint32))
    codes = np.zeros(32, dtype=np.uint8)
    s = _load().or_quantize_block(_fmt(fmt), int(bool(sr)), _ptr(v), _ptr(u), _ptr(codes))
    return codes, s


# ---------------------------------------------------------------- tensors
def out_shapes(rows, cols, axis, fmt):
    """(q shape, scales shape) of the stored copy."""
    bits = elem_bits(fmt)
    if axis == AXIS_ROW:
        return (rows, cols * bits // 8), (rows, cols // 32)
    return (cols, rows * bits // 8), (cols, rows // 32)


def quantize(x, axis, fmt, two_level=0, sr=False, hadamard=False, seed=0, offset=0,
             tensor_scale=None, nthreads=None):
    """Quantize a 2-D source.  two_level: 0 none, 1 compute s_t, 2 use given s_t.
    Returns (q, scales, s_t)."""
    fmt = _fmt(fmt)
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    qs, ss = out_shapes(rows, cols, axis, fmt)
    q = np.zeros(qs, dtype=np.uint8)
    s = np.zeros(ss, dtype=np.uint8)
    ts = np.array([1.0 if tensor_scale is None else tensor_scale], dtype=np.float32)
    rc = _load().or_quantize(_ptr(x), _src(x), rows, cols, cols, axis, fmt, int(two_level),
                             int(bool(sr)), int(bool(hadamard)), int(seed), int(offset),
                             _ptr(q), _ptr(s), _ptr(ts), nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle: shape not defined for this axis")
    return q, s, float(ts[0])


def quantize_blocks(x, axis, fmt, r0, c0, two_level=0, s_t=1.0, sr=False, hadamard=False,
                    seed=0, offset=0):
    """Quantize only the blocks starting at (r0[b], c0[b]).  Returns (codes[n][32], scales[n])."""
    fmt = _fmt(fmt)
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    r0 = np.ascontiguousarray(np.asarray(r0, dtype=np.int64))
    c0 = np.ascontiguousarray(np.asarray(c0, dtype=np.int64))
    n = r0.size
    codes = np.zeros((n, 32), dtype=np.uint8)
    s = np.zeros(n, dtype=np.uint8)
    rc = _load().or_quantize_blocks(_ptr(x), _src(x), rows, cols, cols, axis, fmt,
                                    int(two_level), float(s_t), int(bool(sr)),
                                    int(bool(hadamard)), int(seed), int(offset), _ptr(r0),
                                    _ptr(c0), n, _ptr(codes), _ptr(s))
    if rc != 0:
        raise ValueError("oracle: bad block list")
    return codes, s


def unpack_codes(q, fmt):
    """[R][bytes] packed -> [R][elements] one code per byte."""
    if elem_bits(fmt) == 8:
        return q.copy()
    lo = q & 0xF
    hi = q >> 4
    return np.stack([lo, hi], axis=-1).reshape(q.shape[0], q.shape[1] * 2)


def dequantize(q, scales, tensor_scale, fmt, rows, cols, axis, hadamard=False, nthreads=None):
    fmt = _fmt(fmt)
    q = np.ascontiguousarray(q, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    ts = None if tensor_scale is None else np.array([tensor_scale], dtype=np.float32)
    out = np.zeros((rows, cols), dtype=np.float32)
    rc = _load().or_dequantize(_ptr(q), _ptr(scales), _ptr(ts), fmt, rows, cols, axis,
                               int(bool(hadamard)), _ptr(out), nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle: bad dequantize shape")
    return out


def _ts(t):
    return None if t is None else np.array([t], dtype=np.float32)


def gemm(qa, sa, ta, fa, qb, sb, tb, fb, M, N, K, alpha=1.0, hadamard_k=False, nthreads=None):
    """C[M][N] (float64) and the error-bound scale |alpha'| (|A|.|B|) (float64)."""
    qa = np.ascontiguousarray(qa, dtype=np.uint8)
    sa = np.ascontiguousarray(sa, dtype=np.uint8)
    qb = np.ascontiguousarray(qb, dtype=np.uint8)
    sb = np.ascontiguousarray(sb, dtype=np.uint8)
    ta_, tb_ = _ts(ta), _ts(tb)
    C = np.zeros((M, N), dtype=np.float64)
    bound = np.zeros((M, N), dtype=np.float64)
    rc = _load().or_gemm(_ptr(qa), _ptr(sa), _ptr(ta_), _fmt(fa), _ptr(qb), _ptr(sb), _ptr(tb_),
                         _fmt(fb), M, N, K, float(alpha), int(bool(hadamard_k)), _ptr(C),
                         _ptr(bound), nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle: bad gemm arguments")
    return C, bound


def gemm_entries(qa, sa, ta, fa, qb, sb, tb, fb, M, N, K, ii, jj, alpha=1.0, hadamard_k=False,
                 nthreads=None):
    qa = np.ascontiguousarray(qa, dtype=np.uint8)
    sa = np.ascontiguousarray(sa, dtype=np.uint8)
    qb = np.ascontiguousarray(qb, dtype=np.uint8)
    sb = np.ascontiguousarray(sb, dtype=np.uint8)
    ii = np.ascontiguousarray(np.asarray(ii, dtype=np.int64))
    jj = np.ascontiguousarray(np.asarray(jj, dtype=np.int64))
    ta_, tb_ = _ts(ta), _ts(tb)
    n = ii.size
    C = np.zeros(n, dtype=np.float64)
    bound = np.zeros(n, dtype=np.float64)
    rc = _load().or_gemm_entries(_ptr(qa), _ptr(sa), _ptr(ta_), _fmt(fa), _ptr(qb), _ptr(sb),
                                 _ptr(tb_), _fmt(fb), M, N, K, float(alpha),
                                 int(bool(hadamard_k)), _ptr(ii), _ptr(jj), n, _ptr(C),
                                 _ptr(bound), nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle: bad gemm_entries arguments")
    return C, bound


# ---------------------------------------------------------------- COAT optimizer states
def log2_fp32(x):
    return _load().or_log2_fp32(float(x))


def exp2_fp32(y):
    return _load().or_exp2_fp32(float(y))


def pow_fp32(u, k):
    return _load().or_pow_fp32(float(u), float(k))


def optstate_quantize(x, fmt="e4m3", group=128, nthreads=None):
    """[COAT, "解決方案：動態範圍擴充套件"]: FP8 codes of an fp32 optimizer state
    after the per-group expansion u^k.  Returns (codes uint8 [n], amax
    float32 [n/group], k float32 [n/group]) for the flattened x."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32).ravel())
    n = x.size
    q = np.zeros(n, np.uint8)
    amax = np.zeros(n // group, np.float32)
    k = np.zeros(n // group, np.float32)
    rc = _load().or_optstate_quantize(_ptr(x), n, group, _fmt(fmt), _ptr(q), _ptr(amax), _ptr(k),
                                      nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle: bad optimizer-state arguments")
    return q, amax, k


def optstate_dequantize(q, amax, k, fmt="e4m3", group=128, nthreads=None):
    q = np.ascontiguousarray(np.asarray(q, dtype=np.uint8).ravel())
    amax = np.ascontiguousarray(amax, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    out = np.zeros(q.size, np.float32)
    rc = _load().or_optstate_dequantize(_ptr(q), _ptr(amax), _ptr(k), q.size, group, _fmt(fmt), _ptr(out),
                                        nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle: bad optimizer-state arguments")
    return out


# ---------------------------------------------------------------- nvfp routes
NV_PANEL = 32


def nvfp_shapes(rows, cols, axis, local):
    """(codes shape, block-scale shape, tensor-scale count) of a stored nvfp copy."""
    SR, L = (rows, cols) if axis == AXIS_ROW else (cols, rows)
    return (SR, L // 2), (SR, L // 16), ((SR + NV_PANEL - 1) // NV_PANEL if local else 1)


def nvfp_quantize(x, axis, local=False, nthreads=None):
    """[FAF, "格式感知融合的设计思路"]: NVFP4 copy (E2M1, E4M3 scale per 16,
    FP32 second-level scale global or per 32 stored rows).  Returns
    (codes, block scales, second-level scales)."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    qs, ss, nt = nvfp_shapes(rows, cols, axis, local)
    q = np.zeros(qs, np.uint8)
    s = np.zeros(ss, np.uint8)
    t = np.zeros(nt, np.float32)
    rc = _load().or_nvfp_quantize(_ptr(x), _src(x), rows, cols, cols, axis, int(bool(local)), _ptr(q), _ptr(s),
                                  _ptr(t), nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle: bad nvfp shape")
    return q, s, t


def nvfp_dequantize(q, s16, tscale, rows, cols, axis, local=False):
    q = np.ascontiguousarray(q, np.uint8)
    s16 = np.ascontiguousarray(s16, np.uint8)
    t = np.ascontiguousarray(tscale, np.float32)
    out = np.zeros((rows, cols), np.float32)
    rc = _load().or_nvfp_dequantize(_ptr(q), _ptr(s16), _ptr(t), rows, cols, axis, int(bool(local)), _ptr(out))
    if rc != 0:
        raise ValueError("oracle: bad nvfp shape")
    return out


def nvfp_gemm(qa, sa, ta, local_a, qb, sb, tb, local_b, M, N, K, alpha=1.0, nthreads=None):
    """C[M][N] (float64) and the bound |alpha'| (|A|.|B|) of the nvfp GEMM."""
    qa, sa, qb, sb = (np.ascontiguousarray(a, np.uint8) for a in (qa, sa, qb, sb))
    ta, tb = np.ascontiguousarray(ta, np.float32), np.ascontiguousarray(tb, np.float32)
    C = np.zeros((M, N))
    bound = np.zeros((M, N))
    rc = _load().or_nvfp_gemm(_ptr(qa), _ptr(sa), _ptr(ta), int(bool(local_a)), _ptr(qb), _ptr(sb), _ptr(tb),
                              int(bool(local_b)), M, N, K, float(alpha), _ptr(C), _ptr(bound),
                              nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle: bad nvfp gemm arguments")
    return C, bound


def nvfp_gemm_entries(qa, sa, ta, local_a, qb, sb, tb, local_b, M, N, K, ii, jj, alpha=1.0, nthreads=None):
    """Entries (ii, jj) of nvfp_gemm's C and bound."""
    qa, sa, qb, sb = (np.ascontiguousarray(a, np.uint8) for a in (qa, sa, qb, sb))
    ta, tb = np.ascontiguousarray(ta, np.float32), np.ascontiguousarray(tb, np.float32)
    ii = np.ascontiguousarray(np.asarray(ii, np.int64))
    jj = np.ascontiguousarray(np.asarray(jj, np.int64))
    C = np.zeros(ii.size)
    bound = np.zeros(ii.size)
    rc = _load().or_nvfp_gemm_entries(_ptr(qa), _ptr(sa), _ptr(ta), int(bool(local_a)), _ptr(qb), _ptr(sb),
                                      _ptr(tb), int(bool(local_b)), M, N, K, float(alpha), _ptr(ii), _ptr(jj),
                                      ii.size, _ptr(C), _ptr(bound), nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle: bad nvfp_gemm_entries arguments")
    return C, bound

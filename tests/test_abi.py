"""The C ABI on the CPU: libmx.so loads, exports every function declared in
include/mx.h, and rejects bad arguments before any HIP call (so these calls
are safe without a GPU: nothing is launched)."""
import ctypes
import os
import re

import pytest

from fp4_quantization_block_amd import mx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mx.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:mx_status|const char\*|int64_t)\s+(mx_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mx.LIB_PATH):
        pytest.skip("libmx.so not built")
    return mx.load()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert set(names) == set(mx.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for s, name in enumerate(["MX_OK", "MX_ERR_INVALID_ARG", "MX_ERR_UNSUPPORTED",
                              "MX_ERR_ALIGNMENT", "MX_ERR_HIP"]):
        assert lib.mx_status_string(s).decode() == name


FAKE = 0x10000          # 16-byte aligned, never dereferenced: validation fails first
FAKE_ODD = 0x10008


def _q(lib, x=FAKE, src=1, rows=64, cols=64, ld=64, axis=0, cfg=None, q=FAKE, s=FAKE, ts=None):
    cfg = cfg if cfg is not None else mx.qconfig("e4m3")
    return lib.mx_quantize(x, src, rows, cols, ld, axis, ctypes.byref(cfg), q, s, ts, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), mx.MX_ERR_INVALID_ARG),
    (dict(q=None), mx.MX_ERR_INVALID_ARG),
    (dict(s=None), mx.MX_ERR_INVALID_ARG),
    (dict(src=7), mx.MX_ERR_INVALID_ARG),
    (dict(rows=0), mx.MX_ERR_INVALID_ARG),
    (dict(cols=-3), mx.MX_ERR_INVALID_ARG),
    (dict(ld=32), mx.MX_ERR_INVALID_ARG),
    (dict(axis=2), mx.MX_ERR_INVALID_ARG),
    (dict(cols=48, ld=48), mx.MX_ERR_INVALID_ARG),              # row blocks need cols % 32
    (dict(axis=1, rows=40), mx.MX_ERR_INVALID_ARG),             # col blocks need rows % 32
    (dict(x=FAKE + 1), mx.MX_ERR_ALIGNMENT),                   # bf16 source on an odd address
    (dict(x=FAKE + 2, src=0), mx.MX_ERR_ALIGNMENT),            # fp32 source not 4-byte aligned
    (dict(q=FAKE_ODD), mx.MX_ERR_ALIGNMENT),
])
def test_quantize_validation(lib, kw, status):
    assert _q(lib, **kw) == status
    assert lib.mx_last_error_message().decode() != ""


@pytest.mark.parametrize("field,value", [("fmt", 9), ("block", 16), ("scale_fmt", 5),
                                         ("tscale", 3), ("rounding", 4), ("hadamard", 2),
                                         ("reserved", 1)])
def test_quantize_bad_config(lib, field, value):
    cfg = mx.qconfig("e2m1")
    setattr(cfg, field, value)
    assert _q(lib, cfg=cfg) == mx.MX_ERR_INVALID_ARG


def test_two_level_needs_tensor_scale(lib):
    cfg = mx.qconfig("e4m3", two_level=True)
    assert _q(lib, cfg=cfg, ts=None) == mx.MX_ERR_INVALID_ARG
    assert _q(lib, cfg=cfg, ts=FAKE + 2) == mx.MX_ERR_ALIGNMENT
    assert lib.mx_quantize(FAKE, 1, 64, 64, 64, 0, None, FAKE, FAKE, None, None) == mx.MX_ERR_INVALID_ARG


def test_dual_layout_validation(lib):
    cfg = mx.qconfig("e4m3")
    f = lib.mx_quantize_dual_layout
    assert f(FAKE, 1, 40, 64, 64, ctypes.byref(cfg), FAKE, FAKE, FAKE, FAKE, None, None) == mx.MX_ERR_INVALID_ARG
    assert f(FAKE, 1, 64, 40, 40, ctypes.byref(cfg), FAKE, FAKE, FAKE, FAKE, None, None) == mx.MX_ERR_INVALID_ARG
    assert f(FAKE, 1, 64, 64, 64, ctypes.byref(cfg), FAKE, FAKE, None, FAKE, None, None) == mx.MX_ERR_INVALID_ARG
    assert f(FAKE, 1, 64, 64, 64, ctypes.byref(cfg), FAKE, FAKE, FAKE_ODD, FAKE, None, None) == mx.MX_ERR_ALIGNMENT


def _g(lib, qa=FAKE, sa=FAKE, ta=None, fa=0, qb=FAKE, sb=FAKE, tb=None, fb=0, M=64, N=64, K=64,
       alpha=1.0, hk=0, c=FAKE, out=1, ldc=64):
    return lib.mx_gemm(qa, sa, ta, fa, qb, sb, tb, fb, M, N, K, alpha, hk, c, out, ldc, None)


@pytest.mark.parametrize("kw,status", [
    (dict(qa=None), mx.MX_ERR_INVALID_ARG),
    (dict(sb=None), mx.MX_ERR_INVALID_ARG),
    (dict(c=None), mx.MX_ERR_INVALID_ARG),
    (dict(fa=5), mx.MX_ERR_INVALID_ARG),
    (dict(out=3), mx.MX_ERR_INVALID_ARG),
    (dict(M=0), mx.MX_ERR_INVALID_ARG),
    (dict(K=48), mx.MX_ERR_INVALID_ARG),
    (dict(ldc=32), mx.MX_ERR_INVALID_ARG),
    (dict(hk=2), mx.MX_ERR_INVALID_ARG),
    (dict(fa=0, fb=2), mx.MX_ERR_UNSUPPORTED),
    (dict(qa=FAKE_ODD), mx.MX_ERR_ALIGNMENT),
    (dict(c=FAKE + 1), mx.MX_ERR_ALIGNMENT),
    (dict(ta=FAKE + 2), mx.MX_ERR_ALIGNMENT),
    (dict(K=(1 << 23) + 32), mx.MX_ERR_INVALID_ARG),      # 32-bit tile offsets
    (dict(M=1 << 31), mx.MX_ERR_INVALID_ARG),
    (dict(N=(1 << 31) - 255), mx.MX_ERR_INVALID_ARG),
    (dict(M=1 << 30, N=1 << 30), mx.MX_ERR_INVALID_ARG),  # 2^40 tiles
])
def test_gemm_validation(lib, kw, status):
    assert _g(lib, **kw) == status


def _gnv(lib, M=64, N=64, K=64, la=0, lb=0, out=1, ldc=None, c=FAKE):
    return lib.mx_gemm_nvfp(FAKE, FAKE, FAKE, la, FAKE, FAKE, FAKE, lb, M, N, K, 1.0, c, out,
                            N if ldc is None else ldc, None)


@pytest.mark.parametrize("kw,status", [
    (dict(c=None), mx.MX_ERR_INVALID_ARG),
    (dict(la=2), mx.MX_ERR_INVALID_ARG),
    (dict(out=3), mx.MX_ERR_INVALID_ARG),
    (dict(K=96), mx.MX_ERR_INVALID_ARG),                   # K % 64
    (dict(K=(1 << 24) + 64), mx.MX_ERR_INVALID_ARG),
    (dict(M=1 << 31), mx.MX_ERR_INVALID_ARG),
    (dict(M=1 << 30, N=1 << 30), mx.MX_ERR_INVALID_ARG),   # 2^44 output tiles
    (dict(ldc=32), mx.MX_ERR_INVALID_ARG),
])
def test_gemm_nvfp_validation(lib, kw, status):
    assert _gnv(lib, **kw) == status


def test_dequantize_validation(lib):
    f = lib.mx_dequantize
    assert f(None, FAKE, None, 0, 64, 64, 0, 0, FAKE, 0, None) == mx.MX_ERR_INVALID_ARG
    assert f(FAKE, FAKE, None, 7, 64, 64, 0, 0, FAKE, 0, None) == mx.MX_ERR_INVALID_ARG
    assert f(FAKE, FAKE, None, 0, 64, 48, 0, 0, FAKE, 0, None) == mx.MX_ERR_INVALID_ARG
    assert f(FAKE, FAKE, None, 0, 40, 64, 1, 0, FAKE, 0, None) == mx.MX_ERR_INVALID_ARG
    assert f(FAKE, FAKE, None, 0, 64, 64, 0, 0, FAKE_ODD, 0, None) == mx.MX_ERR_ALIGNMENT
    assert f(FAKE, FAKE, None, 0, 64, 64, 0, 3, FAKE, 0, None) == mx.MX_ERR_INVALID_ARG


def _predict(lib, w=None, ldw=64, g=None, ldg=64, src=1, rows=64, cols=64, lr=1e-3, fmt=0, work=None,
             nbytes=4096, out=None):
    FAKE = ctypes.c_void_p(0x10000)
    return lib.mx_predict_tensor_scale(FAKE if w is None else w, ldw, FAKE if g is None else g, ldg, src, rows,
                                       cols, lr, fmt, FAKE if work is None else work, nbytes,
                                       FAKE if out is None else out, None)


@pytest.mark.parametrize("kw,status", [
    (dict(w=ctypes.c_void_p(0)), mx.MX_ERR_INVALID_ARG),
    (dict(g=ctypes.c_void_p(0)), mx.MX_ERR_INVALID_ARG),
    (dict(work=ctypes.c_void_p(0)), mx.MX_ERR_INVALID_ARG),
    (dict(out=ctypes.c_void_p(0)), mx.MX_ERR_INVALID_ARG),
    (dict(src=7), mx.MX_ERR_INVALID_ARG),
    (dict(fmt=9), mx.MX_ERR_INVALID_ARG),
    (dict(rows=0), mx.MX_ERR_INVALID_ARG),
    (dict(ldw=32), mx.MX_ERR_INVALID_ARG),
    (dict(ldg=63), mx.MX_ERR_INVALID_ARG),
    (dict(lr=-1e-3), mx.MX_ERR_INVALID_ARG),
    (dict(lr=float("nan")), mx.MX_ERR_INVALID_ARG),
    (dict(lr=float("inf")), mx.MX_ERR_INVALID_ARG),
    (dict(nbytes=4095), mx.MX_ERR_INVALID_ARG),
    (dict(work=ctypes.c_void_p(0x10002)), mx.MX_ERR_ALIGNMENT),
    (dict(out=ctypes.c_void_p(0x10001)), mx.MX_ERR_ALIGNMENT),
    (dict(w=ctypes.c_void_p(0x10001)), mx.MX_ERR_ALIGNMENT),
])
def test_predict_tensor_scale_validation(lib, kw, status):
    assert _predict(lib, **kw) == status
    assert lib.mx_last_error_message().decode() != ""


def test_predict_workspace_bytes(lib):
    assert lib.mx_predict_workspace_bytes() == 4096


def _gemmq(lib, M=64, N=64, K=128, fa=0, fb=0, out_fmt=0, qc=None, sc=None, sa=None):
    FAKE = ctypes.c_void_p(0x10000)
    return lib.mx_gemm_quantized(FAKE, FAKE if sa is None else sa, None, fa, FAKE, FAKE, None, fb, M, N, K, 1.0, 0,
                                 out_fmt, FAKE if qc is None else qc, FAKE if sc is None else sc, None)


@pytest.mark.parametrize("kw,status", [
    (dict(qc=ctypes.c_void_p(0)), mx.MX_ERR_INVALID_ARG),
    (dict(sc=ctypes.c_void_p(0)), mx.MX_ERR_INVALID_ARG),
    (dict(out_fmt=7), mx.MX_ERR_INVALID_ARG),
    (dict(out_fmt=2), mx.MX_ERR_UNSUPPORTED),          # E2M1 output
    (dict(N=48), mx.MX_ERR_INVALID_ARG),               # N % 32
    (dict(qc=ctypes.c_void_p(0x10008)), mx.MX_ERR_ALIGNMENT),
    (dict(K=96), mx.MX_ERR_UNSUPPORTED),               # FP8 needs K % 128
    (dict(fa=2, fb=2, K=128), mx.MX_ERR_UNSUPPORTED),  # FP4 needs K % 256
    (dict(sa=ctypes.c_void_p(0x10002)), mx.MX_ERR_UNSUPPORTED),
    (dict(fa=0, fb=2), mx.MX_ERR_UNSUPPORTED),         # mixed FP8 x FP4
    (dict(K=100), mx.MX_ERR_INVALID_ARG),
])
def test_gemm_quantized_validation(lib, kw, status):
    assert _gemmq(lib, **kw) == status
    assert lib.mx_last_error_message().decode() != ""


def _predict_noalloc(lib, w=None, ldw=64, g=None, ldg=64, src=1, rows=64, cols=64, lr=1e-3, fmt=0, out=None):
    FAKE = ctypes.c_void_p(0x10000)
    return lib.mx_predict_tensor_scale_noalloc(FAKE if w is None else w, ldw, FAKE if g is None else g, ldg, src,
                                               rows, cols, lr, fmt, FAKE if out is None else out, None)


@pytest.mark.parametrize("kw,status", [
    (dict(w=ctypes.c_void_p(0)), mx.MX_ERR_INVALID_ARG),
    (dict(g=ctypes.c_void_p(0)), mx.MX_ERR_INVALID_ARG),
    (dict(out=ctypes.c_void_p(0)), mx.MX_ERR_INVALID_ARG),
    (dict(src=7), mx.MX_ERR_INVALID_ARG),
    (dict(fmt=9), mx.MX_ERR_INVALID_ARG),
    (dict(cols=0), mx.MX_ERR_INVALID_ARG),
    (dict(ldg=63), mx.MX_ERR_INVALID_ARG),
    (dict(lr=-1e-3), mx.MX_ERR_INVALID_ARG),
    (dict(lr=float("nan")), mx.MX_ERR_INVALID_ARG),
    (dict(out=ctypes.c_void_p(0x10001)), mx.MX_ERR_ALIGNMENT),
    (dict(g=ctypes.c_void_p(0x10001)), mx.MX_ERR_ALIGNMENT),
])
def test_predict_tensor_scale_noalloc_validation(lib, kw, status):
    """The no-allocation variant validates like the workspace version (no
    HIP call is made for any of these)."""
    assert _predict_noalloc(lib, **kw) == status
    assert lib.mx_last_error_message().decode() != ""

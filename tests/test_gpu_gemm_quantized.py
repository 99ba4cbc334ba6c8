"""GPU parity of mx_gemm_quantized: the GEMM epilogue that writes C already
MX-quantized (1x32 row blocks, E8M0 scales) for the next layer
([FAF, "格式感知融合的设计思路"]).  The fp32 values the epilogue encodes
are the ones mx_gemm writes with fp32 output (checked against the oracle's
GEMM by the GEMM tests and again here); the oracle's row quantizer applied
to those fp32 values must give the fused codes and scales bit for bit."""
import numpy as np
import pytest
import torch

import oracle as O
from fp4_quantization_block_amd import mx
from gpu_util import assert_codes_equal, gemm_check, log, mfma_allowance, require_gpu, to_device, u8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _operands(rng, fa, fb, M, N, K, two_level=False, hadamard=False):
    a = (rng.standard_normal((M, K)) * np.exp2(rng.integers(-3, 4, (M, 1)))).astype(np.float32)
    b = (rng.standard_normal((K, N)) * 0.05).astype(np.float32)
    ca = mx.qconfig(fa, two_level=two_level, hadamard=hadamard)
    cb = mx.qconfig(fb, two_level=two_level, hadamard=hadamard)
    qa, sa, ta = mx.mx_quantize(to_device(a), mx.MX_AXIS_ROW, ca)
    qb, sb, tb = mx.mx_quantize(to_device(b), mx.MX_AXIS_COL, cb)
    return (qa, sa, ta), (qb, sb, tb)


CASES = [
    # (fa, fb, M, N, K, out_fmt, alpha, two_level, hadamard)
    ("e4m3", "e4m3", 300, 288, 256, "e4m3", 1.0, False, False),
    ("e5m2", "e4m3", 257, 96, 640, "e5m2", 0.75, False, False),
    ("e4m3", "e5m2", 64, 544, 1152, "e4m3", 3.0, True, False),
    ("e2m1", "e2m1", 130, 320, 512, "e4m3", 1.0, False, True),
    ("e4m3", "e4m3", 33, 32, 128, "e5m2", 1e-30, False, False),     # tiny outputs: small shared exponents
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}x{c[1]}->{c[5]}_{c[2]}x{c[3]}x{c[4]}" for c in CASES])
def test_fused_output_is_the_quantized_fp32_output(case):
    fa, fb, M, N, K, of, alpha, tl, had = case
    rng = np.random.default_rng(M * 7 + N + K)
    (qa, sa, ta), (qb, sb, tb) = _operands(rng, fa, fb, M, N, K, tl, had)
    c32 = mx.mx_gemm(qa, sa, ta, fa, qb, sb, tb, fb, M, N, K, alpha=alpha, hadamard_k=had,
                     out_dtype=mx.MX_OUT_F32)
    qc, sc = mx.mx_gemm_quantized(qa, sa, ta, fa, qb, sb, tb, fb, M, N, K, out_fmt=of, alpha=alpha,
                                  hadamard_k=had)
    torch.cuda.synchronize()
    c = c32.cpu().numpy()
    q, s, _ = O.quantize(c, O.AXIS_ROW, of)
    assert_codes_equal(u8(qc), q, "fused codes")
    assert_codes_equal(u8(sc), s, "fused scales")
    # and the fp32 values themselves are the GEMM the oracle defines
    qao, sao = u8(qa), u8(sa)
    qbo, sbo = u8(qb), u8(sb)
    tao = None if ta is None else float(ta.item())
    tbo = None if tb is None else float(tb.item())
    C, bound = O.gemm(qao, sao, tao, fa, qbo, sbo, tbo, fb, M, N, K, alpha=alpha, hadamard_k=had)
    allow = None
    if O.elem_bits(fa) == 8:
        ap = alpha * (tao or 1.0) * (tbo or 1.0)
        allow = mfma_allowance(O.unpack_codes(qao, fa), sao, fa, O.unpack_codes(qbo, fb), sbo, fb, ap)
    gemm_check(c.astype(np.float64), C, bound, False, "fp32 values", allow)


def test_non_finite_outputs_give_nan_blocks():
    rng = np.random.default_rng(1)
    (qa, sa, ta), (qb, sb, tb) = _operands(rng, "e4m3", "e4m3", 64, 64, 128)
    qc, sc = mx.mx_gemm_quantized(qa, sa, None, "e4m3", qb, sb, None, "e4m3", 64, 64, 128, alpha=float("inf"))
    c32 = mx.mx_gemm(qa, sa, None, "e4m3", qb, sb, None, "e4m3", 64, 64, 128, alpha=float("inf"),
                     out_dtype=mx.MX_OUT_F32)
    torch.cuda.synchronize()
    q, s, _ = O.quantize(c32.cpu().numpy(), O.AXIS_ROW, "e4m3")
    assert_codes_equal(u8(qc), q, "codes")
    assert_codes_equal(u8(sc), s, "scales")
    assert np.all(u8(sc) == 0xFF)


def test_full_moss_4096_fused_e4m3():
    from fp4_quantization_block_amd import inputs as I
    w = I.make("moss_two_level_4096")
    A, B = w.tensors["A"], w.tensors["B"]
    cfg = mx.qconfig("e4m3", two_level=True)
    qa, sa, ta = mx.mx_quantize(to_device(A), mx.MX_AXIS_ROW, cfg)
    qb, sb, tb = mx.mx_quantize(to_device(B), mx.MX_AXIS_COL, cfg)
    M, K = A.shape
    N = B.shape[1]
    c32 = mx.mx_gemm(qa, sa, ta, "e4m3", qb, sb, tb, "e4m3", M, N, K, out_dtype=mx.MX_OUT_F32)
    qc, sc = mx.mx_gemm_quantized(qa, sa, ta, "e4m3", qb, sb, tb, "e4m3", M, N, K, out_fmt="e4m3")
    torch.cuda.synchronize()
    q, s, _ = O.quantize(c32.cpu().numpy(), O.AXIS_ROW, "e4m3")
    assert_codes_equal(u8(qc), q, "fused codes 4096")
    assert_codes_equal(u8(sc), s, "fused scales 4096")
    log("fused E4M3 output of the 4096^3 MOSS GEMM matches the oracle's quantization of its fp32 output")

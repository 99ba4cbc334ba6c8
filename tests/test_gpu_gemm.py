"""GPU parity of the block-scaled GEMM, end to end: the HIP path quantizes
and multiplies on the device; the oracle quantizes and multiplies on the
CPU from the same seeded inputs.  Codes must agree bit for bit; the GEMM
output must satisfy |C_gpu - C_ref| <= 1e-5 (|A|.|B|)_ij + 1e-6 (fp32
output), and for bf16 output lie in [RNE_bf16(C_ref - tol),
RNE_bf16(C_ref + tol)]."""
import numpy as np
import pytest
import torch

import oracle as O
from fp4_quantization_block_amd import inputs as I
from fp4_quantization_block_amd import mx
from gpu_util import (DEV, assert_codes_equal, gemm_check, log, mfma_allowance,
                      mfma_allowance_entries, mfma_model, require_gpu, to_device, u8)

pytestmark = pytest.mark.gpu
SEED = I.SR_SEED


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def quant_both(x, axis, fmt, **opts):
    """GPU and oracle quantization of the same source; checks codes agree."""
    cfg = mx.qconfig(fmt, two_level=opts.get("two_level", False), sr=opts.get("sr", False),
                     hadamard=opts.get("hadamard", False), seed=SEED)
    q, s, ts = mx.mx_quantize(to_device(x), axis, cfg)
    qo, so, st = O.quantize(x, axis, fmt, two_level=1 if opts.get("two_level") else 0,
                            sr=opts.get("sr", False), hadamard=opts.get("hadamard", False),
                            seed=SEED)
    torch.cuda.synchronize()
    assert_codes_equal(u8(q), qo, "operand codes")
    assert_codes_equal(u8(s), so, "operand scales")
    return (q, s, ts), (qo, so, st if opts.get("two_level") else None)


CASES = [
    # (name, fa, fb, M, N, K, out, opts)
    ("e4m3_ragged", "e4m3", "e4m3", 300, 200, 96, "f32", {}),
    ("e4m3_bf16", "e4m3", "e4m3", 257, 513, 384, "bf16", {}),
    ("e5m2_e4m3", "e5m2", "e4m3", 129, 260, 224, "f32", {}),
    ("e4m3_e5m2", "e4m3", "e5m2", 64, 96, 1024, "f32", {}),
    ("e5m2_e5m2", "e5m2", "e5m2", 33, 31, 160, "f32", {}),
    ("e2m1", "e2m1", "e2m1", 300, 280, 320, "f32", {}),
    ("e2m1_had_sr", "e2m1", "e2m1", 256, 256, 512, "f32", dict(hadamard=True, sr=True)),
    ("two_level", "e4m3", "e4m3", 200, 300, 256, "f32", dict(two_level=True)),
    ("two_level_bf16", "e4m3", "e4m3", 512, 512, 512, "bf16", dict(two_level=True)),
    ("tiny", "e4m3", "e4m3", 1, 1, 32, "f32", {}),
    # FP8 with K a multiple of 128 runs the one-wave-per-SIMD kernel: one
    # stage, an odd stage count, ragged M and N, bf16 output
    ("k128_one_stage", "e4m3", "e4m3", 300, 200, 128, "f32", {}),
    ("e5m2_e4m3_five_stages", "e5m2", "e4m3", 129, 260, 640, "f32", {}),
    ("e4m3_e5m2_bf16_ragged", "e4m3", "e5m2", 257, 300, 1152, "bf16", {}),
    # FP4 with K a multiple of 256 runs it too (four k-steps per stage)
    ("e2m1_three_stages_ragged", "e2m1", "e2m1", 300, 280, 768, "f32", {}),
    ("e2m1_one_stage_bf16", "e2m1", "e2m1", 257, 200, 256, "bf16", dict(hadamard=True)),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_gemm_small(case):
    name, fa, fb, M, N, K, out, opts = case
    rng = np.random.default_rng(len(name) * 1000 + M)
    a = (rng.standard_normal((M, K)) * np.exp2(rng.integers(-3, 4, (M, 1)))).astype(np.float32)
    b = (rng.standard_normal((K, N)) * 0.05).astype(np.float32)
    (qa, sa, ta), (qao, sao, tao) = quant_both(a, O.AXIS_ROW, fa, **opts)
    (qb, sb, tb), (qbo, sbo, tbo) = quant_both(b, O.AXIS_COL, fb, **opts)
    alpha = 0.75
    hk = bool(opts.get("hadamard"))
    od = mx.MX_OUT_F32 if out == "f32" else mx.MX_OUT_BF16
    c = mx.mx_gemm(qa, sa, ta, fa, qb, sb, tb, fb, M, N, K, alpha=alpha, hadamard_k=hk, out_dtype=od)
    torch.cuda.synchronize()
    C, bound = O.gemm(qao, sao, tao, fa, qbo, sbo, tbo, fb, M, N, K, alpha=alpha, hadamard_k=hk)
    got = c.float().cpu().numpy()
    allow = None
    if O.elem_bits(fa) == 8:
        ap = _alpha_prime(alpha, tao, tbo, hk)
        allow = mfma_allowance(O.unpack_codes(qao, fa), sao, fa, O.unpack_codes(qbo, fb), sbo, fb, ap)
        if out == "f32":
            # the kernel computes exactly what the matrix cores define
            model = mfma_model(O.unpack_codes(qao, fa), sao, fa, O.unpack_codes(qbo, fb), sbo, fb, ap)
            dev_ = np.abs(got - model)
            lim = (K / 64 + 2) * 2.0 ** -24 * bound + 1e-30
            assert np.all(dev_ <= lim), f"{name}: kernel differs from the MFMA arithmetic by {np.max(dev_ / lim):.2f}x"
    r = gemm_check(got, C, bound, out == "bf16", name, allow)
    log(f"{name}: (max err / stated tol, fraction within stated tol) = {r}")


def _alpha_prime(alpha, ta, tb, hk):
    ap = float(alpha)
    if ta is not None:
        ap *= float(ta)
    if tb is not None:
        ap *= float(tb)
    return ap / 32.0 if hk else ap


@pytest.mark.parametrize("K", [64, 256])
def test_gemm_ldc(K):
    rng = np.random.default_rng(9)
    M, N = 70, 50
    a = rng.standard_normal((M, K)).astype(np.float32)
    b = rng.standard_normal((K, N)).astype(np.float32)
    (qa, sa, _), (qao, sao, _) = quant_both(a, O.AXIS_ROW, "e4m3")
    (qb, sb, _), (qbo, sbo, _) = quant_both(b, O.AXIS_COL, "e4m3")
    big = torch.full((M, 80), 7.0, dtype=torch.float32, device=DEV)
    mx.mx_gemm(qa, sa, None, "e4m3", qb, sb, None, "e4m3", M, N, K, out_dtype=mx.MX_OUT_F32,
               c=big, ldc=80)
    torch.cuda.synchronize()
    C, bound = O.gemm(qao, sao, None, "e4m3", qbo, sbo, None, "e4m3", M, N, K)
    g = big.cpu().numpy()
    gemm_check(g[:, :N], C, bound, False, "ldc", mfma_allowance(qao, sao, "e4m3", qbo, sbo, "e4m3", 1.0))
    assert np.all(g[:, N:] == 7.0)                      # outside N untouched


def _sample_entries(rng, M, N, n):
    ii = np.concatenate([rng.integers(0, M, n), [0, 0, M - 1, M - 1]])
    jj = np.concatenate([rng.integers(0, N, n), [0, N - 1, 0, N - 1]])
    return ii, jj


def _pick(c, ii, jj):
    t = c[torch.from_numpy(ii).to(DEV), torch.from_numpy(jj).to(DEV)]
    return t.float().cpu().numpy().astype(np.float64)


def test_full_mxfp8_gemm_256():
    w = I.make("mxfp8_gemm_256")
    (qa, sa, _), (qao, sao, _) = quant_both(w.tensors["A"], O.AXIS_ROW, "e4m3")
    (qb, sb, _), (qbo, sbo, _) = quant_both(w.tensors["B"], O.AXIS_COL, "e4m3")
    allow = mfma_allowance(qao, sao, "e4m3", qbo, sbo, "e4m3", 1.0)
    for od in (mx.MX_OUT_F32, mx.MX_OUT_BF16):
        c = mx.mx_gemm(qa, sa, None, "e4m3", qb, sb, None, "e4m3", 256, 256, 256, out_dtype=od)
        torch.cuda.synchronize()
        C, bound = O.gemm(qao, sao, None, "e4m3", qbo, sbo, None, "e4m3", 256, 256, 256)
        r = gemm_check(c.float().cpu().numpy(), C, bound, od == mx.MX_OUT_BF16, "256^3", allow)
        log("256^3 (max err / stated tol, fraction within stated tol)", r)


def test_full_moss_two_level_4096_sampled():
    w = I.make("moss_two_level_4096")
    (qa, sa, ta), (qao, sao, tao) = quant_both(w.tensors["A"], O.AXIS_ROW, "e4m3", two_level=True)
    (qb, sb, tb), (qbo, sbo, tbo) = quant_both(w.tensors["B"], O.AXIS_COL, "e4m3", two_level=True)
    n = 4096
    c32 = mx.mx_gemm(qa, sa, ta, "e4m3", qb, sb, tb, "e4m3", n, n, n, out_dtype=mx.MX_OUT_F32)
    c16 = mx.mx_gemm(qa, sa, ta, "e4m3", qb, sb, tb, "e4m3", n, n, n, out_dtype=mx.MX_OUT_BF16)
    torch.cuda.synchronize()
    rng = np.random.default_rng(22)
    ii, jj = _sample_entries(rng, n, n, 4000)
    C, bound = O.gemm_entries(qao, sao, tao, "e4m3", qbo, sbo, tbo, "e4m3", n, n, n, ii, jj)
    allow = mfma_allowance_entries(qao, sao, "e4m3", qbo, sbo, "e4m3", float(tao) * float(tbo), ii, jj)
    r = gemm_check(_pick(c32, ii, jj), C, bound, False, "4096^3 two-level fp32", allow)
    log("4096^3 (max err / stated tol, fraction within stated tol)", r)
    gemm_check(_pick(c16, ii, jj), C, bound, True, "4096^3 two-level bf16", allow)


def test_full_mxfp4_wgrad_sampled():
    w = I.make("mxfp4_wgrad_qkv")
    dY, X = w.tensors["dY"], w.tensors["X"]        # [T][Q], [T][H]; K = T
    T, Q = dY.shape
    H = X.shape[1]
    (qa, sa, _), (qao, sao, _) = quant_both_sampled(dY, "e2m1")
    (qb, sb, _), (qbo, sbo, _) = quant_both_sampled(X, "e2m1")
    c = mx.mx_gemm(qa, sa, None, "e2m1", qb, sb, None, "e2m1", Q, H, T, hadamard_k=True,
                   out_dtype=mx.MX_OUT_F32)
    torch.cuda.synchronize()
    rng = np.random.default_rng(21)
    ii, jj = _sample_entries(rng, Q, H, 3000)
    C, bound = O.gemm_entries(qao, sao, None, "e2m1", qbo, sbo, None, "e2m1", Q, H, T, ii, jj,
                              hadamard_k=True)
    r = gemm_check(_pick(c, ii, jj), C, bound, False, "fp4 wgrad")
    log("fp4 wgrad max err/tol", r)


def quant_both_sampled(x, fmt):
    """Column copy (K = rows) with Hadamard + SR on both sides; the oracle
    quantizes the whole tensor (its C loop is fast enough at this size)."""
    cfg = mx.qconfig(fmt, sr=True, hadamard=True, seed=SEED)
    q, s, _ = mx.mx_quantize(to_device(x), mx.MX_AXIS_COL, cfg)
    qo, so, _ = O.quantize(x, O.AXIS_COL, fmt, sr=True, hadamard=True, seed=SEED)
    torch.cuda.synchronize()
    assert_codes_equal(u8(q), qo, "codes")
    assert_codes_equal(u8(s), so, "scales")
    return (q, s, None), (qo, so, None)


MLP = [  # (name, A tensor, A axis, fa, B tensor, B axis, fb)
    ("fprop_gate_up", "X", "row", "e4m3", "W_gu", "col", "e4m3"),
    ("fprop_down", "Xp", "row", "e4m3", "W_d", "col", "e4m3"),
    ("dgrad_gate_up", "dY_gu", "row", "e5m2", "W_gu", "row", "e4m3"),
    ("dgrad_down", "dY_d", "row", "e5m2", "W_d", "row", "e4m3"),
    ("wgrad_gate_up", "X", "col", "e4m3", "dY_gu", "col", "e5m2"),
    ("wgrad_down", "Xp", "col", "e4m3", "dY_d", "col", "e5m2"),
]


def test_full_llama3_8b_mlp_sampled():
    """The six training GEMMs from dual-layout operands (each source tensor
    read once); each checked on sampled entries against the oracle."""
    w = I.make("llama3_8b_mlp")
    fmts = {"X": "e4m3", "Xp": "e4m3", "W_gu": "e4m3", "W_d": "e4m3", "dY_gu": "e5m2", "dY_d": "e5m2"}
    dev = {}
    for name, fmt in fmts.items():
        qr, sr_, qc, sc, _ = mx.mx_quantize_dual_layout(to_device(w.tensors[name]), mx.qconfig(fmt))
        dev[name] = {"row": (qr, sr_), "col": (qc, sc)}
    torch.cuda.synchronize()
    rng = np.random.default_rng(23)
    for gname, an, aax, fa, bn, bax, fb in MLP:
        A, B = w.tensors[an], w.tensors[bn]
        qa, sa = dev[an][aax]
        qb, sb = dev[bn][bax]
        M = A.shape[0] if aax == "row" else A.shape[1]
        K = A.shape[1] if aax == "row" else A.shape[0]
        N = B.shape[1] if bax == "col" else B.shape[0]
        c = mx.mx_gemm(qa, sa, None, fa, qb, sb, None, fb, M, N, K, out_dtype=mx.MX_OUT_F32)
        torch.cuda.synchronize()
        ii, jj = _sample_entries(rng, M, N, 600)
        # oracle operands: only the rows the sampled entries touch
        ua, ia = np.unique(ii, return_inverse=True)
        ub, ib = np.unique(jj, return_inverse=True)
        qao, sao = _oracle_rows(A, aax, fa, ua)
        qbo, sbo = _oracle_rows(B, bax, fb, ub)
        C, bound = O.gemm_entries(qao, sao, None, fa, qbo, sbo, None, fb, len(ua), len(ub), K,
                                  ia, ib)
        allow = mfma_allowance_entries(qao, sao, fa, qbo, sbo, fb, 1.0, ia, ib)
        r = gemm_check(_pick(c, ii, jj), C, bound, False, gname, allow)
        log(f"{gname} ({M},{N},{K}) max err/tol {r}")
        del c


def _oracle_rows(x, axis, fmt, rows):
    """Oracle-quantized stored rows `rows` of a copy (row copy: source rows;
    column copy: source columns), packed as the quantizer writes them."""
    R, Cc = x.shape
    if axis == "row":
        r0 = np.repeat(rows, Cc // 32)
        c0 = np.tile(np.arange(0, Cc, 32), len(rows))
        codes, scales = O.quantize_blocks(x, O.AXIS_ROW, fmt, r0, c0)
        kblk = Cc // 32
    else:
        c0 = np.repeat(rows, R // 32)
        r0 = np.tile(np.arange(0, R, 32), len(rows))
        codes, scales = O.quantize_blocks(x, O.AXIS_COL, fmt, r0, c0)
        kblk = R // 32
    codes = codes.reshape(len(rows), kblk * 32)
    if O.elem_bits(fmt) == 4:
        codes = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return codes, scales.reshape(len(rows), kblk)

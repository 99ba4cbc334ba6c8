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
from gpu_util import (DEV, assert_codes_equal, check_model, gemm_check, log, mfma_rule, record,
                      require_gpu, tile_samples, to_device, u8)

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
        model, allow = mfma_rule(O.unpack_codes(qao, fa), sao, fa, O.unpack_codes(qbo, fb), sbo, fb, ap)
        if out == "f32":
            check_model(got, model, bound, K, name)   # the kernel computes what the matrix cores define
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
    model, allow = mfma_rule(qao, sao, "e4m3", qbo, sbo, "e4m3", 1.0)
    gemm_check(g[:, :N], C, bound, False, "ldc", allow)
    check_model(g[:, :N], model, bound, K, "ldc")
    assert np.all(g[:, N:] == 7.0)                      # outside N untouched


def _pick(c, ii, jj):
    t = c[torch.from_numpy(ii).to(DEV), torch.from_numpy(jj).to(DEV)]
    return t.float().cpu().numpy().astype(np.float64)


def _report(config, gemm, shape, fa, fb, got, C, bound, K, ap, qa_u=None, sa=None, qb_u=None, sb=None,
            ii=None, jj=None, sampled="all outputs"):
    """fp32-output parity of one GEMM against the oracle, and a record of
    its largest error relative to the stated bound and the fraction of
    outputs inside that bound.  FP8: the stated bound plus the MFMA rule's
    worst-case truncation, and agreement with the rule up to fp32
    accumulation.  FP4: the stated bound alone."""
    entry = {"config": config, "gemm": gemm, "shape_MNK": list(shape), "formats": [fa, fb],
             "checked": sampled, "n": int(np.size(got))}
    if O.elem_bits(fa) == 8:
        model, allow = mfma_rule(qa_u, sa, fa, qb_u, sb, fb, ap, ii, jj)
        entry["max_dev_vs_rule_over_accum_limit"] = check_model(got, model, bound, K, f"{config} {gemm}")
        ratio, frac = gemm_check(got, C, bound, False, f"{config} {gemm}", allow)
    else:
        ratio, frac = gemm_check(got, C, bound, False, f"{config} {gemm}")
    entry["max_err_over_stated_bound"] = ratio
    entry["frac_within_stated_bound"] = frac
    log(f"{config} {gemm} {shape}: max err / stated bound {ratio:.3f}, within stated bound {frac:.4%} "
        f"({sampled}, {entry['n']} entries)")
    record(entry)
    return entry


def test_full_mxfp8_gemm_256():
    w = I.make("mxfp8_gemm_256")
    (qa, sa, _), (qao, sao, _) = quant_both(w.tensors["A"], O.AXIS_ROW, "e4m3")
    (qb, sb, _), (qbo, sbo, _) = quant_both(w.tensors["B"], O.AXIS_COL, "e4m3")
    C, bound = O.gemm(qao, sao, None, "e4m3", qbo, sbo, None, "e4m3", 256, 256, 256)
    c32 = mx.mx_gemm(qa, sa, None, "e4m3", qb, sb, None, "e4m3", 256, 256, 256, out_dtype=mx.MX_OUT_F32)
    c16 = mx.mx_gemm(qa, sa, None, "e4m3", qb, sb, None, "e4m3", 256, 256, 256, out_dtype=mx.MX_OUT_BF16)
    torch.cuda.synchronize()
    _report("mxfp8_256", "gemm", (256, 256, 256), "e4m3", "e4m3", c32.cpu().numpy(), C, bound, 256, 1.0,
            qao, sao, qbo, sbo)
    allow = mfma_rule(qao, sao, "e4m3", qbo, sbo, "e4m3", 1.0)[1]
    gemm_check(c16.float().cpu().numpy(), C, bound, True, "256^3 bf16", allow)


def test_full_moss_two_level_4096():
    """Every output of the 4096^3 two-level GEMM, fp32 and bf16."""
    w = I.make("moss_two_level_4096")
    (qa, sa, ta), (qao, sao, tao) = quant_both(w.tensors["A"], O.AXIS_ROW, "e4m3", two_level=True)
    (qb, sb, tb), (qbo, sbo, tbo) = quant_both(w.tensors["B"], O.AXIS_COL, "e4m3", two_level=True)
    n = 4096
    c32 = mx.mx_gemm(qa, sa, ta, "e4m3", qb, sb, tb, "e4m3", n, n, n, out_dtype=mx.MX_OUT_F32)
    c16 = mx.mx_gemm(qa, sa, ta, "e4m3", qb, sb, tb, "e4m3", n, n, n, out_dtype=mx.MX_OUT_BF16)
    torch.cuda.synchronize()
    C, bound = O.gemm(qao, sao, tao, "e4m3", qbo, sbo, tbo, "e4m3", n, n, n)
    ap = float(np.float32(tao)) * float(np.float32(tbo))
    _report("moss_two_level_4096", "gemm", (n, n, n), "e4m3", "e4m3", c32.cpu().numpy(), C, bound, n, ap,
            qao, sao, qbo, sbo)
    allow = mfma_rule(qao, sao, "e4m3", qbo, sbo, "e4m3", ap)[1]
    gemm_check(c16.float().cpu().numpy(), C, bound, True, "4096^3 two-level bf16", allow)


def test_full_mxfp4_wgrad():
    """Every output of the FP4 wgrad GEMM (M 6144, N 4096, K 16384) against
    the stated bound alone (FP4 products are exact)."""
    w = I.make("mxfp4_wgrad_qkv")
    dY, X = w.tensors["dY"], w.tensors["X"]        # [T][Q], [T][H]; K = T
    T, Q = dY.shape
    H = X.shape[1]
    (qa, sa, _), (qao, sao, _) = quant_both_sampled(dY, "e2m1")
    (qb, sb, _), (qbo, sbo, _) = quant_both_sampled(X, "e2m1")
    c = mx.mx_gemm(qa, sa, None, "e2m1", qb, sb, None, "e2m1", Q, H, T, hadamard_k=True,
                   out_dtype=mx.MX_OUT_F32)
    torch.cuda.synchronize()
    got = c.cpu().numpy()
    del c
    C, bound = O.gemm(qao, sao, None, "e2m1", qbo, sbo, None, "e2m1", Q, H, T, hadamard_k=True)
    _report("mxfp4_wgrad_qkv", "wgrad", (Q, H, T), "e2m1", "e2m1", got, C, bound, T, 1.0 / 32)


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
MLP_FMTS = {"X": "e4m3", "Xp": "e4m3", "W_gu": "e4m3", "W_d": "e4m3", "dY_gu": "e5m2", "dY_d": "e5m2"}


def test_full_llama3_8b_mlp():
    """The Llama-3-8B MLP training step: all six dual-layout quantizations
    compared in full (both copies, codes and scales), then the six GEMMs
    from those operands, each checked on 16 entries of every 128x128 output
    tile (its four corners included) against the oracle and the MFMA rule."""
    w = I.make("llama3_8b_mlp")
    dev, ora = {}, {}
    for name, fmt in MLP_FMTS.items():
        x = w.tensors[name]
        qr, sr_, qc, sc, _ = mx.mx_quantize_dual_layout(to_device(x), mx.qconfig(fmt))
        torch.cuda.synchronize()
        qro, sro, _ = O.quantize(x, O.AXIS_ROW, fmt)
        qco, sco, _ = O.quantize(x, O.AXIS_COL, fmt)
        assert_codes_equal(u8(qr), qro, f"{name} row codes")
        assert_codes_equal(u8(sr_), sro, f"{name} row scales")
        assert_codes_equal(u8(qc), qco, f"{name} col codes")
        assert_codes_equal(u8(sc), sco, f"{name} col scales")
        dev[name] = {"row": (qr, sr_), "col": (qc, sc)}
        ora[name] = {"row": (qro, sro), "col": (qco, sco)}
        log(f"mlp {name} {x.shape}: both copies equal the oracle's")
    w.tensors.clear()
    rng = np.random.default_rng(23)
    for gname, an, aax, fa, bn, bax, fb in MLP:
        qa, sa = dev[an][aax]
        qb, sb = dev[bn][bax]
        qao, sao = ora[an][aax]
        qbo, sbo = ora[bn][bax]
        M, K = qao.shape
        N = qbo.shape[0]
        c = mx.mx_gemm(qa, sa, None, fa, qb, sb, None, fb, M, N, K, out_dtype=mx.MX_OUT_F32)
        torch.cuda.synchronize()
        ii, jj = tile_samples(rng, M, N)
        got = _pick(c, ii, jj)
        del c
        C, bound = O.gemm_entries(qao, sao, None, fa, qbo, sbo, None, fb, M, N, K, ii, jj)
        _report("llama3_8b_mlp", gname, (M, N, K), fa, fb, got, C, bound, K, 1.0, qao, sao, qbo, sbo, ii, jj,
                sampled="16 per 128x128 tile incl. corners")


@pytest.mark.parametrize("fmt,K,out", [("e4m3", 256, "f32"), ("e4m3", 384, "bf16"), ("e2m1", 512, "f32"),
                                       ("e2m1", 768, "bf16")])
def test_last_round_half_tiles(fmt, K, out):
    """A grid of one full round of 256 x 256 tiles plus one tile row: the
    last tile row runs as a second launch of 256 x 128 half tiles.  Ragged M
    (the tail row holds 100 rows) and N (300: the third half tile holds 44
    columns).  Every output of the tail rows, the rows next to the seam and
    a sample of the rest are checked."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tiles_m = cus // 2 + 1                                  # x 2 tile columns = cus + 2 tiles
    M, N = (tiles_m - 1) * 256 + 100, 300
    rng = np.random.default_rng(K + len(fmt))
    a = (rng.standard_normal((M, K)) * np.exp2(rng.integers(-3, 4, (M, 1)))).astype(np.float32)
    b = (rng.standard_normal((K, N)) * 0.05).astype(np.float32)
    log(f"half-tile tail {fmt} {M}x{N}x{K} out={out} ({cus} CUs)")
    (qa, sa, _), (qao, sao, _) = quant_both(a, O.AXIS_ROW, fmt)
    (qb, sb, _), (qbo, sbo, _) = quant_both(b, O.AXIS_COL, fmt)
    od = mx.MX_OUT_F32 if out == "f32" else mx.MX_OUT_BF16
    c = mx.mx_gemm(qa, sa, None, fmt, qb, sb, None, fmt, M, N, K, alpha=0.5, out_dtype=od)
    torch.cuda.synchronize()
    seam = (tiles_m - 1) * 256
    rows = np.concatenate([np.arange(seam - 8, M), rng.integers(0, seam - 8, 64)])
    ii = np.repeat(rows, N).astype(np.int64)
    jj = np.tile(np.arange(N), rows.size).astype(np.int64)
    C, bound = O.gemm_entries(qao, sao, None, fmt, qbo, sbo, None, fmt, M, N, K, ii, jj, alpha=0.5)
    got = _pick(c, ii, jj)
    if out == "f32":
        _report("half_tile_tail", fmt, (M, N, K), fmt, fmt, got, C, bound, K, 0.5,
                O.unpack_codes(qao, fmt) if O.elem_bits(fmt) == 8 else None, sao,
                O.unpack_codes(qbo, fmt) if O.elem_bits(fmt) == 8 else None, sbo, ii, jj,
                sampled="tail rows, seam rows, 64 random rows")
    else:
        allow = None
        if O.elem_bits(fmt) == 8:
            allow = mfma_rule(O.unpack_codes(qao, fmt), sao, fmt, O.unpack_codes(qbo, fmt), sbo, fmt, 0.5,
                              ii, jj)[1]
        gemm_check(got, C, bound, True, f"half-tile tail {fmt} bf16", allow)

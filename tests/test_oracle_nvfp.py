"""Pins of the oracle's nvfp routes ([FAF, "格式感知融合的设计思路"]: global
and CTA-local nvfp beside native mxfp).  CPU only.

The pages fix neither block size nor scale format ("parity unpinned" for
the reading itself); the reading -- NVFP4: E2M1 in blocks of 16, an E4M3
scale per block, an FP32 second-level scale amax / (6 * 448), over the tensor
(global) or per 32 stored rows (local) -- is pinned by the properties that
define it: exact round trips of representable blocks, block scales that
reach but never exceed E4M3's top, a half-step error bound, the panel
structure of the local scales, and a float64 library matmul for the GEMM."""
import numpy as np
import pytest

import oracle as O

E2M1 = np.array([O.decode("e2m1", c) for c in range(8)])        # 0, .5, 1, 1.5, 2, 3, 4, 6
E4M3 = np.array([O.decode("e4m3", c) for c in range(0x7F)])      # finite non-negative values


def _representable(rng, srows, L, j):
    """Stored rows of E2M1 codes with a 6 in every block, E4M3 block
    scales, the largest block scale 448 and second-level scale 2^j."""
    nb = L // 16
    codes = rng.integers(0, 16, (srows, L)).astype(np.uint8)
    codes[:, ::16] = 0x7                                          # +6 leads every block
    sb = rng.integers(1, 0x7F, (srows, nb)).astype(np.uint8)
    sb[0, 0] = 0x7E                                               # 448
    val = np.array([O.decode("e2m1", c) for c in range(16)])[codes] * \
        np.repeat(E4M3[sb].astype(np.float64), 16, axis=1) * 2.0 ** j
    return codes, sb, val.astype(np.float32)


@pytest.mark.parametrize("axis", [O.AXIS_ROW, O.AXIS_COL])
def test_representable_round_trip_is_exact(axis):
    rng = np.random.default_rng(1 + axis)
    codes, sb, val = _representable(rng, 48, 64, -3)
    x = val if axis == O.AXIS_ROW else np.ascontiguousarray(val.T)
    q, s, t = O.nvfp_quantize(x, axis)
    assert t[0] == 2.0 ** -3                                      # 6 * 448 * 2^-3 / 2688
    assert np.array_equal(s, sb)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    assert np.array_equal(q, packed)
    back = O.nvfp_dequantize(q, s, t, x.shape[0], x.shape[1], axis)
    assert np.array_equal(back, x)


@pytest.mark.parametrize("local", [False, True])
def test_block_scales_fill_e4m3_and_errors_stay_within_half_step(local):
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((96, 128)) * np.exp2(rng.integers(-8, 8, (96, 1)))).astype(np.float32)
    q, s, t = O.nvfp_quantize(x, O.AXIS_ROW, local=local)
    sv = E4M3[s]
    assert np.all(s < 0x7F)                                       # never the NaN code
    # the domain holding the largest magnitude gets the top block scale, up to E4M3 rounding
    dom = np.repeat(t, 32)[:96] if local else np.full(96, t[0])
    for p in range(len(t)):
        rows = slice(32 * p, 32 * p + 32) if local else slice(0, 96)
        assert sv[rows].max() >= 448.0 / (1 + 2.0 ** -3)
    back = O.nvfp_dequantize(q, s, t, 96, 128, O.AXIS_ROW, local=local)
    # half an E2M1 step at the value, at the block's effective scale (plus the
    # reciprocal's and the final product's roundings)
    step = np.array([0.5, 0.5, 0.5, 0.5, 1.0, 1.0, 2.0, 2.0])
    mag = np.abs(x) / (np.repeat(sv, 16, axis=1) * dom[:, None])
    idx = np.clip(np.searchsorted(E2M1, mag), 0, 7)
    tol = 0.5 * step[idx] * np.repeat(sv, 16, axis=1) * dom[:, None] * (1 + 2.0 ** -20) + \
        np.abs(x) * 2.0 ** -21
    assert np.all(np.abs(back.astype(np.float64) - x) <= tol)


def test_local_scales_are_per_panel():
    """Local: each 32-row panel is quantized exactly as a tensor of its own
    (global route); one panel: local equals global."""
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((80, 64)) * np.exp2(rng.integers(-5, 6, (80, 1)))).astype(np.float32)
    q, s, t = O.nvfp_quantize(x, O.AXIS_ROW, local=True)
    assert t.shape == (3,)
    for p in range(3):
        rows = slice(32 * p, min(32 * p + 32, 80))
        qp, sp, tp = O.nvfp_quantize(np.ascontiguousarray(x[rows]), O.AXIS_ROW, local=False)
        assert tp[0] == t[p] and np.array_equal(qp, q[rows]) and np.array_equal(sp, s[rows])
    qc, sc, tc = O.nvfp_quantize(x, O.AXIS_COL, local=True)      # 64 stored rows: 2 panels
    for p in range(2):
        cols = slice(32 * p, 32 * p + 32)
        qp, sp, tp = O.nvfp_quantize(np.ascontiguousarray(x[:, cols]), O.AXIS_COL, local=False)
        assert tp[0] == tc[p] and np.array_equal(qp, qc[cols]) and np.array_equal(sp, sc[cols])


def test_special_blocks():
    x = np.ones((32, 64), np.float32)
    x[0, :16] = 0.0
    x[1, :16] = -0.0
    x[2, 3] = np.nan
    q, s, t = O.nvfp_quantize(x, O.AXIS_ROW)
    assert np.isnan(t[0]) and np.all(s == 0x7F) and np.all(q == 0)
    x[2, 3] = 1.0
    q, s, t = O.nvfp_quantize(x, O.AXIS_ROW)
    assert t[0] == np.float32(1.0) / np.float32(2688.0)
    assert s[0, 0] == 0 and np.all(q[0, :8] == 0)                 # zero block: zero scale, +0 codes
    assert s[1, 0] == 0 and np.all(q[1, :8] == 0x88)              # signed zeros kept
    z = np.zeros((32, 32), np.float32)
    q, s, t = O.nvfp_quantize(z, O.AXIS_ROW)
    assert t[0] == 1.0 and np.all(s == 0) and np.all(q == 0)


@pytest.mark.parametrize("la,lb", [(False, False), (True, False), (True, True)])
def test_gemm_equals_float64_matmul(la, lb):
    rng = np.random.default_rng(5)
    M, N, K = 70, 40, 96
    a = (rng.standard_normal((M, K)) * np.exp2(rng.integers(-4, 5, (M, 1)))).astype(np.float32)
    b = (rng.standard_normal((K, N)) * 0.05).astype(np.float32)
    qa, sa, ta = O.nvfp_quantize(a, O.AXIS_ROW, local=la)
    qb, sb, tb = O.nvfp_quantize(b, O.AXIS_COL, local=lb)
    C, bound = O.nvfp_gemm(qa, sa, ta, la, qb, sb, tb, lb, M, N, K, alpha=0.5)
    # dequantized operands without the second-level scales, which factor out of the sum
    A = O.nvfp_dequantize(qa, sa, np.ones_like(ta), M, K, O.AXIS_ROW, local=la).astype(np.float64)
    B = O.nvfp_dequantize(qb, sb, np.ones_like(tb), K, N, O.AXIS_COL, local=lb).astype(np.float64)
    sA = (np.repeat(ta, 32)[:M] if la else np.full(M, ta[0])).astype(np.float64)
    sB = (np.repeat(tb, 32)[:N] if lb else np.full(N, tb[0])).astype(np.float64)
    ref = 0.5 * (sA[:, None] * sB[None, :]) * (A @ B)
    assert np.allclose(C, ref, rtol=1e-12, atol=1e-300)
    assert np.allclose(bound, 0.5 * np.abs(sA)[:, None] * np.abs(sB)[None, :] * (np.abs(A) @ np.abs(B)), rtol=1e-12)


def test_gemm_entries_equal_full_gemm():
    rng = np.random.default_rng(6)
    M, N, K = 45, 37, 64
    a = rng.standard_normal((M, K)).astype(np.float32)
    b = rng.standard_normal((K, N)).astype(np.float32)
    qa, sa, ta = O.nvfp_quantize(a, O.AXIS_ROW, local=True)
    qb, sb, tb = O.nvfp_quantize(b, O.AXIS_COL)
    C, bound = O.nvfp_gemm(qa, sa, ta, True, qb, sb, tb, False, M, N, K, alpha=2.0)
    ii, jj = rng.integers(0, M, 50), rng.integers(0, N, 50)
    Ce, be = O.nvfp_gemm_entries(qa, sa, ta, True, qb, sb, tb, False, M, N, K, ii, jj, alpha=2.0)
    assert np.array_equal(Ce, C[ii, jj]) and np.array_equal(be, bound[ii, jj])

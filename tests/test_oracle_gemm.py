"""Pins of the oracle GEMM ([MOSS] "GEMM Kernel 优化": scaled codes in the
main loop, per-tensor scales once at the end).

Checks: a float64 library matmul (numpy/BLAS) on independently dequantized
operands; pure-Python brute force on tiny integer cases; the effect of one
scale byte; the per-tensor / Hadamard factors; the bound; sampled entries.
"""
import numpy as np
import pytest

import oracle as O


def _rand_operand(fmt, rows, K, rng, byte_lo=120, byte_hi=135):
    bits = O.elem_bits(fmt)
    n = 1 << bits
    codes = rng.integers(0, n, size=(rows, K)).astype(np.uint8)
    nan = {O.E4M3: [0x7F, 0xFF], O.E5M2: list(range(0x7C, 0x80)) + list(range(0xFC, 0x100)),
           O.E2M1: []}[fmt]
    for c in nan:
        codes[codes == c] = 0
    if bits == 4:
        q = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    else:
        q = codes
    s = rng.integers(byte_lo, byte_hi, size=(rows, K // 32)).astype(np.uint8)
    return codes, q, s


def _dq(fmt, codes, s):
    lut = np.array([O.decode(fmt, c) for c in range(1 << O.elem_bits(fmt))])
    return lut[codes] * np.repeat(np.exp2(s.astype(np.float64) - 127), 32, axis=1)


@pytest.mark.parametrize("fa,fb", [(O.E4M3, O.E4M3), (O.E5M2, O.E4M3), (O.E4M3, O.E5M2),
                                   (O.E2M1, O.E2M1), (O.E5M2, O.E5M2)])
def test_gemm_matches_float64_matmul(fa, fb):
    rng = np.random.default_rng(10)
    M, N, K = 37, 29, 160
    ca, qa, sa = _rand_operand(fa, M, K, rng)
    cb, qb, sb = _rand_operand(fb, N, K, rng)
    C, bound = O.gemm(qa, sa, 0.75, fa, qb, sb, 1.5, fb, M, N, K, alpha=2.0)
    A = _dq(fa, ca, sa)
    B = _dq(fb, cb, sb)
    ref = (A @ B.T) * (2.0 * 0.75 * 1.5)
    assert np.allclose(C, ref, rtol=1e-12, atol=0)
    assert np.allclose(bound, np.abs(A) @ np.abs(B).T * 2.25, rtol=1e-12, atol=0)


def test_gemm_brute_force_small_integers():
    """Codes for small integers, scale 2^0: pure-Python integer sums."""
    ints = {0: 0x00, 1: 0x38, 2: 0x40, 3: 0x44, 4: 0x48, -1: 0xB8, -2: 0xC0, -3: 0xC4}
    for v, c in ints.items():
        assert O.decode(O.E4M3, c) == v
    rng = np.random.default_rng(11)
    M, N, K = 3, 4, 64
    va = rng.choice(list(ints), size=(M, K))
    vb = rng.choice(list(ints), size=(N, K))
    qa = np.vectorize(ints.get)(va).astype(np.uint8)
    qb = np.vectorize(ints.get)(vb).astype(np.uint8)
    sa = np.full((M, K // 32), 127, np.uint8)
    sb = np.full((N, K // 32), 127, np.uint8)
    C, _ = O.gemm(qa, sa, None, O.E4M3, qb, sb, None, O.E4M3, M, N, K)
    for i in range(M):
        for j in range(N):
            assert C[i, j] == sum(int(va[i, k]) * int(vb[j, k]) for k in range(K))


def test_one_scale_byte_doubles_one_block():
    rng = np.random.default_rng(12)
    M, N, K = 8, 8, 128
    ca, qa, sa = _rand_operand(O.E4M3, M, K, rng)
    cb, qb, sb = _rand_operand(O.E4M3, N, K, rng)
    C0, _ = O.gemm(qa, sa, None, O.E4M3, qb, sb, None, O.E4M3, M, N, K)
    sa2 = sa.copy()
    sa2[2, 1] += 1                                   # row 2, block k in [32, 64)
    C1, _ = O.gemm(qa, sa2, None, O.E4M3, qb, sb, None, O.E4M3, M, N, K)
    A = _dq(O.E4M3, ca, sa)
    B = _dq(O.E4M3, cb, sb)
    block = A[2, 32:64] @ B[:, 32:64].T
    assert np.array_equal(np.delete(C1, 2, 0), np.delete(C0, 2, 0))
    assert np.allclose(C1[2] - C0[2], block, rtol=1e-12, atol=1e-300)


def test_tensor_scales_and_hadamard_factor():
    rng = np.random.default_rng(13)
    M, N, K = 5, 6, 64
    _, qa, sa = _rand_operand(O.E2M1, M, K, rng)
    _, qb, sb = _rand_operand(O.E2M1, N, K, rng)
    C, _ = O.gemm(qa, sa, None, O.E2M1, qb, sb, None, O.E2M1, M, N, K)
    C2, _ = O.gemm(qa, sa, 4.0, O.E2M1, qb, sb, 0.125, O.E2M1, M, N, K)
    C3, _ = O.gemm(qa, sa, None, O.E2M1, qb, sb, None, O.E2M1, M, N, K, hadamard_k=True)
    assert np.array_equal(C, C2 * 2.0)
    assert np.array_equal(C3 * 32.0, C)


def test_hadamard_gemm_recovers_plain_product():
    """Quantize both operands with the Hadamard along K: the GEMM with the
    1/32 factor approximates A.B^T of the sources (H^T H = 32 I)."""
    rng = np.random.default_rng(14)
    M, N, K = 16, 16, 256
    a = rng.integers(-3, 4, size=(M, K)).astype(np.float32)
    b = rng.integers(-3, 4, size=(N, K)).astype(np.float32)
    qa, sa, _ = O.quantize(a, O.AXIS_ROW, O.E4M3, hadamard=True)
    qb, sb, _ = O.quantize(b, O.AXIS_ROW, O.E4M3, hadamard=True)
    C, bound = O.gemm(qa, sa, None, O.E4M3, qb, sb, None, O.E4M3, M, N, K, hadamard_k=True)
    ref = a.astype(np.float64) @ b.astype(np.float64).T
    # E4M3 keeps 3 mantissa bits: relative error per element <= 2^-4
    assert np.all(np.abs(C - ref) <= 2.0 ** -4 * bound * 32 / 32 + 1e-9)


def test_gemm_entries_match_full():
    rng = np.random.default_rng(15)
    M, N, K = 33, 21, 96
    _, qa, sa = _rand_operand(O.E5M2, M, K, rng)
    _, qb, sb = _rand_operand(O.E4M3, N, K, rng)
    C, bound = O.gemm(qa, sa, 2.0, O.E5M2, qb, sb, None, O.E4M3, M, N, K, alpha=-0.5)
    ii = rng.integers(0, M, 50)
    jj = rng.integers(0, N, 50)
    Ce, be = O.gemm_entries(qa, sa, 2.0, O.E5M2, qb, sb, None, O.E4M3, M, N, K, ii, jj,
                            alpha=-0.5)
    assert np.array_equal(Ce, C[ii, jj]) and np.array_equal(be, bound[ii, jj])


def test_round_bf16_matches_torch_on_float32_inputs():
    import torch
    rng = np.random.default_rng(16)
    x = (rng.standard_normal(20000) * np.exp2(rng.uniform(-60, 60, 20000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([O.round_bf16(float(v)) for v in x])
    assert np.array_equal(got, ref)

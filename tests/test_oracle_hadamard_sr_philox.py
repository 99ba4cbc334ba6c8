"""Pins of the oracle's Hadamard transform, stochastic rounding and Philox.

Hadamard ([FAF] "两个关键的数值技巧": fixed-sign 32-point transform): rows of
scipy's Sylvester Hadamard matrix, orthogonality H.H^T = 32 I, involution.
SR (same passage: round up with probability proportional to the distance,
unbiased): measured mean over 10^6 draws, f = 0 invariance, round-up rate.
Philox4x32-10: rocRAND's engine (built from its header) as a black box.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle as O


def test_fwht_basis_vectors_are_hadamard_rows():
    scipy_linalg = pytest.importorskip("scipy.linalg")
    H = scipy_linalg.hadamard(32)
    for i in range(32):
        e = np.zeros(32, np.float32)
        e[i] = 1.0
        assert np.array_equal(O.fwht32(e), H[:, i].astype(np.float32))


def test_fwht_orthogonality_and_involution():
    M = np.stack([O.fwht32(np.eye(32, dtype=np.float32)[i]) for i in range(32)]).astype(np.int64)
    assert np.array_equal(M @ M.T, 32 * np.eye(32, dtype=np.int64))
    rng = np.random.default_rng(0)
    for _ in range(50):
        x = rng.integers(-1000, 1000, 32).astype(np.float32)
        assert np.array_equal(O.fwht32(O.fwht32(x)), 32 * x)


def test_fwht_float_close_to_exact_product():
    scipy_linalg = pytest.importorskip("scipy.linalg")
    H = scipy_linalg.hadamard(32).astype(np.float64)
    rng = np.random.default_rng(1)
    for _ in range(100):
        x = rng.standard_normal(32).astype(np.float32)
        exact = H @ x.astype(np.float64)
        got = O.fwht32(x).astype(np.float64)
        # 5 stages, each one fp32 rounding of values bounded by sum|x|
        assert np.all(np.abs(got - exact) <= 5 * 2.0 ** -24 * np.abs(x).sum() * 2)


@pytest.mark.parametrize("fmt,y", [(O.E2M1, 2.3), (O.E2M1, 0.1), (O.E4M3, 0.0123),
                                   (O.E4M3, 300.0), (O.E5M2, 3e-6), (O.E2M1, -4.75)])
def test_sr_unbiased_over_1e6_draws(fmt, y):
    rng = np.random.default_rng(2)
    n = 1_000_000
    u = rng.integers(0, 2 ** 32, size=n, dtype=np.uint64).astype(np.uint32)
    codes = O.encode_array(fmt, np.full(n, y, np.float32), u)
    lut = np.array([O.decode(fmt, c) for c in range(1 << O.elem_bits(fmt))])
    vals = lut[codes]
    yv = float(np.float32(y))
    lo, hi = np.sort(np.unique(vals))[[0, -1]]
    assert set(np.unique(vals)) <= {lo, hi}
    f = (yv - lo) / (hi - lo) if hi != lo else 0.0
    sigma = (hi - lo) * np.sqrt(max(f * (1 - f), 1e-12) / n)
    assert abs(vals.mean() - yv) <= 5 * sigma


@pytest.mark.parametrize("fmt", [O.E4M3, O.E5M2, O.E2M1])
def test_sr_leaves_representable_values(fmt):
    rng = np.random.default_rng(3)
    n = 1 << (O.elem_bits(fmt) - 1)
    vals = np.array([O.decode(fmt, c) for c in range(n)])
    vals = vals[np.isfinite(vals)].astype(np.float32)
    for v in vals:
        u = rng.integers(0, 2 ** 32, size=64, dtype=np.uint64).astype(np.uint32)
        assert np.all(O.encode_array(fmt, np.full(64, v, np.float32), u) == O.encode_rne(fmt, v))


def test_sr_round_up_rate_follows_distance():
    # E2M1 between 2 and 3: y = 2 + f
    rng = np.random.default_rng(4)
    u = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    for f in (0.125, 0.25, 0.5, 0.75, 0.9):
        codes = O.encode_array(O.E2M1, np.full(u.size, 2 + f, np.float32), u)
        rate = (codes == O.encode_rne(O.E2M1, 3.0)).mean()
        assert abs(rate - f) < 5 * np.sqrt(f * (1 - f) / u.size)


def test_sr_decision_threshold_reading():
    """Round up iff u < floor(frac * 2^32): at frac = 1/4, u = 2^30 - 1 rounds
    up and u = 2^30 does not."""
    assert O.encode_sr(O.E2M1, 2.25, (1 << 30) - 1) == O.encode_rne(O.E2M1, 3.0)
    assert O.encode_sr(O.E2M1, 2.25, 1 << 30) == O.encode_rne(O.E2M1, 2.0)


def _rocrand_tool(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available to build the rocRAND reference")
    d = tmp_path_factory.mktemp("rr")
    exe = str(d / "rocrand_philox_ref")
    src = os.path.join(os.path.dirname(__file__), "rocrand_philox_ref.cpp")
    subprocess.run([hipcc, "--offload-arch=gfx950", "-O1", "-o", exe, src], check=True,
                   capture_output=True)
    return exe


def test_philox_matches_rocrand_engine(tmp_path_factory):
    """rocRAND's Philox4x32-10 with (seed, subsequence, offset) produces the
    block for counter (offset/4 + call, 0 + carry, subsequence lo, hi) and
    key (seed lo, seed hi)."""
    exe = _rocrand_tool(tmp_path_factory)
    cases = [(0, 0, 0), (0x00C0FFEE5EED0004, 3, 0), (123456789, 0x1234, 40),
             (0xDEADBEEFCAFEF00D, 0xFFFFFFFF00000007, 4 << 32), (7, 1 << 33, 4 * 1000003)]
    for seed, sub, off in cases:
        out = subprocess.run([exe, str(seed), str(sub), str(off), "3"], check=True,
                             capture_output=True, text=True).stdout.split()
        got = np.array(out, dtype=np.uint64).reshape(3, 4).astype(np.uint32)
        for call in range(3):
            n = off // 4 + call
            ctr = [n & 0xFFFFFFFF, n >> 32, sub & 0xFFFFFFFF, sub >> 32]
            key = [seed & 0xFFFFFFFF, seed >> 32]
            assert np.array_equal(O.philox4x32_10(ctr, key), got[call]), (seed, sub, off, call)


def test_sr_stream_in_quantizer_is_unbiased():
    """The quantizer's own Philox stream: a constant value in many blocks
    (each block anchored by one max element) averages to the value."""
    rows, cols = 512, 2048
    x = np.full((rows, cols), 2.6, np.float32)
    x[:, ::32] = 6.0                               # anchors: block exponent 0
    q, s, _ = O.quantize(x, O.AXIS_ROW, O.E2M1, sr=True, seed=0x1234, offset=9)
    assert np.all(s == 127)
    vals = np.array([O.decode(O.E2M1, c) for c in range(16)])[O.unpack_codes(q, O.E2M1)]
    body = np.delete(vals, np.s_[::32], axis=1).ravel()
    n = body.size
    sigma = 1.0 * np.sqrt(0.6 * 0.4 / n)
    assert abs(body.mean() - 2.6) < 5 * sigma
    # a different axis word or offset draws a different stream
    q2, _, _ = O.quantize(x, O.AXIS_ROW, O.E2M1, sr=True, seed=0x1234, offset=10)
    assert not np.array_equal(q, q2)

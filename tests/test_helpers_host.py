"""CPU checks of host-side facts the GPU code and tests lean on: the
vectorised bf16 rounding against the oracle's scalar routine, the stratified
output sampler, and the fp32 identity behind the Hadamard quantizers' block
maximum."""
import numpy as np

import oracle as O
from gpu_util import round_bf16_array, tile_samples


def test_round_bf16_array_matches_oracle():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(20000) * np.exp2(rng.integers(-130, 130, 20000))
    # exact ties and near-ties of bf16 (8 significant bits)
    base = np.ldexp(rng.integers(128, 256, 2000).astype(np.float64), rng.integers(-20, 20, 2000))
    ties = np.concatenate([base + np.ldexp(1.0, np.frexp(base)[1] - 9),
                           base + np.ldexp(1.0, np.frexp(base)[1] - 9) * (1 + 2.0 ** -40),
                           base + np.ldexp(1.0, np.frexp(base)[1] - 9) * (1 - 2.0 ** -40)])
    x = np.concatenate([x, ties, -ties, [0.0, -0.0, np.inf, -np.inf, 3.4e38, 1e-39, 2.0 ** -126]])
    got = round_bf16_array(x)
    ref = np.array([O.round_bf16(v) for v in x])
    assert np.array_equal(got, ref)


def test_tile_samples_cover_every_tile_with_corners():
    rng = np.random.default_rng(1)
    M, N = 300, 520                           # ragged last tiles in both directions
    ii, jj = tile_samples(rng, M, N)
    assert ii.min() >= 0 and ii.max() < M and jj.min() >= 0 and jj.max() < N
    tiles = set(zip((ii // 128).tolist(), (jj // 128).tolist()))
    assert len(tiles) == 3 * 5 and ii.size == 16 * 15
    for r0 in range(0, M, 128):
        for c0 in range(0, N, 128):
            r1, c1 = min(r0 + 128, M) - 1, min(c0 + 128, N) - 1
            got = set(zip(ii.tolist(), jj.tolist()))
            assert {(r0, c0), (r0, c1), (r1, c0), (r1, c1)} <= got


def _key(x):
    return x.view(np.uint32) & np.uint32(0x7FFFFFFF)


def test_butterfly_pair_max_is_sum_of_magnitudes():
    # The Hadamard quantizers take a block's |max| from the transform's last
    # stage: of a pair (a + b, a - b) rounded to fp32, the larger magnitude is
    # RN(|a| + |b|).  Checked here in IEEE float32 over wide exponents, exact
    # ties, subnormals, overflow and the non-finite cases, where only "at
    # least Inf" is needed.
    rng = np.random.default_rng(7)
    n = 400000
    with np.errstate(over="ignore"):          # a few draws overflow to +-Inf in the cast
        a = (rng.standard_normal(n) * np.exp2(rng.integers(-150, 128, n))).astype(np.float32)
        b = (rng.standard_normal(n) * np.exp2(rng.integers(-150, 128, n))).astype(np.float32)
    # near neighbours (cancellation), equal magnitudes, and ulp-level ties
    with np.errstate(over="ignore"):
        c = a[: n // 4] * np.float32(1 + 2.0 ** -20)
    d = np.nextafter(a[: n // 4], np.float32(np.inf))
    a = np.concatenate([a, a[: n // 4], a[: n // 4], a[: n // 4], np.float32([3e38, -3e38, np.inf, np.inf, np.nan, 1e-45, 0.0, -0.0])])
    b = np.concatenate([b, c, -d, a[: n // 4] * np.float32(2.0 ** -24), np.float32([3e38, 3e38, -np.inf, 1.0, 1.0, 1e-45, -0.0, -0.0])])
    with np.errstate(over="ignore", invalid="ignore"):
        s, t = a + b, a - b
        m = np.abs(a) + np.abs(b)
    both = np.maximum(_key(s), _key(t))
    finite = np.isfinite(s) & np.isfinite(t)
    assert np.array_equal(both[finite], _key(m)[finite])
    assert (_key(m)[~finite] >= 0x7F800000).all() and (both[~finite] >= 0x7F800000).all()
    assert (~finite).sum() >= 4

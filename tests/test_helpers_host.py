"""CPU checks of the GPU tests' own helpers: the vectorised bf16 rounding
against the oracle's scalar routine, and the stratified output sampler."""
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

"""The seeded input generators: determinism and the stated distributions."""
import numpy as np

from fp4_quantization_block_amd import inputs as I


def test_deterministic_and_distinct_streams():
    a = I.make("moss_two_level_4096", M=64, N=64, K=64)
    b = I.make("moss_two_level_4096", M=64, N=64, K=64)
    assert np.array_equal(a.tensors["A"], b.tensors["A"])
    assert not np.array_equal(a.tensors["A"], a.tensors["B"])


def test_distributions():
    w = I.make("moss_two_level_4096", M=512, N=512, K=4096)
    A = I.bf16_bits_to_f32(w.tensors["A"])
    colmax = np.abs(A).max(axis=0)
    # 0.1% of 4096 K-channels = 4 columns scaled x100
    assert (colmax > 20 * np.median(colmax)).sum() == 4
    B = I.bf16_bits_to_f32(w.tensors["B"])
    assert abs(B.std() - 0.02) < 0.001
    d = I.make("dual_layout_16384x14336", R=256, C=512)
    X = I.bf16_bits_to_f32(d.tensors["X"])
    frac = (np.abs(X) > 6).mean()
    assert 0.005 < frac < 0.015
    l = I.make("mxfp4_wgrad_qkv", T=256, H=128, Q=192)
    L = I.bf16_bits_to_f32(l.tensors["dY"])
    assert abs(np.abs(L).mean() - 1e-3) < 1e-4          # Laplace(b): E|x| = b


def test_bf16_rounding_is_rne():
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -0.0], np.float32)
    bits = I.to_bf16_bits(x)
    assert list(bits) == [0x3F80, 0x3F82, 0x8000]

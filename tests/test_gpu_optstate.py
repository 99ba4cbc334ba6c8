"""GPU parity of the FP8 optimizer-state quantization with dynamic range
expansion ([COAT, "解決方案：動態範圍擴充套件"]): codes, the per-group amax and
expansion exponent k, and the dequantized values must equal the oracle's
bit for bit (both evaluate the expansion as the same fixed sequence of fp32
operations)."""
import numpy as np
import pytest
import torch

import oracle as O
from fp4_quantization_block_amd import inputs as I
from fp4_quantization_block_amd import mx
from gpu_util import DEV, assert_codes_equal, assert_same_f32, log, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _run(x, fmt, group):
    xd = torch.from_numpy(np.ascontiguousarray(x.ravel())).to(DEV)
    q, amax, k = mx.mx_quantize_optstate(xd, fmt, group)
    back = mx.mx_dequantize_optstate(q, amax, k, fmt, group)
    torch.cuda.synchronize()
    return q.cpu().numpy(), amax.cpu().numpy(), k.cpu().numpy(), back.cpu().numpy()


def _compare(x, fmt, group, what):
    q, amax, k, back = _run(x, fmt, group)
    qo, amaxo, ko = O.optstate_quantize(x, fmt, group)
    assert_codes_equal(q.reshape(-1, group), qo.reshape(-1, group), f"{what} codes")
    assert_same_f32(amax, amaxo)
    assert_same_f32(k, ko)
    backo = O.optstate_dequantize(qo, amaxo, ko, fmt, group)
    assert_same_f32(back, backo)


def _mixed(rng, ngroups, group):
    """Groups spanning 0.2 to 40 decades, with zeros, signed zeros and fp32
    subnormals sprinkled in."""
    dec = rng.uniform(0.2, 40.0, (ngroups, 1))
    lo = rng.uniform(-30.0, 10.0, (ngroups, 1))
    mag = 10.0 ** (lo + dec * rng.random((ngroups, group)))
    x = (mag * rng.choice([-1.0, 1.0], (ngroups, group))).astype(np.float32)
    m = rng.random((ngroups, group))
    x[m < 0.03] = 0.0
    x[(m >= 0.03) & (m < 0.05)] = -0.0
    sub = (m >= 0.05) & (m < 0.06)
    x[sub] = (rng.standard_normal(sub.sum()) * 2.0 ** -135).astype(np.float32)
    return x


@pytest.mark.parametrize("group", [32, 64, 128, 256])
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_mixed_groups(fmt, group):
    rng = np.random.default_rng(group + len(fmt))
    _compare(_mixed(rng, 389, group), fmt, group, f"{fmt} G={group}")


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_degenerate_groups(fmt):
    x = np.full((8, 128), 0.25, np.float32)
    x[0] = 0.0
    x[1] = -0.0
    x[1, 3] = 0.0
    x[2, 5] = -0.25                      # one magnitude: k = 1
    x[3, 7] = np.nan
    x[4, 9] = np.inf
    x[5] = 0.0
    x[5, 11] = -3e-3                     # one nonzero element
    x[6] = 2.0 ** -149                   # smallest subnormal everywhere
    x[6, 0] = 3.0e38                     # ratio beyond fp32: k from log2(inf)
    x[7, :64] = 1e-30
    _compare(x, fmt, 128, f"{fmt} degenerate")


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_dequantize_any_parameters(fmt):
    """Every code under per-group parameters no quantizer produces: k of 0,
    negative, tiny, huge or infinite, and amax negative, zero, subnormal or
    infinite.  The powers then overflow, underflow or turn NaN, and the
    dequantizer must take each case as the oracle does."""
    params = [(1.0, 0.0), (1.0, -2.0), (1.0, np.inf), (1.0, 1e-30), (1.0, 1e30), (-3.0, 0.5), (np.inf, 1.0),
              (0.0, 1.0), (2.0 ** -140, 3.0), (1e30, 0.05), (7.5, 1.0), (1.0, -np.inf)]
    group = 256
    q = np.tile(np.arange(256, dtype=np.uint8), len(params))
    amax = np.array([a for a, _ in params], np.float32)
    k = np.array([kk for _, kk in params], np.float32)
    back = mx.mx_dequantize_optstate(torch.from_numpy(q).to(DEV), torch.from_numpy(amax).to(DEV),
                                     torch.from_numpy(k).to(DEV), fmt, group)
    torch.cuda.synchronize()
    assert_same_f32(back.cpu().numpy(), O.optstate_dequantize(q, amax, k, fmt, group))


@pytest.mark.parametrize("n_groups", [1, 3, 63, 1025])
def test_ragged_grid(n_groups):
    """Group counts that leave waves and workgroups partly empty."""
    rng = np.random.default_rng(n_groups)
    _compare(_mixed(rng, n_groups, 64), "e4m3", 64, f"{n_groups} groups")


def test_full_llama_wgu_moments():
    """Adam's first and second moments of the Llama-3-8B gate-up weight
    (4096 x 28672 fp32 each), E4M3 + E4M3 as the page recommends, group 128:
    every code, amax, k and dequantized value."""
    w = I.make("coat_optstate_llama_wgu")
    for name in ("m", "v"):
        _compare(w.tensors[name], "e4m3", 128, f"moment {name}")
        log(f"optimizer state {name}: all {w.tensors[name].size} elements equal the oracle")

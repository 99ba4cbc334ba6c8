"""Pins of the oracle's FP8 optimizer-state quantization with dynamic range
expansion ([COAT, "解決方案：動態範圍擴充套件"]).  CPU only.

The page keeps the goal but not the formula: an expansion function applied
before quantization, one parameter k per quantization group computed on the
fly, stretching the group's max/min ratio to E4M3's range (about 2e5) so
that the group spans the format from its smallest subnormal (0.00195) to
its maximum (448); k > 1 expands.  The reading (the COAT paper's f(x) =
sign(x)|x|^k, normalised by the group maximum) is pinned here by exactly
those stated properties, by its inverse, and by the library routines its
fp32 log2 / exp2 approximate."""
import math

import numpy as np
import pytest

import oracle as O

FMAX = {"e4m3": 448.0, "e5m2": 57344.0}
TOP = {"e4m3": 0x7E, "e5m2": 0x7B}                 # largest finite code
RANGE = {"e4m3": 448.0 / 2.0 ** -9, "e5m2": 57344.0 / 2.0 ** -16}


def ulp32(v):
    v = np.abs(np.asarray(v, np.float32))
    return np.spacing(v).astype(np.float64)


def test_log2_fp32_against_numpy():
    rng = np.random.default_rng(1)
    e = rng.uniform(-149, 128, 20000)
    x = np.exp2(e).astype(np.float32)
    x = x[(x > 0) & np.isfinite(x)]
    got = np.array([O.log2_fp32(v) for v in x])
    ref = np.log2(x.astype(np.float64))
    assert np.all(np.abs(got - ref) <= 2.0 * ulp32(ref) + 2.0 ** -23)
    for j in range(-149, 128):                           # powers of two are exact
        assert O.log2_fp32(np.float32(2.0 ** j)) == j


def test_exp2_fp32_against_numpy():
    rng = np.random.default_rng(2)
    y = rng.uniform(-125, 127, 20000).astype(np.float32)
    got = np.array([O.exp2_fp32(v) for v in y])
    ref = np.exp2(y.astype(np.float64))
    assert np.all(np.abs(got / ref - 1.0) <= 3 * 2.0 ** -23)
    for j in range(-149, 128):                           # integers are exact
        assert O.exp2_fp32(float(j)) == 2.0 ** j
    assert O.exp2_fp32(-151.0) == 0.0 and O.exp2_fp32(128.0) == math.inf
    sub = np.float32(-140.3)                             # subnormal results: one rounding
    assert abs(O.exp2_fp32(sub) - 2.0 ** float(sub)) <= 2.0 ** -149


def test_pow_fp32_against_float64():
    rng = np.random.default_rng(3)
    u = np.exp2(rng.uniform(-40, 0, 5000)).astype(np.float32)
    k = rng.uniform(0.3, 6.0, 5000).astype(np.float32)
    got = np.array([O.pow_fp32(a, b) for a, b in zip(u, k)])
    ref = u.astype(np.float64) ** k.astype(np.float64)
    ok = ref > 2.0 ** -120
    assert np.all(np.abs(got[ok] / ref[ok] - 1.0) <= 2e-5)
    assert O.pow_fp32(0.0, 2.5) == 0.0 and O.pow_fp32(1.0, 3.7) == 1.0


def _groups(rng, ngroups, group, lo_dec, hi_dec):
    """Values log-uniform over [10^lo, 10^hi] with random signs."""
    mag = 10.0 ** rng.uniform(lo_dec, hi_dec, (ngroups, group))
    return (mag * rng.choice([-1.0, 1.0], (ngroups, group))).astype(np.float32)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("decades", [0.5, 1.0, 3.0, 5.0, 8.0, 12.0])
def test_group_spans_the_format(fmt, decades):
    """The page's aim: after expansion each group covers the format from
    its maximum to its smallest subnormal -- the largest magnitude gets the
    top code, the smallest nonzero one the smallest subnormal code."""
    rng = np.random.default_rng(int(decades * 10) + len(fmt))
    x = _groups(rng, 64, 128, -6.0, -6.0 + decades)
    q, amax, k = O.optstate_quantize(x, fmt)
    q = q.reshape(64, 128)
    for g in range(64):
        a = np.abs(x[g])
        i_max, i_min = np.argmax(a), np.argmin(a)
        sign_max = 0x80 if x[g, i_max] < 0 else 0
        sign_min = 0x80 if x[g, i_min] < 0 else 0
        assert q[g, i_max] == TOP[fmt] | sign_max
        assert q[g, i_min] == 0x01 | sign_min
        assert amax[g] == a.max()
        r = float(a.max()) / float(a.min())
        assert abs(k[g] - math.log(RANGE[fmt]) / math.log(r)) <= 1e-5 * k[g]


def test_page_ratios_give_expanding_k():
    """First-moment groups with max/min ~1e3 and second-moment groups with
    ~10 (the page's typical ratios) get k > 1: the range is expanded."""
    for r, kk in ((1000.0, math.log(RANGE["e4m3"]) / math.log(1000.0)),
                  (10.0, math.log(RANGE["e4m3"]) / math.log(10.0))):
        x = np.linspace(1.0, r, 128).astype(np.float32) * np.float32(1e-4)
        _, _, k = O.optstate_quantize(x, "e4m3")
        assert k[0] > 1.0 and abs(k[0] - kk) <= 1e-5 * kk
    # wider than the format: k < 1 compresses
    x = np.exp2(np.linspace(-30, 0, 128)).astype(np.float32)
    _, _, k = O.optstate_quantize(x, "e4m3")
    assert k[0] < 1.0


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_codes_monotone_in_magnitude(fmt):
    rng = np.random.default_rng(7)
    x = _groups(rng, 32, 128, -8, -3)
    q, _, _ = O.optstate_quantize(x, fmt)
    q = q.reshape(32, 128)
    for g in range(32):
        order = np.argsort(np.abs(x[g]), kind="stable")
        mags = np.array([abs(O.decode(fmt, c)) for c in q[g][order]])
        assert np.all(np.diff(mags) >= 0)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_round_trip_error_bound(fmt):
    """dequantize(quantize(x)): the FP8 rounding error of y = u^k Fmax
    (half a code step relative to y) shrinks by the 1/k root; fp32 slack 1e-5."""
    rng = np.random.default_rng(8)
    x = _groups(rng, 64, 128, -7, -3)
    q, amax, k = O.optstate_quantize(x, fmt)
    back = O.optstate_dequantize(q, amax, k, fmt)
    xs = x.ravel().astype(np.float64)
    kk = np.repeat(k.astype(np.float64), 128)
    am = np.repeat(amax.astype(np.float64), 128)
    y = (np.abs(xs) / am) ** kk * FMAX[fmt]
    codes = np.array([O.decode(fmt, c) for c in range(128)])          # positive code values
    codes = codes[np.isfinite(codes)]
    n = codes.size
    i = np.searchsorted(codes, y, side="right")
    step = codes[np.minimum(i, n - 1)] - codes[np.maximum(i - 1, 0)]  # spacing around y
    step = np.where(i >= n, codes[n - 1] - codes[n - 2], step)        # at the top code
    delta = 0.5 * step / y
    # rounded down or up by at most delta relative, then the 1/k root
    bound = np.maximum(1.0 - (1.0 - delta) ** (1.0 / kk), (1.0 + delta) ** (1.0 / kk) - 1.0) + 1e-5
    rel = np.abs(back.astype(np.float64) / xs - 1.0)
    assert np.all(rel <= bound)
    assert np.all(np.sign(back) == np.sign(xs))


@pytest.mark.parametrize("decades,factor", [(3.0, 1.0), (1.0, 0.35)])
def test_expansion_beats_plain_group_scaling(decades, factor):
    """The page: expansion greatly reduces the quantization error.  Against
    the same groups quantized with k = 1 (plain per-group absmax scaling to
    448): at the page's typical max/min ratios, ~1e3 (first moment, three
    decades: k ~ 1.8) it is lower, and ~10 (second moment, one decade:
    k ~ 5.4) less than a third, since the 1/k root divides the FP8
    relative error by k."""
    rng = np.random.default_rng(9)
    x = _groups(rng, 256, 128, -6, -6 + decades).astype(np.float32)
    q, amax, k = O.optstate_quantize(x, "e4m3")
    back = O.optstate_dequantize(q, amax, k, "e4m3")
    ones = np.ones_like(k)
    q1 = O.encode_array("e4m3", (x.reshape(256, 128) / amax[:, None] * 448.0).ravel())
    back1 = O.optstate_dequantize(q1, amax, ones, "e4m3")
    e_exp = np.mean(np.abs(back / x.ravel() - 1))
    e_plain = np.mean(np.abs(back1 / x.ravel() - 1))
    assert e_exp < factor * e_plain, (e_exp, e_plain)


def test_degenerate_groups():
    x = np.zeros((4, 128), np.float32)
    x[0, :] = -0.0
    x[1, :] = 3.0                                         # one magnitude: k = 1, all top codes
    x[1, 5] = -3.0
    x[2, 7] = np.nan
    x[3, 9] = 2.5e-3                                      # one nonzero element
    q, amax, k = O.optstate_quantize(x, "e4m3")
    q = q.reshape(4, 128)
    assert np.all(q[0] == 0x80) and amax[0] == 1.0 and k[0] == 1.0
    assert np.all(q[1][np.arange(128) != 5] == 0x7E) and q[1, 5] == 0xFE and k[1] == 1.0
    assert np.all(q[2] == 0x7F) and np.isnan(amax[2]) and np.isnan(k[2])
    assert q[3, 9] == 0x7E and np.all(np.delete(q[3], 9) == 0) and k[3] == 1.0
    back = O.optstate_dequantize(q.ravel(), amax, k, "e4m3").reshape(4, 128)
    assert np.all(back[1] == np.where(np.arange(128) == 5, -3.0, 3.0))
    assert np.all(np.isnan(back[2]))
    assert back[3, 9] == np.float32(2.5e-3)

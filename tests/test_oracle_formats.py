"""Pins of the oracle's element formats and rounding against sources other
than the oracle itself: torch's float8 dtypes (an independent encoder and
decoder), transformers' MXFP4 value table, and the constants the pages print.
"""
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split()[:2]
                vals[k] = float(v)
    return vals


def _torch_decode(dtype, codes):
    t = torch.tensor(codes, dtype=torch.uint8).view(dtype).to(torch.float64)
    return t.numpy()


@pytest.mark.parametrize("fmt,dtype", [(O.E4M3, torch.float8_e4m3fn),
                                       (O.E5M2, torch.float8_e5m2)])
def test_fp8_decode_all_codes_matches_torch(fmt, dtype):
    codes = list(range(256))
    ref = _torch_decode(dtype, codes)
    got = np.array([O.decode(fmt, c) for c in codes])
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.all(both_nan | (ref == got))
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    # signed zero
    assert np.signbit(got[0x80]) and not np.signbit(got[0])


def test_e8m0_decode_all_bytes_matches_torch():
    ref = _torch_decode(torch.float8_e8m0fnu, list(range(256)))
    got = np.array([O.decode_e8m0(b) for b in range(256)])
    assert np.isnan(ref[255]) and np.isnan(got[255])
    assert np.array_equal(ref[:255], got[:255])


def test_e2m1_decode_matches_mxfp4_library_table():
    mx = pytest.importorskip("transformers.integrations.mxfp4")
    table = np.array(mx.FP4_VALUES, dtype=np.float64)
    got = np.array([O.decode(O.E2M1, c) for c in range(16)])
    assert np.array_equal(got, table)
    assert np.array_equal(np.signbit(got), np.signbit(table))


def test_page_constants():
    g = _golden("page_constants.txt")
    assert O.fmax(O.E4M3) == g["e4m3_max"]
    min_sub = O.decode(O.E4M3, 0x01)
    assert abs(min_sub - g["e4m3_min_subnormal"]) < 5e-6          # page prints 0.00195
    assert min_sub == 2.0 ** -9
    ratio = O.fmax(O.E4M3) / min_sub
    assert ratio == 229376.0
    assert 0.5 * g["e4m3_dynamic_range"] < ratio < 2 * g["e4m3_dynamic_range"]
    # E2M1: 1 sign + 2 exponent + 1 mantissa bits
    assert O.elem_bits(O.E2M1) == 1 + int(g["e2m1_exponent_bits"]) + int(g["e2m1_mantissa_bits"])
    # power-of-two illustration: scale 2^3 times a value is an exponent shift
    k = int(g["pow2_example_k"])
    assert O.decode_e8m0(127 + k) * g["pow2_example_value"] == g["pow2_example_product"]


def test_page_example_value_is_not_e4m3():
    """The page's illustrative fp8 value 50 is not an E4M3 value: RNE gives 48
    (code 0x64), the same as torch's cast."""
    g = _golden("page_constants.txt")
    c = O.encode_rne(O.E4M3, g["pow2_example_value"])
    t = torch.tensor([g["pow2_example_value"]], dtype=torch.float32).to(torch.float8_e4m3fn)
    assert c == t.view(torch.uint8).item() == 0x64
    assert O.decode(O.E4M3, c) == 48.0


def _sweep_values(fmt, rng):
    """fp32 values around every code value and every midpoint (+-1, +-2 ulp),
    plus random values across the whole finite range, both signs."""
    n = {O.E4M3: 127, O.E5M2: 124, O.E2M1: 8}[fmt]
    t = np.array([O.decode(fmt, k) for k in range(n)], dtype=np.float64)
    pts = list(t) + list(0.5 * (t[1:] + t[:-1]))
    vals = []
    for p in pts:
        f = np.float32(p)
        vals.append(f)
        up, dn = f, f
        for _ in range(2):
            up = np.nextafter(up, np.float32(np.inf))
            dn = np.nextafter(dn, np.float32(-np.inf))
            vals += [up, dn]
    fmax = t[-1]
    lo_exp = np.log2(t[1]) - 4
    mags = np.exp2(rng.uniform(lo_exp, np.log2(fmax), 20000)).astype(np.float32)
    vals = np.array(vals + list(mags), dtype=np.float32)
    vals = vals[(vals >= 0) & (vals <= fmax)]
    return np.concatenate([vals, -vals])


@pytest.mark.parametrize("fmt,dtype", [(O.E4M3, torch.float8_e4m3fn),
                                       (O.E5M2, torch.float8_e5m2)])
def test_fp8_rne_matches_torch_cast_in_range(fmt, dtype):
    rng = np.random.default_rng(11)
    y = _sweep_values(fmt, rng)
    got = O.encode_array(fmt, y)
    ref = torch.from_numpy(y).to(dtype).view(torch.uint8).numpy()
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, (y[bad[:5]], got[bad[:5]], ref[bad[:5]])


@pytest.mark.parametrize("fmt,dtype", [(O.E4M3, torch.float8_e4m3fn),
                                       (O.E5M2, torch.float8_e5m2)])
def test_fp8_rne_strided_fp32_patterns(fmt, dtype):
    """Every 211th fp32 bit pattern from 0 up to the format's maximum."""
    top = np.float32(O.fmax(fmt)).view(np.uint32)
    bits = np.arange(0, int(top) + 1, 211, dtype=np.uint32)
    y = bits.view(np.float32)
    got = O.encode_array(fmt, y)
    ref = torch.from_numpy(y.copy()).to(dtype).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


def test_e2m1_rne_brute_force():
    """Nearest value over the library table, ties to the even code."""
    mx = pytest.importorskip("transformers.integrations.mxfp4")
    table = np.array(mx.FP4_VALUES[:8], dtype=np.float64)
    rng = np.random.default_rng(12)
    y = _sweep_values(O.E2M1, rng)
    got = O.encode_array(O.E2M1, y)
    a = np.abs(y.astype(np.float64))
    d = np.abs(a[:, None] - table[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among tied candidates prefer the even code index
    even = cand & (np.arange(8)[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    ref = pick | np.where(np.signbit(y), 8, 0)
    assert np.array_equal(got, ref.astype(np.uint8))


@pytest.mark.parametrize("fmt", [O.E4M3, O.E5M2, O.E2M1])
def test_saturation_and_signed_zero(fmt):
    fm = O.fmax(fmt)
    top = {O.E4M3: 0x7E, O.E5M2: 0x7B, O.E2M1: 0x7}[fmt]
    sbit = 0x80 if fmt != O.E2M1 else 0x8
    for y in (fm, fm * 1.03, fm * 1.2, fm * 1.99, 1e30):
        assert O.encode_rne(fmt, y) == top
        assert O.encode_rne(fmt, -y) == top | sbit
        for u in (0, 1 << 31, 0xFFFFFFFF):
            assert O.encode_sr(fmt, y, u) == top
    assert O.encode_rne(fmt, -0.0) == sbit
    assert O.encode_rne(fmt, -1e-30) == sbit
    assert O.encode_rne(fmt, 1e-30) == 0


def test_e4m3_overflow_differs_from_torch_only_by_saturation():
    """Above 464 torch's non-saturating cast gives NaN; the oracle saturates."""
    assert torch.tensor([470.0]).to(torch.float8_e4m3fn).view(torch.uint8).item() == 0x7F
    assert O.encode_rne(O.E4M3, 470.0) == 0x7E


def test_table_strictly_increasing():
    for fmt, n in ((O.E4M3, 127), (O.E5M2, 124), (O.E2M1, 8)):
        t = [O.decode(fmt, k) for k in range(n)]
        assert all(b > a for a, b in zip(t, t[1:]))
        assert O.emax(fmt) == int(np.floor(np.log2(O.fmax(fmt))))

"""Pins of the oracle's scale rule, quantizer, layouts and dequantizer.

Each check leans on something other than the oracle: the defining property
of the OCP shared exponent (the block max lands in the element format's top
binade), exactness of power-of-two scaling ([MOSS] "Power-of-Two 的关键优势"),
round-trip identity on representable blocks, numpy's IEEE float32 division
for the two-level step ([MOSS] "两级缩放实现"), transposition symmetry, and
transformers' MXFP4 dequantizer for the FP4 packing.
"""
import numpy as np
import pytest
import torch

import oracle as O

FMTS = [O.E4M3, O.E5M2, O.E2M1]
TOP_CODE = {O.E4M3: 0x7E, O.E5M2: 0x7B, O.E2M1: 0x7}
NCODE = {O.E4M3: 127, O.E5M2: 124, O.E2M1: 8}


def _bf16_bits(a32):
    return torch.from_numpy(np.ascontiguousarray(a32, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def _bf16_to_f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("fmt,amax,byte", [(O.E4M3, 448.0, 127), (O.E4M3, 1.0, 119),
                                           (O.E2M1, 6.0, 127), (O.E5M2, 2.5e-3, 103),
                                           (O.E4M3, 0.0, 0), (O.E4M3, 2.0 ** -140, 0),
                                           (O.E2M1, 3.0e38, 252)])
def test_block_exponent_hand_cases(fmt, amax, byte):
    assert O.block_exponent(fmt, amax) + 127 == byte


@pytest.mark.parametrize("fmt", FMTS)
def test_block_max_lands_in_top_binade(fmt):
    """OCP rule: after dividing by 2^e the block max lies in [2^emax, 2^(emax+1))."""
    rng = np.random.default_rng(1)
    amax = np.exp2(rng.uniform(-100, 100, 5000)).astype(np.float32)
    em = O.emax(fmt)
    for a in amax:
        e = O.block_exponent(fmt, float(a))
        y = float(a) * 2.0 ** (-e)
        assert 2.0 ** em <= y < 2.0 ** (em + 1)


@pytest.mark.parametrize("fmt", FMTS)
def test_dequant_exact_for_all_codes_and_bytes(fmt):
    """decode(code) * 2^(byte-127) is exact in fp32 for every byte the
    quantizer can emit (<= 254 - emax), and overflows beyond."""
    bits = O.elem_bits(fmt)
    ncodes = 1 << bits
    limit = 254 - O.emax(fmt)
    codes = np.arange(ncodes, dtype=np.uint8)
    vals = np.array([O.decode(fmt, c) for c in codes])
    for byte in list(range(0, limit + 1)):
        blk = np.resize(codes, 32)
        if bits == 4:
            q = (blk[0::2] | (blk[1::2] << 4)).astype(np.uint8)[None, :]
        else:
            q = blk[None, :]
        out = O.dequantize(q, np.array([[byte]], np.uint8), None, fmt, 1, 32, O.AXIS_ROW)
        ref = np.resize(vals, 32) * 2.0 ** (byte - 127)
        fin = np.isfinite(ref)
        assert np.array_equal(out[0][fin].astype(np.float64), ref[fin])
        assert np.array_equal(np.isnan(out[0]), np.isnan(ref))


def _representable_blocks(fmt, rng, nblk, byte_lo=60, byte_hi=180):
    """Blocks of random codes whose largest magnitude has the top exponent
    field, with random scale bytes: quantization must reproduce them."""
    bits = O.elem_bits(fmt)
    nmag = NCODE[fmt]
    mbits = {O.E4M3: 3, O.E5M2: 2, O.E2M1: 1}[fmt]
    top_binade = range(nmag - (1 << mbits) + 1, nmag) if fmt == O.E4M3 else \
        range(nmag - (1 << mbits), nmag)
    codes = rng.integers(0, nmag, size=(nblk, 32))
    pos = rng.integers(0, 32, size=nblk)
    codes[np.arange(nblk), pos] = rng.choice(list(top_binade), size=nblk)
    signs = rng.integers(0, 2, size=(nblk, 32)) << (bits - 1)
    codes = (codes | signs).astype(np.uint8)
    scales = rng.integers(byte_lo, byte_hi, size=nblk).astype(np.uint8)
    return codes, scales


@pytest.mark.parametrize("fmt", FMTS)
def test_round_trip_identity_on_representable_blocks(fmt):
    rng = np.random.default_rng(2)
    codes, scales = _representable_blocks(fmt, rng, 512)
    vals = np.array([[O.decode(fmt, c) for c in row] for row in codes]) * \
        np.exp2(scales.astype(np.float64) - 127)[:, None]
    x = vals.astype(np.float32).reshape(16, 32 * 32)       # 16 rows x 32 blocks
    q, s, _ = O.quantize(x, O.AXIS_ROW, fmt)
    got = O.unpack_codes(q, fmt).reshape(512, 32)
    # -0 codes stay -0; +0 stays +0
    assert np.array_equal(got, codes)
    assert np.array_equal(s.reshape(-1), scales)


def test_e4m3_1p875_significand_exception():
    """A block whose max is 1.875*2^k rescales to 480, which E4M3 cannot hold
    (1.875*2^8 is its NaN pattern): it saturates to 448, so the value-level
    round trip fails for exactly this case."""
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 240.0
    x[0, 1] = 3.0
    q, s, _ = O.quantize(x, O.AXIS_ROW, O.E4M3)
    assert s[0, 0] == 127 - 1
    assert q[0, 0] == 0x7E
    back = O.dequantize(q, s, None, O.E4M3, 1, 32, O.AXIS_ROW)
    assert back[0, 0] == 224.0 and back[0, 1] == 3.0


@pytest.mark.parametrize("fmt", FMTS)
def test_two_level_equals_float32_division_then_mx(fmt):
    rng = np.random.default_rng(3)
    x = _bf16_bits(rng.standard_t(3, size=(64, 128)).astype(np.float32) * 7)
    q2, s2, st = O.quantize(x, O.AXIS_ROW, fmt, two_level=1)
    xf = _bf16_to_f32(x)
    amax = np.float32(np.abs(xf).max())
    st_ref = amax / np.float32(O.fmax(fmt))            # numpy float32 IEEE division
    assert np.float32(st) == st_ref
    q1, s1, _ = O.quantize((xf / np.float32(st_ref)).astype(np.float32), O.AXIS_ROW, fmt)
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)
    # provided-scale mode reproduces it
    q3, s3, _ = O.quantize(x, O.AXIS_ROW, fmt, two_level=2, tensor_scale=st)
    assert np.array_equal(q3, q2) and np.array_equal(s3, s2)


def test_two_level_zero_tensor_unit_scale():
    x = np.zeros((32, 32), np.float32)
    q, s, st = O.quantize(x, O.AXIS_ROW, O.E4M3, two_level=1)
    assert st == 1.0 and not q.any() and np.all(s == 0)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("src", ["f32", "bf16"])
def test_col_layout_is_row_layout_of_transpose(fmt, src):
    rng = np.random.default_rng(4)
    x = rng.standard_normal((96, 64)).astype(np.float32)
    if src == "bf16":
        x = _bf16_bits(x)
    qc, sc, _ = O.quantize(x, O.AXIS_COL, fmt)
    qr, sr_, _ = O.quantize(np.ascontiguousarray(x.T), O.AXIS_ROW, fmt)
    assert np.array_equal(qc, qr) and np.array_equal(sc, sr_)
    # the sampled-block entry point agrees with the whole-tensor one
    r0 = np.array([0, 32, 64, 32]); c0 = np.array([0, 5, 63, 17])
    codes, s = O.quantize_blocks(x, O.AXIS_COL, fmt, r0, c0)
    uc = O.unpack_codes(qc, fmt)
    for b in range(4):
        assert np.array_equal(codes[b], uc[c0[b], r0[b]:r0[b] + 32])
        assert s[b] == sc[c0[b], r0[b] // 32]


def test_fp4_packing_matches_mxfp4_library_dequant():
    """transformers' MXFP4 dequantizer (low nibble = even element, E8M0 bias
    127) reproduces the oracle's own dequantization of its packed output."""
    mx = pytest.importorskip("transformers.integrations.mxfp4")
    rng = np.random.default_rng(5)
    x = rng.laplace(0, 1e-3, size=(8, 256)).astype(np.float32)
    q, s, _ = O.quantize(x, O.AXIS_ROW, O.E2M1)
    # the library takes (experts, rows, groups, 16 bytes) and returns the
    # (experts, cols, rows) transpose
    blocks = torch.from_numpy(q.reshape(1, 8, 8, 16).copy())
    scales = torch.from_numpy(s.reshape(1, 8, 8).copy())
    lib = mx._convert_moe_packed_tensors(blocks, scales, dtype=torch.float32)
    lib = lib[0].T.contiguous().numpy()
    ours = O.dequantize(q, s, None, O.E2M1, 8, 256, O.AXIS_ROW)
    assert np.array_equal(lib, ours)


def test_nonfinite_block_reading():
    x = np.ones((2, 32), np.float32)
    x[0, 3] = np.nan
    x[1, 4] = -np.inf
    x[1, 5] = -2.0
    for fmt in (O.E4M3, O.E5M2):
        q, s, _ = O.quantize(x, O.AXIS_ROW, fmt)
        assert s[0, 0] == 0xFF and s[1, 0] == 0xFF
        # every element of a non-finite block: the canonical NaN, no sign
        assert np.all(q[0] == 0x7F) and np.all(q[1] == 0x7F)
    q, s, _ = O.quantize(x, O.AXIS_ROW, O.E2M1)
    assert s[0, 0] == 0xFF and not q.any()


def test_signed_zero_survives():
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 1.0
    x[0, 1] = -0.0
    x[0, 2] = -1e-12
    q, s, _ = O.quantize(x, O.AXIS_ROW, O.E4M3)
    assert q[0, 1] == 0x80 and q[0, 2] == 0x80 and q[0, 3] == 0x00


def test_subnormal_source_values():
    """bf16 / fp32 subnormals are exact reals: a block of them scales up to
    a normal range and quantizes like any other block."""
    x = np.zeros((1, 32), np.float32)
    x[0, :] = np.float32(2.0 ** -140) * np.arange(1, 33, dtype=np.float32)
    q, s, _ = O.quantize(x, O.AXIS_ROW, O.E4M3)
    assert s[0, 0] == 0       # clamped at 2^-127
    y = x[0].astype(np.float64) * 2.0 ** 127
    assert np.array_equal(q[0], O.encode_array(O.E4M3, y.astype(np.float32)))


def test_hadamard_quantization_equals_matrix_product_on_integers():
    """With small-integer inputs the fp32 transform is exact, so quantizing
    with the Hadamard flag equals quantizing H@x computed by scipy."""
    scipy_linalg = pytest.importorskip("scipy.linalg")
    H = scipy_linalg.hadamard(32).astype(np.float64)
    rng = np.random.default_rng(6)
    x = rng.integers(-8, 9, size=(64, 32)).astype(np.float32)       # col blocks of 32 rows
    q, s, _ = O.quantize(x, O.AXIS_COL, O.E4M3, hadamard=True)
    hx = (H @ x.astype(np.float64)[0:32]).astype(np.float32)
    hx2 = (H @ x.astype(np.float64)[32:64]).astype(np.float32)
    q2, s2, _ = O.quantize(np.vstack([hx, hx2]), O.AXIS_COL, O.E4M3)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)


@pytest.mark.parametrize("fmt", FMTS)
def test_dequantize_inverts_quantize_within_half_step(fmt):
    """|x - dq(q(x))| <= half a code step at the block scale (RNE), and the
    inverse Hadamard / tensor scale recover the source layout."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((64, 96)).astype(np.float32)
    for axis in (O.AXIS_ROW, O.AXIS_COL):
        for had in (False, True):
            q, s, st = O.quantize(x, axis, fmt, two_level=1, hadamard=had)
            back = O.dequantize(q, s, st, fmt, 64, 96, axis, hadamard=had)
            assert back.shape == x.shape
            err = np.abs(back.astype(np.float64) - x)
            # relative to each block's max: at most one element step of the
            # format (2^-mbits of the top binade), times sqrt(32) spread by H
            mb = {O.E4M3: 3, O.E5M2: 2, O.E2M1: 1}[fmt]
            tol = np.abs(x).max() * 2.0 ** (-mb) * (6.0 if had else 1.0)
            assert err.max() <= tol


@pytest.mark.parametrize("axis", [O.AXIS_ROW, O.AXIS_COL])
def test_dequantize_hadamard_tensor_scale_exact(axis):
    """The Hadamard + tensor-scale branch of dequantize on a case whose
    every intermediate is exact: small-integer E4M3 codes, power-of-two
    block scales, so x_hat, H.x_hat (scipy's Sylvester matrix) and the 1/32
    are exact and the result is one rounding of H.x_hat/32 * s_t.  With an
    s_t of long significand this fixes the order (inverse transform first,
    then the tensor scale once): scaling each element before the transform
    gives different bits."""
    scipy_linalg = pytest.importorskip("scipy.linalg")
    H = scipy_linalg.hadamard(32).astype(np.float64)
    rng = np.random.default_rng(12)
    rows, cols = 64, 96
    v = rng.integers(-15, 16, (rows, cols)).astype(np.float64)     # exact in E4M3
    codes = np.array([O.encode_rne(O.E4M3, t) for t in v.ravel()], np.uint8).reshape(rows, cols)
    st = np.float32(0.1)
    if axis == O.AXIS_ROW:
        bytes_ = rng.integers(124, 131, (rows, cols // 32)).astype(np.uint8)
        xhat = v * np.exp2(np.repeat(bytes_, 32, 1).astype(np.float64) - 127)
        blocks = xhat.reshape(rows, cols // 32, 32)
        exact = np.einsum("ij,rbj->rbi", H, blocks).reshape(rows, cols) / 32
        q, s = codes, bytes_
    else:
        bytes_ = rng.integers(124, 131, (cols, rows // 32)).astype(np.uint8)      # [col][row block]
        xhat = v * np.exp2(np.repeat(bytes_.T, 32, 0).astype(np.float64) - 127)
        blocks = xhat.reshape(rows // 32, 32, cols)
        exact = np.einsum("ij,bjc->bic", H, blocks).reshape(rows, cols) / 32
        q, s = np.ascontiguousarray(codes.T), bytes_
    got = O.dequantize(q, s, float(st), O.E4M3, rows, cols, axis, hadamard=True)
    want = (exact * np.float64(st)).astype(np.float32)              # one rounding of an exact product
    assert np.array_equal(got, want)
    # the other order: each element scaled (rounded) first, then the transform
    xs = (xhat * np.float64(st)).astype(np.float32).astype(np.float64)
    if axis == O.AXIS_ROW:
        other = np.einsum("ij,rbj->rbi", H, xs.reshape(rows, cols // 32, 32)).reshape(rows, cols) / 32
    else:
        other = np.einsum("ij,bjc->bic", H, xs.reshape(rows // 32, 32, cols)).reshape(rows, cols) / 32
    assert not np.array_equal(got, other.astype(np.float32))

"""GPU parity of the nvfp routes ([FAF, "格式感知融合的设计思路"]: global and
CTA-local nvfp beside native mxfp; [FAF, "FP4加速为何常常纸上富贵"]: nvfp is
one scale per block).  Codes, E4M3 block scales and FP32 second-level
scales must equal the oracle's bit for bit, dequantized values too; the
GEMM must stay within the stated bound |C - C_ref| <= 1e-5 (|A||B|) + 1e-6
of the oracle's float64 product of the same copies."""
import numpy as np
import pytest
import torch

import oracle as O
from fp4_quantization_block_amd import inputs as I
from fp4_quantization_block_amd import mx
from gpu_util import DEV, assert_codes_equal, assert_same_f32, gemm_check, log, record, to_device, u8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    from gpu_util import require_gpu
    require_gpu()


def _source(rng, rows, cols, src):
    """Rows and columns of widely different magnitudes (so that local
    domains differ from the global one and block scales reach E4M3's
    subnormals and zero), zero blocks, signed zeros."""
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    # magnitudes constant over 16-row groups, so that column blocks (16
    # rows) differ as much as row blocks
    x *= np.exp2(np.repeat(rng.integers(-14, 4, (rows + 15) // 16), 16)[:rows, None]).astype(np.float32)
    x *= np.exp2(rng.integers(-6, 2, (1, cols))).astype(np.float32)
    x[rng.random((rows, cols)) < 0.02] = 0.0
    x[rng.random((rows, cols)) < 0.01] = -0.0
    if rows > 2 and cols >= 32:
        x[1, :16] = 0.0
        x[2, 16:32] = -0.0
    return I.to_bf16_bits(x) if src == "bf16" else x


def _quantize_gpu(x, axis, local, ld_pad=0):
    xd = to_device(x)
    if ld_pad:
        big = torch.zeros((x.shape[0], x.shape[1] + ld_pad), dtype=xd.dtype, device=DEV)
        big[:, : x.shape[1]] = xd
        xd = big[:, : x.shape[1]]
    q, s, t = mx.mx_quantize_nvfp(xd, axis, local)
    torch.cuda.synchronize()
    return q, s, t


def _compare_copy(x, axis, local, what, ld_pad=0):
    q, s, t = _quantize_gpu(x, axis, local, ld_pad)
    qo, so, to = O.nvfp_quantize(x, axis, local)
    assert_same_f32(t.cpu().numpy(), to)
    assert_codes_equal(u8(s), so, f"{what} block scales")
    assert_codes_equal(u8(q), qo, f"{what} codes")
    return q, s, t, qo, so, to


@pytest.mark.parametrize("src", ["f32", "bf16"])
@pytest.mark.parametrize("local", [False, True])
@pytest.mark.parametrize("axis", [mx.MX_AXIS_ROW, mx.MX_AXIS_COL])
def test_quantize_and_dequantize_match_oracle(axis, local, src):
    """Several panels and a ragged last panel (SR = 200 or 216 stored rows),
    a strided source."""
    rng = np.random.default_rng(10 + 4 * axis + 2 * local + (src == "bf16"))
    rows, cols = (200, 384) if axis == mx.MX_AXIS_ROW else (384, 216)
    x = _source(rng, rows, cols, src)
    log(f"nvfp quantize axis={axis} local={local} src={src} {rows}x{cols}")
    q, s, t, qo, so, to = _compare_copy(x, axis, local, f"axis={axis} local={local} {src}", ld_pad=48)
    back = mx.mx_dequantize_nvfp(q, s, t, rows, cols, axis, local, mx.MX_OUT_F32)
    ref = O.nvfp_dequantize(qo, so, to, rows, cols, axis, local)
    assert_same_f32(back.cpu().numpy(), ref)
    back16 = mx.mx_dequantize_nvfp(q, s, t, rows, cols, axis, local, mx.MX_OUT_BF16)
    ref16 = torch.from_numpy(ref).to(torch.bfloat16)                 # round to nearest even
    assert torch.equal(back16.cpu().view(torch.int16), ref16.view(torch.int16))
    # the block scales reach E4M3 subnormals and zero in this input
    assert (so == 0).any() and ((so > 0) & (so < 8)).any()


@pytest.mark.parametrize("local", [False, True])
@pytest.mark.parametrize("axis", [mx.MX_AXIS_ROW, mx.MX_AXIS_COL])
def test_unaligned_rows(axis, local):
    """Row starts off 16-byte alignment (ld = cols + 3): the element-wise
    load path, bit-exact as the vector one."""
    rng = np.random.default_rng(50 + 2 * axis + local)
    rows, cols = (96, 208) if axis == mx.MX_AXIS_ROW else (208, 100)
    x = _source(rng, rows, cols, "bf16")
    _compare_copy(x, axis, local, f"unaligned axis={axis} local={local}", ld_pad=3)


@pytest.mark.parametrize("local", [False, True])
def test_special_values(local):
    """A NaN poisons its domain: the whole tensor (global) or its panel
    (local); Inf likewise; an all-zero domain gets scale 1."""
    rng = np.random.default_rng(21)
    x = rng.standard_normal((96, 64)).astype(np.float32)
    x[40, 5] = np.nan
    x[70, 9] = np.inf
    x[:32] = 0.0
    x[0, 0] = -0.0
    q, s, t, qo, so, to = _compare_copy(x, mx.MX_AXIS_ROW, local, f"special local={local}")
    if local:
        assert to[0] == 1.0 and np.isnan(to[1]) and np.isnan(to[2])
    else:
        assert np.isnan(to[0]) and np.all(so == 0x7F)
    z = np.zeros((64, 32), np.float32)
    _compare_copy(z, mx.MX_AXIS_COL, local, f"zeros local={local}")


def test_single_row_and_block():
    """Degenerate sizes: one stored row of one block; one source row."""
    rng = np.random.default_rng(22)
    _compare_copy(rng.standard_normal((1, 16)).astype(np.float32), mx.MX_AXIS_ROW, True, "1x16 row")
    _compare_copy(rng.standard_normal((16, 1)).astype(np.float32), mx.MX_AXIS_COL, False, "16x1 col")
    _compare_copy(rng.standard_normal((16, 3)).astype(np.float32), mx.MX_AXIS_COL, True, "16x3 col")
    # bf16, CTA-local: the one-pass kernel (one stored row; one 8-column panel)
    _compare_copy(I.to_bf16_bits(rng.standard_normal((1, 16)).astype(np.float32)), mx.MX_AXIS_ROW, True, "1x16 bf16")
    _compare_copy(I.to_bf16_bits(rng.standard_normal((16, 8)).astype(np.float32)), mx.MX_AXIS_COL, True, "16x8 bf16")


@pytest.mark.parametrize("axis", [mx.MX_AXIS_ROW, mx.MX_AXIS_COL])
def test_local_one_pass_shapes(axis):
    """The one-pass CTA-local kernel (bf16, blocked length <= 4096) at its
    limit and with ragged panels: L = 4096 with 40 stored rows, and a short
    L = 48 (only 6 chunks of a 32-lane row group in use)."""
    rng = np.random.default_rng(60 + axis)
    for SR, L in ((40, 4096), (72, 48)):
        rows, cols = (SR, L) if axis == mx.MX_AXIS_ROW else (L, SR)
        x = _source(rng, rows, cols, "bf16")
        log(f"one-pass local axis={axis} {rows}x{cols}")
        _compare_copy(x, axis, True, f"one-pass axis={axis} {rows}x{cols}")


def test_invalid_arguments():
    x = torch.zeros((32, 24), dtype=torch.float32, device=DEV)
    with pytest.raises(mx.MXError, match="multiple of 16"):
        mx.mx_quantize_nvfp(x, mx.MX_AXIS_ROW)
    q = torch.zeros((32, 32), dtype=torch.uint8, device=DEV)
    s = torch.zeros((32, 4), dtype=torch.uint8, device=DEV)
    t = torch.ones(1, dtype=torch.float32, device=DEV)
    with pytest.raises(mx.MXError, match="multiple of 64"):
        mx.mx_gemm_nvfp(q, s, t, False, q, s, t, False, 32, 32, 48)
    c = torch.empty((32, 16), dtype=torch.float32, device=DEV)
    with pytest.raises(mx.MXError, match="ldc"):
        mx.mx_gemm_nvfp(q, s, t, False, q, s, t, False, 32, 32, 64, out_dtype=mx.MX_OUT_F32, c=c)


def _gemm_case(rng, M, N, K, la, lb, out, alpha, what, full=True, ii=None, jj=None):
    a = _source(rng, M, K, "bf16")
    b = I.to_bf16_bits((rng.standard_normal((K, N)) * 0.05).astype(np.float32))
    qa, sa, ta = mx.mx_quantize_nvfp(to_device(a), mx.MX_AXIS_ROW, la)
    qb, sb, tb = mx.mx_quantize_nvfp(to_device(b), mx.MX_AXIS_COL, lb)
    c = mx.mx_gemm_nvfp(qa, sa, ta, la, qb, sb, tb, lb, M, N, K, alpha, out)
    torch.cuda.synchronize()
    got = c.float().cpu().numpy().astype(np.float64)
    args = (u8(qa), u8(sa), ta.cpu().numpy(), la, u8(qb), u8(sb), tb.cpu().numpy(), lb, M, N, K)
    if full:
        C, bound = O.nvfp_gemm(*args, alpha=alpha)
    else:
        C, bound = O.nvfp_gemm_entries(*args, ii, jj, alpha=alpha)
        got = got[ii, jj]
    r = gemm_check(got, C, bound, out == mx.MX_OUT_BF16, what)
    if r is not None:
        log(f"{what}: max err / stated tolerance {r[0]:.3g}")
        record({"test": "nvfp_gemm", "case": what, "max_err_over_stated": r[0], "inside_stated": r[1]})
    return r


@pytest.mark.parametrize("la,lb", [(False, False), (True, False), (False, True), (True, True)])
@pytest.mark.parametrize("out", [mx.MX_OUT_F32, mx.MX_OUT_BF16])
def test_gemm_matches_oracle(la, lb, out):
    """Ragged M and N (partial 256 x 256 tiles in both directions), K of 16
    stages."""
    rng = np.random.default_rng(30 + 2 * la + lb + 4 * out)
    M, N, K = 300, 520, 1024
    log(f"nvfp gemm la={la} lb={lb} out={out} {M}x{N}x{K}")
    _gemm_case(rng, M, N, K, la, lb, out, 0.75, f"nvfp gemm la={la} lb={lb} out={out}")


def test_gemm_one_stage_and_tiny():
    rng = np.random.default_rng(40)
    _gemm_case(rng, 1, 1, 64, True, True, mx.MX_OUT_F32, 1.0, "nvfp gemm 1x1x64")
    _gemm_case(rng, 33, 257, 64, False, True, mx.MX_OUT_F32, -2.0, "nvfp gemm 33x257x64")


@pytest.mark.parametrize("K", [128, 192, 320])
def test_gemm_few_and_odd_stages(K):
    """2, 3 and 5 K stages of 64: the stage loop runs in pairs and loads two
    stages ahead, so short and odd stage counts take its edge paths."""
    rng = np.random.default_rng(41 + K)
    _gemm_case(rng, 130, 300, K, True, False, mx.MX_OUT_BF16, 0.5, f"nvfp gemm 130x300x{K}")


def test_gemm_nan_scale_propagates():
    """A NaN second-level scale (its domain held a NaN) makes exactly the
    outputs that use that domain NaN."""
    rng = np.random.default_rng(41)
    M, N, K = 96, 64, 128
    a = rng.standard_normal((M, K)).astype(np.float32)
    a[40, 3] = np.nan                                                 # panel 1 of A
    b = rng.standard_normal((K, N)).astype(np.float32)
    qa, sa, ta = mx.mx_quantize_nvfp(to_device(a), mx.MX_AXIS_ROW, True)
    qb, sb, tb = mx.mx_quantize_nvfp(to_device(b), mx.MX_AXIS_COL, False)
    c = mx.mx_gemm_nvfp(qa, sa, ta, True, qb, sb, tb, False, M, N, K, 1.0, mx.MX_OUT_F32).cpu().numpy()
    assert np.all(np.isnan(c[32:64])) and np.all(np.isfinite(c[:32])) and np.all(np.isfinite(c[64:]))


@pytest.mark.parametrize("local", [False, True])
def test_full_llama3_8b_gate(local):
    """Llama-3-8B gate projection at full size (X [8192][4096] activations with
    outlier channels, W [4096][14336]): both copies bit-exact against the
    oracle in full, the GEMM on stratified samples of every 128 x 128 output
    tile."""
    w = I.make("nvfp_llama3_8b_gate")
    T, H, F = w.meta["T"], w.meta["H"], w.meta["F"]
    X, W = w.tensors["X"], w.tensors["W"]
    log(f"nvfp llama3-8b gate local={local}: quantize {T}x{H} row, {H}x{F} col")
    qa, sa, ta, _, _, _ = _compare_copy(X, mx.MX_AXIS_ROW, local, f"X local={local}")
    qb, sb, tb, _, _, _ = _compare_copy(W, mx.MX_AXIS_COL, local, f"W local={local}")
    c = mx.mx_gemm_nvfp(qa, sa, ta, local, qb, sb, tb, local, T, F, H, 1.0, mx.MX_OUT_F32)
    torch.cuda.synchronize()
    ii, jj = I.sample_tile_entries(np.random.default_rng(8), T, F, per_tile=8)
    got = c.cpu().numpy()[ii, jj].astype(np.float64)
    args = (u8(qa), u8(sa), ta.cpu().numpy(), local, u8(qb), u8(sb), tb.cpu().numpy(), local, T, F, H)
    C, bound = O.nvfp_gemm_entries(*args, ii, jj)
    r = gemm_check(got, C, bound, False, f"llama gate local={local}")
    log(f"llama gate local={local}: {ii.size} sampled outputs, max err / stated tolerance {r[0]:.3g}")
    record({"test": "nvfp_gemm", "case": f"llama3_8b_gate local={local}", "sampled": int(ii.size),
            "max_err_over_stated": r[0], "inside_stated": r[1]})


def test_gemm_dequantizes_every_code_exactly():
    """The GEMM's in-loop dequantization is exact for every E4M3 block scale
    (subnormals and NaN included) times every E2M1 code: hand-built operands
    with A row i using scale code i on all its blocks and code k % 16 at
    position k, against a B that selects one position per column (code 1.0
    under scale 1.0).  Each output is then a single product, which the f16
    matrix cores and the fp32 accumulator carry without rounding, so C must
    equal e2m1(k % 16) * e4m3(i) bit for bit (NaN for the NaN scale code)."""
    M, N, K = 128, 64, 64
    kk = np.arange(K)
    codes = np.tile((kk % 16).astype(np.uint8), (M, 1))                       # [M][K] nibbles
    qa = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)            # element 2j low nibble
    sa = np.repeat(np.arange(M, dtype=np.uint8)[:, None], K // 16, axis=1)    # scale code i on row i
    bc = np.zeros((N, K), np.uint8)
    bc[np.arange(N), np.arange(N)] = 0x2                                      # E2M1 1.0 at k = j
    qb = (bc[:, 0::2] | (bc[:, 1::2] << 4)).astype(np.uint8)
    sb = np.full((N, K // 16), 0x38, np.uint8)                                # E4M3 1.0
    one = torch.ones(1, dtype=torch.float32, device=DEV)
    dv = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    c = mx.mx_gemm_nvfp(dv(qa), dv(sa), one, False, dv(qb), dv(sb), one, False, M, N, K, 1.0, mx.MX_OUT_F32)
    got = c.cpu().numpy()
    e2m1 = np.array([O.decode("e2m1", v) for v in range(16)])
    e4m3 = np.array([O.decode("e4m3", v) for v in range(128)])
    # exact in fp32; a signed zero product sums to +0 with the accumulator's +0
    ref = (e4m3[:, None] * e2m1[kk[:N] % 16][None, :]).astype(np.float32) + np.float32(0.0)
    assert_same_f32(got, ref)
    assert np.isnan(got[0x7F]).all() and (got[0] == 0).all()

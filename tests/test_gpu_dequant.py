"""GPU parity of mx_dequantize: the inverse of each quantized copy (exact
power-of-two scaling, inverse Hadamard, tensor scale) must match the oracle
bit for bit in fp32, and its bfloat16 output must be the RNE of that."""
import numpy as np
import pytest
import torch

import oracle as O
from fp4_quantization_block_amd import inputs as I
from fp4_quantization_block_amd import mx
from gpu_util import DEV, assert_codes_equal, assert_same_f32, require_gpu, to_device, u8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2", "e2m1"])
@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("opts", [dict(), dict(hadamard=True), dict(two_level=True),
                                  dict(hadamard=True, two_level=True, sr=True)],
                         ids=["plain", "had", "two", "had_two_sr"])
def test_dequantize(fmt, axis, opts):
    rng = np.random.default_rng(31 + axis)
    rows, cols = (96, 160)
    x = (rng.standard_normal((rows, cols)) * np.exp2(rng.integers(-20, 20, (rows, 1)))).astype(np.float32)
    cfg = mx.qconfig(fmt, two_level=opts.get("two_level", False), sr=opts.get("sr", False),
                     hadamard=opts.get("hadamard", False), seed=I.SR_SEED)
    q, s, ts = mx.mx_quantize(to_device(x), axis, cfg)
    qo, so, st = O.quantize(x, axis, fmt, two_level=1 if opts.get("two_level") else 0,
                            sr=opts.get("sr", False), hadamard=opts.get("hadamard", False),
                            seed=I.SR_SEED)
    torch.cuda.synchronize()
    assert_codes_equal(u8(q), qo, "codes")
    had = opts.get("hadamard", False)
    out32 = mx.mx_dequantize(q, s, ts, fmt, rows, cols, axis, hadamard=had, out_dtype=mx.MX_OUT_F32)
    out16 = mx.mx_dequantize(q, s, ts, fmt, rows, cols, axis, hadamard=had, out_dtype=mx.MX_OUT_BF16)
    torch.cuda.synchronize()
    ref = O.dequantize(qo, so, st if opts.get("two_level") else None, fmt, rows, cols, axis,
                       hadamard=had)
    assert_same_f32(out32.cpu().numpy(), ref)
    ref16 = torch.from_numpy(ref).to(torch.bfloat16)
    assert torch.equal(out16.cpu().view(torch.int16), ref16.view(torch.int16))


def test_dequantize_every_code_and_extreme_bytes():
    """All codes with scale bytes 0, 1, 127, 200 and 0xFF (NaN)."""
    for fmt in ("e4m3", "e5m2", "e2m1"):
        bits = O.elem_bits(fmt)
        codes = np.arange(1 << bits, dtype=np.uint8)
        blk = np.resize(codes, 32 * 10).reshape(10, 32)
        q = blk if bits == 8 else (blk[:, 0::2] | (blk[:, 1::2] << 4)).astype(np.uint8)
        q = np.ascontiguousarray(np.repeat(q, 1, axis=0))
        s = np.array([[0], [1], [127], [200], [255], [3], [250], [128], [126], [90]], np.uint8)
        qd = torch.from_numpy(q).to(DEV)
        sd = torch.from_numpy(s).to(DEV)
        out = mx.mx_dequantize(qd, sd, None, fmt, 10, 32, 0, out_dtype=mx.MX_OUT_F32)
        torch.cuda.synchronize()
        ref = O.dequantize(q, s, None, fmt, 10, 32, 0)
        assert_same_f32(out.cpu().numpy(), ref)

"""GPU parity of mx_predict_tensor_scale (MOSS weight auto-scaling,
[MOSS, "创新 2：权重自动缩放"]) against the oracle: the predicted scale
(max|W| + lr*max|g|)/Fmax bit for bit, and the next step's weights
quantized with it (MX_TSCALE_PROVIDED) code for code."""
import numpy as np
import pytest
import torch

import oracle as O
from fp4_quantization_block_amd import inputs as I
from fp4_quantization_block_amd import mx
from gpu_util import DEV, assert_codes_equal, log, require_gpu, to_device, u8

pytestmark = pytest.mark.gpu
FMTS = ["e4m3", "e5m2", "e2m1"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _pair(rng, rows, cols, src, wscale=0.02, gscale=1e-3):
    w = (rng.standard_normal((rows, cols)) * wscale).astype(np.float32)
    g = rng.laplace(0.0, gscale, (rows, cols)).astype(np.float32)
    if src == "bf16":
        return I.to_bf16_bits(w), I.to_bf16_bits(g)
    return w, g


def _same(a, b):
    a, b = np.float32(a), np.float32(b)
    assert (np.isnan(a) and np.isnan(b)) or a.view(np.uint32) == b.view(np.uint32), (float(a), float(b))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("src", ["f32", "bf16"])
def test_predicted_scale_matches_oracle(fmt, src):
    rng = np.random.default_rng(11 + FMTS.index(fmt) + 10 * (src == "bf16"))
    for rows, cols in [(1, 1), (3, 70), (64, 96), (257, 33), (512, 1024)]:
        for lr in (0.0, 1e-3, 0.5, 3.0):
            w, g = _pair(rng, rows, cols, src)
            got = mx.mx_predict_tensor_scale(to_device(w), to_device(g), lr, fmt)
            torch.cuda.synchronize()
            _same(got.item(), O.predict_tensor_scale(w, g, lr, fmt))


def test_strided_views_and_special_values():
    rng = np.random.default_rng(3)
    w, g = _pair(rng, 96, 200, "bf16")
    wb = to_device(I.to_bf16_bits(np.zeros((96, 256), np.float32)))
    gb = to_device(I.to_bf16_bits(np.zeros((96, 232), np.float32)))
    wb[:, :200] = to_device(w)
    gb[:, :200] = to_device(g)
    got = mx.mx_predict_tensor_scale(wb[:, :200], gb[:, :200], 0.25, "e4m3")
    torch.cuda.synchronize()
    _same(got.item(), O.predict_tensor_scale(w, g, 0.25, "e4m3"))
    z = np.zeros((64, 64), np.float32)
    one = np.full((64, 64), 0.5, np.float32)
    gn = z.copy()
    gn[7, 9] = np.nan
    wi = one.copy()
    wi[1, 2] = -np.inf
    gi = z.copy()
    gi[5, 6] = np.inf
    for a, b, lr in [(z, z, 0.5), (one, z, 0.5), (one, gn, 0.5), (wi, z, 0.5), (one, gi, 0.5), (one, gi, 0.0),
                     (wi, z, 0.0)]:
        got = mx.mx_predict_tensor_scale(to_device(a), to_device(b), lr, "e4m3")
        torch.cuda.synchronize()
        _same(got.item(), O.predict_tensor_scale(a, b, lr, "e4m3"))


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_next_step_weights_quantized_with_the_prediction(fmt):
    rng = np.random.default_rng(21)
    w, g = _pair(rng, 256, 192, "f32")
    lr = 0.05
    s = mx.mx_predict_tensor_scale(to_device(w), to_device(g), lr, fmt)
    w2 = (w - np.float32(lr) * g).astype(np.float32)             # the step's update, fp32
    cfg = mx.qconfig(fmt, two_level=True, tscale_provided=True)
    q, sc, ts = mx.mx_quantize(to_device(w2), mx.MX_AXIS_COL, cfg, tensor_scale=s)
    torch.cuda.synchronize()
    s_or = O.predict_tensor_scale(w, g, lr, fmt)
    _same(ts.item(), s_or)
    qo, so, _ = O.quantize(w2, O.AXIS_COL, fmt, two_level=2, tensor_scale=s_or)
    assert_codes_equal(u8(q), qo, "codes")
    assert_codes_equal(u8(sc), so, "scales")
    # the bound the prediction rests on: no element of the new weights exceeds it
    assert np.abs(w2).max() <= np.float32(O.predict_max(w, g, lr))


def test_full_weight_4096_bf16():
    rng = np.random.default_rng(2)
    w, g = _pair(rng, 4096, 4096, "bf16")
    got = mx.mx_predict_tensor_scale(to_device(w), to_device(g), 1e-3, "e4m3")
    torch.cuda.synchronize()
    want = O.predict_tensor_scale(w, g, 1e-3, "e4m3")
    _same(got.item(), want)
    log(f"predicted scale 4096x4096: {got.item()!r}")

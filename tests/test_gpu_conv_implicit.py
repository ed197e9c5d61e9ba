"""ConvInteger's implicit-GEMM path (group channels a multiple of 64, at
most nine taps) on the GPU against the oracle, bit for bit, and against the
im2col path on the same inputs: tile shapes with ragged output rows and
columns (16- and 32-wide tiles), output channels past one 128-row tile and
short of one, strides, dilations, asymmetric pads, groups, 1x1 / 1x3 / 3x1 /
2x2 / 3x3 kernels, every operand dtype pairing and weight zero-point form,
several 64-channel blocks, odd output widths (scalar stores), and the
benchmark's 3x3 layer (sampled images); inputs whose rows are whole 16-byte
vectors (W % 16 == 0) also through the one-launch fused form."""
import numpy as np
import pytest

import oracle
import quantized_int8_gemm_amd as q
import seeded_inputs as si
from gpu_util import case, to_dev
from test_oracle_pins import _conv_case

pytestmark = pytest.mark.gpu


def both_paths(monkeypatch, x, w, x_zp, w_zp, **kw):
    """The default path (one fused launch where x's rows are 16-byte
    aligned, W % 16 == 0; else the padded-copy pass and the implicit GEMM),
    the two-pass form and the im2col path, each against the oracle."""
    ref = oracle.conv_integer(x, w, x_zp, w_zp, **kw)
    zw = None if w_zp is None else to_dev(np.asarray(w_zp).astype(w.dtype))
    tx, tw = to_dev(x), to_dev(w)
    y = q.conv_integer(tx, tw, x_zp, zw, **kw)
    assert q.last_kernel() == ("conv_fused" if x.shape[-1] % 16 == 0 else "conv_implicit"), q.last_kernel()
    np.testing.assert_array_equal(y.cpu().numpy(), ref)
    monkeypatch.setenv("QGEMM_CONV", "twopass")
    y1 = q.conv_integer(tx, tw, x_zp, zw, **kw)
    assert q.last_kernel() == "conv_implicit", q.last_kernel()
    np.testing.assert_array_equal(y1.cpu().numpy(), ref)
    monkeypatch.setenv("QGEMM_CONV", "im2col")
    y2 = q.conv_integer(tx, tw, x_zp, zw, **kw)
    monkeypatch.delenv("QGEMM_CONV")
    assert q.last_kernel().startswith("conv_im2col+"), q.last_kernel()
    np.testing.assert_array_equal(y2.cpu().numpy(), ref)


# (N, C, H, W, M, kH, kW, group, pads, strides, dilations)
SHAPES = [
    (2, 64, 32, 32, 128, 3, 3, 1, (1, 1, 1, 1), (1, 1), (1, 1)),     # whole 4x32 tiles
    (2, 64, 19, 37, 40, 3, 3, 1, (1, 1, 1, 1), (1, 1), (1, 1)),      # ragged rows / columns, Mg < 128
    (1, 64, 9, 14, 200, 3, 3, 1, (1, 2, 0, 1), (1, 1), (1, 1)),      # 16-wide tiles, two m tiles, odd pads
    (2, 128, 12, 12, 72, 3, 3, 1, (1, 1, 1, 1), (2, 2), (1, 1)),     # stride 2, two channel blocks
    (2, 64, 20, 21, 64, 3, 3, 1, (2, 2, 2, 2), (1, 1), (2, 2)),      # dilation 2
    (2, 128, 10, 18, 96, 3, 3, 2, (1, 1, 1, 1), (1, 1), (1, 1)),     # two groups of 64 channels
    (3, 64, 7, 33, 48, 1, 1, 1, (0, 0, 0, 0), (1, 1), (1, 1)),       # 1x1
    (2, 64, 8, 20, 32, 1, 3, 1, (0, 1, 0, 1), (1, 2), (1, 1)),       # 1x3, column stride 2
    (2, 64, 15, 6, 32, 3, 1, 1, (1, 0, 1, 0), (2, 1), (1, 1)),       # 3x1, row stride 2
    (2, 64, 11, 11, 24, 2, 2, 1, (0, 0, 1, 1), (1, 1), (1, 1)),      # 2x2, even kernel
    (1, 192, 6, 7, 130, 3, 3, 1, (1, 1, 1, 1), (1, 1), (1, 1)),      # three channel blocks, OW = 7
    # W % 16 == 0: the fused launch
    (2, 64, 19, 48, 40, 3, 3, 1, (1, 1, 1, 1), (1, 1), (1, 1)),      # ragged rows, Mg < 128
    (2, 128, 12, 16, 72, 3, 3, 1, (1, 1, 1, 1), (2, 2), (1, 1)),     # stride 2, two channel blocks
    (2, 64, 20, 32, 64, 3, 3, 1, (2, 2, 2, 2), (1, 1), (2, 2)),      # dilation 2
    (2, 128, 10, 16, 96, 3, 3, 2, (1, 1, 1, 1), (1, 1), (1, 1)),     # two groups of 64 channels
    (3, 64, 7, 48, 48, 1, 1, 1, (0, 0, 0, 0), (1, 1), (1, 1)),       # 1x1
    (2, 64, 8, 32, 32, 1, 3, 1, (0, 1, 0, 1), (1, 2), (1, 1)),       # 1x3, column stride 2
    (2, 64, 11, 16, 24, 2, 2, 1, (0, 0, 1, 1), (1, 1), (1, 1)),      # 2x2 (four taps: byte-wise weights)
    (1, 192, 6, 16, 130, 3, 3, 1, (1, 2, 1, 0), (1, 1), (1, 1)),     # three channel blocks, asymmetric pads
    (1, 64, 9, 64, 200, 3, 3, 1, (0, 3, 2, 0), (1, 1), (1, 1)),      # wide pads, two m tiles
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"s{i}" for i in range(len(SHAPES))])
def test_conv_implicit_shapes(monkeypatch, shape):
    N, C, H, W, M, kH, kW, group, pads, strides, dil = shape
    case(f"conv implicit {shape}")
    x, w, x_zp, w_zp = _conv_case(sum(shape[:7]) + 17, N, C, H, W, M, kH, kW, group, True, False, True)
    both_paths(monkeypatch, x, w, x_zp, w_zp, pads=pads, strides=strides, dilations=dil, group=group)


@pytest.mark.parametrize("x_u8,w_u8", [(True, False), (False, True), (True, True), (False, False)])
@pytest.mark.parametrize("zp_form", ["none", "scalar", "per_channel"])
def test_conv_implicit_dtypes_and_zero_points(monkeypatch, x_u8, w_u8, zp_form):
    case(f"conv implicit dtypes x_u8={x_u8} w_u8={w_u8} zp={zp_form}")
    x, w, x_zp, w_zp = _conv_case(31 + x_u8 + 2 * w_u8, 2, 64, 13, 18, 72, 3, 3, 1, x_u8, w_u8, True)
    wz = {"none": None, "scalar": int(w_zp[0]), "per_channel": w_zp}[zp_form]
    both_paths(monkeypatch, x, w, x_zp, wz, pads=(1, 1, 1, 1))


def test_conv_implicit_extreme_values_wrap():
    """All-255 uint8 operands with zero points 0 over 64 * 9 * 48 terms per
    output stay exact; a 1x1 reduction of 40000 channels of 255 * 255 wraps
    int32 like the oracle."""
    case("conv implicit extreme values")
    x = np.full((1, 64 * 48, 5, 5), 255, np.uint8)
    w = np.full((4, 64 * 48, 3, 3), 255, np.uint8)
    y = q.conv_integer(to_dev(x), to_dev(w), 0, None, pads=(1, 1, 1, 1))
    assert q.last_kernel() == "conv_implicit"
    np.testing.assert_array_equal(y.cpu().numpy(), oracle.conv_integer(x, w, 0, None, pads=(1, 1, 1, 1)))
    case("conv implicit int32 wrap, reduction 40000")
    x = np.full((1, 40000, 1, 1), 255, np.uint8)
    w = np.full((2, 40000, 1, 1), 255, np.uint8)
    y = q.conv_integer(to_dev(x), to_dev(w), 0, None)
    assert q.last_kernel() == "conv_implicit"
    np.testing.assert_array_equal(y.cpu().numpy(), oracle.conv_integer(x, w, 0, None))


def test_conv_implicit_tokenizer_layer_sampled(monkeypatch):
    """The benchmark's layer through both paths; the oracle checks images 0,
    31 and 63, and the two GPU paths agree on all 64."""
    case("conv implicit tokenizer layer 64x64x32x32 * 128x64x3x3")
    x, w, zw = si.conv_integer_inputs(64, 64, 32, 32, 128, 3, 3, seed=808)
    tx, tw, tz = to_dev(x), to_dev(w), to_dev(zw)
    y = q.conv_integer(tx, tw, 128, tz, pads=(1, 1, 1, 1))
    assert q.last_kernel() == "conv_fused", q.last_kernel()
    yc = y.cpu().numpy()
    for n in (0, 31, 63):
        np.testing.assert_array_equal(yc[n:n + 1], oracle.conv_integer(x[n:n + 1], w, 128, zw, pads=(1, 1, 1, 1)))
    monkeypatch.setenv("QGEMM_CONV", "twopass")
    y1 = q.conv_integer(tx, tw, 128, tz, pads=(1, 1, 1, 1))
    assert q.last_kernel() == "conv_implicit", q.last_kernel()
    np.testing.assert_array_equal(y1.cpu().numpy(), yc)
    monkeypatch.setenv("QGEMM_CONV", "im2col")
    y2 = q.conv_integer(tx, tw, 128, tz, pads=(1, 1, 1, 1))
    assert q.last_kernel().startswith("conv_im2col+")
    np.testing.assert_array_equal(y2.cpu().numpy(), yc)

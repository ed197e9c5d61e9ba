"""ConvInteger on the GPU against the oracle, bit for bit: the shapes the
oracle is pinned on (groups, padding, strides, dilations, depthwise), the
page's 259-channel 1x1 convolution and its grouped, padded, stride-2
reduction of 261, rank-3 NCL, every operand dtype pairing and zero-point
form, both GEMM kernel families (P a multiple of 16 or not), the int32
wrap, auto_pad, and the 3x3 tokenizer-sized layer the benchmark times
(sampled images)."""
import numpy as np
import pytest
import torch

import oracle
import quantized_int8_gemm_amd as q
import seeded_inputs as si
from gpu_util import case, to_dev
from test_oracle_pins import CONV_LIBRARY_CASES, _conv_case

pytestmark = pytest.mark.gpu


def run(x, w, x_zp, w_zp, expect=None, **kw):
    ref = oracle.conv_integer(x, w, x_zp, w_zp, **kw)
    zw = None if w_zp is None else to_dev(np.asarray(w_zp).astype(w.dtype))
    y = q.conv_integer(to_dev(x), to_dev(w), x_zp, zw, **kw)
    if expect is not None:
        assert q.last_kernel().startswith("conv_im2col+" + expect), q.last_kernel()
    np.testing.assert_array_equal(y.cpu().numpy(), ref)


@pytest.mark.parametrize("cfg", CONV_LIBRARY_CASES)
def test_conv_integer_library_cases(cfg):
    N, C, H, W, M, kH, kW, group, pads, strides, dil, x_u8, w_u8, per_ch = cfg
    case(f"conv {cfg}")
    x, w, x_zp, w_zp = _conv_case(sum(cfg[:7]), N, C, H, W, M, kH, kW, group, x_u8, w_u8, per_ch)
    run(x, w, x_zp, w_zp if per_ch else int(w_zp[0]), pads=pads, strides=strides, dilations=dil, group=group)


def test_conv_integer_page_shapes():
    case("conv 259-channel 1x1, all 255")
    x = np.full((2, 259, 4, 8), 255, np.uint8)
    w = np.full((3, 259, 1, 1), 255, np.uint8)
    run(x, w, 0, None, expect="int8_dma")        # P = 32
    case("conv 259-channel 1x1, random")
    x, w, x_zp, w_zp = _conv_case(259, 3, 259, 5, 7, 16, 1, 1, 1, True, False, True)
    run(x, w, x_zp, w_zp, expect="int8_staged")   # P = 35
    case("conv grouped padded stride-2 reduction 261")
    x, w, x_zp, w_zp = _conv_case(261, 2, 58, 9, 9, 8, 3, 3, 2, True, False, True)
    run(x, w, x_zp, w_zp, pads=(1, 1, 1, 1), strides=(2, 2), group=2)


@pytest.mark.parametrize("x_u8,w_u8", [(True, False), (False, True), (True, True), (False, False)])
@pytest.mark.parametrize("zp_form", ["none", "scalar", "per_channel"])
def test_conv_integer_dtypes_and_zero_points(x_u8, w_u8, zp_form):
    case(f"conv dtypes x_u8={x_u8} w_u8={w_u8} zp={zp_form}")
    x, w, x_zp, w_zp = _conv_case(11 + x_u8 + 2 * w_u8, 2, 24, 16, 16, 40, 3, 3, 1, x_u8, w_u8, True)
    wz = {"none": None, "scalar": int(w_zp[0]), "per_channel": w_zp}[zp_form]
    run(x, w, x_zp, wz, expect="int8_dma", pads=(1, 1, 1, 1))          # P = 256
    run(x, w, x_zp, wz, expect="int8_staged", pads=(0, 1, 0, 0))       # P = 14 * 15


def test_conv_integer_rank3_ncl_and_auto_pad():
    case("conv rank-3 NCL")
    x, w, x_zp, w_zp = _conv_case(3, 4, 12, 1, 100, 10, 1, 5, 2, True, False, True)
    run(x[:, :, 0, :], w[:, :, 0, :], x_zp, w_zp, pads=(2, 3), strides=(2,), dilations=(2,), group=2)
    case("conv auto_pad SAME_UPPER / SAME_LOWER / VALID")
    x, w, x_zp, w_zp = _conv_case(5, 2, 8, 9, 10, 16, 4, 3, 1, False, False, True)
    for mode, pads in (("SAME_UPPER", None), ("SAME_LOWER", None), ("VALID", (0, 0, 0, 0))):
        y = q.conv_integer(to_dev(x), to_dev(w), x_zp, to_dev(w_zp.astype(np.int8)), strides=(2, 2), auto_pad=mode)
        out = [-(-9 // 2), -(-10 // 2)] if mode != "VALID" else [(9 - 4) // 2 + 1, (10 - 3) // 2 + 1]
        tot = [max(0, (o - 1) * 2 + k - s) for o, k, s in zip(out, (4, 3), (9, 10))]
        if mode == "SAME_UPPER":
            pads = (tot[0] // 2, tot[1] // 2, tot[0] - tot[0] // 2, tot[1] - tot[1] // 2)
        elif mode == "SAME_LOWER":
            pads = (tot[0] - tot[0] // 2, tot[1] - tot[1] // 2, tot[0] // 2, tot[1] // 2)
        ref = oracle.conv_integer(x, w, x_zp, w_zp, pads=pads, strides=(2, 2))
        assert tuple(y.shape[2:]) == tuple(out)
        np.testing.assert_array_equal(y.cpu().numpy(), ref)


def test_conv_integer_wraps():
    case("conv int32 wrap, reduction 40000")
    x = np.full((1, 40000, 1, 1), 255, np.uint8)
    w = np.full((2, 40000, 1, 1), 255, np.uint8)
    run(x, w, 0, None)


def test_conv_integer_tokenizer_layer_sampled(monkeypatch):
    """The benchmark's layer (uint8 [64, 64, 32, 32] activations, int8
    [128, 64, 3, 3] weight, padding 1, zero points 128 and per channel)
    through the im2col path, all 64 images on the GPU; the oracle checks
    images 0, 31 and 63 in full."""
    case("conv tokenizer layer 64x64x32x32 * 128x64x3x3, im2col path")
    monkeypatch.setenv("QGEMM_CONV", "im2col")
    x, w, zw = si.conv_integer_inputs(64, 64, 32, 32, 128, 3, 3, seed=808)
    y = q.conv_integer(to_dev(x), to_dev(w), 128, to_dev(zw), pads=(1, 1, 1, 1))
    assert q.last_kernel().startswith("conv_im2col+int8_dma"), q.last_kernel()
    yc = y.cpu().numpy()
    for n in (0, 31, 63):
        np.testing.assert_array_equal(yc[n:n + 1], oracle.conv_integer(x[n:n + 1], w, 128, zw, pads=(1, 1, 1, 1)))

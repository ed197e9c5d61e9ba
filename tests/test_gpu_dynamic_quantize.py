"""DynamicQuantizeLinear (uint8) on the GPU against the oracle, bit for bit:
y, scale and zero point, on the page's all-zero case, hand-worked ties,
ragged sizes around the kernels' 4- and 16-element vectors, one-signed and
extreme ranges, unaligned views, the empty input, repeated calls, the full
[8, 512, 2048] activation, and the on-device chain into MatMulInteger."""
import numpy as np
import pytest
import torch

import oracle
import quantized_int8_gemm_amd as q
import seeded_inputs as si
from golden_io import load
from gpu_util import case, dev, to_dev

pytestmark = pytest.mark.gpu


def check(x, x_dev=None):
    y_ref, sc_ref, zp_ref = oracle.dynamic_quantize_linear(x)
    xd = to_dev(x) if x_dev is None else x_dev
    y, sc, zp = q.dynamic_quantize_linear(xd)
    assert q.last_kernel() == "dql_minmax+dql_quantize"
    assert sc.item() == float(sc_ref) or (np.isnan(sc.item()) and np.isnan(sc_ref))
    assert np.float32(sc.item()).view(np.uint32) == np.float32(sc_ref).view(np.uint32)
    assert int(zp.item()) == int(zp_ref)
    np.testing.assert_array_equal(y.cpu().numpy(), y_ref)
    return y, sc, zp


def test_dql_golden_cases_from_page_and_hand_worked():
    gv = load("dynamic_quantize_linear.txt")
    case("dql golden all_zero / ties_pos / ties_neg / unit_range / sym_range")
    y, sc, zp = check(np.zeros(8, np.float32))
    assert sc.item() == float(gv["all_zero_scale"]) and int(zp.item()) == int(gv["all_zero_zero_point"])
    assert y.cpu().tolist() == [int(t) for t in gv["all_zero_output"].split()]
    for name in ("ties_pos", "ties_neg", "unit_range", "sym_range"):
        x = np.array([float(t) for t in gv[name + "_input"].split()], dtype=np.float32)
        y, sc, zp = check(x)
        assert sc.item() == float(gv[name + "_scale"]) and int(zp.item()) == int(gv[name + "_zero_point"])
        assert y.cpu().tolist() == [int(t) for t in gv[name + "_output"].split()]


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 15, 16, 17, 31, 4095, 4096, 4097, 65537, 1048579])
def test_dql_ragged_sizes(n):
    case(f"dql n={n}")
    check(si.dql_inputs((n,), seed=8000 + n))


@pytest.mark.parametrize("kind", ["positive", "negative", "huge", "tiny", "subnormal_range", "ties", "offset"])
def test_dql_ranges(kind):
    case(f"dql range kind={kind}")
    g = si.rng(8100)
    n = 70001
    if kind == "positive":      # zero point 0
        x = np.abs(si.dql_inputs((n,), 1)) * 3 + 0.25
    elif kind == "negative":    # zero point 255
        x = -np.abs(si.dql_inputs((n,), 2)) * 7 - 1.0
    elif kind == "huge":
        x = si.dql_inputs((n,), 3) * np.float32(1e36)
    elif kind == "tiny":
        x = si.dql_inputs((n,), 4) * np.float32(1e-36)
    elif kind == "subnormal_range":   # range / 255 underflows to 0: scale 1
        x = np.zeros(n, np.float32)
        x[123] = np.float32(1e-45)
        x[999] = np.float32(-1e-45)
    elif kind == "ties":        # scale exactly 1, many halves
        x = (si.randint(g, (n,), -255, 255, np.int64) * 0.5).astype(np.float32)
        x[0], x[1] = -127.5, 127.5
    else:                       # mostly positive with a small negative tail
        x = si.dql_inputs((n,), 5, mean=6.0, std=2.0)
    check(np.ascontiguousarray(x, dtype=np.float32))


def test_dql_unaligned_views_and_empty():
    d = dev()
    x = si.dql_inputs((40003,), seed=77)
    base = torch.zeros(40003 + 3, dtype=torch.float32, device=d)
    for off in (1, 2, 3):
        case(f"dql unaligned x offset {off}")
        view = base[off:off + 40003]
        view.copy_(to_dev(x))
        check(x, x_dev=view)
    case("dql unaligned y offset")
    out_base = torch.zeros(40003 + 1, dtype=torch.uint8, device=d)
    y, sc, zp = q.dynamic_quantize_linear(to_dev(x), out=out_base[1:])
    np.testing.assert_array_equal(y.cpu().numpy(), oracle.dynamic_quantize_linear(x)[0])
    case("dql n=0")
    y, sc, zp = q.dynamic_quantize_linear(torch.empty(0, dtype=torch.float32, device=d))
    assert y.numel() == 0 and sc.item() == 1.0 and int(zp.item()) == 0


def test_dql_repeated_calls_keep_no_state():
    case("dql repeated calls, shrinking sizes")
    for i, n in enumerate((3 * 1048576 + 5, 70000, 17, 1)):
        check(si.dql_inputs((n,), seed=900 + i, mean=float(i) - 1.5, std=10.0 ** (i - 2)))


def test_dql_full_activation_8x512x2048():
    case("dql full [8,512,2048]")
    x = si.dql_inputs((8, 512, 2048), seed=303)
    check(x)


def test_dql_feeds_matmul_integer_on_device():
    """Quantize fp32 activations, then MatMulInteger with the device zero
    point (no host round trip), against the oracle's two steps."""
    case("dql -> matmul_integer_row_zp 2x64x300x256")
    x = si.dql_inputs((2, 64, 256), seed=31)
    _, B, zb = si.matmul_integer_inputs(1, 1, 300, 256, seed=32)
    y_ref, sc_ref, zp_ref = oracle.dynamic_quantize_linear(x)
    Y_ref = oracle.matmul_integer(y_ref, B, int(zp_ref), zb)
    y, sc, zp = q.dynamic_quantize_linear(to_dev(x))
    Y = q.matmul_integer_row_zp(y, to_dev(B), zp.reshape(1), to_dev(zb))
    np.testing.assert_array_equal(Y.cpu().numpy(), Y_ref)

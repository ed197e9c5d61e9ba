"""The launch-status convention of "feat(onnx-to-hip): lower quantized
integer conv and matmul" ("What", last paragraph): a call clears the HIP
error left pending by earlier, unrelated work, launches, and reports only
its own launch.  A stale error must not fail a valid call, and the call
leaves no error behind.  Every call goes straight through the C ABI with all
buffers allocated beforehand, so nothing else touches the runtime between
the stale error and the call."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from gpu_util import case, dev, to_dev
from quantized_int8_gemm_amd import _binding as b

pytestmark = pytest.mark.gpu


def _hip():
    # the runtime the library and torch already share (one soname, loaded once)
    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipSetDevice.argtypes = [ctypes.c_int]
    hip.hipSetDevice.restype = ctypes.c_int
    hip.hipPeekAtLastError.restype = ctypes.c_int
    hip.hipGetDeviceCount.argtypes = [ctypes.POINTER(ctypes.c_int)]
    hip.hipGetDeviceCount.restype = ctypes.c_int
    return hip


def _leave_stale_error(hip):
    """Make a HIP error pending without touching any device: select a
    device ordinal that does not exist."""
    n = ctypes.c_int(0)
    assert hip.hipGetDeviceCount(ctypes.byref(n)) == 0
    rc = hip.hipSetDevice(n.value + 7)
    assert rc != 0
    assert hip.hipPeekAtLastError() == rc


P = b._ptr


@pytest.mark.parametrize("op", ["a8w8", "decode", "matmul_integer", "w8a32", "dynamic_quantize_linear"])
def test_stale_error_is_cleared_and_does_not_fail_the_call(op):
    case(f"launch convention: stale HIP error before {op}")
    d = dev()
    hip = _hip()
    stream = ctypes.c_void_p(torch.cuda.current_stream(d).cuda_stream)
    if op in ("a8w8", "decode"):
        M, N, K = (64 if op == "a8w8" else 4), 512, 768
        A, W, s_a, s_w = si.a8w8_inputs(M, N, K, seed=31)
        tA, tW, ta, tw = (to_dev(x) for x in (A, W, s_a, s_w))
        out = torch.empty((M, N), dtype=torch.float32, device=d)
        nws = b.workspace_bytes(b.QG_OP_A8W8, 1, M, N, K)
        ws = torch.zeros(max(nws, 256), dtype=torch.uint8, device=d)
        torch.cuda.synchronize()
        _leave_stale_error(hip)
        st = b.lib.qgemm_a8w8(M, N, K, P(tA), K, P(tW), N, 0, P(ta), M, P(tw), N, P(out), b.QG_FP32, N,
                              P(ws), ws.numel(), stream)
        want = oracle.a8w8(A, W, s_a, s_w)["f32"]
    elif op == "matmul_integer":
        bt, M, N, K = 2, 40, 256, 320
        A, B, zb = si.matmul_integer_inputs(bt, M, N, K, seed=32)
        tA, tB, tz = to_dev(A), to_dev(B), to_dev(zb)
        out = torch.empty((bt, M, N), dtype=torch.int32, device=d)
        torch.cuda.synchronize()
        _leave_stale_error(hip)
        st = b.lib.matmul_integer(bt, M, N, K, P(tA), b.QG_UINT8, K, M * K, P(tB), b.QG_INT8, N, 0, 128,
                                  P(tz), N, P(out), N, M * N, None, 0, stream)
        want = oracle.matmul_integer(A, B, 128, zb)
    elif op == "w8a32":
        M, N, K = 64, 64, 128
        A, W = si.w8a32_inputs(M, N, K, seed=33)
        tA, tW = to_dev(A), to_dev(W)
        out = torch.empty((M, N), dtype=torch.float32, device=d)
        torch.cuda.synchronize()
        _leave_stale_error(hip)
        st = b.lib.qgemm_w8a32(M, N, K, P(tA), K, P(tW), N, 0.5, 0, P(out), N, stream)
        want = None
        R, bound = oracle.w8a32(A, W, 0.5, 0)
    else:
        x = si.dql_inputs((3, 1000), seed=34)
        tx = to_dev(x)
        out = torch.empty(x.shape, dtype=torch.uint8, device=d)
        sc = torch.empty((), dtype=torch.float32, device=d)
        zp = torch.empty((), dtype=torch.uint8, device=d)
        ws = torch.empty(8192, dtype=torch.uint8, device=d)
        torch.cuda.synchronize()
        _leave_stale_error(hip)
        st = b.lib.dynamic_quantize_linear(x.size, P(tx), P(out), P(sc), P(zp), P(ws), ws.numel(), stream)
        want = oracle.dynamic_quantize_linear(x)[0]
    assert st == b.QG_OK, b.status_string(st)
    assert hip.hipPeekAtLastError() == 0     # the stale error was cleared, none left behind
    assert b.last_kernel() != ""
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    if want is None:
        assert np.all(np.abs(got.astype(np.float64) - R) <= 1e-5 * bound)
    else:
        np.testing.assert_array_equal(got, want)
    assert torch.cuda.current_device() == d.index

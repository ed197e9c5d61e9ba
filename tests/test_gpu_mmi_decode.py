"""MatMulInteger with at most 16 rows (batches folded) on the decode kernel:
B streamed once with K split across workgroups, row and column sums carried
with the partials.  Every output against the oracle, bit for bit: both
operand types, scalar / per-column / per-row zero points, ragged N, folded
batches, forced split counts, one split, int32 wrap-around, a workspace
reused across shapes, and the shapes it does not take."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import quantized_int8_gemm_amd as q
import seeded_inputs as si
from gpu_util import case, dev, env, to_dev

pytestmark = pytest.mark.gpu

DECODE = "matmul_integer_skinny"


def operands(M, N, K, a_dt, b_dt, seed, batch=None):
    g = si.rng(seed)
    a_shape = (M, K) if batch is None else (batch, M, K)
    A = si.randint(g, a_shape, 0, 255, a_dt) if a_dt == np.uint8 else si.randint(g, a_shape, -128, 127, a_dt)
    B = si.randint(g, (K, N), 0, 255, b_dt) if b_dt == np.uint8 else si.randint(g, (K, N), -128, 127, b_dt)
    return g, A, B


def vals(g, n, dt):
    return si.randint(g, (n,), 0, 255, dt) if dt == np.uint8 else si.randint(g, (n,), -128, 127, dt)


def check(A, B, za, zb, kernel=DECODE):
    za_dev = to_dev(za) if isinstance(za, np.ndarray) else za
    y = q.matmul_integer(to_dev(A), to_dev(B), za_dev, None if zb is None else to_dev(zb))
    assert q.last_kernel() == kernel, q.last_kernel()
    np.testing.assert_array_equal(y.cpu().numpy(), oracle.matmul_integer(A, B, za, zb))


@pytest.mark.parametrize("M,N,K,a_dt,b_dt,zp", [
    (1, 8192, 8192, np.uint8, np.int8, "column"),    # 32 column tiles, 8 splits
    (4, 4096, 4096, np.int8, np.uint8, "scalar"),
    (16, 2000, 2048, np.uint8, np.uint8, "rows"),    # per-row and per-column zero points, ragged N
    (7, 1024, 3072, np.int8, np.int8, "none"),
    (16, 8192, 1024, np.uint8, np.int8, "rows"),
])
def test_matmul_integer_decode_every_output(M, N, K, a_dt, b_dt, zp):
    case(f"matmul_integer decode M={M} N={N} K={K} {np.dtype(a_dt)}x{np.dtype(b_dt)} zp={zp}")
    g, A, B = operands(M, N, K, a_dt, b_dt, seed=M * 7 + N + K)
    za = 128 if a_dt == np.uint8 else -3
    zb = None
    if zp == "scalar":
        zb = np.array([200 if b_dt == np.uint8 else 7], dtype=b_dt)
    elif zp in ("column", "rows"):
        zb = vals(g, N, b_dt)
    if zp == "rows":
        za = vals(g, M, a_dt)
    check(A, B, za, zb)


def test_matmul_integer_decode_folded_batches():
    """Four contiguous batches of 4 rows over a shared B: 16 rows in one call."""
    case("matmul_integer decode batch 4x4x4096x4096")
    g, A, B = operands(4, 4096, 4096, np.uint8, np.int8, seed=801, batch=4)
    check(A, B, 128, vals(g, 4096, np.int8))


def test_matmul_integer_decode_folded_batches_per_row_zero_points():
    """Per-row zero points of a [4, 4, K] activation: after the fold, row m of
    the 16 takes zero point m % 4."""
    case("matmul_integer decode batch 4x4x2048x4096 per-row zp")
    g, A, B = operands(4, 4096, 2048, np.uint8, np.uint8, seed=804, batch=4)
    check(A, B, vals(g, 4, np.uint8), vals(g, 4096, np.uint8))


@pytest.mark.parametrize("splits", [3, 16, 64])
def test_matmul_integer_decode_forced_splits(splits):
    case(f"matmul_integer decode forced splits={splits} 5x2048x8192")
    g, A, B = operands(5, 2048, 8192, np.uint8, np.uint8, seed=802)
    with env(QGEMM_SPLITS=splits):
        check(A, B, vals(g, 5, np.uint8), vals(g, 2048, np.uint8))


def test_matmul_integer_decode_wraps():
    """255 * 255 over K = 65536 exceeds 2^32: the int32 result wraps exactly
    as the oracle's does (128 splits of one column tile)."""
    case("matmul_integer decode wrap 1x256x65536")
    A = np.full((1, 65536), 255, np.uint8)
    B = np.full((65536, 256), 255, np.uint8)
    check(A, B, 0, None)
    g = si.rng(803)
    B[:, ::3] = vals(g, 65536 * 86, np.uint8).reshape(65536, 86)
    check(A, B, 1, np.array([254], np.uint8))


def test_matmul_integer_decode_shapes_in_sequence():
    """Calls of different column-tile and split counts share the binding's
    cached workspace; its ticket header ends at zero."""
    case("matmul_integer decode shape sequence")
    for i, (M, N, K) in enumerate([(1, 8192, 8192), (16, 1024, 4096), (2, 12288, 2048), (1, 8192, 8192)]):
        g, A, B = operands(M, N, K, np.uint8, np.int8, seed=810 + i)
        check(A, B, 128, vals(g, N, np.int8))
    from quantized_int8_gemm_amd import _binding as b
    ws = b._workspaces[(dev(), torch.cuda.current_stream(dev()).cuda_stream)]
    assert int(ws[:1024].sum().item()) == 0


def _abi_call(A, B, za, zb, ws, wsb):
    from quantized_int8_gemm_amd import _binding as b
    M, K = A.shape
    N = B.shape[1]
    tA, tB, tz = to_dev(A), to_dev(B), to_dev(zb)
    y = torch.empty(M, N, dtype=torch.int32, device=dev())
    st = b.lib.matmul_integer(1, M, N, K, b._ptr(tA), b.QG_UINT8, K, 0, b._ptr(tB), b.QG_INT8, N, 0,
                              za, b._ptr(tz), N, b._ptr(y), N, M * N, ws, wsb,
                              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st, y


def test_matmul_integer_decode_single_split():
    """K short enough for one split (no partials): a workspace passed through
    the C ABI still selects the decode kernel, which then runs its epilogue
    directly."""
    case("matmul_integer decode one split 9x512x256")
    g, A, B = operands(9, 512, 256, np.uint8, np.int8, seed=820)
    zb = vals(g, 512, np.int8)
    assert q.workspace_bytes(q.QG_OP_MATMUL_INTEGER, 1, 9, 512, 256) == 0
    ws = torch.zeros(4096, dtype=torch.uint8, device=dev())
    st, y = _abi_call(A, B, 100, zb, ctypes.c_void_p(ws.data_ptr()), ws.numel())
    assert st == 0
    assert q.last_kernel() == DECODE, q.last_kernel()
    np.testing.assert_array_equal(y.cpu().numpy(), oracle.matmul_integer(A, B, 100, zb))


def test_matmul_integer_decode_not_taken():
    """No workspace, or K not whole 64-row steps: the tiled kernels."""
    case("matmul_integer decode-sized shapes on the tiled kernels")
    g, A, B = operands(8, 2048, 4096, np.uint8, np.int8, seed=830)
    zb = vals(g, 2048, np.int8)
    st, y = _abi_call(A, B, 128, zb, None, 0)
    assert st == 0
    assert q.last_kernel() == "int8_dma_64x128k128x3", q.last_kernel()
    np.testing.assert_array_equal(y.cpu().numpy(), oracle.matmul_integer(A, B, 128, zb))
    g, A, B = operands(8, 2048, 4112, np.uint8, np.int8, seed=831)
    zb = vals(g, 2048, np.int8)
    y = q.matmul_integer(to_dev(A), to_dev(B), 128, to_dev(zb))
    assert q.last_kernel() != DECODE
    np.testing.assert_array_equal(y.cpu().numpy(), oracle.matmul_integer(A, B, 128, zb))

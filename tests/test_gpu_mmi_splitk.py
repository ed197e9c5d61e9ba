"""MatMulInteger on outputs of at most 256 tiles of 128 x 128 over a long K:
the three-stage kernel, K split across workgroups (each split's partial tile
and partial row / column sums exchanged through the workspace) for at most
128 tiles.  Every output against the oracle, bit for bit, for both operand
types, scalar / per-column / per-row zero points, ragged M and N, folded
batches, forced split counts and the unsplit forms."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import quantized_int8_gemm_amd as q
import seeded_inputs as si
from gpu_util import case, dev, env, to_dev

pytestmark = pytest.mark.gpu

SPLITK = "int8_dma_128x128k128_splitk"
UNSPLIT = "int8_dma_128x128k128x3"


def operands(M, N, K, a_dt, b_dt, seed, batch=None):
    g = si.rng(seed)
    a_shape = (M, K) if batch is None else (batch, M, K)
    A = si.randint(g, a_shape, 0, 255, a_dt) if a_dt == np.uint8 else si.randint(g, a_shape, -128, 127, a_dt)
    B = si.randint(g, (K, N), 0, 255, b_dt) if b_dt == np.uint8 else si.randint(g, (K, N), -128, 127, b_dt)
    return g, A, B


def column_zp(g, N, b_dt):
    return si.randint(g, (N,), 0, 255, b_dt) if b_dt == np.uint8 else si.randint(g, (N,), -128, 127, b_dt)


def tiles_of(rows, name):
    """At most 64 rows (batches folded) run the same split on 64 x 128
    tiles (same tile count, same plan)."""
    return name.replace("128x128", "64x128") if rows <= 64 else name


def check(A, B, za, zb, kernel):
    za_dev = to_dev(za) if isinstance(za, np.ndarray) else za
    y = q.matmul_integer(to_dev(A), to_dev(B), za_dev, None if zb is None else to_dev(zb))
    rows = A.shape[0] * A.shape[1] if A.ndim == 3 else A.shape[0]
    assert q.last_kernel() == tiles_of(rows, kernel), q.last_kernel()
    np.testing.assert_array_equal(y.cpu().numpy(), oracle.matmul_integer(A, B, za, zb))


@pytest.mark.parametrize("M,N,K,a_dt,b_dt,zp", [
    (17, 4096, 8192, np.uint8, np.int8, "column"),    # 32 tiles, 8 splits of 1024
    (100, 2048, 4096, np.int8, np.uint8, "scalar"),   # 16 tiles, 4 splits
    (256, 1024, 3072, np.uint8, np.uint8, "rows"),    # per-row and per-column zero points, 3 splits
    (33, 2000, 3072, np.int8, np.int8, "none"),       # ragged N, 3 splits of 1024
    (130, 4096, 4096, np.uint8, np.int8, "rows"),     # ragged M, 64 tiles, 4 splits
])
def test_matmul_integer_split_k_every_output(M, N, K, a_dt, b_dt, zp):
    case(f"matmul_integer split-K M={M} N={N} K={K} {np.dtype(a_dt)}x{np.dtype(b_dt)} zp={zp}")
    g, A, B = operands(M, N, K, a_dt, b_dt, seed=M + N + K)
    za = 128 if a_dt == np.uint8 else -3
    zb = None
    if zp == "scalar":
        zb = np.array([200 if b_dt == np.uint8 else 7], dtype=b_dt)
    elif zp in ("column", "rows"):
        zb = column_zp(g, N, b_dt)
    if zp == "rows":
        za = si.randint(g, (M,), 0, 255, a_dt) if a_dt == np.uint8 else si.randint(g, (M,), -128, 127, a_dt)
    check(A, B, za, zb, SPLITK)


def test_matmul_integer_split_k_folded_batches():
    """Contiguous batches of A over a shared B fold into M = 80: one split
    grid covers both batches."""
    case("matmul_integer split-K batch 2x40x1024x4096")
    g, A, B = operands(40, 1024, 4096, np.uint8, np.int8, seed=701, batch=2)
    check(A, B, 128, column_zp(g, 1024, np.int8), SPLITK)


def test_matmul_integer_split_k_folded_batches_per_row_zero_points():
    """Per-row zero points of a [3, 40, K] activation: after the fold, row m
    of the 120 takes zero point m % 40."""
    case("matmul_integer split-K batch 3x40x2048x4096 per-row zp")
    g, A, B = operands(40, 2048, 4096, np.int8, np.int8, seed=703, batch=3)
    check(A, B, vals_i8(g, 40), vals_i8(g, 2048), SPLITK)


def vals_i8(g, n):
    return si.randint(g, (n,), -128, 127, np.int8)


@pytest.mark.parametrize("splits", [2, 3, 5, 8])
def test_matmul_integer_split_k_forced_counts(splits):
    case(f"matmul_integer split-K forced splits={splits} 96x2048x8192")
    g, A, B = operands(96, 2048, 8192, np.uint8, np.int8, seed=702)
    za = si.randint(g, (96,), 0, 255, np.uint8)
    with env(QGEMM_TILE_SPLITS=splits):
        check(A, B, za, column_zp(g, 2048, np.int8), SPLITK)


def test_matmul_integer_split_k_shapes_in_sequence():
    """Calls of different tile and split counts in a row share the binding's
    workspace; its ticket header ends at zero."""
    case("matmul_integer split-K shape sequence")
    for i, (M, N, K) in enumerate([(64, 4096, 8192), (40, 1024, 4096), (64, 4096, 8192), (130, 2048, 3072)]):
        g, A, B = operands(M, N, K, np.uint8, np.int8, seed=710 + i)
        check(A, B, 128, column_zp(g, N, np.int8), SPLITK)
    from quantized_int8_gemm_amd import _binding as b
    ws = b._workspaces[(dev(), torch.cuda.current_stream(dev()).cuda_stream)]
    assert int(ws[:1024].sum().item()) == 0


@pytest.mark.parametrize("M,N,K", [(640, 4096, 2176), (300, 8192, 4096)])
def test_matmul_integer_three_stage_unsplit(M, N, K):
    """129 to 256 output tiles over a long K: the three-stage kernel unsplit."""
    case(f"matmul_integer three-stage unsplit M={M} N={N} K={K}")
    g, A, B = operands(M, N, K, np.uint8, np.int8, seed=M + N + K + 1)
    za = si.randint(g, (M,), 0, 255, np.uint8)
    check(A, B, za, column_zp(g, N, np.int8), UNSPLIT)


def test_matmul_integer_without_workspace_runs_unsplit():
    """A NULL workspace through the C ABI: the same kernel unsplit, same bits."""
    case("matmul_integer 64x2048x4096 NULL workspace")
    from quantized_int8_gemm_amd import _binding as b
    M, N, K = 64, 2048, 4096
    g, A, B = operands(M, N, K, np.uint8, np.int8, seed=720)
    zb = column_zp(g, N, np.int8)
    tA, tB, tz = to_dev(A), to_dev(B), to_dev(zb)
    y = torch.empty(M, N, dtype=torch.int32, device=dev())
    st = b.lib.matmul_integer(1, M, N, K, b._ptr(tA), b.QG_UINT8, K, 0, b._ptr(tB), b.QG_INT8, N, 0,
                              128, b._ptr(tz), N, b._ptr(y), N, M * N, None, 0,
                              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    assert q.last_kernel() == tiles_of(M, UNSPLIT), q.last_kernel()
    np.testing.assert_array_equal(y.cpu().numpy(), oracle.matmul_integer(A, B, 128, zb))

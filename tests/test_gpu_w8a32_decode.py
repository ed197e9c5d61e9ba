"""W8A32 and its input gradient with at most 64 rows on the decode kernel
(the weight streamed once, the contraction split across workgroups, the
fp32 partials added in split order): every output within the bound,
integer activations and an identity weight bit for bit, repeated calls bit
for bit, forced and single splits, a partial last step, a workspace shared
with the tiled kernels, and the shapes and switches that leave it."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import quantized_int8_gemm_amd as q
import seeded_inputs as si
from gpu_util import case, dev, env, to_dev

pytestmark = pytest.mark.gpu

TOL = 1e-5
DECODE = "w8a32_skinny"


def run(A, W, scale, zp, **kw):
    c = q.qgemm_w8a32(to_dev(A), to_dev(W), scale, zp, **kw)
    return c, q.last_kernel()


def within(c, A, W, scale, zp):
    R, bound = oracle.w8a32(A, W, scale, zp)
    err = np.abs(c.cpu().numpy().astype(np.float64) - R)
    worst = float((err / np.maximum(bound, 1e-300)).max())
    assert np.all(err <= TOL * bound), f"worst relative error {worst:.3e}"


@pytest.mark.parametrize("M,N,K,zp", [
    (1, 8192, 8192, 5),      # 32 column tiles, 8 splits
    (4, 4096, 4096, 0),      # 16 tiles, 16 splits, no correction
    (16, 2000, 2048, -3),    # ragged last column tile
    (7, 1024, 3000, 2),      # K not whole 64-row steps: a partial last step
    (16, 8192, 1000, 1),     # 2 splits, the second reaching past K
])
def test_w8a32_decode_every_output(M, N, K, zp):
    case(f"w8a32 decode M={M} N={N} K={K} zp={zp}")
    A, W = si.w8a32_inputs(M, N, K, seed=M * 3 + N + K)
    c, kern = run(A, W, 0.017, zp)
    assert kern == DECODE, kern
    within(c, A, W, 0.017, zp)
    c2, _ = run(A, W, 0.017, zp)
    assert torch.equal(c, c2), "a repeated call differs"


@pytest.mark.parametrize("M", [17, 40, 64])
def test_w8a32_decode_row_blocks(M):
    """17 to 64 rows: blocks of 16 rows on the grid, the last one ragged,
    forward and gradient."""
    case(f"w8a32 decode row blocks M={M} 4096x4096")
    A, W = si.w8a32_inputs(M, 4096, 4096, seed=1030 + M)
    c, kern = run(A, W, 0.01, -2)
    assert kern == DECODE, kern
    within(c, A, W, 0.01, -2)
    dC, _ = si.w8a32_inputs(M, 1, 4096, seed=1040 + M)
    d = q.qgemm_w8a32_input_grad(to_dev(dC), to_dev(W), 0.01, -2)
    assert q.last_kernel() == "w8a32_input_grad_skinny", q.last_kernel()
    R, bound = oracle.w8a32_input_grad(dC, W, 0.01, -2)
    assert np.all(np.abs(d.cpu().numpy().astype(np.float64) - R) <= TOL * bound)


def test_w8a32_decode_integer_activations_bit_exact():
    """Small integer activations: S1 and S2 are exact in fp32 in any order, so
    scale * (S1 - zp * S2) has one rounding and matches the oracle exactly."""
    case("w8a32 decode integer activations 8x4096x2048")
    g = si.rng(41)
    A = g.integers(-3, 4, size=(8, 2048)).astype(np.float32)
    W = si.randint(g, (2048, 4096), -128, 127, np.int8)
    for zp in (3, 0, -5):
        c, kern = run(A, W, 0.02, zp)
        assert kern == DECODE, kern
        R, _ = oracle.w8a32(A, W, 0.02, zp)
        np.testing.assert_array_equal(c.cpu().numpy(), R.astype(np.float32))


@pytest.mark.parametrize("sign", [1, -1])
def test_w8a32_decode_identity_weight_bit_exact(sign):
    """W = +-I: every output is one product, so the three bf16 parts must
    rebuild all 24 significand bits of activations of magnitude 2^-100 ..
    2^101."""
    case(f"w8a32 decode identity weight sign={sign}")
    g = si.rng(79)
    n = 320
    mant = (1.0 + g.random((16, n))).astype(np.float32)
    A = (mant * np.exp2(g.integers(-100, 101, size=(16, n))).astype(np.float32)
         * np.where(g.random((16, n)) < 0.5, -1.0, 1.0).astype(np.float32))
    W = (sign * np.eye(n)).astype(np.int8)
    c, kern = run(A, W, 1.0, 0)
    assert kern == DECODE, kern
    np.testing.assert_array_equal(c.cpu().numpy(), sign * A)


@pytest.mark.parametrize("splits", [2, 5, 16])
def test_w8a32_decode_forced_splits(splits):
    case(f"w8a32 decode forced splits={splits} 3x2048x8192")
    A, W = si.w8a32_inputs(3, 2048, 8192, seed=990 + splits)
    with env(QGEMM_W8A32_SPLITS=splits):
        c, kern = run(A, W, 0.01, 4)
    assert kern == DECODE, kern
    within(c, A, W, 0.01, 4)


def test_w8a32_decode_wide_output_one_split():
    """More than 256 column tiles: one split per tile (no workspace needed)."""
    case("w8a32 decode wide 2x65792x64")
    A, W = si.w8a32_inputs(2, 65792, 64, seed=995)
    assert q.workspace_bytes(q.QG_OP_W8A32, 1, 2, 65792, 64) == 0
    c, kern = run(A, W, 0.01, 1)
    assert kern == DECODE, kern
    within(c, A, W, 0.01, 1)


def test_w8a32_decode_workspace_shared_with_tiled_shapes():
    """One zeroed workspace for decode and tiled split calls in turn; the
    ticket header ends at zero."""
    case("w8a32 decode/tiled workspace sharing")
    shapes = [(1, 8192, 8192), (100, 2048, 4096), (16, 4096, 4096), (1, 8192, 8192)]
    need = max(q.workspace_bytes(q.QG_OP_W8A32, 1, *s) for s in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev())
    for i, (M, N, K) in enumerate(shapes):
        A, W = si.w8a32_inputs(M, N, K, seed=1000 + i)
        c, kern = run(A, W, 0.01, 2, workspace=ws)
        assert kern == (DECODE if M <= 64 else "w8a32_bf16x3_128x128_splitk"), kern
        within(c, A, W, 0.01, 2)
    assert int(ws[:1024].sum().item()) == 0


def test_w8a32_decode_other_routes():
    """No workspace: the decode kernel as one split per column tile.  The
    fp32 matrix-core path, QGEMM_FORCE_KERNEL=tiled and rows that are not
    16-byte aligned leave it; all within the bound."""
    case("w8a32 decode routes 12x2048x2048")
    from quantized_int8_gemm_amd import _binding as b
    M, N, K = 12, 2048, 2048
    A, W = si.w8a32_inputs(M, N, K, seed=1010)
    tA, tW = to_dev(A), to_dev(W)
    C = torch.empty(M, N, dtype=torch.float32, device=dev())
    st = b.lib.qgemm_w8a32(M, N, K, b._ptr(tA), K, b._ptr(tW), N, 0.01, -6, b._ptr(C), N,
                           ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    assert q.last_kernel() == DECODE, q.last_kernel()
    within(C, A, W, 0.01, -6)
    with env(QGEMM_W8A32="fp32"):
        c, kern = run(A, W, 0.01, -6)
    assert kern == "w8a32_tiled_128x128", kern
    within(c, A, W, 0.01, -6)
    with env(QGEMM_FORCE_KERNEL="tiled"):
        c, kern = run(A, W, 0.01, -6)
    assert kern == "w8a32_bf16x3_128x128_splitk", kern
    within(c, A, W, 0.01, -6)
    A2, W2 = si.w8a32_inputs(M, 2040, K, seed=1011)   # N % 16 != 0
    c, kern = run(A2, W2, 0.01, -6)
    assert kern != DECODE, kern
    within(c, A2, W2, 0.01, -6)


GRAD = "w8a32_input_grad_skinny"


def run_grad(dC, W, scale, zp, **kw):
    d = q.qgemm_w8a32_input_grad(to_dev(dC), to_dev(W), scale, zp, **kw)
    return d, q.last_kernel()


def within_grad(d, dC, W, scale, zp):
    R, bound = oracle.w8a32_input_grad(dC, W, scale, zp)
    err = np.abs(d.cpu().numpy().astype(np.float64) - R)
    worst = float((err / np.maximum(bound, 1e-300)).max())
    assert np.all(err <= TOL * bound), f"worst relative error {worst:.3e}"


@pytest.mark.parametrize("M,N,K,zp", [
    (1, 8192, 8192, 3),      # dA 1 x 8192 over a sum of 8192
    (16, 4096, 2000, 0),     # ragged last tile of dA's columns
    (5, 3008, 1024, -4),     # a partial last step of the sum (3008 = 47 x 64)
])
def test_w8a32_input_grad_decode_every_output(M, N, K, zp):
    case(f"w8a32_input_grad decode M={M} N={N} K={K} zp={zp}")
    dC, _ = si.w8a32_inputs(M, 1, N, seed=M + N + K + 7)   # [M, N]
    _, W = si.w8a32_inputs(1, N, K, seed=K + 11)            # [K, N]
    d, kern = run_grad(dC, W, 0.019, zp)
    assert kern == ("w8a32_input_grad_slab" if (M <= 8 and K >= 8192) else GRAD), kern
    within_grad(d, dC, W, 0.019, zp)
    d2, _ = run_grad(dC, W, 0.019, zp)
    assert torch.equal(d, d2), "a repeated call differs"


def test_w8a32_input_grad_decode_identity_bit_exact():
    """W = I: dA = dC exactly (one product per output)."""
    case("w8a32_input_grad decode identity weight")
    g = si.rng(80)
    n = 320
    mant = (1.0 + g.random((16, n))).astype(np.float32)
    dC = (mant * np.exp2(g.integers(-100, 101, size=(16, n))).astype(np.float32)
          * np.where(g.random((16, n)) < 0.5, -1.0, 1.0).astype(np.float32))
    d, kern = run_grad(dC, np.eye(n, dtype=np.int8), 1.0, 0)
    assert kern == GRAD, kern
    np.testing.assert_array_equal(d.cpu().numpy(), dC)


def test_w8a32_input_grad_decode_matches_forward_adjoint():
    """<dC, A W'> == <A, dC W'^T> for W' = (W - zp) * scale: the decode
    forward and gradient kernels are adjoint to within the sums' rounding."""
    case("w8a32 decode adjoint 8x2048x4096")
    A, W = si.w8a32_inputs(8, 2048, 4096, seed=1020)
    dC, _ = si.w8a32_inputs(8, 1, 2048, seed=1021)
    c, kern = run(A, W, 0.01, 3)
    assert kern == DECODE, kern
    d, kern = run_grad(dC, W, 0.01, 3)
    assert kern == GRAD, kern
    lhs = float((dC.astype(np.float64) * c.cpu().numpy().astype(np.float64)).sum())
    rhs = float((A.astype(np.float64) * d.cpu().numpy().astype(np.float64)).sum())
    scale_ = float(np.abs(dC).sum() * np.abs(A).max() * 131 * 0.01)
    assert abs(lhs - rhs) <= 1e-5 * scale_

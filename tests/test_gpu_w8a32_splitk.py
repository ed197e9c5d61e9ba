"""W8A32 and its input gradient with the contraction divided among
workgroups (outputs of at most 128 tiles of 128 x 128, e.g. decode-sized M
at N = K = 8192): every output within the bound, results repeated bit for
bit (the partials are added in split order), forced split counts, ragged
edges and a ragged last split, a workspace reused across shapes, and the
unsplit forms (no workspace, or the fp32 matrix-core path)."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import quantized_int8_gemm_amd as q
import seeded_inputs as si
from gpu_util import case, dev, env, to_dev, w8a32_kernel

pytestmark = pytest.mark.gpu

TOL = 1e-5


def fwd(A, W, scale, zp, **kw):
    c = q.qgemm_w8a32(to_dev(A), to_dev(W), scale, zp, **kw)
    return c, q.last_kernel()


def grad(dC, W, scale, zp, **kw):
    d = q.qgemm_w8a32_input_grad(to_dev(dC), to_dev(W), scale, zp, **kw)
    return d, q.last_kernel()


def within(c, R, bound):
    err = np.abs(c.cpu().numpy().astype(np.float64) - R)
    worst = float((err / np.maximum(bound, 1e-300)).max())
    assert np.all(err <= TOL * bound), f"worst relative error {worst:.3e}"


@pytest.mark.parametrize("M,N,K,zp", [
    (1, 8192, 8192, 5),       # 64 tiles, 4 splits
    (16, 4096, 4096, 0),      # 32 tiles, 8 splits, no correction
    (100, 2048, 8192, -7),    # 16 tiles, 8 splits
    (257, 1000, 3000, 3),     # ragged M, N and K: 24 tiles, 5 splits of 608 (the last 568)
])
def test_w8a32_split_k_every_output(M, N, K, zp):
    """(At most 64 rows would take the decode kernel: the tiled one is forced.)"""
    case(f"w8a32 split-K M={M} N={N} K={K} zp={zp}")
    A, W = si.w8a32_inputs(M, N, K, seed=M + N + K)
    with env(QGEMM_FORCE_KERNEL="tiled"):
        c, kern = fwd(A, W, 0.013, zp)
        c2, _ = fwd(A, W, 0.013, zp)
    assert kern == "w8a32_bf16x3_128x128_splitk", kern
    R, bound = oracle.w8a32(A, W, 0.013, zp)
    within(c, R, bound)
    assert torch.equal(c, c2), "a repeated call differs"


@pytest.mark.parametrize("M,N,K,zp", [
    (1, 8192, 8192, 3),       # dA is 1 x 8192: 64 tiles over a sum of 8192
    (48, 4096, 2048, 0),      # dA 48 x 2048 over a sum of 4096
    (130, 3000, 1000, -2),    # ragged
])
def test_w8a32_input_grad_split_every_output(M, N, K, zp):
    case(f"w8a32_input_grad split M={M} N={N} K={K} zp={zp}")
    dC, _ = si.w8a32_inputs(M, 1, N, seed=M + N + 1)   # [M, N]
    _, W = si.w8a32_inputs(1, N, K, seed=K + 5)         # [K, N]
    with env(QGEMM_FORCE_KERNEL="tiled"):   # at most 64 rows would take the decode kernel
        d, kern = grad(dC, W, 0.021, zp)
        d2, _ = grad(dC, W, 0.021, zp)
        assert kern == w8a32_kernel("bf16x3", M, K, grad=True, k=N), kern
    assert kern.endswith("_splitk"), kern
    R, bound = oracle.w8a32_input_grad(dC, W, 0.021, zp)
    within(d, R, bound)
    assert torch.equal(d, d2), "a repeated call differs"


@pytest.mark.parametrize("splits", [2, 3, 7])
def test_w8a32_split_k_forced_counts(splits):
    case(f"w8a32 split-K forced splits={splits} 64x2048x4096")
    A, W = si.w8a32_inputs(64, 2048, 4096, seed=950 + splits)
    with env(QGEMM_W8A32_SPLITS=splits, QGEMM_FORCE_KERNEL="tiled"):
        c, kern = fwd(A, W, 0.01, 4)
    assert kern == "w8a32_bf16x3_128x128_splitk", kern
    R, bound = oracle.w8a32(A, W, 0.01, 4)
    within(c, R, bound)


def test_w8a32_split_k_workspace_reused_across_shapes():
    """One zeroed workspace for calls of different tile and split counts,
    forward and gradient; its ticket header ends at zero."""
    case("w8a32 split-K workspace reuse")
    shapes = [(1, 8192, 8192), (40, 2048, 4096), (1, 8192, 8192), (200, 1024, 2048)]
    need = max(max(q.workspace_bytes(q.QG_OP_W8A32, 1, *s), q.workspace_bytes(q.QG_OP_W8A32_INPUT_GRAD, 1, *s))
               for s in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev())
    for i, (M, N, K) in enumerate(shapes):
        A, W = si.w8a32_inputs(M, N, K, seed=960 + i)
        with env(QGEMM_FORCE_KERNEL="tiled"):
            c, kern = fwd(A, W, 0.01, 2, workspace=ws)
        assert kern.endswith("_splitk"), kern
        within(c, *oracle.w8a32(A, W, 0.01, 2))
        dC, _ = si.w8a32_inputs(M, 1, N, seed=970 + i)      # [M, N]; dA is [M, K]
        with env(QGEMM_FORCE_KERNEL="tiled"):
            d, kern = grad(dC, W, 0.01, 2, workspace=ws)
        assert kern.endswith("_splitk"), kern
        within(d, *oracle.w8a32_input_grad(dC, W, 0.01, 2))
    assert int(ws[:1024].sum().item()) == 0


def test_w8a32_without_workspace_runs_unsplit():
    """qgemm_w8a32 itself (no workspace) runs the 128 x 128 tiles unsplit,
    and so does the fp32 matrix-core path with one."""
    case("w8a32 80x2048x4096 unsplit forms")
    from quantized_int8_gemm_amd import _binding as b
    M, N, K = 80, 2048, 4096
    A, W = si.w8a32_inputs(M, N, K, seed=980)
    tA, tW = to_dev(A), to_dev(W)
    C = torch.empty(M, N, dtype=torch.float32, device=dev())
    st = b.lib.qgemm_w8a32(M, N, K, b._ptr(tA), K, b._ptr(tW), N, 0.01, 6, b._ptr(C), N,
                           ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    assert q.last_kernel() == "w8a32_bf16x3_128x128", q.last_kernel()
    R, bound = oracle.w8a32(A, W, 0.01, 6)
    within(C, R, bound)
    with env(QGEMM_W8A32="fp32"):
        c, kern = fwd(A, W, 0.01, 6)
    assert kern == "w8a32_tiled_128x128", kern
    within(c, R, bound)


def test_w8a32_split_k_unaligned_rows():
    """Rows of A and W that are not 16-byte aligned (lda = K + 1, ldw = N + 3)
    take the scalar loads, split over K like the vector path."""
    case("w8a32 split-K unaligned 64x2048x4096")
    M, N, K = 64, 2048, 4096
    A, W = si.w8a32_inputs(M, N, K, seed=1100)
    d = dev()
    Ab = torch.zeros(M, K + 1, dtype=torch.float32, device=d)
    Ab[:, :K] = to_dev(A)
    Wb = torch.zeros(K, N + 3, dtype=torch.int8, device=d)
    Wb[:, :N] = to_dev(W)
    c = q.qgemm_w8a32(Ab[:, :K], Wb[:, :N], 0.01, 5)
    assert q.last_kernel() == "w8a32_bf16x3_128x128_splitk", q.last_kernel()
    within(c, *oracle.w8a32(A, W, 0.01, 5))
    dC, _ = si.w8a32_inputs(M, 1, N, seed=1101)
    Cb = torch.zeros(M, N + 1, dtype=torch.float32, device=d)
    Cb[:, :N] = to_dev(dC)
    g = q.qgemm_w8a32_input_grad(Cb[:, :N], Wb[:, :N], 0.01, 5)
    assert q.last_kernel() == "w8a32_input_grad_bf16x3_128x128_splitk", q.last_kernel()
    within(g, *oracle.w8a32_input_grad(dC, W, 0.01, 5))

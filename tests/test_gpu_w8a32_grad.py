"""Input gradient of W8A32 on the GPU against the oracle: |dA - R| <=
1e-5 * bound, R = dC @ ((W - zp) * scale)^T in double, bound = |scale| *
sum_n |dC| |W - zp|; integer-valued dC must match exactly.  Every case runs
on both paths (bf16 matrix cores with the exact split, fp32 matrix cores)."""
import numpy as np
import pytest
import torch

import oracle
import quantized_int8_gemm_amd as q
import seeded_inputs as si
from gpu_util import W8A32_PATHS, case, dev, env, to_dev, w8a32_kernel

pytestmark = pytest.mark.gpu

TOL = 1e-5


@pytest.fixture(params=W8A32_PATHS)
def path(request):
    with env(QGEMM_W8A32=request.param):
        yield request.param


def inputs(M, N, K, seed):
    dC, _ = si.w8a32_inputs(M, K, N, seed=seed)        # dC: [M, N]
    _, W = si.w8a32_inputs(1, N, K, seed=seed + 1)     # W: [K, N], the forward weight
    return dC, W


def check(dC, W, scale, zp, path, dC_dev=None, W_dev=None):
    d = q.qgemm_w8a32_input_grad(to_dev(dC) if dC_dev is None else dC_dev,
                                 to_dev(W) if W_dev is None else W_dev, scale, zp)
    assert q.last_kernel() == w8a32_kernel(path, dC.shape[0], W.shape[0], grad=True, k=W.shape[1]), q.last_kernel()
    d = d.cpu().numpy().astype(np.float64)
    R, bound = oracle.w8a32_input_grad(dC, W, scale, zp)
    err = np.abs(d - R)
    worst = float((err / np.maximum(bound, 1e-300)).max())
    assert np.all(err <= TOL * bound), f"worst relative error {worst:.3e}"


@pytest.mark.parametrize("M,N,K,zp", [(1, 1, 1, 0), (3, 7, 5, -5), (64, 128, 64, 3), (17, 33, 130, 3),
                                      (129, 300, 257, 12), (200, 1027, 64, -128), (64, 4096, 300, 5)])
def test_w8a32_input_grad_ragged(M, N, K, zp, path):
    case(f"w8a32_input_grad M={M} N={N} K={K} zp={zp} {path}")
    dC, W = inputs(M, N, K, seed=M + N + K)
    check(dC, W, 0.01, zp, path)


def test_w8a32_input_grad_integer_gradients_bit_exact(path):
    """Integer-valued dC: both sums are exact integers, one rounding."""
    case(f"w8a32_input_grad integer dC exact {path}")
    g = si.rng(32)
    dC = g.integers(-3, 4, size=(64, 128)).astype(np.float32)
    W = si.randint(g, (96, 128), -128, 127, np.int8)
    for zp in (3, 0, -5):
        d = q.qgemm_w8a32_input_grad(to_dev(dC), to_dev(W), 0.02, zp).cpu().numpy()
        R, _ = oracle.w8a32_input_grad(dC, W, 0.02, zp)
        np.testing.assert_array_equal(d, R.astype(np.float32))


def test_w8a32_input_grad_unaligned_views(path):
    """dC and W as strided views that rule out the vector loads."""
    case(f"w8a32_input_grad unaligned views 70x99x45 {path}")
    M, N, K = 70, 99, 45
    dC, W = inputs(M, N, K, seed=7)
    bigc = torch.zeros((M, N + 3), dtype=torch.float32, device=dev())
    bigw = torch.zeros((K, N + 5), dtype=torch.int8, device=dev())
    vc, vw = bigc[:, 1:1 + N], bigw[:, 3:3 + N]
    vc.copy_(to_dev(dC))
    vw.copy_(to_dev(W))
    check(dC, W, 0.03, -7, path, dC_dev=vc, W_dev=vw)


@pytest.mark.parametrize("zp", [0, -9])
def test_w8a32_input_grad_big_tiles_both_zero_point_forms(zp, path):
    """dA 4096 x 4096 over N = 80 (the split path's 256 x 256 tiles), with
    and without the zero-point correction compiled in."""
    case(f"w8a32_input_grad 4096x80x4096 zp={zp} {path}")
    dC, W = inputs(4096, 80, 4096, seed=904 - zp)
    check(dC, W, 0.02, zp, path)


def test_w8a32_input_grad_4096_every_output(path):
    """4096^3 at full size, the forward workload's weight and scale: all
    16.8M outputs within the bound."""
    case(f"w8a32_input_grad 4096x4096x4096 zp=-5 every output {path}")
    dC, W = inputs(4096, 4096, 4096, seed=506)
    d = q.qgemm_w8a32_input_grad(to_dev(dC), to_dev(W), 0.01, -5).cpu().numpy().astype(np.float64)
    assert q.last_kernel() == w8a32_kernel(path, 4096, 4096, grad=True, k=4096), q.last_kernel()
    R, bound = oracle.w8a32_input_grad(dC, W, 0.01, -5)
    assert np.all(np.abs(d - R) <= TOL * bound)


def test_w8a32_input_grad_matches_forward_adjoint_on_gpu(path):
    """<dC, fwd(A)> == <grad(dC), A> with both products from the GPU."""
    case(f"w8a32 adjoint identity on the GPU 300x500x200 {path}")
    A, W = si.w8a32_inputs(300, 500, 200, seed=41)
    dC, _ = si.w8a32_inputs(300, 200, 500, seed=42)
    fwd = q.qgemm_w8a32(to_dev(A), to_dev(W), 0.02, 4).cpu().numpy().astype(np.float64)
    grad = q.qgemm_w8a32_input_grad(to_dev(dC), to_dev(W), 0.02, 4).cpu().numpy().astype(np.float64)
    _, fb = oracle.w8a32(A, W, 0.02, 4)
    lhs = float((dC.astype(np.float64) * fwd).sum())
    rhs = float((grad * A.astype(np.float64)).sum())
    assert abs(lhs - rhs) <= 2e-5 * float((np.abs(dC.astype(np.float64)) * fb).sum())


def test_w8a32_input_grad_identity_weight_bit_exact(path):
    """W = I, zp = 0, scale = 1: dA = dC bit for bit (full 24-bit
    significands over magnitudes 2^-100 .. 2^101)."""
    case(f"w8a32_input_grad identity weight {path}")
    g = si.rng(78)
    n = 288
    mant = (1.0 + g.random((80, n))).astype(np.float32)
    dC = (mant * np.exp2(g.integers(-100, 101, size=(80, n))).astype(np.float32)
          * np.where(g.random((80, n)) < 0.5, -1.0, 1.0).astype(np.float32))
    W = np.eye(n, dtype=np.int8)
    d = q.qgemm_w8a32_input_grad(to_dev(dC), to_dev(W), 1.0, 0).cpu().numpy()
    assert q.last_kernel() == w8a32_kernel(path, 80, n, grad=True, k=n)
    np.testing.assert_array_equal(d, dC)


def test_w8a32_input_grad_split_big_tiles_ragged():
    """A gradient that takes the 256 x 256 split tiles with ragged edges:
    dA 4099 x 4101 over N = 275."""
    case("w8a32_input_grad split 256x256 ragged 4099x275x4101")
    dC, W = inputs(4099, 275, 4101, seed=902)
    with env(QGEMM_W8A32="bf16x3"):
        check(dC, W, 0.01, -9, "bf16x3")


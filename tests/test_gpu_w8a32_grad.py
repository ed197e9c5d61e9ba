"""Input gradient of W8A32 on the GPU against the oracle: |dA - R| <=
1e-5 * bound, R = dC @ ((W - zp) * scale)^T in double, bound = |scale| *
sum_n |dC| |W - zp|; integer-valued dC must match exactly."""
import numpy as np
import pytest
import torch

import oracle
import quantized_int8_gemm_amd as q
import seeded_inputs as si
from gpu_util import case, dev, to_dev

pytestmark = pytest.mark.gpu

TOL = 1e-5


def inputs(M, N, K, seed):
    dC, _ = si.w8a32_inputs(M, K, N, seed=seed)        # dC: [M, N]
    _, W = si.w8a32_inputs(1, N, K, seed=seed + 1)     # W: [K, N], the forward weight
    return dC, W


def check(dC, W, scale, zp, dC_dev=None, W_dev=None):
    d = q.qgemm_w8a32_input_grad(to_dev(dC) if dC_dev is None else dC_dev,
                                 to_dev(W) if W_dev is None else W_dev, scale, zp)
    assert q.last_kernel() == "w8a32_input_grad_128x128"
    d = d.cpu().numpy().astype(np.float64)
    R, bound = oracle.w8a32_input_grad(dC, W, scale, zp)
    err = np.abs(d - R)
    worst = float((err / np.maximum(bound, 1e-300)).max())
    assert np.all(err <= TOL * bound), f"worst relative error {worst:.3e}"


@pytest.mark.parametrize("M,N,K,zp", [(1, 1, 1, 0), (3, 7, 5, -5), (64, 128, 64, 3), (17, 33, 130, 3),
                                      (129, 300, 257, 12), (200, 1027, 64, -128), (64, 4096, 300, 5)])
def test_w8a32_input_grad_ragged(M, N, K, zp):
    case(f"w8a32_input_grad M={M} N={N} K={K} zp={zp}")
    dC, W = inputs(M, N, K, seed=M + N + K)
    check(dC, W, 0.01, zp)


def test_w8a32_input_grad_integer_gradients_bit_exact():
    """Integer-valued dC: both sums are exact integers, one rounding."""
    case("w8a32_input_grad integer dC exact")
    g = si.rng(32)
    dC = g.integers(-3, 4, size=(64, 128)).astype(np.float32)
    W = si.randint(g, (96, 128), -128, 127, np.int8)
    for zp in (3, 0, -5):
        d = q.qgemm_w8a32_input_grad(to_dev(dC), to_dev(W), 0.02, zp).cpu().numpy()
        R, _ = oracle.w8a32_input_grad(dC, W, 0.02, zp)
        np.testing.assert_array_equal(d, R.astype(np.float32))


def test_w8a32_input_grad_unaligned_views():
    """dC and W as strided views that rule out the vector loads."""
    case("w8a32_input_grad unaligned views 70x99x45")
    M, N, K = 70, 99, 45
    dC, W = inputs(M, N, K, seed=7)
    bigc = torch.zeros((M, N + 3), dtype=torch.float32, device=dev())
    bigw = torch.zeros((K, N + 5), dtype=torch.int8, device=dev())
    vc, vw = bigc[:, 1:1 + N], bigw[:, 3:3 + N]
    vc.copy_(to_dev(dC))
    vw.copy_(to_dev(W))
    check(dC, W, 0.03, -7, dC_dev=vc, W_dev=vw)


def test_w8a32_input_grad_4096_every_output():
    """4096^3 at full size, the forward workload's weight and scale: all
    16.8M outputs within the bound."""
    case("w8a32_input_grad 4096x4096x4096 zp=-5 every output")
    dC, W = inputs(4096, 4096, 4096, seed=506)
    d = q.qgemm_w8a32_input_grad(to_dev(dC), to_dev(W), 0.01, -5).cpu().numpy().astype(np.float64)
    assert q.last_kernel() == "w8a32_input_grad_128x128", q.last_kernel()
    R, bound = oracle.w8a32_input_grad(dC, W, 0.01, -5)
    assert np.all(np.abs(d - R) <= TOL * bound)


def test_w8a32_input_grad_matches_forward_adjoint_on_gpu():
    """<dC, fwd(A)> == <grad(dC), A> with both products from the GPU."""
    case("w8a32 adjoint identity on the GPU 300x500x200")
    A, W = si.w8a32_inputs(300, 500, 200, seed=41)
    dC, _ = si.w8a32_inputs(300, 200, 500, seed=42)
    fwd = q.qgemm_w8a32(to_dev(A), to_dev(W), 0.02, 4).cpu().numpy().astype(np.float64)
    grad = q.qgemm_w8a32_input_grad(to_dev(dC), to_dev(W), 0.02, 4).cpu().numpy().astype(np.float64)
    _, fb = oracle.w8a32(A, W, 0.02, 4)
    lhs = float((dC.astype(np.float64) * fwd).sum())
    rhs = float((grad * A.astype(np.float64)).sum())
    assert abs(lhs - rhs) <= 2e-5 * float((np.abs(dC.astype(np.float64)) * fb).sum())

"""W8A32 on the GPU against the oracle: |C - R| <= 1e-5 * bound, where R is
the double-precision dequantise-then-matmul result and bound is
|scale| * sum_k |a| |b - zp|."""
import numpy as np
import pytest

import oracle
import quantized_int8_gemm_amd as q
import seeded_inputs as si
from gpu_util import case, to_dev

pytestmark = pytest.mark.gpu

TOL = 1e-5


def check(A, W, scale, zp):
    c = q.qgemm_w8a32(to_dev(A), to_dev(W), scale, zp).cpu().numpy().astype(np.float64)
    assert q.last_kernel() == "w8a32_tiled_128x128", q.last_kernel()
    R, bound = oracle.w8a32(A, W, scale, zp)
    err = np.abs(c - R)
    worst = float((err / np.maximum(bound, 1e-300)).max())
    assert np.all(err <= TOL * bound), f"worst relative error {worst:.3e}"
    return worst


@pytest.mark.parametrize("zp", [3, 0])
def test_w8a32_64x128x64(zp):
    case(f"w8a32 64x128x64 zp={zp}")
    A, W = si.w8a32_inputs(64, 64, 128, seed=101)
    check(A, W, 0.02, zp)


def test_w8a32_integer_activations_bit_exact():
    """Integer-valued A: S1 and S2 are exact integers, so the factorised
    result scale * (S1 - zp * S2) has one rounding and must match exactly."""
    case("w8a32 integer activations exact")
    g = si.rng(31)
    A = g.integers(-3, 4, size=(64, 128)).astype(np.float32)
    W = si.randint(g, (128, 64), -128, 127, np.int8)
    for zp in (3, 0, -5):
        c = q.qgemm_w8a32(to_dev(A), to_dev(W), 0.02, zp).cpu().numpy()
        R, _ = oracle.w8a32(A, W, 0.02, zp)
        np.testing.assert_array_equal(c, R.astype(np.float32))


@pytest.mark.parametrize("M,N,K,zp", [(1, 1, 1, 0), (3, 5, 7, -5), (17, 130, 33, 3), (129, 257, 300, 12),
                                      (200, 64, 1027, -128), (64, 300, 4096, 5)])
def test_w8a32_ragged(M, N, K, zp):
    case(f"w8a32 ragged M={M} N={N} K={K} zp={zp}")
    A, W = si.w8a32_inputs(M, N, K, seed=M + N + K)
    check(A, W, 0.01, zp)


def test_w8a32_4096_every_output():
    """The 4096^3 workload at full size: all 16.8M outputs within the bound,
    from the kernel the benchmark times."""
    case("w8a32 4096x4096x4096 zp=-5 every output")
    A, W = si.w8a32_inputs(4096, 4096, 4096, seed=506)
    c = q.qgemm_w8a32(to_dev(A), to_dev(W), 0.01, -5).cpu().numpy().astype(np.float64)
    assert q.last_kernel() == "w8a32_tiled_128x128", q.last_kernel()
    R, bound = oracle.w8a32(A, W, 0.01, -5)
    assert np.all(np.abs(c - R) <= TOL * bound)


def test_w8a32_unaligned_views():
    """Leading dimensions that are not multiples of 4 take the scalar loads."""
    case("w8a32 unaligned lda/ldw")
    A, W = si.w8a32_inputs(50, 61, 77, seed=2)
    import torch
    d = to_dev(A).device
    Ab = torch.zeros(50, 79, dtype=torch.float32, device=d)
    Ab[:, :77] = to_dev(A)
    Wb = torch.zeros(77, 63, dtype=torch.int8, device=d)
    Wb[:, :61] = to_dev(W)
    c = q.qgemm_w8a32(Ab[:, :77], Wb[:, :61], 0.02, 3).cpu().numpy().astype(np.float64)
    R, bound = oracle.w8a32(A, W, 0.02, 3)
    assert np.all(np.abs(c - R) <= TOL * bound)

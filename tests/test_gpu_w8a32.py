"""W8A32 on the GPU against the oracle: |C - R| <= 1e-5 * bound, where R is
the double-precision dequantise-then-matmul result and bound is
|scale| * sum_k |a| |b - zp|.  Every case runs on both paths: the bf16
matrix cores with the exact three-way split of A (the default) and the fp32
matrix cores."""
import numpy as np
import pytest

import oracle
import quantized_int8_gemm_amd as q
import seeded_inputs as si
from gpu_util import W8A32_PATHS, case, env, to_dev, w8a32_kernel

pytestmark = pytest.mark.gpu

TOL = 1e-5


@pytest.fixture(params=W8A32_PATHS)
def path(request):
    with env(QGEMM_W8A32=request.param):
        yield request.param


def check(A, W, scale, zp, path):
    M, N = A.shape[0], W.shape[1]
    c = q.qgemm_w8a32(to_dev(A), to_dev(W), scale, zp).cpu().numpy().astype(np.float64)
    assert q.last_kernel() == w8a32_kernel(path, M, N, k=A.shape[1]), q.last_kernel()
    R, bound = oracle.w8a32(A, W, scale, zp)
    err = np.abs(c - R)
    worst = float((err / np.maximum(bound, 1e-300)).max())
    assert np.all(err <= TOL * bound), f"worst relative error {worst:.3e}"
    return worst


@pytest.mark.parametrize("zp", [3, 0])
def test_w8a32_64x128x64(zp, path):
    case(f"w8a32 64x128x64 zp={zp} {path}")
    A, W = si.w8a32_inputs(64, 64, 128, seed=101)
    check(A, W, 0.02, zp, path)


def test_w8a32_integer_activations_bit_exact(path):
    """Integer-valued A: S1 and S2 are exact integers, so the factorised
    result scale * (S1 - zp * S2) has one rounding and must match exactly."""
    case(f"w8a32 integer activations exact {path}")
    g = si.rng(31)
    A = g.integers(-3, 4, size=(64, 128)).astype(np.float32)
    W = si.randint(g, (128, 64), -128, 127, np.int8)
    for zp in (3, 0, -5):
        c = q.qgemm_w8a32(to_dev(A), to_dev(W), 0.02, zp).cpu().numpy()
        R, _ = oracle.w8a32(A, W, 0.02, zp)
        np.testing.assert_array_equal(c, R.astype(np.float32))


@pytest.mark.parametrize("sign", [1, -1])
def test_w8a32_identity_weight_returns_activations_bit_exact(sign, path):
    """W = +-I, zp = 0, scale = 1: every output is one product a * (+-1)
    plus exact zeros, so C must equal +-A bit for bit.  Activations carry
    all 24 significand bits, magnitudes 2^-100 .. 2^101 with random signs:
    on the split path this fails unless hi + lo + lo2 rebuilds every bit."""
    case(f"w8a32 identity weight sign={sign} {path}")
    g = si.rng(77)
    n = 320
    mant = (1.0 + g.random((96, n))).astype(np.float32)            # [1, 2), 24 random bits
    A = (mant * np.exp2(g.integers(-100, 101, size=(96, n))).astype(np.float32)
         * np.where(g.random((96, n)) < 0.5, -1.0, 1.0).astype(np.float32))
    W = (sign * np.eye(n)).astype(np.int8)
    c = q.qgemm_w8a32(to_dev(A), to_dev(W), 1.0, 0).cpu().numpy()
    assert q.last_kernel() == w8a32_kernel(path, 96, n, k=n)
    np.testing.assert_array_equal(c, sign * A)


@pytest.mark.parametrize("M,N,K,zp", [(1, 1, 1, 0), (3, 5, 7, -5), (17, 130, 33, 3), (129, 257, 300, 12),
                                      (200, 64, 1027, -128), (64, 300, 4096, 5), (300, 520, 200, -3)])
def test_w8a32_ragged(M, N, K, zp, path):
    case(f"w8a32 ragged M={M} N={N} K={K} zp={zp} {path}")
    A, W = si.w8a32_inputs(M, N, K, seed=M + N + K)
    check(A, W, 0.01, zp, path)


def test_w8a32_split_big_tiles_ragged():
    """A shape that takes the 256 x 256 split tiles with ragged edges in M, N
    and K (4100 x 4097 outputs, K = 333)."""
    case("w8a32 split 256x256 ragged 4100x4097x333")
    A, W = si.w8a32_inputs(4100, 4097, 333, seed=901)
    with env(QGEMM_W8A32="bf16x3"):
        check(A, W, 0.01, 7, "bf16x3")


@pytest.mark.parametrize("M,N", [(2560, 4096), (2048, 4096), (2100, 4000)])
def test_w8a32_tile_choice_by_tile_count(M, N):
    """2560 x 4096 (160 tiles of 256 x 256) and 2100 x 4000 (144 ragged ones)
    take the 256 x 256 split tiles, 2048 x 4096 (128) the 128 x 128 ones;
    every output within the bound."""
    case(f"w8a32 tile choice M={M} N={N} K=160")
    A, W = si.w8a32_inputs(M, N, 160, seed=M + N + 905)
    with env(QGEMM_W8A32="bf16x3"):
        check(A, W, 0.01, -4, "bf16x3")


@pytest.mark.parametrize("zp", [0, 9])
def test_w8a32_big_tiles_both_zero_point_forms(zp, path):
    """4096 x 4096 outputs over K = 96 (the split path's 256 x 256 tiles),
    with and without the zero-point correction compiled in."""
    case(f"w8a32 4096x4096x96 zp={zp} {path}")
    A, W = si.w8a32_inputs(4096, 4096, 96, seed=903 + zp)
    check(A, W, 0.02, zp, path)


def test_w8a32_4096_every_output(path):
    """The 4096^3 workload at full size: all 16.8M outputs within the bound,
    from the kernel the benchmark times."""
    case(f"w8a32 4096x4096x4096 zp=-5 every output {path}")
    A, W = si.w8a32_inputs(4096, 4096, 4096, seed=506)
    c = q.qgemm_w8a32(to_dev(A), to_dev(W), 0.01, -5).cpu().numpy().astype(np.float64)
    assert q.last_kernel() == w8a32_kernel(path, 4096, 4096, k=4096), q.last_kernel()
    R, bound = oracle.w8a32(A, W, 0.01, -5)
    assert np.all(np.abs(c - R) <= TOL * bound)


def test_w8a32_unaligned_views(path):
    """Leading dimensions that are not multiples of 4 take the scalar loads."""
    case(f"w8a32 unaligned lda/ldw {path}")
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

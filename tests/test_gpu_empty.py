"""Empty problems through the binding on the GPU: an output with no
elements (zero rows, zero columns or a zero batch) comes back as an empty
tensor of the right shape and dtype without a launch (the last-kernel
record reads "none"), and the next real call still runs and matches the
oracle; an empty reduction under a non-empty output is rejected."""
import numpy as np
import pytest
import torch

import oracle
import quantized_int8_gemm_amd as q
import seeded_inputs as si
from gpu_util import case, dev, to_dev

pytestmark = pytest.mark.gpu


def _i8(*shape):
    return torch.ones(shape, dtype=torch.int8, device=dev())


def _none():
    assert q.last_kernel() == "none", q.last_kernel()


def test_a8w8_and_acc_empty_outputs():
    case("empty: A8W8 and A8W8 acc with M = 0 and N = 0")
    d = dev()
    for M, N in ((0, 32), (5, 0), (0, 0)):
        A, W = _i8(M, 64), _i8(64, N)
        sa, sw = torch.ones(M, device=d), torch.ones(N, device=d)
        for dt in (torch.float32, torch.bfloat16):
            y = q.qgemm_a8w8(A, W, sa, sw, out_dtype=dt)
            _none()
            assert y.shape == (M, N) and y.dtype == dt
            acc = torch.zeros((M, N), dtype=torch.int32, device=d)
            y = q.qgemm_a8w8_acc(acc, A, W, sa, sw, out_dtype=dt)
            _none()
            assert y.shape == (M, N) and y.dtype == dt
    with pytest.raises(ValueError):
        q.qgemm_a8w8(_i8(4, 0), _i8(0, 32), torch.ones(4, device=d), torch.ones(32, device=d))


def test_w8a32_and_input_grad_empty_outputs():
    case("empty: W8A32 and its input gradient with zero rows / columns")
    d = dev()
    y = q.qgemm_w8a32(torch.zeros((0, 64), device=d), _i8(64, 32), 0.5, 3)
    _none()
    assert y.shape == (0, 32)
    y = q.qgemm_w8a32(torch.zeros((7, 64), device=d), _i8(64, 0), 0.5, 3)
    _none()
    assert y.shape == (7, 0)
    dA = q.qgemm_w8a32_input_grad(torch.zeros((0, 32), device=d), _i8(64, 32), 0.5, 3)
    _none()
    assert dA.shape == (0, 64)
    with pytest.raises(ValueError):
        q.qgemm_w8a32(torch.zeros((4, 0), device=d), _i8(0, 32), 0.5, 3)
    with pytest.raises(ValueError):
        q.qgemm_w8a32_input_grad(torch.zeros((4, 0), device=d), _i8(64, 0), 0.5, 3)


def test_matmul_integer_empty_batch_rows_and_columns():
    case("empty: MatMulInteger with a zero batch, zero rows, zero columns")
    d = dev()
    B = _i8(64, 32)
    for a_shape in ((0, 16, 64), (3, 0, 64), (2, 3, 0, 64)):
        A = torch.ones(a_shape, dtype=torch.uint8, device=d)
        y = q.matmul_integer(A, B, 128)
        _none()
        assert tuple(y.shape) == a_shape[:-1] + (32,) and y.dtype == torch.int32
    y = q.matmul_integer(torch.ones((3, 16, 64), dtype=torch.uint8, device=d), _i8(64, 0), 128)
    _none()
    assert tuple(y.shape) == (3, 16, 0)
    # a real call right after still launches and matches the oracle
    a, b, zb = si.matmul_integer_inputs(2, 16, 32, 64, seed=961)
    y = q.matmul_integer(to_dev(a), to_dev(b), 128, to_dev(zb))
    assert q.last_kernel() != "none"
    np.testing.assert_array_equal(y.cpu().numpy(), oracle.matmul_integer(a, b, 128, zb))
    with pytest.raises(ValueError):
        q.matmul_integer(torch.ones((2, 16, 0), dtype=torch.uint8, device=d), _i8(0, 32), 128)

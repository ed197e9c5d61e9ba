"""The calibration kernels behind the measured ceilings: the streaming read
touches every byte (the xor of its per-wave words equals the xor of the
buffer's words), and the matrix-core loop reports the operation count the
header states."""
import numpy as np
import pytest
import torch

import quantized_int8_gemm_amd as q
import seeded_inputs as si
from gpu_util import case, dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096, 1 << 20, (3 << 20) + 48])
def test_calib_read_touches_every_word(nbytes):
    case(f"calib_read {nbytes} bytes")
    g = si.rng(nbytes)
    host = si.randint(g, (nbytes // 4,), 0, 2**31 - 1, np.int64).astype(np.uint32)
    buf = to_dev(host.view(np.int32))
    sink = q.calib_read(buf)
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)


def test_calib_mfma_counts_ops():
    case("calib_mfma_i8 3 rounds")
    ops = torch.ones(4096, dtype=torch.int8, device=dev())
    n = q.calib_mfma_i8(ops, 3)
    torch.cuda.synchronize()
    assert n == 3 * 4294967296


def test_calib_mfma_32x32x32_counts_the_same_ops():
    case("calib_mfma_i8 32x32x32 3 rounds")
    ops = torch.ones(4096, dtype=torch.int8, device=dev())
    sink = torch.full((q._binding.QG_CALIB_SINK_WORDS,), 7, dtype=torch.int32, device=dev())
    n = q.calib_mfma_i8(ops, 3, sink, shape="32x32x32")
    torch.cuda.synchronize()
    assert n == q.calib_mfma_i8(ops, 3) == 3 * 4294967296
    assert q.last_kernel() == "calib_mfma_i8"
    # every wave wrote its word: an even number of equal all-ones sums XOR to 0
    assert int(sink.abs().sum()) == 0
    with pytest.raises(ValueError):
        q.calib_mfma_i8(ops, 3, shape="16x16x32")


def test_calib_mfma_f32_counts_flops_and_stays_finite():
    case("calib_mfma_f32 5 rounds")
    ops = to_dev(si.rng(8).uniform(-1.0, 1.0, size=1024).astype(np.float32))
    sink = torch.zeros(q._binding.QG_CALIB_SINK_WORDS, dtype=torch.int32, device=dev())
    n = q.calib_mfma_f32(ops, 5, sink)
    torch.cuda.synchronize()
    assert n == 5 * 268435456
    # every wave wrote its word; an all-zero operand set gives all-zero sums
    zeros = torch.zeros(1024, dtype=torch.float32, device=dev())
    q.calib_mfma_f32(zeros, 5, sink)
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0


def test_calib_mfma_bf16_counts_flops_and_stays_finite():
    case("calib_mfma_bf16 5 rounds")
    vals = si.rng(9).uniform(-1.0, 1.0, size=2048).astype(np.float32)
    ops = torch.from_numpy(vals).to(dev()).to(torch.bfloat16)
    sink = torch.zeros(q._binding.QG_CALIB_SINK_WORDS, dtype=torch.int32, device=dev())
    n = q.calib_mfma_bf16(ops, 5, sink)
    torch.cuda.synchronize()
    assert n == 5 * 2147483648
    assert q.last_kernel() == "calib_mfma_bf16"
    zeros = torch.zeros(2048, dtype=torch.bfloat16, device=dev())
    q.calib_mfma_bf16(zeros, 5, sink)
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0
    with pytest.raises(ValueError):
        q.calib_mfma_bf16(torch.zeros(100, dtype=torch.bfloat16, device=dev()), 3)


def test_calib_rejects_bad_operands():
    with pytest.raises(ValueError):
        q.calib_mfma_i8(torch.ones(100, dtype=torch.int8, device=dev()), 3)
    with pytest.raises(ValueError):
        q.calib_mfma_f32(torch.ones(100, dtype=torch.float32, device=dev()), 3)
    with pytest.raises(TypeError):
        q.calib_mfma_f32(torch.ones(1024, dtype=torch.int32, device=dev()), 3)

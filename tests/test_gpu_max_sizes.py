"""Parity at the largest operands the library takes.  Its kernels address
operands through 32-bit buffer offsets, and the C ABI accepts an operand
only while its byte span stays below 2^31 (tests/test_abi.py checks that a
larger one is refused).  Here the int8 weight is [131072, 16128], 2.11 GB,
whose last rows sit just under that limit ((K + 256) * ldw = 2,118,057,984
bytes), and every output of the tiled kernel, the decode kernel, the W8A32
kernel and MatMulInteger over it is compared with the oracle.  A weight
given as [N,K] counts only 256 of its rows toward that limit; one of
2.28 GB runs the decode kernel, sampled outputs against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import quantized_int8_gemm_amd as q
import seeded_inputs as si
from gpu_util import bf16_bits, case, dev, to_dev, w8a32_kernel

pytestmark = pytest.mark.gpu

K, N = 131072, 16128
SPAN_LIMIT = 1 << 31


@pytest.fixture(scope="module")
def weight():
    assert (K + 256) * N < SPAN_LIMIT and (K + 256) * (N + 256) >= SPAN_LIMIT - 64 * 1024 * 1024
    dev()
    W = si.randint(si.rng(777), (K, N), -128, 127, np.int8)
    return W, to_dev(W)


def test_a8w8_tiled_at_the_span_limit(weight):
    W, tW = weight
    M = 272                                    # one full 256-row tile band and a ragged one
    case(f"a8w8 max span tiled M={M} N={N} K={K}")
    A = si.randint(si.rng(778), (M, K), -128, 127, np.int8)
    g = si.rng(779)
    s_a = g.uniform(0.001, 0.05, size=M).astype(np.float32)
    s_w = g.uniform(0.001, 0.05, size=N).astype(np.float32)
    tA, ta, tw = to_dev(A), to_dev(s_a), to_dev(s_w)
    h = bf16_bits(q.qgemm_a8w8(tA, tW, ta, tw, out_dtype=torch.bfloat16))
    assert q.last_kernel().startswith("int8_dma"), q.last_kernel()
    f = q.qgemm_a8w8(tA, tW, ta, tw).cpu().numpy()
    ref = oracle.a8w8(A, W, s_a, s_w)
    np.testing.assert_array_equal(h, ref["bf16"])
    np.testing.assert_array_equal(f, ref["f32"])


@pytest.mark.parametrize("M", [1, 16])
def test_a8w8_decode_at_the_span_limit(weight, M):
    W, tW = weight
    case(f"a8w8 max span decode M={M} N={N} K={K}")
    A = si.randint(si.rng(780 + M), (M, K), -128, 127, np.int8)
    g = si.rng(790 + M)
    s_a = g.uniform(0.001, 0.05, size=M).astype(np.float32)
    s_w = g.uniform(0.001, 0.05, size=N).astype(np.float32)
    out = bf16_bits(q.qgemm_a8w8(to_dev(A), tW, to_dev(s_a), to_dev(s_w), out_dtype=torch.bfloat16))
    assert q.last_kernel() == "a8w8_skinny"
    np.testing.assert_array_equal(out, oracle.a8w8(A, W, s_a, s_w)["bf16"])


def test_w8a32_at_the_span_limit(weight):
    W, tW = weight
    M = 64
    case(f"w8a32 max span M={M} N={N} K={K}")
    A = si.rng(781).standard_normal((M, K), dtype=np.float32)
    c = q.qgemm_w8a32(to_dev(A), tW, 0.01, -5).cpu().numpy().astype(np.float64)
    assert q.last_kernel() == w8a32_kernel("bf16x3", M, N, k=K)
    R, bound = oracle.w8a32(A, W, 0.01, -5)
    assert np.all(np.abs(c - R) <= 1e-5 * bound)


def test_matmul_integer_at_the_span_limit(weight):
    W, tW = weight
    M = 20
    case(f"matmul_integer max span M={M} N={N} K={K}")
    A = si.randint(si.rng(782), (1, M, K), 0, 255, np.uint8)
    zb = si.randint(si.rng(783), (N,), -8, 8, np.int8)
    y = q.matmul_integer(to_dev(A), tW, 131, to_dev(zb)).cpu().numpy()
    assert q.last_kernel().startswith("int8_"), q.last_kernel()
    np.testing.assert_array_equal(y, oracle.matmul_integer(A, W, 131, zb))


def test_w8a32_input_grad_at_the_span_limit(weight):
    W, tW = weight
    M = 48
    case(f"w8a32_input_grad max span M={M} N={N} K={K}")
    dC = si.rng(784).standard_normal((M, N), dtype=np.float32)
    d = q.qgemm_w8a32_input_grad(to_dev(dC), tW, 0.02, 3).cpu().numpy().astype(np.float64)
    assert q.last_kernel() == w8a32_kernel("bf16x3", M, K, grad=True, k=N)
    R, bound = oracle.w8a32_input_grad(dC, W, 0.02, 3)
    assert np.all(np.abs(d - R) <= 1e-5 * bound)


NK_N, NK_K = 139264, 16384


@pytest.fixture(scope="module")
def weight_nk():
    assert NK_N * NK_K >= SPAN_LIMIT
    dev()
    Wt = si.randint(si.rng(800), (NK_N, NK_K), -128, 127, np.int8)
    return Wt, to_dev(Wt)


@pytest.mark.parametrize("M", [1, 16])
def test_a8w8_decode_weight_as_n_by_k_past_two_gib(weight_nk, M):
    """A [N,K] weight of 2.28 GB (N = 139264, K = 16384): the C ABI takes it
    (its kernels address such a weight one tile of rows at a time), and the
    column-slab decode kernel's buffer windows cover only its own rows.  The
    first and last 4096 outputs and 2048 others against the oracle."""
    Wt, tW = weight_nk
    case(f"a8w8 [N,K] decode past 2 GiB M={M} N={NK_N} K={NK_K}")
    A = si.randint(si.rng(801 + M), (M, NK_K), -128, 127, np.int8)
    g = si.rng(803 + M)
    s_a = g.uniform(0.001, 0.05, size=M).astype(np.float32)
    s_w = g.uniform(0.001, 0.05, size=NK_N).astype(np.float32)
    out = bf16_bits(q.qgemm_a8w8(to_dev(A), tW, to_dev(s_a), to_dev(s_w), out_dtype=torch.bfloat16, b_trans=True))
    assert q.last_kernel() == "a8w8_slab", q.last_kernel()
    cols = np.unique(np.concatenate([np.arange(4096), np.arange(NK_N - 4096, NK_N),
                                     si.rng(805).integers(0, NK_N, size=2048)]))
    ref = oracle.a8w8(A, np.ascontiguousarray(Wt[cols]), s_a, s_w[cols], b_trans=True)["bf16"]
    np.testing.assert_array_equal(out[:, cols], ref)

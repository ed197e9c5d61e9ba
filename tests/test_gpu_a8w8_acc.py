"""A8W8 with an int32 accumulator input on the GPU against the oracle:
bit-exact accumulators, fp32 and bf16 outputs, on every kernel the
operator can reach (tiled tile shapes with both epilogue modes, the
register-staged family, the decode kernel), with accumulator inputs near
the int32 limits so that the wrapping add is exercised."""
import numpy as np
import pytest
import torch

import oracle
import quantized_int8_gemm_amd as q
import seeded_inputs as si
from gpu_util import bf16_bits, case, dev, env, to_dev

pytestmark = pytest.mark.gpu


def acc_input(M, N, seed):
    g = si.rng(seed)
    edge = np.array([2**31 - 1, -2**31, 2**31 - 5000, -2**31 + 5000], dtype=np.int64)
    pick = si.randint(g, (M, N), 0, 3, np.int64)
    rnd = si.randint(g, (M, N), -2**31, 2**31 - 1, np.int64)
    return np.where(si.randint(g, (M, N), 0, 4, np.int64) == 0, edge[pick], rnd).astype(np.int32)


def check(acc_in, A, W, s_a, s_w, b_trans=False, expect_kernel=None, acc_dev=None):
    ref = oracle.a8w8_acc(acc_in, A, W, s_a, s_w, b_trans=b_trans)
    ai = to_dev(acc_in) if acc_dev is None else acc_dev
    f = q.qgemm_a8w8_acc(ai, to_dev(A), to_dev(W), to_dev(s_a), to_dev(s_w), b_trans=b_trans)
    if expect_kernel:
        assert q.last_kernel().startswith(expect_kernel), q.last_kernel()
    h = q.qgemm_a8w8_acc(ai, to_dev(A), to_dev(W), to_dev(s_a), to_dev(s_w), out_dtype=torch.bfloat16,
                         b_trans=b_trans)
    np.testing.assert_array_equal(f.cpu().numpy(), ref["f32"])
    np.testing.assert_array_equal(bf16_bits(h), ref["bf16"])


@pytest.mark.parametrize("stage", [0, 1, 2])
@pytest.mark.parametrize("tile", range(10))
def test_a8w8_acc_every_tile_shape(tile, stage):
    case(f"a8w8_acc tile {tile} stage {stage} 520x704x512 and 300x700x256 b_trans")
    A, W, s_a, s_w = si.a8w8_inputs(520, 704, 512, seed=60 + tile)
    A2, W2, s_a2, s_w2 = si.a8w8_inputs(300, 700, 256, seed=70 + tile)
    with env(QGEMM_TILE=tile, QGEMM_STAGE=stage):
        check(acc_input(520, 704, tile), A, W, s_a, s_w, expect_kernel="int8_dma")
        check(acc_input(300, 700, 10 + tile), A2, np.ascontiguousarray(W2.T), s_a2, s_w2, b_trans=True,
              expect_kernel="int8_dma")


@pytest.mark.parametrize("M,N,K", [(256, 256, 512), (130, 96, 208), (64, 40, 50)])
def test_a8w8_acc_register_staged_family(M, N, K):
    case(f"a8w8_acc staged M={M} N={N} K={K}")
    A, W, s_a, s_w = si.a8w8_inputs(M, N, K, seed=M + N + K)
    with env(QGEMM_FAMILY="staged"):
        check(acc_input(M, N, 5), A, W, s_a, s_w, expect_kernel="int8_staged")


@pytest.mark.parametrize("M", [1, 4, 16])
def test_a8w8_acc_decode(M):
    case(f"a8w8_acc decode M={M} 8192x8192")
    A, W, s_a, s_w = si.a8w8_inputs(M, 8192, 8192, seed=404 + M)
    check(acc_input(M, 8192, M), A, W, s_a, s_w, expect_kernel="a8w8_skinny")


def test_a8w8_acc_decode_ragged_and_unaligned_accumulator():
    """Decode with N not a multiple of 4 and an accumulator view whose rows
    are neither contiguous nor 16-byte aligned (scalar loads)."""
    case("a8w8_acc decode 7x1000x640, acc_in view with row stride 1003 at offset 1")
    M, N, K = 7, 1000, 640
    A, W, s_a, s_w = si.a8w8_inputs(M, N, K, seed=3)
    acc = acc_input(M, N, 9)
    big = torch.zeros((M, 1003), dtype=torch.int32, device=dev())
    view = big[:, 1:1 + N]
    view.copy_(to_dev(acc))
    check(acc, A, W, s_a, s_w, expect_kernel="a8w8_skinny", acc_dev=view)


def test_a8w8_acc_tiled_accumulator_view():
    case("a8w8_acc tiled 300x512x256, acc_in view with row stride 520")
    M, N, K = 300, 512, 256
    A, W, s_a, s_w = si.a8w8_inputs(M, N, K, seed=4)
    acc = acc_input(M, N, 11)
    big = torch.zeros((M, 520), dtype=torch.int32, device=dev())
    view = big[:, :N]
    view.copy_(to_dev(acc))
    for stage in (0, 1, 2):
        with env(QGEMM_STAGE=stage):
            check(acc, A, W, s_a, s_w, expect_kernel="int8_dma", acc_dev=view)


@pytest.mark.parametrize("M", [3, 512])
def test_a8w8_acc_chains_k_chunks_on_the_gpu(M):
    """The int32 accumulator of the first K chunk (MatMulInteger with int8
    operands and zero points 0) fed into qgemm_a8w8_acc for the rest of K
    gives the bits of one A8W8 call over the whole K."""
    case(f"a8w8_acc K chaining M={M} N=1024 K=1536")
    A, W, s_a, s_w = si.a8w8_inputs(M, 1024, 1536, seed=8, lo=-128, hi=127)
    tA, tW, ta, tw = to_dev(A), to_dev(W), to_dev(s_a), to_dev(s_w)
    first = q.matmul_integer(tA[:, :512].contiguous(), tW[:512].contiguous())
    y = q.qgemm_a8w8_acc(first, tA[:, 512:].contiguous(), tW[512:].contiguous(), ta, tw)
    whole = q.qgemm_a8w8(tA, tW, ta, tw)
    np.testing.assert_array_equal(y.cpu().numpy(), whole.cpu().numpy())
    np.testing.assert_array_equal(whole.cpu().numpy(), oracle.a8w8(A, W, s_a, s_w)["f32"])


def test_a8w8_acc_prefill_8192_every_output():
    """The accumulator-input workload at full size (8192^3, the benchmark's
    inputs: accumulators uniform over [-2^20, 2^20]) in the launch
    configuration the benchmark times, bf16 and fp32 out: all 67.1M outputs
    against the oracle."""
    case("a8w8_acc 8192x8192x8192 every output")
    M = N = K = 8192
    A, W, s_a, s_w = si.a8w8_inputs(M, N, K, seed=505)
    acc = si.randint(si.rng(606), (M, N), -2**20, 2**20, np.int32)
    tacc, tA, tW, ta, tw = (to_dev(x) for x in (acc, A, W, s_a, s_w))
    h = bf16_bits(q.qgemm_a8w8_acc(tacc, tA, tW, ta, tw, out_dtype=torch.bfloat16))
    assert q.last_kernel() == "int8_dma_256x256w8k128", q.last_kernel()
    f = q.qgemm_a8w8_acc(tacc, tA, tW, ta, tw).cpu().numpy()
    assert q.last_kernel() == "int8_dma_256x256w8k128", q.last_kernel()
    del tacc, tA, tW
    ref = oracle.a8w8_acc(acc, A, W, s_a, s_w)
    np.testing.assert_array_equal(h, ref["bf16"])
    np.testing.assert_array_equal(f, ref["f32"])

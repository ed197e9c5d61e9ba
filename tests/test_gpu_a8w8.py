"""A8W8 on the GPU against the oracle: bit-exact fp32 and bf16 outputs
(the stated bar is 1 ulp; the fixed epilogue order makes them exact)."""
import numpy as np
import pytest
import torch

import oracle
import quantized_int8_gemm_amd as q
import seeded_inputs as si
from gpu_util import bf16_bits, case, dev, env, to_dev, ulp_diff_bf16, ulp_diff_f32

pytestmark = pytest.mark.gpu


def run(A, W, s_a, s_w, out_dtype, b_trans=False, **kw):
    return q.qgemm_a8w8(to_dev(A), to_dev(W), to_dev(s_a), to_dev(s_w), out_dtype=out_dtype,
                        b_trans=b_trans, **kw)


def check(A, W, s_a, s_w, b_trans=False, expect_kernel=None):
    ref = oracle.a8w8(A, W, s_a, s_w, b_trans=b_trans)
    f = run(A, W, s_a, s_w, torch.float32, b_trans).cpu().numpy()
    if expect_kernel:
        assert q.last_kernel().startswith(expect_kernel), q.last_kernel()
    h = bf16_bits(run(A, W, s_a, s_w, torch.bfloat16, b_trans))
    assert ulp_diff_f32(f, ref["f32"]).max() <= 1
    assert ulp_diff_bf16(h, ref["bf16"]).max() <= 1
    # the epilogue order is fixed, so the results are in fact identical
    np.testing.assert_array_equal(f, ref["f32"])
    np.testing.assert_array_equal(h, ref["bf16"])


def test_a8w8_256x1024x1024_all_scale_forms():
    case("a8w8 256x1024x1024 seed 202")
    A, W, s_a, s_w = si.a8w8_inputs(256, 1024, 1024, seed=202)
    check(A, W, s_a, s_w, expect_kernel="int8_")
    ref = run(A, W, s_a, s_w, torch.float32).cpu().numpy()
    # [M,1] / [1,N] scales give the same bits as [M] / [N]
    two_d = q.qgemm_a8w8(to_dev(A), to_dev(W), to_dev(s_a).reshape(-1, 1), to_dev(s_w).reshape(1, -1))
    np.testing.assert_array_equal(two_d.cpu().numpy(), ref)
    # a scalar scale equals a broadcast vector of that value
    one = q.qgemm_a8w8(to_dev(A), to_dev(W), to_dev(s_a[:1]), to_dev(s_w[:1])).cpu().numpy()
    vec = q.qgemm_a8w8(to_dev(A), to_dev(W), to_dev(np.full(256, s_a[0], np.float32)),
                       to_dev(np.full(1024, s_w[0], np.float32))).cpu().numpy()
    np.testing.assert_array_equal(one, vec)
    np.testing.assert_array_equal(one, oracle.a8w8(A, W, s_a[:1], s_w[:1])["f32"])


def test_a8w8_raw_accumulator():
    """The int32 accumulator itself (MatMulInteger with zero zero-points on
    int8 operands runs the same matrix-core loop)."""
    case("a8w8 raw accumulator 256x1024x1024")
    A, W, s_a, s_w = si.a8w8_inputs(256, 1024, 1024, seed=202)
    acc = q.matmul_integer(to_dev(A), to_dev(W)).cpu().numpy()
    np.testing.assert_array_equal(acc, oracle.a8w8(A, W, s_a, s_w)["acc"])


def test_a8w8_square_rank1_act_scale_scales_rows():
    case("a8w8 square 512 rank-1 row scale")
    A, W, _, _ = si.a8w8_inputs(512, 512, 256, seed=17)
    s_a = np.linspace(0.5, 2.0, 512).astype(np.float32)
    s_w = np.ones(512, np.float32)
    out = run(A, W, s_a, s_w, torch.float32).cpu().numpy()
    acc = (A.astype(np.int64) @ W.astype(np.int64)).astype(np.float32)
    np.testing.assert_array_equal(out, acc * s_a[:, None])


@pytest.mark.parametrize("M,N,K", [
    (1, 1, 1), (2, 7, 7), (4, 65, 258), (16, 64, 259), (17, 128, 261), (33, 520, 1100),
    (300, 130, 129), (257, 255, 512), (64, 1024, 16), (129, 384, 4096),
])
@pytest.mark.parametrize("kernel", ["auto", "tiled"])
def test_a8w8_ragged(M, N, K, kernel):
    case(f"a8w8 ragged M={M} N={N} K={K} kernel={kernel}")
    A, W, s_a, s_w = si.a8w8_inputs(M, N, K, seed=M * 7 + N * 3 + K, lo=-128, hi=127)
    with env(QGEMM_FORCE_KERNEL=kernel):
        check(A, W, s_a, s_w, expect_kernel="a8w8_skinny" if (kernel == "auto" and M <= 16) else "int8_")


@pytest.mark.parametrize("M,N,K", [(3, 40, 50), (64, 256, 512), (200, 300, 259)])
def test_a8w8_b_trans(M, N, K):
    case(f"a8w8 b_trans M={M} N={N} K={K}")
    A, W, s_a, s_w = si.a8w8_inputs(M, N, K, seed=5 + M)
    check(A, np.ascontiguousarray(W.T), s_a, s_w, b_trans=True, expect_kernel="int8_")


@pytest.mark.parametrize("M", [1, 4, 16])
def test_a8w8_decode_8192(M):
    """Decode shapes at full size, every output compared."""
    case(f"a8w8 decode M={M} K=N=8192")
    A, W, s_a, s_w = si.a8w8_inputs(M, 8192, 8192, seed=404 + M)
    ref = oracle.a8w8(A, W, s_a, s_w)
    out = bf16_bits(run(A, W, s_a, s_w, torch.bfloat16))
    assert q.last_kernel() == "a8w8_skinny"
    np.testing.assert_array_equal(out, ref["bf16"])


def test_a8w8_decode_split_counts_agree():
    """Integer partial sums: any split of K gives identical bits."""
    case("a8w8 decode M=16 splits 1/2/7/16/32")
    A, W, s_a, s_w = si.a8w8_inputs(16, 2048, 8192, seed=9)
    outs = []
    for s in (1, 2, 7, 16, 32):
        with env(QGEMM_SPLITS=s):
            outs.append(bf16_bits(run(A, W, s_a, s_w, torch.bfloat16)))
    for o in outs[1:]:
        np.testing.assert_array_equal(o, outs[0])
    np.testing.assert_array_equal(outs[0], oracle.a8w8(A, W, s_a, s_w)["bf16"])


def test_a8w8_decode_without_workspace_and_tickets_reset():
    case("a8w8 decode M=4 no workspace / workspace reuse")
    A, W, s_a, s_w = si.a8w8_inputs(4, 4096, 4096, seed=10)
    d = dev()
    ref = oracle.a8w8(A, W, s_a, s_w)["f32"]
    nbytes = q.workspace_bytes(q.QG_OP_A8W8, 1, 4, 4096, 4096)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=d)
    for _ in range(3):
        out = run(A, W, s_a, s_w, torch.float32, workspace=ws)
        np.testing.assert_array_equal(out.cpu().numpy(), ref)
    # the split tickets in the fixed 1 KiB header of the workspace are back at zero
    assert int(ws[:1024].sum().item()) == 0
    from quantized_int8_gemm_amd import _binding as b
    # NULL workspace: single-pass kernel, same bits
    out = torch.empty(4, 4096, dtype=torch.float32, device=d)
    tA, tW, ta, tw = to_dev(A), to_dev(W), to_dev(s_a), to_dev(s_w)
    import ctypes
    st = b.lib.qgemm_a8w8(4, 4096, 4096, b._ptr(tA), 4096, b._ptr(tW), 4096, 0, b._ptr(ta), 4,
                          b._ptr(tw), 4096, b._ptr(out), b.QG_FP32, 4096, None, 0,
                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    np.testing.assert_array_equal(out.cpu().numpy(), ref)


def test_a8w8_decode_workspace_reused_across_shapes():
    """The binding caches one workspace per stream and reuses it for any
    shape that fits.  N = 12288 (48 column tiles, 6 splits) leaves nonzero
    partial sums behind; N = 32768 (128 tiles, 2 splits) then runs in the same
    buffer.  Its tickets live in the same fixed header, which the first call
    returned to zero, so every output still matches."""
    for N in (12288, 32768, 12288):
        case(f"a8w8 decode M=1 N={N} K=8192 cached workspace")
        A, W, s_a, s_w = si.a8w8_inputs(1, N, 8192, seed=N + 1)
        out = bf16_bits(run(A, W, s_a, s_w, torch.bfloat16))
        assert q.last_kernel() == "a8w8_skinny"
        np.testing.assert_array_equal(out, oracle.a8w8(A, W, s_a, s_w)["bf16"])


def test_a8w8_large_8192_every_output():
    """8192^3 at full size in the launch configuration the benchmark times:
    all 67.1M outputs, bf16 and fp32, and the raw int32 accumulator (the
    same matrix-core kernel with the integer epilogue), against the oracle."""
    case("a8w8 8192x8192x8192 every output")
    A, W, s_a, s_w = si.a8w8_inputs(8192, 8192, 8192, seed=505)
    tA, tW, ta, tw = to_dev(A), to_dev(W), to_dev(s_a), to_dev(s_w)
    out16 = bf16_bits(q.qgemm_a8w8(tA, tW, ta, tw, out_dtype=torch.bfloat16))
    assert q.last_kernel() == "int8_dma_256x256w8k128", q.last_kernel()   # the kernel the benchmark times
    out32 = q.qgemm_a8w8(tA, tW, ta, tw).cpu().numpy()
    assert q.last_kernel() == "int8_dma_256x256w8k128", q.last_kernel()
    acc = q.matmul_integer(tA, tW).cpu().numpy()
    assert q.last_kernel() == "int8_dma_256x256w8k128", q.last_kernel()
    del tA, tW
    ref = oracle.a8w8(A, W, s_a, s_w)
    np.testing.assert_array_equal(acc, ref["acc"])
    np.testing.assert_array_equal(out16, ref["bf16"])
    np.testing.assert_array_equal(out32, ref["f32"])


def test_a8w8_output_guard_band():
    """Writes stay inside [M, N] of a wider output buffer."""
    case("a8w8 guard band 70x100x300 ldo=128")
    A, W, s_a, s_w = si.a8w8_inputs(70, 100, 300, seed=3)
    d = dev()
    big = torch.full((70, 128), -7.0, dtype=torch.float32, device=d)
    view = big[:, :100]
    q.qgemm_a8w8(to_dev(A), to_dev(W), to_dev(s_a), to_dev(s_w), out=view)
    got = big.cpu().numpy()
    np.testing.assert_array_equal(got[:, :100], oracle.a8w8(A, W, s_a, s_w)["f32"])
    assert (got[:, 100:] == -7.0).all()


def test_a8w8_repeatable():
    case("a8w8 repeat 10x")
    A, W, s_a, s_w = si.a8w8_inputs(300, 640, 1000, seed=4)
    first = run(A, W, s_a, s_w, torch.float32).cpu().numpy()
    for _ in range(9):
        np.testing.assert_array_equal(run(A, W, s_a, s_w, torch.float32).cpu().numpy(), first)


@pytest.mark.parametrize("stage", [0, 1, 2])
@pytest.mark.parametrize("tile", range(10))
def test_a8w8_every_tile_shape(tile, stage):
    """Every tile configuration, with the output written straight from the
    fragments (stage 0) and through LDS in whole rows (stage 1); ragged M and
    N edges, and (B as [N,K], N = 700) an output row pitch that rules out
    16-byte stores."""
    case(f"a8w8 tile cfg {tile} stage {stage} 520x704x1024 and 300x700x512 b_trans")
    A, W, s_a, s_w = si.a8w8_inputs(520, 704, 1024, seed=40 + tile)
    A2, W2, s_a2, s_w2 = si.a8w8_inputs(300, 700, 512, seed=50 + tile)
    with env(QGEMM_TILE=tile, QGEMM_STAGE=stage):
        check(A, W, s_a, s_w, expect_kernel="int8_dma")
        check(A2, np.ascontiguousarray(W2.T), s_a2, s_w2, b_trans=True, expect_kernel="int8_dma")


@pytest.mark.parametrize("M,N,K", [(256, 256, 512), (300, 384, 320), (64, 128, 208)])
@pytest.mark.parametrize("family", ["dma", "staged"])
def test_a8w8_both_kernel_families(M, N, K, family):
    """The multi-stage direct-to-LDS kernel and the register-staged kernel
    give the same bits (K = 208 is not a multiple of 64)."""
    case(f"a8w8 family={family} M={M} N={N} K={K}")
    A, W, s_a, s_w = si.a8w8_inputs(M, N, K, seed=M + N + K)
    with env(QGEMM_FAMILY=family):
        check(A, W, s_a, s_w, expect_kernel="int8_dma" if family == "dma" else "int8_staged")
        check(A, np.ascontiguousarray(W.T), s_a, s_w, b_trans=True,
              expect_kernel="int8_dma" if (family == "dma" and K % 64 == 0) else "int8_staged")


@pytest.mark.parametrize("tile", [6, 7, 8])
def test_a8w8_k128_stages_partial_last_chunk_and_fallback(tile):
    """128-byte k stages: K = 1088 is not whole stages.  With B as [K,N] the
    bytes past K meet zero weight rows, so the 128-byte kernel runs; with B
    as [N,K] they would not, so its 64-byte sibling runs."""
    case(f"a8w8 k128 tile {tile} 260x384x1088 and b_trans")
    A, W, s_a, s_w = si.a8w8_inputs(260, 384, 1088, seed=90 + tile)
    with env(QGEMM_TILE=tile, QGEMM_STAGE=0):
        check(A, W, s_a, s_w, expect_kernel="int8_dma")
        assert q.last_kernel().endswith("k128"), q.last_kernel()
        check(A, np.ascontiguousarray(W.T), s_a, s_w, b_trans=True, expect_kernel="int8_dma")
        assert not q.last_kernel().endswith("k128"), q.last_kernel()


@pytest.mark.parametrize("M,N,K,kernel", [
    (2560, 4096, 256, "int8_dma_256x256w8k128"),   # 160 tiles of 256x256: one round of them
    (3000, 4000, 384, "int8_dma_256x256w8k128"),   # 12 x 16 = 192 tiles, ragged in M and N
    (5120, 4096, 128, "int8_dma_128x128k128"),     # 320: a second round at most 3/8 full
    (2048, 4096, 256, "int8_dma_128x128k128"),     # 128: half a round
    (256, 1024, 1024, "int8_dma_64x128k128"),      # 16 tiles of 128x128 over K <= 2048: 64x128 tiles
    (2000, 2032, 2048, "int8_dma_64x128k128"),     # 256 of them, ragged M and N
    (4096, 2048, 2048, "int8_dma_128x128k128"),    # 512: 128x128 tiles again
    (256, 2048, 2064, "int8_dma_128x128k128_splitk"),   # K past 2048: the split tiles
])
def test_a8w8_tile_choice_by_tile_count(M, N, K, kernel):
    """The tile is chosen by its count (and, for 64x128 tiles, by K); every
    output of each choice against the oracle."""
    case(f"a8w8 tile choice M={M} N={N} K={K}")
    A, W, s_a, s_w = si.a8w8_inputs(M, N, K, seed=M + N + K + 3)
    check(A, W, s_a, s_w, expect_kernel=kernel)


@pytest.mark.parametrize("M,N,K,kernel", [
    (2560, 4096, 256, "int8_dma_256x256w8k128"),
    (5120, 4096, 128, "int8_dma_128x128k128"),
    (256, 1024, 2048, "int8_dma_64x128k128"),
])
def test_matmul_integer_tile_choice_by_tile_count(M, N, K, kernel):
    """MatMulInteger (uint8 A with a per-row zero point, per-column weight
    zero points: both sums) on the same tile choice."""
    case(f"matmul_integer tile choice M={M} N={N} K={K}")
    g = si.rng(M + K)
    A = si.randint(g, (M, K), 0, 255, np.uint8)
    B = si.randint(g, (K, N), -128, 127, np.int8)
    za = si.randint(g, (M,), 0, 255, np.uint8)
    zb = si.randint(g, (N,), -128, 127, np.int8)
    y = q.matmul_integer(to_dev(A), to_dev(B), to_dev(za), to_dev(zb))
    assert q.last_kernel() == kernel, q.last_kernel()
    np.testing.assert_array_equal(y.cpu().numpy(), oracle.matmul_integer(A, B, za, zb))


@pytest.mark.parametrize("M,N,K,out,forced", [
    (1, 8192, 8192, "bf16", True),    # 32 column tiles, 8 splits
    (4, 4096, 4096, "f32", True),
    (16, 2000, 2048, "bf16", False),  # ragged last column tile
    (7, 1000, 3024, "f32", False),    # K % 64 == 16: a piece of the last step lies past K
])
def test_a8w8_decode_weight_as_n_by_k(M, N, K, out, forced):
    """W given as [N,K] (b_trans) at decode shapes: the split-K decode kernel
    reads each weight row's k-bytes directly (N >= 4096 takes column slabs
    unless the split kernel is asked for); every output against the oracle."""
    case(f"a8w8 decode b_trans M={M} N={N} K={K} {out}")
    A, W, s_a, s_w = si.a8w8_inputs(M, N, K, seed=M + N + K + 9)
    Wt = np.ascontiguousarray(W.T)
    ref = oracle.a8w8(A, Wt, s_a, s_w, b_trans=True)
    with env(**({"QGEMM_FORCE_KERNEL": "skinny"} if forced else {})):
        res = run(A, Wt, s_a, s_w, torch.bfloat16 if out == "bf16" else torch.float32, b_trans=True)
    assert q.last_kernel() == "a8w8_skinny", q.last_kernel()
    got = bf16_bits(res) if out == "bf16" else res.cpu().numpy()
    np.testing.assert_array_equal(got, ref[out])


def test_a8w8_decode_weight_as_n_by_k_splits_acc_noalloc():
    """[N,K] decode: every split count gives the same bits, as do the
    accumulator-input form and the workspace-free entry point."""
    case("a8w8 decode b_trans M=16 N=2048 K=8192 splits / acc / noalloc")
    A, W, s_a, s_w = si.a8w8_inputs(16, 2048, 8192, seed=19)
    Wt = np.ascontiguousarray(W.T)
    ref = oracle.a8w8(A, Wt, s_a, s_w, b_trans=True)["bf16"]
    for s in (1, 3, 16, 64):
        with env(QGEMM_SPLITS=s):
            np.testing.assert_array_equal(bf16_bits(run(A, Wt, s_a, s_w, torch.bfloat16, b_trans=True)), ref)
        assert q.last_kernel() == "a8w8_skinny", q.last_kernel()
    acc = si.randint(si.rng(20), (16, 2048), -(1 << 28), 1 << 28, np.int32)
    out = q.qgemm_a8w8_acc(to_dev(acc), to_dev(A), to_dev(Wt), to_dev(s_a), to_dev(s_w),
                           out_dtype=torch.float32, b_trans=True)
    assert q.last_kernel() == "a8w8_skinny", q.last_kernel()
    np.testing.assert_array_equal(out.cpu().numpy(), oracle.a8w8_acc(acc, A, W, s_a, s_w)["f32"])
    out = q.qgemm_a8w8_noalloc(to_dev(A), to_dev(Wt), to_dev(s_a), to_dev(s_w), out_dtype=torch.bfloat16,
                               b_trans=True)
    assert q.last_kernel() == "a8w8_skinny", q.last_kernel()
    np.testing.assert_array_equal(bf16_bits(out), ref)

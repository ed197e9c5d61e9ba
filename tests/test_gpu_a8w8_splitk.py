"""A8W8 with K split across workgroups (outputs of at most 128 tiles of
128 x 128 and a long K): every output against the oracle, bit for bit, for
both output types, both weight layouts, the accumulator input, ragged last
splits, forced split counts, a workspace reused across shapes, the
workspace-free entry point, and the same three-stage kernel unsplit (without
a workspace, or for 129 to 256 tiles)."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import quantized_int8_gemm_amd as q
import seeded_inputs as si
from gpu_util import bf16_bits, case, dev, env, to_dev

pytestmark = pytest.mark.gpu

SPLITK = "int8_dma_128x128k128_splitk"


def tiles_of(M, name):
    """At most 64 rows run the same split on 64 x 128 tiles (same tile
    count, same plan)."""
    return name.replace("128x128", "64x128") if M <= 64 else name


def run(A, W, s_a, s_w, out_dtype, b_trans=False, **kw):
    return q.qgemm_a8w8(to_dev(A), to_dev(W), to_dev(s_a), to_dev(s_w), out_dtype=out_dtype,
                        b_trans=b_trans, **kw)


def check(A, W, s_a, s_w, b_trans=False, out_dtype=torch.bfloat16, kernel=SPLITK, **kw):
    ref = oracle.a8w8(A, W, s_a, s_w, b_trans=b_trans)
    out = run(A, W, s_a, s_w, out_dtype, b_trans, **kw)
    assert q.last_kernel() == tiles_of(A.shape[0], kernel), q.last_kernel()
    if out_dtype == torch.bfloat16:
        np.testing.assert_array_equal(bf16_bits(out), ref["bf16"])
    else:
        np.testing.assert_array_equal(out.cpu().numpy(), ref["f32"])


@pytest.mark.parametrize("M,N,K,b_trans,out", [
    (17, 8192, 8192, False, "bf16"),     # 64 tiles, 4 splits of 2048
    (64, 4096, 8208, False, "f32"),      # 32 tiles, 8 splits; the last holds 1 whole stage + 16 rows
    (128, 1024, 4096, True, "bf16"),     # W as [N,K], 8 tiles, 4 splits
    (200, 8192, 3072, False, "bf16"),    # 128 tiles, 2 splits, ragged M
    (256, 2000, 8192, False, "f32"),     # ragged N
    (33, 8192, 3072, True, "f32"),       # 3 splits of 1024
])
def test_a8w8_split_k_every_output(M, N, K, b_trans, out):
    case(f"a8w8 split-K M={M} N={N} K={K} b_trans={b_trans} {out}")
    A, W, s_a, s_w = si.a8w8_inputs(M, N, K, seed=M + N + K)
    if b_trans:
        W = np.ascontiguousarray(W.T)
    check(A, W, s_a, s_w, b_trans=b_trans, out_dtype=torch.bfloat16 if out == "bf16" else torch.float32)


@pytest.mark.parametrize("splits", [2, 3, 5, 8])
def test_a8w8_split_k_forced_counts(splits):
    case(f"a8w8 split-K forced splits={splits} 96x4096x8192")
    A, W, s_a, s_w = si.a8w8_inputs(96, 4096, 8192, seed=611)
    with env(QGEMM_TILE_SPLITS=splits):
        check(A, W, s_a, s_w)


def test_a8w8_acc_split_k():
    """The accumulator input is added once, by the split that reduces."""
    case("a8w8_acc split-K 96x4096x4096")
    A, W, s_a, s_w = si.a8w8_inputs(96, 4096, 4096, seed=612)
    g = si.rng(613)
    acc = si.randint(g, (96, 4096), -(1 << 28), (1 << 28), np.int32)
    ref = oracle.a8w8_acc(acc, A, W, s_a, s_w)
    for dt, key in ((torch.bfloat16, "bf16"), (torch.float32, "f32")):
        out = q.qgemm_a8w8_acc(to_dev(acc), to_dev(A), to_dev(W), to_dev(s_a), to_dev(s_w), out_dtype=dt)
        assert q.last_kernel() == SPLITK, q.last_kernel()
        got = bf16_bits(out) if key == "bf16" else out.cpu().numpy()
        np.testing.assert_array_equal(got, ref[key])


def test_a8w8_split_k_workspace_reused_across_shapes():
    """One zeroed workspace for three calls of different tile and split
    counts; the tickets in its fixed 1 KiB header end at zero."""
    case("a8w8 split-K workspace reuse")
    shapes = [(64, 8192, 8192), (40, 2048, 8192), (64, 8192, 8192), (130, 4096, 4096)]
    need = max(q.workspace_bytes(q.QG_OP_A8W8, 1, *s) for s in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev())
    for i, (M, N, K) in enumerate(shapes):
        A, W, s_a, s_w = si.a8w8_inputs(M, N, K, seed=620 + i)
        check(A, W, s_a, s_w, workspace=ws)
    assert int(ws[:1024].sum().item()) == 0


def test_a8w8_noalloc_split_k():
    """The workspace-free entry point splits within its static scratch (2
    splits of 64 tiles here, 64 x 128 ones for 64 rows) and gives the same
    bits."""
    case("a8w8 noalloc split-K 64x8192x8192")
    A, W, s_a, s_w = si.a8w8_inputs(64, 8192, 8192, seed=630)
    ref = oracle.a8w8(A, W, s_a, s_w)
    for _ in range(2):
        out = q.qgemm_a8w8_noalloc(to_dev(A), to_dev(W), to_dev(s_a), to_dev(s_w), out_dtype=torch.bfloat16)
        assert q.last_kernel() == tiles_of(64, SPLITK), q.last_kernel()
        np.testing.assert_array_equal(bf16_bits(out), ref["bf16"])


@pytest.mark.parametrize("M,N,K", [(384, 8192, 4096), (512, 4112, 2064), (300, 8192, 4096)])
def test_a8w8_three_stage_unsplit_every_output(M, N, K):
    """129 to 256 output tiles over a long K: the three-stage kernel without
    a split (no workspace needed)."""
    case(f"a8w8 three-stage unsplit M={M} N={N} K={K}")
    A, W, s_a, s_w = si.a8w8_inputs(M, N, K, seed=M + N + K + 1)
    for dt in (torch.bfloat16, torch.float32):
        check(A, W, s_a, s_w, out_dtype=dt, kernel="int8_dma_128x128k128x3")


def test_a8w8_without_workspace_runs_unsplit():
    """A NULL workspace through the C ABI: the same three-stage kernel
    unsplit, same bits."""
    case("a8w8 64x4096x4096 NULL workspace")
    from quantized_int8_gemm_amd import _binding as b
    M, N, K = 64, 4096, 4096
    A, W, s_a, s_w = si.a8w8_inputs(M, N, K, seed=640)
    tA, tW, ta, tw = to_dev(A), to_dev(W), to_dev(s_a), to_dev(s_w)
    out = torch.empty(M, N, dtype=torch.float32, device=dev())
    st = b.lib.qgemm_a8w8(M, N, K, b._ptr(tA), K, b._ptr(tW), N, 0, b._ptr(ta), M, b._ptr(tw), N,
                          b._ptr(out), b.QG_FP32, N, None, 0,
                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    assert q.last_kernel() == tiles_of(M, "int8_dma_128x128k128x3"), q.last_kernel()
    np.testing.assert_array_equal(out.cpu().numpy(), oracle.a8w8(A, W, s_a, s_w)["f32"])

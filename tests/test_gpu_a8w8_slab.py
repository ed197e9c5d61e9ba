"""A8W8 decode rows with the weight given as [N,K] (b_trans) across a wide N:
the column-slab kernel (each workgroup owns 16 or 32 output columns over all
of K, no workspace).  Every output against the oracle, bit for bit, for both
output types, both slab widths, ragged N and K, padded row strides, the
accumulator input, the workspace-free entry point and HIP graph replays."""
import numpy as np
import pytest
import torch

import oracle
import quantized_int8_gemm_amd as q
import seeded_inputs as si
from gpu_util import bf16_bits, case, dev, env, to_dev

pytestmark = pytest.mark.gpu

SLAB = "a8w8_slab"


def run(A, Wt, s_a, s_w, out_dtype, **kw):
    return q.qgemm_a8w8(to_dev(A), to_dev(Wt), to_dev(s_a), to_dev(s_w), out_dtype=out_dtype, b_trans=True, **kw)


def check(A, Wt, s_a, s_w, out):
    ref = oracle.a8w8(A, Wt, s_a, s_w, b_trans=True)
    res = run(A, Wt, s_a, s_w, torch.bfloat16 if out == "bf16" else torch.float32)
    assert q.last_kernel() == SLAB, q.last_kernel()
    got = bf16_bits(res) if out == "bf16" else res.cpu().numpy()
    np.testing.assert_array_equal(got, ref[out])


@pytest.mark.parametrize("M,N,K,out", [
    (1, 8192, 8192, "bf16"),     # 512 slabs of 16 columns
    (4, 4096, 4096, "f32"),
    (16, 8192, 8192, "bf16"),    # 256 slabs of 32 columns
    (8, 4112, 2064, "f32"),      # 257 slabs; K % 128 == 16: the last step's pieces past K cleared
    (12, 8208, 1040, "bf16"),    # 32-column slabs, the last one half full
    (16, 4096, 16, "f32"),       # one 16-byte piece of K
    (3, 4096, 24592, "bf16"),    # long K, not a whole number of steps
])
def test_slab_every_output(M, N, K, out):
    case(f"a8w8 slab M={M} N={N} K={K} {out}")
    A, W, s_a, s_w = si.a8w8_inputs(M, N, K, seed=M + N + K + 31)
    check(A, np.ascontiguousarray(W.T), s_a, s_w, out)


@pytest.mark.parametrize("tn", [16, 32])
def test_slab_widths_same_bits(tn):
    """Both slab widths give the oracle's bits at every decode row count."""
    case(f"a8w8 slab forced width {tn}, M = 1, 9, 16 at 4096 x 4096")
    for M in (1, 9, 16):
        A, W, s_a, s_w = si.a8w8_inputs(M, 4096, 4096, seed=700 + M)
        with env(QGEMM_SLAB_TN=tn):
            check(A, np.ascontiguousarray(W.T), s_a, s_w, "bf16")


def test_slab_padded_strides_and_scalar_scales():
    """Row strides past K for A, the weight and the output; one activation
    scale for every row."""
    case("a8w8 slab padded strides 5x4096x2048")
    M, N, K = 5, 4096, 2048
    A, W, s_a, s_w = si.a8w8_inputs(M, N, K, seed=733)
    Wt = np.ascontiguousarray(W.T)
    s_a1 = s_a[:1].copy()
    ref = oracle.a8w8(A, Wt, np.full(M, s_a1[0], np.float32), s_w, b_trans=True)["f32"]
    Ap = torch.zeros(M, K + 48, dtype=torch.int8, device=dev())
    Ap[:, :K] = to_dev(A)
    Wp = torch.zeros(N, K + 80, dtype=torch.int8, device=dev())
    Wp[:, :K] = to_dev(Wt)
    outp = torch.full((M, N + 12), -1.0, dtype=torch.float32, device=dev())
    q.qgemm_a8w8(Ap[:, :K], Wp[:, :K], to_dev(s_a1), to_dev(s_w), out_dtype=torch.float32, b_trans=True,
                 out=outp[:, :N])
    assert q.last_kernel() == SLAB, q.last_kernel()
    np.testing.assert_array_equal(outp[:, :N].cpu().numpy(), ref)
    assert bool((outp[:, N:] == -1.0).all())


def test_slab_acc_and_noalloc():
    """The accumulator-input form and the workspace-free entry point take the
    same kernel and give the oracle's bits."""
    case("a8w8 slab acc / noalloc 16x8192x4096")
    M, N, K = 16, 8192, 4096
    A, W, s_a, s_w = si.a8w8_inputs(M, N, K, seed=741)
    Wt = np.ascontiguousarray(W.T)
    acc = si.randint(si.rng(742), (M, N), -(1 << 28), 1 << 28, np.int32)
    for dt, key in ((torch.float32, "f32"), (torch.bfloat16, "bf16")):
        out = q.qgemm_a8w8_acc(to_dev(acc), to_dev(A), to_dev(Wt), to_dev(s_a), to_dev(s_w), out_dtype=dt,
                               b_trans=True)
        assert q.last_kernel() == SLAB, q.last_kernel()
        got = out.cpu().numpy() if key == "f32" else bf16_bits(out)
        np.testing.assert_array_equal(got, oracle.a8w8_acc(acc, A, W, s_a, s_w)[key])
    out = q.qgemm_a8w8_noalloc(to_dev(A), to_dev(Wt), to_dev(s_a), to_dev(s_w), out_dtype=torch.bfloat16,
                               b_trans=True)
    assert q.last_kernel() == SLAB, q.last_kernel()
    np.testing.assert_array_equal(bf16_bits(out), oracle.a8w8(A, W, s_a, s_w)["bf16"])


def test_slab_narrow_n_keeps_split_kernel():
    """Below 256 slabs of 16 columns the split-K decode kernel keeps the
    shape (QGEMM_FORCE_KERNEL=slab still takes it, same bits)."""
    case("a8w8 [N,K] decode 4x2048x4096: split kernel, and forced slab")
    A, W, s_a, s_w = si.a8w8_inputs(4, 2048, 4096, seed=751)
    Wt = np.ascontiguousarray(W.T)
    ref = oracle.a8w8(A, Wt, s_a, s_w, b_trans=True)["bf16"]
    np.testing.assert_array_equal(bf16_bits(run(A, Wt, s_a, s_w, torch.bfloat16)), ref)
    assert q.last_kernel() == "a8w8_skinny", q.last_kernel()
    with env(QGEMM_FORCE_KERNEL="slab"):
        np.testing.assert_array_equal(bf16_bits(run(A, Wt, s_a, s_w, torch.bfloat16)), ref)
        assert q.last_kernel() == SLAB, q.last_kernel()


def test_slab_graph_replays_match_eager():
    """Three slab calls captured in one HIP graph, replayed three times with
    eager work in between: every replay gives the eager bits."""
    case("a8w8 slab graph replays")
    shapes = [(1, 8192, 4096), (16, 8192, 2048), (6, 4096, 8192)]
    ins, outs, refs = [], [], []
    for i, (M, N, K) in enumerate(shapes):
        A, W, s_a, s_w = si.a8w8_inputs(M, N, K, seed=760 + i)
        ins.append((to_dev(A), to_dev(np.ascontiguousarray(W.T)), to_dev(s_a), to_dev(s_w)))
        outs.append(torch.empty(M, N, dtype=torch.bfloat16, device=dev()))
        refs.append(oracle.a8w8(A, W, s_a, s_w)["bf16"])
    calls = [lambda i=i: q.qgemm_a8w8(*ins[i], out_dtype=torch.bfloat16, b_trans=True, out=outs[i])
             for i in range(len(shapes))]
    for c in calls:   # eager, and every workspace the binding may use exists before capture
        c()
        assert q.last_kernel() == SLAB, q.last_kernel()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in calls:
            c()
    for r in range(3):
        for o in outs:
            o.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        for o, ref in zip(outs, refs):
            np.testing.assert_array_equal(bf16_bits(o), ref)
        calls[r % len(calls)]()   # eager work between replays
        torch.cuda.synchronize()

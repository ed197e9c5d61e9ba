"""The W8A32 input gradient's slab form (at most 8 rows of dC across at least
8192 outputs: each workgroup owns 32 of dA's columns, i.e. 32 weight rows,
over the whole contraction, no workspace).  Every output within the bound
1e-5 * scale * sum |dC| |W - zp|, integer gradients and an identity weight
bit for bit, repeated calls bit for bit, a ragged last slab and contraction,
padded strides, the forced form at 16 rows, and HIP graph replays."""
import numpy as np
import pytest
import torch

import oracle
import quantized_int8_gemm_amd as q
import seeded_inputs as si
from gpu_util import case, dev, env, to_dev

pytestmark = pytest.mark.gpu

TOL = 1e-5
SLAB = "w8a32_input_grad_slab"


def grad(dC, W, scale, zp, **kw):
    d = q.qgemm_w8a32_input_grad(to_dev(dC), to_dev(W), scale, zp, **kw)
    return d, q.last_kernel()


def within(d, dC, W, scale, zp):
    R, bound = oracle.w8a32_input_grad(dC, W, scale, zp)
    err = np.abs(d.cpu().numpy().astype(np.float64) - R)
    worst = float((err / np.maximum(bound, 1e-300)).max())
    assert np.all(err <= TOL * bound), f"worst relative error {worst:.3e}"


@pytest.mark.parametrize("M,N,K,zp", [
    (1, 8192, 8192, -5),     # 256 slabs, the bench shape
    (2, 4096, 8192, 0),      # no zero-point correction
    (5, 1008, 8208, 3),      # 257 slabs, the last one half full; 1008 = 15.75 steps of 64
    (8, 8192, 12288, -1),
])
def test_grad_slab_every_output(M, N, K, zp):
    case(f"w8a32_input_grad slab M={M} N={N} K={K} zp={zp}")
    dC, _ = si.w8a32_inputs(M, 1, N, seed=M + N + K + 41)   # [M, N]
    _, W = si.w8a32_inputs(1, N, K, seed=K + 43)            # [K, N]
    d, kern = grad(dC, W, 0.013, zp)
    assert kern == SLAB, kern
    within(d, dC, W, 0.013, zp)
    d2, _ = grad(dC, W, 0.013, zp)
    assert torch.equal(d, d2), "a repeated call differs"


def test_grad_slab_integer_gradients_bit_exact():
    """Small integer dC: every product and partial sum is an exact integer
    in fp32, so the result is the oracle's to the bit."""
    case("w8a32_input_grad slab integer dC 3x2048x8192")
    g = si.rng(45)
    dC = g.integers(-3, 4, size=(3, 2048)).astype(np.float32)
    _, W = si.w8a32_inputs(1, 2048, 8192, seed=46)
    d, kern = grad(dC, W, 1.0, 2)
    assert kern == SLAB, kern
    R, _ = oracle.w8a32_input_grad(dC, W, 1.0, 2)
    np.testing.assert_array_equal(d.cpu().numpy().astype(np.float64), R)


def test_grad_slab_identity_weight_bit_exact():
    """W = I: dA = dC exactly (one product per output, every other one 0)."""
    case("w8a32_input_grad slab identity 8192")
    g = si.rng(47)
    n = 8192
    mant = (1.0 + g.random((4, n))).astype(np.float32)
    dC = (mant * np.exp2(g.integers(-100, 101, size=(4, n))).astype(np.float32)
          * np.where(g.random((4, n)) < 0.5, -1.0, 1.0).astype(np.float32))
    W = torch.eye(n, dtype=torch.int8, device=dev())
    d = q.qgemm_w8a32_input_grad(to_dev(dC), W, 1.0, 0)
    assert q.last_kernel() == SLAB, q.last_kernel()
    np.testing.assert_array_equal(d.cpu().numpy(), dC)


def test_grad_slab_padded_strides():
    """Row strides past the contraction for dC and the weight, and past the
    outputs for dA; nothing outside the view is written."""
    case("w8a32_input_grad slab padded strides 6x2048x8192")
    M, N, K = 6, 2048, 8192
    dC, _ = si.w8a32_inputs(M, 1, N, seed=48)
    _, W = si.w8a32_inputs(1, N, K, seed=49)
    dCp = torch.zeros(M, N + 20, device=dev())
    dCp[:, :N] = to_dev(dC)
    Wp = torch.zeros(K, N + 48, dtype=torch.int8, device=dev())
    Wp[:, :N] = to_dev(W)
    out = torch.full((M, K + 8), 7.0, device=dev())
    q.qgemm_w8a32_input_grad(dCp[:, :N], Wp[:, :N], 0.02, 4, out=out[:, :K])
    assert q.last_kernel() == SLAB, q.last_kernel()
    within(out[:, :K], dC, W, 0.02, 4)
    assert bool((out[:, K:] == 7.0).all())


def test_grad_slab_forced_at_16_rows_and_narrow():
    """QGEMM_FORCE_KERNEL=slab takes 16 rows and a narrow output as well;
    the default keeps the split decode kernel there."""
    case("w8a32_input_grad slab forced 16x4096x8192 and 3x1024x2048")
    for (M, N, K) in ((16, 4096, 8192), (3, 1024, 2048)):
        dC, _ = si.w8a32_inputs(M, 1, N, seed=50 + M)
        _, W = si.w8a32_inputs(1, N, K, seed=51 + M)
        d, kern = grad(dC, W, 0.01, -2)
        assert kern == "w8a32_input_grad_skinny", kern
        with env(QGEMM_FORCE_KERNEL="slab"):
            d, kern = grad(dC, W, 0.01, -2)
        assert kern == SLAB, kern
        within(d, dC, W, 0.01, -2)


def test_grad_slab_graph_replays_match_eager():
    """Two slab calls captured in one HIP graph and replayed three times,
    with eager work between replays: every replay gives the eager bits."""
    case("w8a32_input_grad slab graph replays")
    ins, outs = [], []
    for i, (M, N, K) in enumerate(((1, 4096, 8192), (7, 2048, 8192))):
        dC, _ = si.w8a32_inputs(M, 1, N, seed=60 + i)
        _, W = si.w8a32_inputs(1, N, K, seed=62 + i)
        ins.append((to_dev(dC), to_dev(W)))
        outs.append(torch.empty(M, K, device=dev()))
    calls = [lambda i=i: q.qgemm_w8a32_input_grad(ins[i][0], ins[i][1], 0.01, 3, out=outs[i]) for i in range(2)]
    eager = []
    for c, o in zip(calls, outs):
        c()
        assert q.last_kernel() == SLAB, q.last_kernel()
        eager.append(o.clone())
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
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), f"replay {r} differs"
        calls[r % 2]()
        torch.cuda.synchronize()

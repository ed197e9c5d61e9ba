"""Calls captured in a HIP graph replay with the same bits as eager calls:
the decode kernel (whose split-K tickets live in the workspace and are
returned to zero by every call) and the tiled kernel, each replay checked
against the eager results, with eager calls on the same workspace and
synchronisations between the replays.  The benchmark times its
launch-bound rows this way."""
import numpy as np
import pytest
import torch

import oracle
import quantized_int8_gemm_amd as q
import seeded_inputs as si
from gpu_util import bf16_bits, case, to_dev

pytestmark = pytest.mark.gpu


def _replay_and_check(calls, outs, eager, extra_eager):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in calls:
            c()
    for rep in range(4):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, eager)):
            assert torch.equal(o.view(torch.int16) if o.dtype == torch.bfloat16 else o,
                               e.view(torch.int16) if e.dtype == torch.bfloat16 else e), (rep, i)
        extra_eager()
        torch.cuda.synchronize()


def test_decode_graph_replays_match_eager():
    case("graph: decode M=4 K=N=8192, three inputs")
    m, n, k = 4, 8192, 8192
    sets = []
    for seed in (911, 912, 913):
        A, W, s_a, s_w = si.a8w8_inputs(m, n, k, seed=seed)
        sets.append((A, W, s_a, s_w, tuple(to_dev(x) for x in (A, W, s_a, s_w))))
    ws = torch.zeros(q.workspace_bytes(q.QG_OP_A8W8, 1, m, n, k), dtype=torch.uint8, device="cuda:0")
    eager = []
    for A, W, s_a, s_w, t in sets:
        out = q.qgemm_a8w8(*t, out_dtype=torch.bfloat16, workspace=ws)
        assert q.last_kernel() == "a8w8_skinny"
        eager.append(out.clone())
    np.testing.assert_array_equal(bf16_bits(eager[0]), oracle.a8w8(*sets[0][:4])["bf16"])
    outs = [torch.empty((m, n), dtype=torch.bfloat16, device="cuda:0") for _ in sets]
    calls = [lambda t=s[4], o=o: q.qgemm_a8w8(*t, out_dtype=torch.bfloat16, out=o, workspace=ws)
             for s, o in zip(sets, outs)]
    tmp = torch.empty((m, n), dtype=torch.bfloat16, device="cuda:0")

    def extra():
        q.qgemm_a8w8(*sets[1][4], out_dtype=torch.bfloat16, out=tmp, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(tmp.view(torch.int16), eager[1].view(torch.int16))

    _replay_and_check(calls, outs, eager, extra)


def test_tiled_graph_replays_match_eager():
    case("graph: A8W8 256x1024x1024 fp32 and MatMulInteger 2x64x256x128")
    A, W, s_a, s_w = si.a8w8_inputs(256, 1024, 1024, seed=914)
    t = tuple(to_dev(x) for x in (A, W, s_a, s_w))
    e1 = q.qgemm_a8w8(*t)
    a, b, zb = si.matmul_integer_inputs(2, 64, 256, 128, seed=915)
    ta, tb, tzb = to_dev(a), to_dev(b), to_dev(zb)
    e2 = q.matmul_integer(ta, tb, 128, tzb)
    np.testing.assert_array_equal(e2.cpu().numpy(), oracle.matmul_integer(a, b, 128, zb))
    o1 = torch.empty_like(e1)
    o2 = torch.empty_like(e2)
    calls = [lambda: q.qgemm_a8w8(*t, out=o1), lambda: q.matmul_integer(ta, tb, 128, tzb, out=o2)]

    def extra():
        q.matmul_integer(ta, tb, 128, tzb)
        torch.cuda.synchronize()

    _replay_and_check(calls, [o1, o2], [e1, e2], extra)


def test_split_and_decode_kernels_graph_replays_match_eager():
    """The other kernels whose tickets live in the workspace, captured
    together in one graph sharing one workspace: the W8A32 decode kernel and
    its gradient, the W8A32 split tiles, the MatMulInteger decode kernel, the
    int8 split tiles and the [N,K] A8W8 decode kernel."""
    case("graph: W8A32 decode/split, MatMulInteger decode, A8W8 split-K and [N,K] decode")
    d = torch.device("cuda:0")
    Aw, Ww = si.w8a32_inputs(4, 4096, 4096, seed=920)
    Aw2, Ww2 = si.w8a32_inputs(96, 2048, 4096, seed=921)
    dC, _ = si.w8a32_inputs(4, 1, 4096, seed=922)
    Am, Bm, zb = si.matmul_integer_inputs(1, 8, 4096, 4096, seed=923)
    A8, W8, s_a, s_w = si.a8w8_inputs(64, 4096, 4096, seed=924)
    A9, W9, s_a9, s_w9 = si.a8w8_inputs(8, 2048, 4096, seed=925)
    t = {k: to_dev(v) for k, v in dict(Aw=Aw, Ww=Ww, Aw2=Aw2, Ww2=Ww2, dC=dC, Am=Am[0], Bm=Bm, zb=zb, A8=A8, W8=W8,
                                        s_a=s_a, s_w=s_w, A9=A9, W9t=np.ascontiguousarray(W9.T), s_a9=s_a9,
                                        s_w9=s_w9).items()}
    need = max(q.workspace_bytes(q.QG_OP_W8A32, 1, 4, 4096, 4096), q.workspace_bytes(q.QG_OP_W8A32, 1, 96, 2048, 4096),
               q.workspace_bytes(q.QG_OP_W8A32_INPUT_GRAD, 1, 4, 4096, 4096),
               q.workspace_bytes(q.QG_OP_MATMUL_INTEGER, 1, 8, 4096, 4096),
               q.workspace_bytes(q.QG_OP_A8W8, 1, 64, 4096, 4096), q.workspace_bytes(q.QG_OP_A8W8, 1, 8, 2048, 4096))
    ws = torch.zeros(need, dtype=torch.uint8, device=d)
    outs = [torch.empty(4, 4096, device=d), torch.empty(96, 2048, device=d), torch.empty(4, 4096, device=d),
            torch.empty(8, 4096, dtype=torch.int32, device=d), torch.empty(64, 4096, dtype=torch.bfloat16, device=d),
            torch.empty(8, 2048, dtype=torch.float32, device=d)]
    calls = [
        lambda: q.qgemm_w8a32(t["Aw"], t["Ww"], 0.01, 3, out=outs[0], workspace=ws),
        lambda: q.qgemm_w8a32(t["Aw2"], t["Ww2"], 0.01, 3, out=outs[1], workspace=ws),
        lambda: q.qgemm_w8a32_input_grad(t["dC"], t["Ww"], 0.01, 3, out=outs[2], workspace=ws),
        lambda: q.matmul_integer(t["Am"], t["Bm"], 128, t["zb"], out=outs[3], workspace=ws),
        lambda: q.qgemm_a8w8(t["A8"], t["W8"], t["s_a"], t["s_w"], out_dtype=torch.bfloat16, out=outs[4],
                             workspace=ws),
        lambda: q.qgemm_a8w8(t["A9"], t["W9t"], t["s_a9"], t["s_w9"], b_trans=True, out=outs[5], workspace=ws),
    ]
    kernels = ["w8a32_skinny", "w8a32_bf16x3_128x128_splitk", "w8a32_input_grad_skinny", "matmul_integer_skinny",
               "int8_dma_64x128k128_splitk", "a8w8_skinny"]
    eager = []
    for c, o, k in zip(calls, outs, kernels):
        c()
        assert q.last_kernel() == k, (q.last_kernel(), k)
        eager.append(o.clone())
    np.testing.assert_array_equal(eager[3].cpu().numpy(), oracle.matmul_integer(Am[0], Bm, 128, zb))
    np.testing.assert_array_equal(bf16_bits(eager[4]), oracle.a8w8(A8, W8, s_a, s_w)["bf16"])
    tmp = torch.empty(4, 4096, device=d)

    def extra():
        q.qgemm_w8a32(t["Aw"], t["Ww"], 0.01, 3, out=tmp, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(tmp, eager[0])

    _replay_and_check(calls, outs, eager, extra)
    assert int(ws[:1024].sum().item()) == 0

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

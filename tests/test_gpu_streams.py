"""Calls that overlap on two HIP streams (default priority) give the same
bits as calls on one stream, as long as they do not share a workspace: the
decode kernel keeps its split-K tickets and partials, DynamicQuantizeLinear
its min/max partials, in the caller's workspace (or, without one, in the
binding's workspace for that stream).  The per-thread record of the last
kernel launched stays per thread while two host threads call the library at
once (ctypes releases the GIL around each call)."""
import threading

import numpy as np
import pytest
import torch

import oracle
import quantized_int8_gemm_amd as q
import seeded_inputs as si
from gpu_util import bf16_bits, case, to_dev

pytestmark = pytest.mark.gpu


def test_decode_on_two_streams_with_their_own_workspaces():
    case("streams: decode M=4 K=N=8192 on two streams, 8 calls each")
    m, n, k = 4, 8192, 8192
    sets = []
    for seed in (931, 932):
        A, W, s_a, s_w = si.a8w8_inputs(m, n, k, seed=seed)
        sets.append(((A, W, s_a, s_w), tuple(to_dev(x) for x in (A, W, s_a, s_w))))
    ref = [q.qgemm_a8w8(*t, out_dtype=torch.bfloat16).clone() for _, t in sets]
    assert q.last_kernel() == "a8w8_skinny"
    np.testing.assert_array_equal(bf16_bits(ref[0]), oracle.a8w8(*sets[0][0])["bf16"])
    nbytes = q.workspace_bytes(q.QG_OP_A8W8, 1, m, n, k)
    ws = [torch.zeros(nbytes, dtype=torch.uint8, device="cuda:0") for _ in range(2)]
    outs = [[torch.empty((m, n), dtype=torch.bfloat16, device="cuda:0") for _ in range(8)] for _ in range(2)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for it in range(8):
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                q.qgemm_a8w8(*sets[i][1], out_dtype=torch.bfloat16, out=outs[i][it], workspace=ws[i])
    torch.cuda.synchronize()
    for i in range(2):
        for it in range(8):
            assert torch.equal(outs[i][it].view(torch.int16), ref[i].view(torch.int16)), (i, it)
    # every call returned its tickets to zero
    tiles_n = (n + 255) // 256
    for w in ws:
        assert int(w[:4 * tiles_n].view(torch.int32).abs().sum()) == 0


def test_w8a32_and_matmul_integer_split_kernels_on_two_streams():
    """The W8A32 decode and split kernels and the MatMulInteger decode kernel
    on two streams at once, each stream with the binding's own workspace:
    the same bits as one-stream calls, every ticket back at zero."""
    case("streams: W8A32 decode / split and MatMulInteger decode on two streams, 6 rounds")
    from quantized_int8_gemm_amd import _binding as b
    d = torch.device("cuda:0")
    Aw, Ww = si.w8a32_inputs(8, 4096, 4096, seed=950)
    Aw2, Ww2 = si.w8a32_inputs(100, 2048, 4096, seed=951)
    Am, Bm, zb = si.matmul_integer_inputs(1, 4, 4096, 4096, seed=952)
    t = [to_dev(x) for x in (Aw, Ww, Aw2, Ww2, Am[0], Bm, zb)]
    calls = [lambda: q.qgemm_w8a32(t[0], t[1], 0.01, 2), lambda: q.qgemm_w8a32(t[2], t[3], 0.01, 2),
             lambda: q.matmul_integer(t[4], t[5], 128, t[6])]
    ref = [c().clone() for c in calls]
    np.testing.assert_array_equal(ref[2].cpu().numpy(), oracle.matmul_integer(Am[0], Bm, 128, zb))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    res = [[], []]
    torch.cuda.synchronize()
    for it in range(6):
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                res[i].append([c() for c in calls])
    torch.cuda.synchronize()
    for i in range(2):
        for it in range(6):
            for j in range(3):
                assert torch.equal(res[i][it][j], ref[j]), (i, it, j)
    for i in range(2):
        ws = b._workspaces[(d, streams[i].cuda_stream)]
        assert int(ws[:1024].sum().item()) == 0


def test_dynamic_quantize_on_two_streams_with_the_bindings_workspaces():
    case("streams: DynamicQuantizeLinear [8, 512, 2048] on two streams, 6 calls each")
    xs = [si.dql_inputs((8, 512, 2048), seed=s) for s in (941, 942)]
    refs = [oracle.dynamic_quantize_linear(x) for x in xs]
    tx = [to_dev(x) for x in xs]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    res = [[], []]
    torch.cuda.synchronize()
    for it in range(6):
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                res[i].append(q.dynamic_quantize_linear(tx[i]))
    torch.cuda.synchronize()
    for i in range(2):
        y_ref, s_ref, z_ref = refs[i]
        for it, (y, s, z) in enumerate(res[i]):
            np.testing.assert_array_equal(y.cpu().numpy(), y_ref, err_msg=f"stream {i} call {it}")
            assert s.item() == float(s_ref) and z.item() == int(z_ref), (i, it)


def test_last_kernel_record_is_per_thread():
    case("streams: two host threads, decode and MatMulInteger, 20 calls each")
    A, W, s_a, s_w = si.a8w8_inputs(1, 4096, 4096, seed=951)
    td = tuple(to_dev(x) for x in (A, W, s_a, s_w))
    a, b, zb = si.matmul_integer_inputs(2, 64, 256, 128, seed=952)
    ta, tb, tzb = to_dev(a), to_dev(b), to_dev(zb)
    ref_d = q.qgemm_a8w8(*td, out_dtype=torch.bfloat16).clone()
    ref_m = q.matmul_integer(ta, tb, 128, tzb).clone()
    np.testing.assert_array_equal(ref_m.cpu().numpy(), oracle.matmul_integer(a, b, 128, zb))
    torch.cuda.synchronize()
    errors = []
    start = threading.Barrier(2)

    def worker(kind):
        try:
            s = torch.cuda.Stream()
            start.wait()
            with torch.cuda.stream(s):
                for _ in range(20):
                    if kind == "decode":
                        y = q.qgemm_a8w8(*td, out_dtype=torch.bfloat16)
                        name, want = q.last_kernel(), "a8w8_skinny"
                    else:
                        y = q.matmul_integer(ta, tb, 128, tzb)
                        name, want = q.last_kernel(), "int8_"
                    if not name.startswith(want):
                        errors.append((kind, name))
                s.synchronize()
                ref = ref_d if kind == "decode" else ref_m
                same = torch.equal(y.view(torch.int16), ref.view(torch.int16)) if kind == "decode" \
                    else torch.equal(y, ref)
                if not same:
                    errors.append((kind, "result"))
        except Exception as e:  # reported below, in the test's thread
            errors.append((kind, repr(e)))

    threads = [threading.Thread(target=worker, args=(k,)) for k in ("decode", "mmi")]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not any(t.is_alive() for t in threads)
    assert errors == [], errors

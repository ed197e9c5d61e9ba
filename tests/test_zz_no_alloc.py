"""The A8W8 entry point that allocates nothing (qgemm_a8w8_noalloc): called
through the C ABI, its outputs equal qgemm_a8w8's bit for bit (and the
oracle's) on two calls in a row, the second smaller, with the decode split-K
scratch held in the library's static device array.  CPU checks: argument
validation happens before any HIP call, and a split-K plan larger than the
static scratch is refused."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from quantized_int8_gemm_amd import _binding as b

FAKE = ctypes.c_void_p(4096)   # never dereferenced: validation fails first
SCRATCH_BYTES = 1024 + (8 << 20)


def noalloc_raw(M, N, K, A, W, sa, sw, out, od, stream, lda=None, ldw=None, ldo=None, bt=0):
    return b.lib.qgemm_a8w8_noalloc(M, N, K, A, K if lda is None else lda, W, N if ldw is None else ldw, bt,
                                    sa, M, sw, N, out, od, N if ldo is None else ldo, stream)


def test_noalloc_rejects_before_any_hip_call():
    INV = b.QG_ERR_INVALID_ARGUMENT
    assert noalloc_raw(4, 4, 4, None, FAKE, FAKE, FAKE, FAKE, b.QG_FP32, None) == INV
    assert noalloc_raw(4, 4, 4, FAKE, FAKE, FAKE, FAKE, FAKE, b.QG_INT32, None) == INV
    assert noalloc_raw(4, 4, 4, FAKE, FAKE, FAKE, FAKE, FAKE, b.QG_FP32, None, lda=3) == INV
    assert noalloc_raw(0, 4, 4, None, None, None, None, None, b.QG_FP32, None) == b.QG_OK


def test_noalloc_refuses_plans_beyond_the_scratch(monkeypatch):
    # 64 forced splits of 64 column tiles want 64 MiB of partial sums
    monkeypatch.setenv("QGEMM_SPLITS", "64")
    need = b.lib.qgemm_workspace_bytes(b.QG_OP_A8W8, 1, 16, 16384, 65536)
    assert need > SCRATCH_BYTES
    assert noalloc_raw(16, 16384, 65536, FAKE, FAKE, FAKE, FAKE, FAKE, b.QG_BF16, None) == b.QG_ERR_WORKSPACE


def test_default_plans_fit_the_scratch():
    for M in (1, 16):
        for N in range(256, 70000, 256 * 7):
            for K in (64, 4096, 8192, 65536):
                assert b.lib.qgemm_workspace_bytes(b.QG_OP_A8W8, 1, M, N, K) <= SCRATCH_BYTES, (M, N, K)


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _inputs(M, N, K, seed, d):
    A, W, sa, sw = si.a8w8_inputs(M, N, K, seed=seed)
    t = [torch.from_numpy(x).to(d) for x in (A, W, sa, sw)]
    return (A, W, sa, sw), t


@pytest.mark.gpu
@pytest.mark.parametrize("shapes", [
    ((16, 8192, 8192, torch.bfloat16), (4, 4096, 2048, torch.float32)),   # decode, split-K scratch
    ((3, 12288, 8192, torch.float32), (1, 1000, 777, torch.bfloat16)),    # ragged second call
    ((300, 640, 1024, torch.bfloat16), (40, 256, 512, torch.float32)),    # tiled kernel, no scratch
])
def test_noalloc_matches_workspace_entry_point(shapes):
    d = _dev()
    stream = ctypes.c_void_p(torch.cuda.current_stream(d).cuda_stream)
    for i, (M, N, K, dt) in enumerate(shapes):
        import sys
        sys.stderr.write(f"[case] a8w8_noalloc call {i} M={M} N={N} K={K} {dt}\n")
        sys.stderr.flush()
        (A, W, sa, sw), (tA, tW, ta, tw) = _inputs(M, N, K, 900 + 7 * i + M, d)
        ref_out = torch.empty((M, N), dtype=dt, device=d)
        ws_bytes = b.lib.qgemm_workspace_bytes(b.QG_OP_A8W8, 1, M, N, K)
        ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device=d)
        od = b.QG_FP32 if dt == torch.float32 else b.QG_BF16
        assert b.lib.qgemm_a8w8(M, N, K, b._ptr(tA), K, b._ptr(tW), N, 0, b._ptr(ta), M, b._ptr(tw), N,
                                b._ptr(ref_out), od, N, b._ptr(ws) if ws_bytes else None, ws_bytes,
                                stream) == b.QG_OK
        out = torch.full((M, N), -3.0, dtype=dt, device=d)
        assert noalloc_raw(M, N, K, b._ptr(tA), b._ptr(tW), b._ptr(ta), b._ptr(tw), b._ptr(out), od,
                           stream) == b.QG_OK
        kernel = b.last_kernel()
        # decode rows, else (K <= 2048, at most 256 tiles of 128 x 128) 64 x 128 tiles
        assert kernel == ("a8w8_skinny" if M <= 16 else "int8_dma_64x128k128"), kernel
        torch.cuda.synchronize()
        if dt == torch.float32:
            got, want = out.cpu().numpy(), ref_out.cpu().numpy()
            np.testing.assert_array_equal(got, oracle.a8w8(A, W, sa, sw)["f32"])
        else:
            got = out.cpu().view(torch.int16).numpy().view(np.uint16)
            want = ref_out.cpu().view(torch.int16).numpy().view(np.uint16)
            np.testing.assert_array_equal(got, oracle.a8w8(A, W, sa, sw)["bf16"])
        np.testing.assert_array_equal(got, want)

"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
rejects bad arguments before any HIP call.  No compute call is made here."""
import ctypes
import threading
import os
import re

import pytest
import torch

import quantized_int8_gemm_amd as q
from quantized_int8_gemm_amd import _binding as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qgemm.h")
FAKE = ctypes.c_void_p(4096)   # never dereferenced: validation fails first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q\w+|matmul_integer\w*|dynamic_quantize_linear|conv_integer\w*)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert set(names) == {"qgemm_w8a32", "qgemm_a8w8", "matmul_integer", "qgemm_workspace_bytes",
                          "qgemm_status_string", "qgemm_last_kernel", "qgemm_version",
                          "qgemm_calib_read", "qgemm_calib_mfma_i8", "qgemm_calib_mfma_i8_32x32", "qgemm_calib_mfma_f32", "qgemm_calib_mfma_bf16", "qgemm_a8w8_acc",
                          "matmul_integer_row_zp", "qgemm_w8a32_input_grad", "dynamic_quantize_linear",
                          "conv_integer", "conv_integer_workspace_bytes", "qgemm_a8w8_noalloc",
                          "qgemm_w8a32_ws", "qgemm_w8a32_input_grad_ws"}
    lib = ctypes.CDLL(b.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(b.PROTOTYPES) == set(names)


def test_status_strings_and_version():
    assert q.status_string(0) == "ok"
    assert q.status_string(1) == "invalid argument"
    assert q.status_string(2) == "unsupported"
    assert q.status_string(3) == "workspace too small"
    assert q.status_string(4) == "HIP launch error"
    assert "gfx950" in q.version()
    # the record is per thread: a thread that has launched nothing reads ""
    seen = []
    t = threading.Thread(target=lambda: seen.append(q.last_kernel()))
    t.start()
    t.join()
    assert seen == [""]


def test_workspace_bytes():
    # decode shapes split K and want a workspace; large shapes need none
    assert q.workspace_bytes(q.QG_OP_A8W8, 1, 16, 8192, 8192) > 0
    assert q.workspace_bytes(q.QG_OP_A8W8, 1, 1, 8192, 8192) > 0
    assert q.workspace_bytes(q.QG_OP_A8W8, 1, 8192, 8192, 8192) == 0
    # a tiled output of 64 tiles over K = 8192 splits K four ways: the ticket
    # header and four 64 KiB partial tiles per output tile
    assert q.workspace_bytes(q.QG_OP_A8W8, 1, 64, 8192, 8192) == 1024 + 64 * 4 * 128 * 128 * 4
    assert q.workspace_bytes(q.QG_OP_A8W8, 1, 64, 8192, 1024) == 0      # K too short to split
    assert q.workspace_bytes(q.QG_OP_A8W8, 1, 2048, 4096, 8192) == 0    # 512 tiles fill the chip
    # W8A32: 128x128 tiles over K split eight ways at M = 16, N = K = 8192 (64
    # tiles, two workgroups per CU): the ticket header, then per split a 64 KiB
    # fp32 tile and 512 bytes of row sums
    assert q.workspace_bytes(q.QG_OP_W8A32, 1, 16, 8192, 8192) == 1024 + 64 * 8 * (65536 + 512)
    # 256 tiles (M = 512) still split, two ways; 512 do not
    assert q.workspace_bytes(q.QG_OP_W8A32, 1, 512, 8192, 8192) == 1024 + 256 * 2 * (65536 + 512)
    assert q.workspace_bytes(q.QG_OP_W8A32, 1, 1024, 8192, 8192) == 0
    # at most 16 rows the size covers both the decode kernel (17 rows of 256
    # floats per split and column tile) and the tiled one, which unaligned
    # rows take: here the tiled one's 2 splits of 64 tiles
    assert q.workspace_bytes(q.QG_OP_W8A32, 1, 16, 8192, 1024) == 1024 + 64 * 2 * (65536 + 512)
    # wide outputs: the decode kernel alone splits nothing past 256 column tiles
    assert q.workspace_bytes(q.QG_OP_W8A32, 1, 2, 65792, 64) == 0
    assert q.workspace_bytes(q.QG_OP_W8A32, 1, 4096, 4096, 4096) == 0     # 256x256 tiles, unsplit
    assert q.workspace_bytes(q.QG_OP_W8A32, 1, 16, 8192, 512) == 0        # K too short to split
    # the input gradient's outputs are dA's K columns, its sum runs over N
    assert q.workspace_bytes(q.QG_OP_W8A32_INPUT_GRAD, 1, 16, 8192, 4096) == 1024 + 32 * 8 * (65536 + 512)
    assert q.workspace_bytes(q.QG_OP_MATMUL_INTEGER, 8, 512, 2048, 2048) == 0
    # MatMulInteger splits like A8W8, each partial tile followed by its row
    # and column sums (8 KiB); batches are folded into M
    mmi_split = 1024 + 64 * 4 * (128 * 128 * 4 + 8192)
    assert q.workspace_bytes(q.QG_OP_MATMUL_INTEGER, 1, 64, 8192, 8192) == mmi_split
    assert q.workspace_bytes(q.QG_OP_MATMUL_INTEGER, 4, 16, 8192, 8192) == mmi_split
    assert q.workspace_bytes(q.QG_OP_MATMUL_INTEGER, 1, 64, 8192, 1024) == 0
    assert q.workspace_bytes(q.QG_OP_MATMUL_INTEGER, 0, 64, 8192, 8192) == 0
    # at most 16 rows: the decode kernel's partials, 16 output rows plus a row
    # of column sums and one of row sums per split and 256-column tile
    assert q.workspace_bytes(q.QG_OP_MATMUL_INTEGER, 1, 1, 8192, 8192) == 1024 + 32 * 8 * 18 * 256 * 4
    assert q.workspace_bytes(q.QG_OP_MATMUL_INTEGER, 4, 4, 8192, 8192) == 1024 + 32 * 8 * 18 * 256 * 4
    assert q.workspace_bytes(q.QG_OP_MATMUL_INTEGER, 1, 16, 8192, 8160) == 0   # K not whole 64-row steps
    assert q.workspace_bytes(q.QG_OP_A8W8, 1, 0, 8192, 8192) == 0
    # DynamicQuantizeLinear: one (min, max) float pair per 128 KiB of x, at most 2 KiB
    assert q.workspace_bytes(q.QG_OP_DYNAMIC_QUANTIZE_LINEAR, 1, 1, 0, 1) == 8
    assert q.workspace_bytes(q.QG_OP_DYNAMIC_QUANTIZE_LINEAR, 1, 1, 32768, 1) == 8
    assert q.workspace_bytes(q.QG_OP_DYNAMIC_QUANTIZE_LINEAR, 1, 1, 32769, 1) == 16
    assert q.workspace_bytes(q.QG_OP_DYNAMIC_QUANTIZE_LINEAR, 1, 1, 8 * 512 * 2048, 1) == 2048
    assert q.workspace_bytes(q.QG_OP_DYNAMIC_QUANTIZE_LINEAR, 1, 1, 1 << 34, 1) == 2048


def w8a32(**kw):
    a = dict(M=4, N=4, K=4, A=FAKE, lda=4, W=FAKE, ldw=4, scale=1.0, zp=0, C=FAKE, ldc=4, stream=None)
    a.update(kw)
    return b.lib.qgemm_w8a32(a["M"], a["N"], a["K"], a["A"], a["lda"], a["W"], a["ldw"], a["scale"],
                             a["zp"], a["C"], a["ldc"], a["stream"])


def a8w8(**kw):
    a = dict(M=4, N=4, K=4, A=FAKE, lda=4, W=FAKE, ldw=4, bt=0, s_a=FAKE, n_a=4, s_w=FAKE, n_w=4,
             out=FAKE, dt=b.QG_FP32, ldo=4, ws=None, wsb=0, stream=None)
    a.update(kw)
    return b.lib.qgemm_a8w8(a["M"], a["N"], a["K"], a["A"], a["lda"], a["W"], a["ldw"], a["bt"],
                            a["s_a"], a["n_a"], a["s_w"], a["n_w"], a["out"], a["dt"], a["ldo"],
                            a["ws"], a["wsb"], a["stream"])


def mmi(**kw):
    a = dict(batch=1, M=4, N=4, K=4, A=FAKE, adt=b.QG_UINT8, lda=4, abs=0, B=FAKE, bdt=b.QG_INT8,
             ldb=4, bbs=0, za=0, zb=None, nzb=0, Y=FAKE, ldy=4, ybs=16, ws=None, wsb=0, stream=None)
    a.update(kw)
    return b.lib.matmul_integer(a["batch"], a["M"], a["N"], a["K"], a["A"], a["adt"], a["lda"], a["abs"],
                                a["B"], a["bdt"], a["ldb"], a["bbs"], a["za"], a["zb"], a["nzb"],
                                a["Y"], a["ldy"], a["ybs"], a["ws"], a["wsb"], a["stream"])


INV, UNS, OK = b.QG_ERR_INVALID_ARGUMENT, b.QG_ERR_UNSUPPORTED, b.QG_OK


@pytest.mark.parametrize("kw,code", [
    (dict(M=0), OK), (dict(N=0), OK), (dict(M=0, A=None, C=None), OK), (dict(N=0, K=0), OK),
    (dict(K=0), INV), (dict(M=-3), INV), (dict(M=0, N=-1), INV),
    (dict(A=None), INV), (dict(W=None), INV), (dict(C=None), INV),
    (dict(lda=3), INV), (dict(ldw=3), INV), (dict(ldc=3), INV),
    (dict(scale=float("nan")), INV), (dict(scale=float("inf")), INV),
    (dict(K=70000, ldw=40000, N=40000, lda=70000, ldc=40000), UNS),
])
def test_w8a32_rejects(kw, code):
    assert w8a32(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(M=0), OK), (dict(N=0), OK), (dict(M=0, A=None, out=None, s_a=None), OK),
    (dict(K=0), INV), (dict(M=-1, N=0), INV),
    (dict(A=None), INV), (dict(W=None), INV), (dict(s_a=None), INV), (dict(s_w=None), INV),
    (dict(out=None), INV),
    (dict(lda=3), INV), (dict(ldw=3), INV), (dict(ldo=3), INV),
    (dict(n_a=2), INV), (dict(n_a=0), INV), (dict(n_w=3), INV), (dict(n_w=5), INV),
    (dict(dt=b.QG_INT32), INV), (dict(dt=b.QG_INT8), INV), (dict(dt=7), INV),
    (dict(bt=2), INV), (dict(bt=1, ldw=3), INV),
    (dict(ws=ctypes.c_void_p(4096 + 16), wsb=1 << 20), INV), (dict(ws=ctypes.c_void_p(4096 + 128), wsb=1 << 20), INV),
    (dict(K=100000, ldw=40000, N=40000, lda=100000, ldo=40000, n_a=1, n_w=1), UNS),
])
def test_a8w8_rejects(kw, code):
    assert a8w8(**kw) == code


def test_a8w8_split_k_workspace_too_small():
    # a tiled shape whose split-K plan needs more workspace than was passed
    M, N, K = 64, 8192, 8192
    need = q.workspace_bytes(q.QG_OP_A8W8, 1, M, N, K)
    st = a8w8(M=M, N=N, K=K, lda=K, ldw=N, ldo=N, n_a=M, n_w=N, ws=FAKE, wsb=need - 1)
    assert st == b.QG_ERR_WORKSPACE


def test_matmul_integer_split_k_workspace_checks():
    M, N, K = 64, 8192, 8192
    need = q.workspace_bytes(q.QG_OP_MATMUL_INTEGER, 1, M, N, K)
    kw = dict(M=M, N=N, K=K, lda=K, ldb=N, ldy=N, ybs=M * N, ws=FAKE)
    assert mmi(wsb=need - 1, **kw) == b.QG_ERR_WORKSPACE
    kw["ws"] = ctypes.c_void_p(4096 + 16)   # not 256-byte aligned
    assert mmi(wsb=need, **kw) == b.QG_ERR_INVALID_ARGUMENT


def test_w8a32_ws_workspace_checks():
    M, N, K = 80, 8192, 8192   # tiled, K split four ways
    need = q.workspace_bytes(q.QG_OP_W8A32, 1, M, N, K)
    args = (M, N, K, FAKE, K, FAKE, N, 1.0, 0, FAKE, N)
    assert b.lib.qgemm_w8a32_ws(*args, FAKE, need - 1, None) == b.QG_ERR_WORKSPACE
    assert b.lib.qgemm_w8a32_ws(*args, ctypes.c_void_p(4096 + 64), need, None) == b.QG_ERR_INVALID_ARGUMENT
    # 16 aligned rows: the decode kernel, 8 splits of 32 column tiles
    M = 16
    decode_need = 1024 + 32 * 8 * 17 * 1024
    args = (M, N, K, FAKE, K, FAKE, N, 1.0, 0, FAKE, N)
    assert b.lib.qgemm_w8a32_ws(*args, FAKE, decode_need - 1, None) == b.QG_ERR_WORKSPACE
    M, N, K = 80, 8192, 8192
    need = q.workspace_bytes(q.QG_OP_W8A32_INPUT_GRAD, 1, M, N, K)
    gargs = (M, N, K, FAKE, N, FAKE, N, 1.0, 0, FAKE, K)
    assert b.lib.qgemm_w8a32_input_grad_ws(*gargs, FAKE, need - 1, None) == b.QG_ERR_WORKSPACE
    M = 16   # the decode kernel: 8 splits of 32 tiles of dA's columns
    gargs = (M, N, K, FAKE, N, FAKE, N, 1.0, 0, FAKE, K)
    assert b.lib.qgemm_w8a32_input_grad_ws(*gargs, FAKE, decode_need - 1, None) == b.QG_ERR_WORKSPACE
    # the same argument checks as the calls without a workspace
    assert b.lib.qgemm_w8a32_ws(M, N, K, FAKE, K - 1, FAKE, N, 1.0, 0, FAKE, N, None, 0, None) == \
        b.QG_ERR_INVALID_ARGUMENT


def test_a8w8_workspace_too_small():
    # a decode shape whose split-K workspace is larger than what was passed
    M, N, K = 16, 8192, 8192
    need = q.workspace_bytes(q.QG_OP_A8W8, 1, M, N, K)
    assert need > 0
    st = a8w8(M=M, N=N, K=K, lda=K, ldw=N, ldo=N, n_a=M, n_w=N, ws=FAKE, wsb=need - 1)
    assert st == b.QG_ERR_WORKSPACE


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), OK), (dict(M=0), OK), (dict(N=0), OK), (dict(batch=0, A=None, Y=None), OK),
    (dict(K=0), INV), (dict(batch=-1), INV), (dict(batch=0, M=-2), INV),
    (dict(A=None), INV), (dict(B=None), INV), (dict(Y=None), INV),
    (dict(adt=b.QG_FP32), UNS), (dict(bdt=b.QG_BF16), UNS), (dict(adt=b.QG_INT32), UNS),
    (dict(adt=7), INV), (dict(bdt=-1), INV),
    (dict(lda=3), INV), (dict(ldb=3), INV), (dict(ldy=3), INV),
    (dict(za=256), INV), (dict(za=-1), INV), (dict(adt=b.QG_INT8, za=128), INV),
    (dict(adt=b.QG_INT8, za=-129), INV),
    (dict(zb=FAKE, nzb=2), INV), (dict(zb=FAKE, nzb=0), INV),
    (dict(abs=-1), INV), (dict(bbs=-4), INV), (dict(ybs=-16), INV),
    (dict(batch=2, ybs=15), INV), (dict(batch=2, abs=15), INV), (dict(batch=2, bbs=3), INV),
    (dict(K=70000, ldb=40000, N=40000, lda=70000, ldy=40000), UNS),
])
def test_matmul_integer_rejects(kw, code):
    assert mmi(**kw) == code


# -- binding-level checks (raise before any device work) --------------------

def test_binding_rejects_float_weight_as_int8():
    """An fp32 tensor passed where the int8 weight belongs is a TypeError,
    never a silent reinterpretation of its bytes."""
    A = torch.zeros(4, 8, dtype=torch.int8)
    with pytest.raises(TypeError):
        q.qgemm_a8w8(A, torch.zeros(8, 4), torch.ones(4), torch.ones(4))
    with pytest.raises(TypeError):
        q.qgemm_w8a32(torch.zeros(4, 8), torch.zeros(8, 4), 0.1, 0)
    with pytest.raises(TypeError):
        q.matmul_integer(torch.zeros(4, 8), torch.zeros(8, 4, dtype=torch.int8))


def test_binding_rejects_bad_shapes():
    A = torch.zeros(4, 8, dtype=torch.int8)
    W = torch.zeros(8, 5, dtype=torch.int8)
    with pytest.raises(ValueError):
        q.qgemm_a8w8(A, torch.zeros(7, 5, dtype=torch.int8), torch.ones(4), torch.ones(5))
    with pytest.raises(ValueError):   # act_scale of length N != M
        q.qgemm_a8w8(A, W, torch.ones(5), torch.ones(5))
    with pytest.raises(ValueError):   # weight_scale of length M != N
        q.qgemm_a8w8(A, W, torch.ones(4), torch.ones(4))
    with pytest.raises(ValueError):   # [1, M] is not a row-scale shape
        q.qgemm_a8w8(A, W, torch.ones(1, 4), torch.ones(5))
    with pytest.raises(ValueError):   # rank 1 MatMulInteger
        q.matmul_integer(torch.zeros(8, dtype=torch.uint8), torch.zeros(8, 3, dtype=torch.int8))
    with pytest.raises(ValueError):   # rank 5
        q.matmul_integer(torch.zeros(1, 1, 1, 2, 8, dtype=torch.uint8), torch.zeros(8, 3, dtype=torch.int8))
    with pytest.raises(ValueError):   # per-row activation zero point of the wrong length
        q.matmul_integer(torch.zeros(4, 8, dtype=torch.uint8), torch.zeros(8, 3, dtype=torch.int8),
                         torch.zeros(3, dtype=torch.uint8))
    with pytest.raises(ValueError):   # [1, M] is not a per-row shape
        q.matmul_integer(torch.zeros(4, 8, dtype=torch.uint8), torch.zeros(8, 3, dtype=torch.int8),
                         torch.zeros(1, 4, dtype=torch.uint8))
    with pytest.raises(ValueError):   # acc_in of the wrong shape
        q.qgemm_a8w8_acc(torch.zeros(4, 5, dtype=torch.int32), A, torch.zeros(8, 4, dtype=torch.int8),
                         torch.ones(4), torch.ones(4))
    with pytest.raises(TypeError):    # acc_in must be int32
        q.qgemm_a8w8_acc(torch.zeros(4, 5), A, W, torch.ones(4), torch.ones(5))
    with pytest.raises(ValueError):   # per-column zero point of the wrong length
        q.matmul_integer(torch.zeros(4, 8, dtype=torch.uint8), torch.zeros(8, 3, dtype=torch.int8),
                         0, torch.zeros(2, dtype=torch.int8))


def test_binding_requires_gpu_tensors():
    A = torch.zeros(4, 8, dtype=torch.int8)
    W = torch.zeros(8, 4, dtype=torch.int8)
    with pytest.raises(ValueError):
        q.qgemm_a8w8(A, W, torch.ones(4), torch.ones(4))


def test_calibration_rejects_bad_arguments():
    lib = b.lib
    ops = ctypes.c_int64(0)
    assert lib.qgemm_calib_read(None, 4096, FAKE, None) == b.QG_ERR_INVALID_ARGUMENT
    assert lib.qgemm_calib_read(FAKE, 0, FAKE, None) == b.QG_ERR_INVALID_ARGUMENT
    assert lib.qgemm_calib_read(FAKE, 4100, FAKE, None) == b.QG_ERR_INVALID_ARGUMENT
    assert lib.qgemm_calib_read(ctypes.c_void_p(4104), 4096, FAKE, None) == b.QG_ERR_INVALID_ARGUMENT
    assert lib.qgemm_calib_read(FAKE, 4096, None, None) == b.QG_ERR_INVALID_ARGUMENT
    assert lib.qgemm_calib_mfma_i8(FAKE, 0, FAKE, None, ctypes.byref(ops)) == b.QG_ERR_INVALID_ARGUMENT
    assert lib.qgemm_calib_mfma_i8(FAKE, (1 << 20) + 1, FAKE, None, ctypes.byref(ops)) == b.QG_ERR_INVALID_ARGUMENT
    assert lib.qgemm_calib_mfma_i8(None, 10, FAKE, None, ctypes.byref(ops)) == b.QG_ERR_INVALID_ARGUMENT
    assert lib.qgemm_calib_mfma_i8(FAKE, 10, FAKE, None, None) == b.QG_ERR_INVALID_ARGUMENT
    for fn in (lib.qgemm_calib_mfma_f32, lib.qgemm_calib_mfma_bf16):
        assert fn(FAKE, 0, FAKE, None, ctypes.byref(ops)) == b.QG_ERR_INVALID_ARGUMENT
        assert fn(FAKE, (1 << 20) + 1, FAKE, None, ctypes.byref(ops)) == b.QG_ERR_INVALID_ARGUMENT
        assert fn(None, 10, FAKE, None, ctypes.byref(ops)) == b.QG_ERR_INVALID_ARGUMENT
        assert fn(FAKE, 10, None, None, ctypes.byref(ops)) == b.QG_ERR_INVALID_ARGUMENT
        assert fn(FAKE, 10, FAKE, None, None) == b.QG_ERR_INVALID_ARGUMENT


def test_a8w8_acc_and_row_zero_point_reject_bad_arguments():
    lib = b.lib
    # qgemm_a8w8_acc: NULL acc_in, ld_acc < N
    for acc, ld in ((None, 16), (FAKE, 15)):
        assert lib.qgemm_a8w8_acc(4, 16, 32, FAKE, 32, FAKE, 16, 0, acc, ld, FAKE, 4, FAKE, 16,
                                  FAKE, b.QG_FP32, 16, None, 0, None) == b.QG_ERR_INVALID_ARGUMENT
    # an empty output launches nothing, NULL pointers included
    assert lib.qgemm_a8w8_acc(0, 16, 32, None, 32, FAKE, 16, 0, None, 16, None, 0, FAKE, 16,
                              None, b.QG_FP32, 16, None, 0, None) == b.QG_OK
    assert lib.matmul_integer_row_zp(1, 0, 16, 32, None, b.QG_UINT8, 32, 0, FAKE, b.QG_INT8, 16, 0,
                                     None, 0, None, 0, None, 16, 0, None, 0, None) == b.QG_OK
    # the checks of qgemm_a8w8 still apply (act_scale length)
    assert lib.qgemm_a8w8_acc(4, 16, 32, FAKE, 32, FAKE, 16, 0, FAKE, 16, FAKE, 3, FAKE, 16,
                              FAKE, b.QG_FP32, 16, None, 0, None) == b.QG_ERR_INVALID_ARGUMENT
    # matmul_integer_row_zp: NULL zero points, a length other than 1 or M
    for za, n in ((None, 4), (FAKE, 3), (FAKE, 0)):
        assert lib.matmul_integer_row_zp(1, 4, 16, 32, FAKE, b.QG_UINT8, 32, 0, FAKE, b.QG_INT8, 16, 0,
                                         za, n, None, 0, FAKE, 16, 0, None, 0, None) == b.QG_ERR_INVALID_ARGUMENT


def test_w8a32_input_grad_rejects_bad_arguments():
    lib = b.lib
    ok = dict(M=4, N=16, K=8, dC=FAKE, lddc=16, W=FAKE, ldw=16, scale=0.5, zp=0, dA=FAKE, ldda=8)

    def call(**kw):
        a = dict(ok, **kw)
        return lib.qgemm_w8a32_input_grad(a["M"], a["N"], a["K"], a["dC"], a["lddc"], a["W"], a["ldw"],
                                          a["scale"], a["zp"], a["dA"], a["ldda"], None)
    for kw in (dict(N=0), dict(M=-1), dict(dC=None), dict(W=None), dict(dA=None), dict(lddc=15), dict(ldw=15),
               dict(ldda=7), dict(scale=float("inf")), dict(scale=float("nan"))):
        assert call(**kw) == b.QG_ERR_INVALID_ARGUMENT, kw
    # an empty dA ([M, K] with M or K zero) is a call with nothing to do
    for kw in (dict(M=0), dict(K=0), dict(M=0, dC=None, dA=None)):
        assert call(**kw) == b.QG_OK, kw
        assert q.last_kernel() == "none"
    with pytest.raises(ValueError):
        q.qgemm_w8a32_input_grad(torch.zeros(4, 16), torch.zeros(8, 15, dtype=torch.int8), 0.5)
    with pytest.raises(TypeError):
        q.qgemm_w8a32_input_grad(torch.zeros(4, 16), torch.zeros(8, 16), 0.5)


def test_dynamic_quantize_linear_rejects_bad_arguments():
    lib = b.lib
    ok = dict(n=16, x=FAKE, y=FAKE, sc=FAKE, zp=FAKE, ws=FAKE, wsz=8)

    def call(**kw):
        a = dict(ok, **kw)
        return lib.dynamic_quantize_linear(a["n"], a["x"], a["y"], a["sc"], a["zp"], a["ws"], a["wsz"], None)
    for kw in (dict(n=-1), dict(x=None), dict(y=None), dict(sc=None), dict(zp=None), dict(ws=None),
               dict(ws=ctypes.c_void_p(4100))):
        assert call(**kw) == b.QG_ERR_INVALID_ARGUMENT, kw
    assert call(wsz=7) == b.QG_ERR_WORKSPACE
    assert call(n=32769, wsz=8) == b.QG_ERR_WORKSPACE
    with pytest.raises(TypeError):
        q.dynamic_quantize_linear(torch.zeros(8, dtype=torch.float64))
    with pytest.raises(ValueError):
        q.dynamic_quantize_linear(torch.zeros(8))   # a CPU tensor


def _i64a(*v):
    return (ctypes.c_int64 * len(v))(*v)


def test_conv_integer_workspace_and_rejects(monkeypatch):
    lib = b.lib
    P0, S1, D1 = _i64a(0, 0, 0, 0), _i64a(1, 1), _i64a(1, 1)
    # 1 x 64 x 32 x 32 input, 128 x 64 x 3 x 3 weight, pad 1.  Implicit GEMM
    # (channels per group a multiple of 64): packed w (128 x 576), row sums
    # (128 int32), then the padded channel-minor input: 4 x 32 output tiles
    # read padded rows and columns 0..33, 64 channels each.
    P1 = _i64a(1, 1, 1, 1)
    assert lib.conv_integer_workspace_bytes(1, 64, 32, 32, 128, 3, 3, 1, P1, S1, D1) == \
        128 * 576 + 128 * 4 + 34 * 34 * 64
    # the im2col path: K = 576 (a multiple of 64), P = 1024; packed w
    # (128 x 576) + columns (576 x 1024)
    monkeypatch.setenv("QGEMM_CONV", "im2col")
    assert lib.conv_integer_workspace_bytes(1, 64, 32, 32, 128, 3, 3, 1, P1, S1, D1) == 128 * 576 + 576 * 1024
    monkeypatch.delenv("QGEMM_CONV")
    # K padded to 64, P padded to 16: C/group*kH*kW = 29*9 = 261 -> 320; P = 4*4 -> 16
    assert lib.conv_integer_workspace_bytes(1, 58, 7, 7, 6, 3, 3, 2, P1, _i64a(2, 2), D1) == \
        256 * ((2 * 3 * 320 + 255) // 256) + 2 * 320 * 16
    bad_geoms = [
        (0, 4, 5, 5, 4, 3, 3, 1, P0, S1, D1), (1, 4, 5, 5, 4, 3, 3, 3, P0, S1, D1),   # N = 0; group does not divide C
        (1, 4, 5, 5, 6, 3, 3, 4, P0, S1, D1),                                          # group does not divide M
        (1, 4, 2, 5, 4, 3, 3, 1, P0, S1, D1),                                          # window taller than the input
        (1, 4, 5, 5, 4, 3, 3, 1, _i64a(-1, 0, 0, 0), S1, D1), (1, 4, 5, 5, 4, 3, 3, 1, P0, _i64a(0, 1), D1),
        (1, 4, 5, 5, 4, 3, 3, 1, P0, S1, _i64a(1, 0)), (1, 4, 5, 5, 4, 3, 3, 1, None, S1, D1),
        (65536, 4, 5, 5, 4, 3, 3, 1, P0, S1, D1),
    ]
    for gm in bad_geoms:
        assert lib.conv_integer_workspace_bytes(*gm) == 0, gm
        assert lib.conv_integer(*gm[:4], FAKE, b.QG_UINT8, *gm[4:7], FAKE, b.QG_INT8, gm[7], gm[8], gm[9], gm[10],
                                0, None, 0, FAKE, ctypes.c_void_p(4096), 1 << 30, None) == b.QG_ERR_INVALID_ARGUMENT, gm
    ok = (1, 4, 5, 5, 4, 3, 3, 1)
    WS = ctypes.c_void_p(1 << 20)

    def call(**kw):
        a = dict(x=FAKE, xd=b.QG_UINT8, w=FAKE, wd=b.QG_INT8, xz=0, wz=None, wzl=0, y=FAKE, ws=WS, wsz=1 << 30)
        a.update(kw)
        return lib.conv_integer(*ok[:4], a["x"], a["xd"], *ok[4:7], a["w"], a["wd"], ok[7], P0, S1, D1, a["xz"],
                                a["wz"], a["wzl"], a["y"], a["ws"], a["wsz"], None)
    for kw in (dict(x=None), dict(w=None), dict(y=None), dict(ws=None), dict(ws=ctypes.c_void_p(4096 + 16)),
               dict(xd=b.QG_FP32), dict(wd=b.QG_BF16), dict(xz=256), dict(xz=-1), dict(xd=b.QG_INT8, xz=128),
               dict(wz=FAKE, wzl=2), dict(wz=None, wzl=1), dict(wz=FAKE, wzl=0)):
        assert call(**kw) == b.QG_ERR_INVALID_ARGUMENT, kw
    assert call(wsz=100) == b.QG_ERR_WORKSPACE
    with pytest.raises(TypeError):
        q.conv_integer(torch.zeros(1, 4, 5, 5), torch.zeros(4, 4, 3, 3, dtype=torch.int8))
    with pytest.raises(ValueError):
        q.conv_integer(torch.zeros(1, 4, 5, 5, dtype=torch.uint8), torch.zeros(4, 3, 3, 3, dtype=torch.int8))
    with pytest.raises(ValueError):
        q.conv_integer(torch.zeros(1, 4, 5, dtype=torch.uint8), torch.zeros(4, 4, 3, 3, dtype=torch.int8))

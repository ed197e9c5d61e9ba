"""ctypes binding of libqgemm.so: argument marshalling only.

Each function checks dtypes (TypeError) and shapes (ValueError), maps the
tensors to pointers, leading dimensions and batch strides, allocates the
output with torch on the tensors' device, and calls the C entry point of the
same name on torch's current stream.  All arithmetic runs in the HIP
kernels; there is no fallback.  If the library is missing, importing this
module raises.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqgemm.so")

QG_OK, QG_ERR_INVALID_ARGUMENT, QG_ERR_UNSUPPORTED, QG_ERR_WORKSPACE, QG_ERR_HIP = range(5)
QG_FP32, QG_BF16, QG_INT32, QG_INT8, QG_UINT8 = range(5)
QG_OP_W8A32, QG_OP_A8W8, QG_OP_MATMUL_INTEGER, QG_OP_DYNAMIC_QUANTIZE_LINEAR, QG_OP_W8A32_INPUT_GRAD = range(5)

_p, _i64, _i32, _int, _f32, _sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int,
                                   ctypes.c_float, ctypes.c_size_t)

# C prototypes, in the order of include/qgemm.h.
PROTOTYPES = {
    "qgemm_w8a32": ([_i64, _i64, _i64, _p, _i64, _p, _i64, _f32, _i32, _p, _i64, _p], _int),
    "qgemm_w8a32_input_grad": ([_i64, _i64, _i64, _p, _i64, _p, _i64, _f32, _i32, _p, _i64, _p], _int),
    "qgemm_w8a32_ws": ([_i64, _i64, _i64, _p, _i64, _p, _i64, _f32, _i32, _p, _i64, _p, _sz, _p], _int),
    "qgemm_w8a32_input_grad_ws": ([_i64, _i64, _i64, _p, _i64, _p, _i64, _f32, _i32, _p, _i64, _p, _sz, _p], _int),
    "qgemm_a8w8": ([_i64, _i64, _i64, _p, _i64, _p, _i64, _int, _p, _i64, _p, _i64,
                    _p, _int, _i64, _p, _sz, _p], _int),
    "matmul_integer": ([_i64, _i64, _i64, _i64, _p, _int, _i64, _i64, _p, _int, _i64, _i64,
                        _i32, _p, _i64, _p, _i64, _i64, _p, _sz, _p], _int),
    "qgemm_a8w8_noalloc": ([_i64, _i64, _i64, _p, _i64, _p, _i64, _int, _p, _i64, _p, _i64,
                            _p, _int, _i64, _p], _int),
    "qgemm_a8w8_acc": ([_i64, _i64, _i64, _p, _i64, _p, _i64, _int, _p, _i64, _p, _i64, _p, _i64,
                        _p, _int, _i64, _p, _sz, _p], _int),
    "matmul_integer_row_zp": ([_i64, _i64, _i64, _i64, _p, _int, _i64, _i64, _p, _int, _i64, _i64,
                               _p, _i64, _p, _i64, _p, _i64, _i64, _p, _sz, _p], _int),
    "dynamic_quantize_linear": ([_i64, _p, _p, _p, _p, _p, _sz, _p], _int),
    "conv_integer": ([_i64, _i64, _i64, _i64, _p, _int, _i64, _i64, _i64, _p, _int, _i64, _p, _p, _p,
                      _i32, _p, _i64, _p, _p, _sz, _p], _int),
    "conv_integer_workspace_bytes": ([_i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _p, _p, _p], _sz),
    "qgemm_workspace_bytes": ([_int, _i64, _i64, _i64, _i64], _sz),
    "qgemm_status_string": ([_int], ctypes.c_char_p),
    "qgemm_last_kernel": ([], ctypes.c_char_p),
    "qgemm_version": ([], ctypes.c_char_p),
    "qgemm_calib_read": ([_p, _sz, _p, _p], _int),
    "qgemm_calib_mfma_i8": ([_p, _int, _p, _p, ctypes.POINTER(ctypes.c_int64)], _int),
    "qgemm_calib_mfma_i8_32x32": ([_p, _int, _p, _p, ctypes.POINTER(ctypes.c_int64)], _int),
    "qgemm_calib_mfma_f32": ([_p, _int, _p, _p, ctypes.POINTER(ctypes.c_int64)], _int),
    "qgemm_calib_mfma_bf16": ([_p, _int, _p, _p, ctypes.POINTER(ctypes.c_int64)], _int),
}
QG_CALIB_SINK_WORDS = 8192


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                          "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (args, res) in PROTOTYPES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


lib = _load()


class QGemmError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {lib.qgemm_status_string(status).decode()} (status {status})")


def _check(status, where):
    if status == QG_OK:
        return
    if status == QG_ERR_INVALID_ARGUMENT:
        raise ValueError(f"{where}: invalid argument")
    if status == QG_ERR_UNSUPPORTED:
        raise NotImplementedError(f"{where}: unsupported form")
    raise QGemmError(status, where)


def status_string(status):
    return lib.qgemm_status_string(int(status)).decode()


def last_kernel():
    """Name of the kernel the calling thread's last successful call launched."""
    return lib.qgemm_last_kernel().decode()


def version():
    return lib.qgemm_version().decode()


def workspace_bytes(op, batch, M, N, K):
    return int(lib.qgemm_workspace_bytes(int(op), batch, M, N, K))


def _need(t, dtypes, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}; expected one of {dtypes}")


def _on_gpu(*ts):
    dev = ts[0].device
    for t in ts:
        if t.device.type != "cuda":
            raise ValueError("tensors must be on a GPU device")
        if t.device != dev:
            raise ValueError("tensors must be on the same device")
    return dev


def _rows(t, name):
    """Leading dimension of a row-major 2-D view with unit column stride."""
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if t.stride(1) != 1 and t.size(1) > 1:
        raise ValueError(f"{name} must have unit column stride")
    return max(t.stride(0), t.size(1)) if t.size(0) > 1 else t.size(1)


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


# ---------------------------------------------------------------------------
# W8A32
# ---------------------------------------------------------------------------

def qgemm_w8a32(A, W, scale, zero_point=0, out=None, workspace=None):
    """C = A @ ((W - zero_point) * scale) with the dequantisation folded in.

    A: fp32 [M, K]; W: int8 [K, N]; scale: Python float (per tensor);
    zero_point: Python int (per tensor, default 0).  Returns fp32 [M, N].
    workspace: None (a cached, zeroed buffer per device and stream) or a
    zero-filled uint8 tensor of at least workspace_bytes(QG_OP_W8A32, 1, M,
    N, K) bytes; it lets small outputs divide K among workgroups.
    """
    _need(A, (torch.float32,), "A")
    _need(W, (torch.int8,), "W")
    if A.dim() != 2 or W.dim() != 2:
        raise ValueError("A and W must be 2-D")
    M, K = A.shape
    K2, N = W.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: A is {tuple(A.shape)}, W is {tuple(W.shape)}")
    dev = _on_gpu(A, W)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=dev)
    else:
        _need(out, (torch.float32,), "out")
        if tuple(out.shape) != (M, N):
            raise ValueError("out has the wrong shape")
    ws = _w8a32_workspace(dev, workspace, QG_OP_W8A32, M, N, K)
    st = lib.qgemm_w8a32_ws(M, N, K, _ptr(A), _rows(A, "A"), _ptr(W), _rows(W, "W"),
                            float(scale), int(zero_point), _ptr(out), _rows(out, "out"),
                            _ptr(ws), 0 if ws is None else ws.numel(), _stream(dev))
    _check(st, "qgemm_w8a32_ws")
    return out


def _w8a32_workspace(dev, workspace, op, M, N, K):
    if workspace is not None:
        _need(workspace, (torch.uint8, torch.int8), "workspace")
        return workspace
    return _workspace(dev, workspace_bytes(op, 1, M, N, K))




def qgemm_w8a32_input_grad(dC, W, scale, zero_point=0, out=None, workspace=None):
    """dA = dC @ ((W - zero_point) * scale)^T: the gradient of qgemm_w8a32
    with respect to its activations, W in its forward [K, N] layout.

    dC: fp32 [M, N]; W: int8 [K, N]; returns fp32 [M, K].  workspace: as in
    qgemm_w8a32, sized by workspace_bytes(QG_OP_W8A32_INPUT_GRAD, 1, M, N, K).
    """
    _need(dC, (torch.float32,), "dC")
    _need(W, (torch.int8,), "W")
    if dC.dim() != 2 or W.dim() != 2:
        raise ValueError("dC and W must be 2-D")
    M, N = dC.shape
    K, N2 = W.shape
    if N != N2:
        raise ValueError(f"dC is {tuple(dC.shape)} but W is {tuple(W.shape)}; both need N columns")
    dev = _on_gpu(dC, W)
    if out is None:
        out = torch.empty((M, K), dtype=torch.float32, device=dev)
    else:
        _need(out, (torch.float32,), "out")
        if tuple(out.shape) != (M, K):
            raise ValueError("out has the wrong shape")
    ws = _w8a32_workspace(dev, workspace, QG_OP_W8A32_INPUT_GRAD, M, N, K)
    st = lib.qgemm_w8a32_input_grad_ws(M, N, K, _ptr(dC), _rows(dC, "dC"), _ptr(W), _rows(W, "W"),
                                       float(scale), int(zero_point), _ptr(out), _rows(out, "out"),
                                       _ptr(ws), 0 if ws is None else ws.numel(), _stream(dev))
    _check(st, "qgemm_w8a32_input_grad_ws")
    return out
# ---------------------------------------------------------------------------
# A8W8
# ---------------------------------------------------------------------------

_workspaces = {}


def _workspace(dev, nbytes):
    """A zero-filled workspace per (device, stream); the library leaves it zeroed."""
    if nbytes == 0:
        return None
    key = (dev, torch.cuda.current_stream(dev).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
        _workspaces[key] = ws
    return ws


def _act_scale(s, M):
    """act_scale as [M] / [M,1] / [1] / scalar -> (contiguous fp32, length).

    A rank-1 [M] act_scale scales rows, never columns (also when M == N)."""
    _need(s, (torch.float32,), "act_scale")
    if s.dim() == 0 or (s.dim() == 1 and s.numel() in (1, M)) or (s.dim() == 2 and s.shape[1] == 1
                                                                   and s.shape[0] in (1, M)):
        flat = s.reshape(-1).contiguous()
        return flat, flat.numel()
    raise ValueError(f"act_scale of shape {tuple(s.shape)} is not [M], [M,1] or scalar (M={M})")


def _weight_scale(s, N):
    _need(s, (torch.float32,), "weight_scale")
    if s.dim() == 0 or (s.dim() == 1 and s.numel() in (1, N)) or (s.dim() == 2 and s.shape[0] == 1
                                                                   and s.shape[1] in (1, N)):
        flat = s.reshape(-1).contiguous()
        return flat, flat.numel()
    raise ValueError(f"weight_scale of shape {tuple(s.shape)} is not [N], [1,N] or scalar (N={N})")


def qgemm_a8w8(A, W, act_scale, weight_scale, out_dtype=torch.float32, b_trans=False, out=None,
               workspace=None):
    """out = cast(((float)(A @ W)_int32 * act_scale[m]) * weight_scale[n]).

    A: int8 [M, K]; W: int8 [K, N] (or [N, K] with b_trans=True);
    act_scale: fp32 [M], [M, 1] or scalar; weight_scale: fp32 [N], [1, N] or
    scalar; out_dtype: torch.float32 (default) or torch.bfloat16.
    """
    return _a8w8(None, A, W, act_scale, weight_scale, out_dtype, b_trans, out, workspace)


def qgemm_a8w8_noalloc(A, W, act_scale, weight_scale, out_dtype=torch.float32, b_trans=False, out=None):
    """qgemm_a8w8 through the C entry point that allocates nothing: the
    decode split-K scratch is the library's static device array (shared by
    every call on the GPU; overlapping calls race).  Pass `out` to keep the
    call itself free of allocations."""
    return _a8w8(None, A, W, act_scale, weight_scale, out_dtype, b_trans, out, None, noalloc=True)


def qgemm_a8w8_acc(acc_in, A, W, act_scale, weight_scale, out_dtype=torch.float32, b_trans=False, out=None,
                   workspace=None):
    """out = cast(((float)(acc_in + A @ W)_int32 * act_scale[m]) * weight_scale[n]).

    acc_in: int32 [M, N] (unit column stride), added to the int8 product
    (wrapping) before the cast.  Other arguments as qgemm_a8w8.
    """
    _need(acc_in, (torch.int32,), "acc_in")
    return _a8w8(acc_in, A, W, act_scale, weight_scale, out_dtype, b_trans, out, workspace)


def _a8w8(acc_in, A, W, act_scale, weight_scale, out_dtype, b_trans, out, workspace, noalloc=False):
    _need(A, (torch.int8,), "A")
    _need(W, (torch.int8,), "W")
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out_dtype must be torch.float32 or torch.bfloat16")
    if A.dim() != 2 or W.dim() != 2:
        raise ValueError("A and W must be 2-D")
    M, K = A.shape
    N, K2 = (W.shape[0], W.shape[1]) if b_trans else (W.shape[1], W.shape[0])
    if K != K2:
        raise ValueError(f"inner dimensions differ: A is {tuple(A.shape)}, W is {tuple(W.shape)}")
    s_a, n_a = _act_scale(act_scale, M)
    s_w, n_w = _weight_scale(weight_scale, N)
    if acc_in is not None and tuple(acc_in.shape) != (M, N):
        raise ValueError(f"acc_in must be [M, N] = [{M}, {N}]")
    dev = _on_gpu(*([A, W, s_a, s_w] + ([acc_in] if acc_in is not None else [])))
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=dev)
    else:
        _need(out, (out_dtype,), "out")
        if tuple(out.shape) != (M, N):
            raise ValueError("out has the wrong shape")
    od = QG_FP32 if out_dtype == torch.float32 else QG_BF16
    if noalloc:
        st = lib.qgemm_a8w8_noalloc(M, N, K, _ptr(A), _rows(A, "A"), _ptr(W), _rows(W, "W"), int(bool(b_trans)),
                                    _ptr(s_a), n_a, _ptr(s_w), n_w, _ptr(out), od, _rows(out, "out"),
                                    _stream(dev))
        _check(st, "qgemm_a8w8_noalloc")
        return out
    if workspace is None:
        ws = _workspace(dev, workspace_bytes(QG_OP_A8W8, 1, M, N, K))
    else:
        ws = workspace
    wsz = 0 if ws is None else ws.numel()
    if acc_in is None:
        st = lib.qgemm_a8w8(M, N, K, _ptr(A), _rows(A, "A"), _ptr(W), _rows(W, "W"), int(bool(b_trans)),
                            _ptr(s_a), n_a, _ptr(s_w), n_w, _ptr(out), od, _rows(out, "out"),
                            _ptr(ws), wsz, _stream(dev))
        _check(st, "qgemm_a8w8")
    else:
        st = lib.qgemm_a8w8_acc(M, N, K, _ptr(A), _rows(A, "A"), _ptr(W), _rows(W, "W"), int(bool(b_trans)),
                                _ptr(acc_in), _rows(acc_in, "acc_in"),
                                _ptr(s_a), n_a, _ptr(s_w), n_w, _ptr(out), od, _rows(out, "out"),
                                _ptr(ws), wsz, _stream(dev))
        _check(st, "qgemm_a8w8_acc")
    return out


# ---------------------------------------------------------------------------
# MatMulInteger
# ---------------------------------------------------------------------------

_QG_OF = {torch.uint8: QG_UINT8, torch.int8: QG_INT8}


def _batch_view(t, name, batch_shape):
    """(batch stride, leading dim) of t broadcast to batch_shape + t.shape[-2:]."""
    lead = t.shape[:-2]
    if all(d == 1 for d in lead):
        return 0
    if tuple(lead) != tuple(batch_shape):
        # a size-1 batch broadcast against a larger one is covered above; any
        # other mismatch would need a per-dimension stride the ABI lacks
        raise ValueError(f"{name} batch dimensions {tuple(lead)} do not match {tuple(batch_shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous when batched")
    return t.shape[-2] * t.shape[-1]


def matmul_integer(A, B, a_zero_point=0, b_zero_point=None, out=None, workspace=None):
    """ONNX MatMulInteger: int32 wrap(sum_k (A - a_zp) * (B - b_zp)).

    A: uint8/int8 of rank 2-4, [..., M, K]; B: uint8/int8 of rank 2-4,
    [..., K, N].  A rank-2 B, or one whose batch dimensions are all 1, is
    shared by every batch without a copy; a size-1 batch of A is likewise
    reused.  a_zero_point: scalar of A's range, or a tensor of A's dtype
    with M per-row values ([M] or [M, 1]; calls matmul_integer_row_zp);
    b_zero_point: None, scalar, [N] or [..., 1, N] per-column values of B's
    dtype.  Returns int32 [*batch, M, N].  workspace: None (a cached,
    zeroed buffer per device and stream) or a zero-filled uint8 tensor of at
    least workspace_bytes(QG_OP_MATMUL_INTEGER, batch, M, N, K) bytes, which
    calls on one stream may share.
    """
    _need(A, (torch.uint8, torch.int8), "A")
    _need(B, (torch.uint8, torch.int8), "B")
    if not (2 <= A.dim() <= 4 and 2 <= B.dim() <= 4):
        raise ValueError("MatMulInteger operands must have rank 2 to 4")
    M, K = A.shape[-2:]
    K2, N = B.shape[-2:]
    if K != K2:
        raise ValueError(f"inner dimensions differ: A is {tuple(A.shape)}, B is {tuple(B.shape)}")
    za_rows = None
    if isinstance(a_zero_point, torch.Tensor):
        _need(a_zero_point, (A.dtype,), "a_zero_point")
        if a_zero_point.numel() == 1 and a_zero_point.dim() == 0:
            a_zero_point = int(a_zero_point.item())
        elif a_zero_point.numel() == 1:
            # one value for every row, read on the device (no host round trip)
            za_rows = a_zero_point.reshape(-1).contiguous()
        else:
            if a_zero_point.numel() != M or (a_zero_point.dim() == 2 and a_zero_point.shape[1] != 1) \
                    or a_zero_point.dim() > 2:
                raise ValueError(f"a per-row a_zero_point must be [M] or [M, 1] with M={M}")
            za_rows = a_zero_point.reshape(-1).contiguous()
    zb, zb_len = None, 0
    if b_zero_point is not None:
        if isinstance(b_zero_point, torch.Tensor):
            _need(b_zero_point, (B.dtype,), "b_zero_point")
            if b_zero_point.numel() not in (1, N):
                raise ValueError(f"b_zero_point has {b_zero_point.numel()} values; expected 1 or N={N}")
            if b_zero_point.dim() >= 2 and b_zero_point.shape[-2] != 1:
                raise ValueError("a per-column b_zero_point must have shape [..., 1, N]")
            zb = b_zero_point.reshape(-1).contiguous()
        else:
            zb = torch.tensor([int(b_zero_point)], dtype=B.dtype, device=B.device)
        zb_len = zb.numel()
    batch_shape = torch.broadcast_shapes(A.shape[:-2], B.shape[:-2])
    batch = 1
    for d in batch_shape:
        batch *= d
    a_bs = _batch_view(A, "A", batch_shape)
    b_bs = _batch_view(B, "B", batch_shape)
    A2 = A.reshape(-1, A.shape[-1]) if a_bs else A.reshape(A.shape[-2:])
    B2 = B.reshape(-1, B.shape[-1]) if b_bs else B.reshape(B.shape[-2:])
    dev = _on_gpu(*([A, B] + ([zb] if zb is not None else []) + ([za_rows] if za_rows is not None else [])))
    if out is None:
        out = torch.empty(tuple(batch_shape) + (M, N), dtype=torch.int32, device=dev)
    else:
        _need(out, (torch.int32,), "out")
        if tuple(out.shape) != tuple(batch_shape) + (M, N) or not out.is_contiguous():
            raise ValueError("out has the wrong shape or is not contiguous")
    if workspace is None:
        ws = _workspace(dev, workspace_bytes(QG_OP_MATMUL_INTEGER, batch, M, N, K))
    else:
        _need(workspace, (torch.uint8, torch.int8), "workspace")
        ws = workspace
    wsz = 0 if ws is None else ws.numel()
    if za_rows is None:
        st = lib.matmul_integer(batch, M, N, K,
                                _ptr(A2), _QG_OF[A.dtype], _rows(A2, "A"), a_bs,
                                _ptr(B2), _QG_OF[B.dtype], _rows(B2, "B"), b_bs,
                                int(a_zero_point), _ptr(zb), zb_len,
                                _ptr(out), N, M * N, _ptr(ws), wsz, _stream(dev))
        _check(st, "matmul_integer")
    else:
        st = lib.matmul_integer_row_zp(batch, M, N, K,
                                       _ptr(A2), _QG_OF[A.dtype], _rows(A2, "A"), a_bs,
                                       _ptr(B2), _QG_OF[B.dtype], _rows(B2, "B"), b_bs,
                                       _ptr(za_rows), za_rows.numel(), _ptr(zb), zb_len,
                                       _ptr(out), N, M * N, _ptr(ws), wsz, _stream(dev))
        _check(st, "matmul_integer_row_zp")
    return out


def matmul_integer_row_zp(A, B, a_zero_point, b_zero_point=None, out=None, workspace=None):
    """MatMulInteger with one activation zero point per row of A
    (a_zero_point: [M] or [M, 1] of A's dtype); see matmul_integer."""
    if not isinstance(a_zero_point, torch.Tensor) or a_zero_point.dim() == 0:
        raise ValueError("a_zero_point must be a tensor of M per-row values")
    return matmul_integer(A, B, a_zero_point, b_zero_point, out, workspace)


# ---------------------------------------------------------------------------
# ConvInteger
# ---------------------------------------------------------------------------

def _i64x(vals):
    arr = (ctypes.c_int64 * len(vals))(*[int(v) for v in vals])
    return arr


def _auto_pads(auto_pad, sizes, kernel, strides, dilations):
    """ONNX auto_pad: explicit (begin..., end...) pads for SAME_UPPER /
    SAME_LOWER / VALID."""
    begins, ends = [], []
    for size, k, st, d in zip(sizes, kernel, strides, dilations):
        if auto_pad == "VALID":
            begins.append(0)
            ends.append(0)
            continue
        out = -(-size // st)
        total = max(0, (out - 1) * st + (k - 1) * d + 1 - size)
        lo = total // 2 if auto_pad == "SAME_UPPER" else total - total // 2
        begins.append(lo)
        ends.append(total - lo)
    return begins + ends


def conv_integer(x, w, x_zero_point=0, w_zero_point=None, pads=None, strides=None, dilations=None, group=1,
                 auto_pad="NOTSET", out=None, workspace=None):
    """ONNX ConvInteger on the GPU: int32 y = sum (x - x_zp)(w - w_zp[m]) over
    each output channel's group, taps outside the input contributing nothing.

    x: uint8/int8 [N, C, H, W] (or [N, C, L]); w: uint8/int8
    [M, C/group, kH, kW] (or [M, C/group, kL]).  pads in ONNX order
    (begins then ends: top, left, bottom, right; or left, right), strides and
    dilations per spatial axis, auto_pad NOTSET / SAME_UPPER / SAME_LOWER /
    VALID.  x_zero_point: a scalar (int or one-element tensor of x's dtype);
    w_zero_point: None, a scalar, or M values of w's dtype.
    Returns int32 [N, M, OH, OW] (or [N, M, OL])."""
    _need(x, (torch.uint8, torch.int8), "x")
    _need(w, (torch.uint8, torch.int8), "w")
    if x.dim() not in (3, 4) or w.dim() != x.dim():
        raise ValueError("ConvInteger takes rank-3 (NCL) or rank-4 (NCHW) x and w of the same rank")
    if not x.is_contiguous() or not w.is_contiguous():
        raise ValueError("x and w must be contiguous")
    nsp = x.dim() - 2
    strides = list(strides) if strides is not None else [1] * nsp
    dilations = list(dilations) if dilations is not None else [1] * nsp
    if len(strides) != nsp or len(dilations) != nsp:
        raise ValueError("strides and dilations need one value per spatial axis")
    if auto_pad not in ("NOTSET", "SAME_UPPER", "SAME_LOWER", "VALID"):
        raise ValueError(f"unknown auto_pad {auto_pad!r}")
    if auto_pad != "NOTSET":
        pads = _auto_pads(auto_pad, x.shape[2:], w.shape[2:], strides, dilations)
    pads = list(pads) if pads is not None else [0] * (2 * nsp)
    if len(pads) != 2 * nsp:
        raise ValueError("pads need a begin and an end per spatial axis")
    if nsp == 1:
        N, C, L = x.shape
        M, Cg, kL = w.shape
        dims = (N, C, 1, L, M, 1, kL)
        pads4, strides2, dil2 = [0, pads[0], 0, pads[1]], [1, strides[0]], [1, dilations[0]]
    else:
        N, C, H, W = x.shape
        M, Cg, kH, kW = w.shape
        dims = (N, C, H, W, M, kH, kW)
        pads4, strides2, dil2 = pads, strides, dilations
    if Cg * group != C or M % group != 0:
        raise ValueError(f"w has {Cg} input channels per group; x has {C} channels in {group} groups")
    if isinstance(x_zero_point, torch.Tensor):
        _need(x_zero_point, (x.dtype,), "x_zero_point")
        if x_zero_point.numel() != 1:
            raise ValueError("x_zero_point must be a scalar")
        x_zero_point = int(x_zero_point.item())
    zw, zw_len = None, 0
    if w_zero_point is not None:
        if isinstance(w_zero_point, torch.Tensor):
            _need(w_zero_point, (w.dtype,), "w_zero_point")
            if w_zero_point.numel() not in (1, M):
                raise ValueError(f"w_zero_point has {w_zero_point.numel()} values; expected 1 or M={M}")
            zw = w_zero_point.reshape(-1).contiguous()
        else:
            zw = torch.tensor([int(w_zero_point)], dtype=w.dtype, device=w.device)
        zw_len = zw.numel()
    dev = _on_gpu(*([x, w] + ([zw] if zw is not None else [])))
    p4, s2, d2 = _i64x(pads4), _i64x(strides2), _i64x(dil2)
    need = lib.conv_integer_workspace_bytes(*dims, group, p4, s2, d2)
    if need == 0:
        raise ValueError("these sizes do not describe a valid convolution")
    OH = (dims[2] + pads4[0] + pads4[2] - dil2[0] * (dims[5] - 1) - 1) // strides2[0] + 1
    OW = (dims[3] + pads4[1] + pads4[3] - dil2[1] * (dims[6] - 1) - 1) // strides2[1] + 1
    shape = (N, M, OW) if nsp == 1 else (N, M, OH, OW)
    if out is None:
        out = torch.empty(shape, dtype=torch.int32, device=dev)
    else:
        _need(out, (torch.int32,), "out")
        if tuple(out.shape) != shape or not out.is_contiguous():
            raise ValueError(f"out must be a contiguous int32 tensor of shape {shape}")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    else:
        _need(workspace, (torch.uint8, torch.int8), "workspace")
    st = lib.conv_integer(*dims[:4], _ptr(x), _QG_OF[x.dtype], *dims[4:], _ptr(w), _QG_OF[w.dtype], group,
                          p4, s2, d2, int(x_zero_point), _ptr(zw), zw_len, _ptr(out),
                          _ptr(workspace), workspace.numel(), _stream(dev))
    _check(st, "conv_integer")
    return out


# ---------------------------------------------------------------------------
# DynamicQuantizeLinear (uint8)
# ---------------------------------------------------------------------------

_dql_workspaces = {}


def dynamic_quantize_linear(x, out=None, workspace=None):
    """ONNX DynamicQuantizeLinear to uint8 on the GPU.

    x: float32 tensor of any shape (contiguous).  Returns (y, scale, zero_point):
    y uint8 of x's shape, scale a 0-d float32 tensor and zero_point a 0-d uint8
    tensor, all on x's device (no host round trip: zero_point can go straight
    to matmul_integer_row_zp).  The min/max partials live in a workspace of
    their own per (device, stream) unless one is passed."""
    _need(x, (torch.float32,), "x")
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    dev = _on_gpu(x)
    n = x.numel()
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=dev)
    else:
        _need(out, (torch.uint8,), "out")
        if tuple(out.shape) != tuple(x.shape) or not out.is_contiguous():
            raise ValueError("out must be a contiguous uint8 tensor of x's shape")
    scale = torch.empty((), dtype=torch.float32, device=dev)
    zp = torch.empty((), dtype=torch.uint8, device=dev)
    need = workspace_bytes(QG_OP_DYNAMIC_QUANTIZE_LINEAR, 1, 1, n, 1)
    if workspace is None:
        key = (dev, torch.cuda.current_stream(dev).cuda_stream)
        ws = _dql_workspaces.get(key)
        if ws is None or ws.numel() < need:
            ws = torch.empty(max(need, 8192), dtype=torch.uint8, device=dev)
            _dql_workspaces[key] = ws
    else:
        _need(workspace, (torch.uint8, torch.int8), "workspace")
        ws = workspace
    st = lib.dynamic_quantize_linear(n, _ptr(x) if n else None, _ptr(out) if n else None, _ptr(scale), _ptr(zp),
                                     _ptr(ws), ws.numel(), _stream(dev))
    _check(st, "dynamic_quantize_linear")
    return out, scale, zp


# ---------------------------------------------------------------------------
# Calibration (roofline ceilings; no part of the matmuls)
# ---------------------------------------------------------------------------

def _sink(dev, sink):
    if sink is None:
        return torch.empty(QG_CALIB_SINK_WORDS, dtype=torch.int32, device=dev)
    _need(sink, (torch.int32,), "sink")
    if sink.numel() < QG_CALIB_SINK_WORDS or not sink.is_contiguous():
        raise ValueError(f"sink must be a contiguous int32 tensor of >= {QG_CALIB_SINK_WORDS} words")
    return sink


def calib_read(buf, sink=None):
    """Read every byte of the contiguous GPU tensor `buf` once (a streaming
    read for the HBM ceiling).  Returns the sink tensor."""
    if not isinstance(buf, torch.Tensor) or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous tensor")
    dev = _on_gpu(buf)
    sink = _sink(dev, sink)
    nbytes = buf.numel() * buf.element_size()
    _check(lib.qgemm_calib_read(_ptr(buf), nbytes, _ptr(sink), _stream(dev)), "qgemm_calib_read")
    return sink


def calib_mfma_i8(operands, iters, sink=None, shape="16x16x64"):
    """Run `iters` rounds of int8 matrix-core multiplies on the 4096 operand
    bytes in `operands` (an int8 or uint8 GPU tensor), as
    v_mfma_i32_16x16x64_i8 (shape "16x16x64") or v_mfma_i32_32x32x32_i8
    ("32x32x32").  Returns the number of int8 operations the launch
    performs (the same for both shapes)."""
    _need(operands, (torch.int8, torch.uint8), "operands")
    if operands.numel() != 4096 or not operands.is_contiguous():
        raise ValueError("operands must be 4096 contiguous bytes")
    if shape not in ("16x16x64", "32x32x32"):
        raise ValueError("shape must be 16x16x64 or 32x32x32")
    dev = _on_gpu(operands)
    sink = _sink(dev, sink)
    ops = ctypes.c_int64(0)
    fn = lib.qgemm_calib_mfma_i8 if shape == "16x16x64" else lib.qgemm_calib_mfma_i8_32x32
    _check(fn(_ptr(operands), int(iters), _ptr(sink), _stream(dev), ctypes.byref(ops)), fn.__name__)
    return int(ops.value)


def calib_mfma_f32(operands, iters, sink=None):
    """Run `iters` rounds of fp32 matrix-core multiplies on the 1024 float32
    operands in `operands` (values in [-1, 1]).  Returns the number of
    floating-point operations the launch performs."""
    _need(operands, (torch.float32,), "operands")
    if operands.numel() != 1024 or not operands.is_contiguous():
        raise ValueError("operands must be 1024 contiguous float32 values")
    dev = _on_gpu(operands)
    sink = _sink(dev, sink)
    flops = ctypes.c_int64(0)
    _check(lib.qgemm_calib_mfma_f32(_ptr(operands), int(iters), _ptr(sink), _stream(dev), ctypes.byref(flops)),
           "qgemm_calib_mfma_f32")
    return int(flops.value)


def calib_mfma_bf16(operands, iters, sink=None):
    """Run `iters` rounds of bf16 matrix-core multiplies on the 2048 bfloat16
    operands in `operands` (values in [-1, 1]).  Returns the number of
    floating-point operations the launch performs."""
    _need(operands, (torch.bfloat16,), "operands")
    if operands.numel() != 2048 or not operands.is_contiguous():
        raise ValueError("operands must be 2048 contiguous bfloat16 values")
    dev = _on_gpu(operands)
    sink = _sink(dev, sink)
    flops = ctypes.c_int64(0)
    _check(lib.qgemm_calib_mfma_bf16(_ptr(operands), int(iters), _ptr(sink), _stream(dev), ctypes.byref(flops)),
           "qgemm_calib_mfma_bf16")
    return int(flops.value)

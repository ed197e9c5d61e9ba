"""CPU oracle for the quantised matrix multiplies -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path never does, and this
package imports nothing from the product package.

Each function computes the plain definition from the pages (cited per
function) with numpy arrays in and out, by calling the plain C loops in
``oracle.c`` (built into ``liboracle.so`` by ``oracle/build.py``):

* ``w8a32``: the naive dequantise-then-matmul form of the W8A32 operator
  ("feat(PULPOpen): matmul that dequantises an int8 weight in-kernel", intro
  and "The kernel"), in double precision, with the tolerance scale
  ``|scale| * sum_k |a| |b - zp|``.
* ``a8w8`` / ``a8w8_at``: int8 x int8 accumulated exactly and wrapped to
  int32, cast to fp32, times act_scale[m], times weight_scale[n], cast to the
  output type ("Feature/a8w8 matmul dequant fusion", sequence diagram and
  "What Changed").
* ``matmul_integer`` / ``matmul_integer_at``: ONNX MatMulInteger with scalar
  or per-column zero points, ranks 2-4 and a shared B
  ("feat(onnx-to-hip): lower quantized integer conv and matmul", "What").
* ``dot_f32acc``: the f32-accumulator form that page selects only while
  65025*K fits fp32's 24-bit mantissa (used to pin that bound).
* ``f32_to_bf16``: round-to-nearest-even conversion to bfloat16 bits.
* ``dynamic_quantize_linear``: ONNX DynamicQuantizeLinear to uint8 as the
  onnx-to-hip page lowers it.
* ``conv_integer``: ONNX ConvInteger (NCHW / NCL, groups, padding, strides,
  dilations, scalar activation and per-channel weight zero points).
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(HERE, "liboracle.so")
_lib = None

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_int = ctypes.c_int
_f32 = ctypes.c_float


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build_oracle()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_f32_to_bf16.argtypes = [_f32]
    lib.oracle_f32_to_bf16.restype = ctypes.c_uint16
    lib.oracle_w8a32.argtypes = [_i64, _i64, _i64, _p, _i64, _p, _i64, _f32, _i32, _p, _p]
    lib.oracle_w8a32.restype = None
    lib.oracle_w8a32_input_grad.argtypes = [_i64, _i64, _i64, _p, _i64, _p, _i64, _f32, _i32, _p, _p]
    lib.oracle_w8a32_input_grad.restype = None
    lib.oracle_a8w8.argtypes = [_i64, _i64, _i64, _p, _i64, _p, _i64, _int,
                                _p, _i64, _p, _i64, _p, _p, _p]
    lib.oracle_a8w8.restype = None
    lib.oracle_a8w8_at.argtypes = [_i64, _i64, _i64, _p, _i64, _p, _i64, _int,
                                   _p, _i64, _p, _i64, _i64, _p, _p, _p, _p, _p]
    lib.oracle_a8w8_at.restype = None
    lib.oracle_a8w8_acc.argtypes = [_i64, _i64, _i64, _p, _i64, _p, _i64, _int, _p, _i64,
                                    _p, _i64, _p, _i64, _p, _p, _p]
    lib.oracle_a8w8_acc.restype = None
    lib.oracle_matmul_integer_rows.argtypes = [_i64, _i64, _i64, _i64,
                                               _p, _int, _i64, _i64,
                                               _p, _int, _i64, _i64,
                                               _p, _i64, _p, _i64, _p, _i64, _i64]
    lib.oracle_matmul_integer_rows.restype = None
    lib.oracle_matmul_integer.argtypes = [_i64, _i64, _i64, _i64,
                                          _p, _int, _i64, _i64,
                                          _p, _int, _i64, _i64,
                                          _i32, _p, _i64, _p, _i64, _i64]
    lib.oracle_matmul_integer.restype = None
    lib.oracle_matmul_integer_at.argtypes = [_i64, _p, _int, _i64, _i64,
                                             _p, _int, _i64, _i64,
                                             _i32, _p, _i64, _i64, _p, _p, _p, _p]
    lib.oracle_matmul_integer_at.restype = None
    lib.oracle_dot_f32acc.argtypes = [_i64, _p, _int, _p, _int, _i64, _i32, _i32]
    lib.oracle_dot_f32acc.restype = _i32
    lib.oracle_dynamic_quantize_linear.argtypes = [_i64, _p, _p, _p, _p]
    lib.oracle_dynamic_quantize_linear.restype = None
    lib.oracle_conv_integer.argtypes = [_i64, _i64, _i64, _i64, _p, _int, _i64, _i64, _i64, _p, _int, _i64,
                                        _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i32, _p, _i64, _p]
    lib.oracle_conv_integer.restype = None
    lib.oracle_threads.argtypes = []
    lib.oracle_threads.restype = _int
    _lib = lib
    return lib


def threads():
    """OpenMP threads the oracle's loops run on."""
    return int(_load().oracle_threads())


def set_threads(n):
    """Run the oracle's loops on n OpenMP threads from now on."""
    lib = _load()
    lib.oracle_set_threads.argtypes = [_int]
    lib.oracle_set_threads.restype = None
    lib.oracle_set_threads(int(n))


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------------------
# bfloat16
# ---------------------------------------------------------------------------

def f32_to_bf16(x):
    """bfloat16 bit patterns (uint16) of fp32 values, round to nearest even."""
    lib = _load()
    x = np.asarray(x, dtype=np.float32)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint16)
    for i in range(flat.size):
        out[i] = lib.oracle_f32_to_bf16(float(flat[i]))
    return out.reshape(x.shape)


def bf16_bits_to_f32(bits):
    """Widen bfloat16 bit patterns to fp32 (exact)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------------------
# W8A32
# ---------------------------------------------------------------------------

def w8a32(A, W, scale, zero_point):
    """R = A @ ((W - zp) * scale) in double, plus the tolerance scale.

    A: fp32 [M,K]; W: int8 [K,N]; scale: fp32 value; zero_point: integer.
    Returns (R float64 [M,N], bound float64 [M,N]).
    """
    lib = _load()
    A = _c(A, np.float32)
    W = _c(W, np.int8)
    M, K = A.shape
    K2, N = W.shape
    assert K == K2
    R = np.empty((M, N), dtype=np.float64)
    B = np.empty((M, N), dtype=np.float64)
    lib.oracle_w8a32(M, N, K, _ptr(A), K, _ptr(W), N, float(np.float32(scale)),
                     int(zero_point), _ptr(R), _ptr(B))
    return R, B


def w8a32_input_grad(dC, W, scale, zero_point):
    """Gradient of the W8A32 matmul with respect to its activations:
    R = dC @ ((W - zp) * scale)^T in double, plus the tolerance scale.

    dC: fp32 [M,N]; W: int8 [K,N] (the forward weight); returns
    (R float64 [M,K], bound float64 [M,K]).
    """
    lib = _load()
    dC = _c(dC, np.float32)
    W = _c(W, np.int8)
    M, N = dC.shape
    K, N2 = W.shape
    assert N == N2
    R = np.empty((M, K), dtype=np.float64)
    B = np.empty((M, K), dtype=np.float64)
    lib.oracle_w8a32_input_grad(M, N, K, _ptr(dC), N, _ptr(W), N, float(np.float32(scale)),
                                int(zero_point), _ptr(R), _ptr(B))
    return R, B


# ---------------------------------------------------------------------------
# A8W8
# ---------------------------------------------------------------------------

def _scales(act_scale, weight_scale, M, N):
    a = _c(np.asarray(act_scale, dtype=np.float32).reshape(-1), np.float32)
    w = _c(np.asarray(weight_scale, dtype=np.float32).reshape(-1), np.float32)
    assert a.size in (1, M) and w.size in (1, N)
    return a, w


def a8w8(A, W, act_scale, weight_scale, b_trans=False):
    """Full A8W8 result.  A int8 [M,K]; W int8 [K,N] (or [N,K] if b_trans).

    act_scale: 1 or M values (rows); weight_scale: 1 or N values (columns).
    Returns dict(acc=int32, f32=float32, bf16=uint16 bits), each [M,N].
    """
    lib = _load()
    A = _c(A, np.int8)
    W = _c(W, np.int8)
    M, K = A.shape
    N = W.shape[0] if b_trans else W.shape[1]
    a, w = _scales(act_scale, weight_scale, M, N)
    acc = np.empty((M, N), dtype=np.int32)
    f = np.empty((M, N), dtype=np.float32)
    h = np.empty((M, N), dtype=np.uint16)
    lib.oracle_a8w8(M, N, K, _ptr(A), K, _ptr(W), W.shape[1], int(bool(b_trans)),
                    _ptr(a), a.size, _ptr(w), w.size, _ptr(acc), _ptr(f), _ptr(h))
    return {"acc": acc, "f32": f, "bf16": h}


def a8w8_at(A, W, act_scale, weight_scale, rows, cols, b_trans=False):
    """A8W8 at chosen output positions (rows[i], cols[i]); 1-D results."""
    lib = _load()
    A = _c(A, np.int8)
    W = _c(W, np.int8)
    M, K = A.shape
    N = W.shape[0] if b_trans else W.shape[1]
    a, w = _scales(act_scale, weight_scale, M, N)
    rows = _c(rows, np.int64)
    cols = _c(cols, np.int64)
    n = rows.size
    acc = np.empty(n, dtype=np.int32)
    f = np.empty(n, dtype=np.float32)
    h = np.empty(n, dtype=np.uint16)
    lib.oracle_a8w8_at(M, N, K, _ptr(A), K, _ptr(W), W.shape[1], int(bool(b_trans)),
                       _ptr(a), a.size, _ptr(w), w.size, n, _ptr(rows), _ptr(cols),
                       _ptr(acc), _ptr(f), _ptr(h))
    return {"acc": acc, "f32": f, "bf16": h}


def a8w8_acc(acc_in, A, W, act_scale, weight_scale, b_trans=False):
    """A8W8 with an int32 accumulator input: the int8 product is added to
    acc_in (int32 [M,N], wrapping) before the cast and the two scales.
    Returns dict(acc=int32, f32=float32, bf16=uint16 bits), each [M,N]."""
    lib = _load()
    A = _c(A, np.int8)
    W = _c(W, np.int8)
    M, K = A.shape
    N = W.shape[0] if b_trans else W.shape[1]
    acc_in = _c(acc_in, np.int32)
    assert acc_in.shape == (M, N)
    a, w = _scales(act_scale, weight_scale, M, N)
    acc = np.empty((M, N), dtype=np.int32)
    f = np.empty((M, N), dtype=np.float32)
    h = np.empty((M, N), dtype=np.uint16)
    lib.oracle_a8w8_acc(M, N, K, _ptr(A), K, _ptr(W), W.shape[1], int(bool(b_trans)),
                        _ptr(acc_in), N, _ptr(a), a.size, _ptr(w), w.size, _ptr(acc), _ptr(f), _ptr(h))
    return {"acc": acc, "f32": f, "bf16": h}


# ---------------------------------------------------------------------------
# MatMulInteger
# ---------------------------------------------------------------------------

def _is_u8(x):
    if x.dtype == np.uint8:
        return 1
    if x.dtype == np.int8:
        return 0
    raise TypeError("MatMulInteger operands are uint8 or int8")


def _b_zero_points(b_zero_point, N):
    if b_zero_point is None:
        return None, 0
    z = np.asarray(b_zero_point).reshape(-1).astype(np.int32)
    assert z.size in (1, N)
    return _c(z, np.int32), z.size


def matmul_integer(A, B, a_zero_point=0, b_zero_point=None):
    """ONNX MatMulInteger: wrap32(sum_k (A - a_zp) * (B - b_zp)).

    A: uint8/int8 of rank 2-4, [..., M, K]; B: uint8/int8 [..., K, N] of rank
    2-4.  Batch dimensions broadcast as in numpy matmul; a size-1 batch of A
    is repeated, and a rank-2 B (or one whose batch dimensions are all 1) is
    one matrix shared by every batch.  a_zero_point: a scalar, or M per-row
    values ([M] or [M, 1]); b_zero_point: None, a scalar, or N per-column
    values ([N] or [1, N]).
    Returns int32 [*batch, M, N].
    """
    lib = _load()
    A = np.asarray(A)
    B = np.asarray(B)
    if not (2 <= A.ndim <= 4 and 2 <= B.ndim <= 4):
        raise ValueError("MatMulInteger operands have rank 2 to 4")
    M, K = A.shape[-2:]
    K2, N = B.shape[-2:]
    if K != K2:
        raise ValueError("inner dimensions differ")
    batch_shape = np.broadcast_shapes(A.shape[:-2], B.shape[:-2])
    nb = int(np.prod(batch_shape)) if batch_shape else 1
    A3 = _c(np.broadcast_to(A, batch_shape + (M, K)).reshape(nb, M, K), A.dtype)
    b_shared = B.ndim == 2 or all(d == 1 for d in B.shape[:-2])
    if b_shared:
        B3 = _c(B.reshape(K, N), B.dtype)
        b_bstride = 0
    else:
        B3 = _c(np.broadcast_to(B, batch_shape + (K, N)).reshape(nb, K, N), B.dtype)
        b_bstride = K * N
    zb, zb_len = _b_zero_points(b_zero_point, N)
    Y = np.empty((nb, M, N), dtype=np.int32)
    za = np.asarray(a_zero_point)
    if za.size > 1 or za.ndim > 0:
        # one zero point per row of A: [M] or [M, 1]
        za = _c(za.astype(np.int64).reshape(-1), np.int32)
        if za.size not in (1, M):
            raise ValueError("a_zero_point has 1 or M values")
        lib.oracle_matmul_integer_rows(nb, M, N, K,
                                       _ptr(A3), _is_u8(A3), K, M * K,
                                       _ptr(B3), _is_u8(B3), N, b_bstride,
                                       _ptr(za), za.size, _ptr(zb), zb_len,
                                       _ptr(Y), N, M * N)
        return Y.reshape(batch_shape + (M, N))
    lib.oracle_matmul_integer(nb, M, N, K,
                              _ptr(A3), _is_u8(A3), K, M * K,
                              _ptr(B3), _is_u8(B3), N, b_bstride,
                              int(a_zero_point), _ptr(zb), zb_len,
                              _ptr(Y), N, M * N)
    return Y.reshape(batch_shape + (M, N))


def matmul_integer_at(A3, B, a_zero_point, b_zero_point, bts, rows, cols, b_shared):
    """MatMulInteger at positions (bts[i], rows[i], cols[i]).

    A3: [batch, M, K]; B: [K, N] when b_shared else [batch, K, N].
    """
    lib = _load()
    A3 = _c(A3, A3.dtype)
    B = _c(B, B.dtype)
    _, M, K = A3.shape
    N = B.shape[-1]
    zb, zb_len = _b_zero_points(b_zero_point, N)
    bts = _c(bts, np.int64)
    rows = _c(rows, np.int64)
    cols = _c(cols, np.int64)
    Y = np.empty(rows.size, dtype=np.int32)
    lib.oracle_matmul_integer_at(K, _ptr(A3), _is_u8(A3), K, M * K,
                                 _ptr(B), _is_u8(B), N, 0 if b_shared else K * N,
                                 int(a_zero_point), _ptr(zb), zb_len,
                                 rows.size, _ptr(bts), _ptr(rows), _ptr(cols), _ptr(Y))
    return Y


def dot_f32acc(a, b, a_zero_point=0, b_zero_point=0):
    """Sequential fp32 accumulation of (a_k - za)(b_k - zb), cast to int32."""
    lib = _load()
    a = _c(a, a.dtype)
    b = _c(b, b.dtype)
    return int(lib.oracle_dot_f32acc(a.size, _ptr(a), _is_u8(a), _ptr(b), _is_u8(b), 1,
                                     int(a_zero_point), int(b_zero_point)))


# ---------------------------------------------------------------------------
# DynamicQuantizeLinear (uint8)
# ---------------------------------------------------------------------------

def dynamic_quantize_linear(x):
    """ONNX DynamicQuantizeLinear to uint8 as the onnx-to-hip page lowers it.

    x: float32 array of any shape.  Returns (y uint8 of x's shape,
    scale float32, zero_point uint8).
    """
    lib = _load()
    xs = _c(np.asarray(x, dtype=np.float32).reshape(-1), np.float32)
    y = np.empty(xs.size, dtype=np.uint8)
    sc = np.empty(1, dtype=np.float32)
    zp = np.empty(1, dtype=np.int32)
    lib.oracle_dynamic_quantize_linear(xs.size, _ptr(xs), _ptr(y), _ptr(sc), _ptr(zp))
    return y.reshape(np.shape(x)), np.float32(sc[0]), np.uint8(zp[0])


# ---------------------------------------------------------------------------
# ConvInteger
# ---------------------------------------------------------------------------

def conv_output_size(size, k, pad_lo, pad_hi, stride, dilation):
    return (size + pad_lo + pad_hi - dilation * (k - 1) - 1) // stride + 1


def conv_integer(x, w, x_zero_point=0, w_zero_point=None, pads=None, strides=None, dilations=None, group=1):
    """ONNX ConvInteger as the onnx-to-hip page lowers it ("What",
    ConvInteger paragraph): int32 y = wrap32(sum (x - x_zp) (w - w_zp[m]))
    over each output channel's group, taps outside the input contributing
    nothing.

    x: uint8/int8 [N, C, H, W] or [N, C, L]; w: uint8/int8 [M, C/group, kH, kW]
    or [M, C/group, kL].  pads: (top, left, bottom, right) for rank 4,
    (left, right) for rank 3; strides / dilations: per spatial axis.
    w_zero_point: None, a scalar, or M values.  Returns int32 [N, M, OH, OW]
    (or [N, M, OL])."""
    lib = _load()
    x = np.asarray(x)
    w = np.asarray(w)
    rank3 = x.ndim == 3
    if rank3:
        x = x[:, :, None, :]
        w = w[:, :, None, :]
        pads = (0, pads[0], 0, pads[1]) if pads is not None else None
        strides = (1, strides[0]) if strides is not None else None
        dilations = (1, dilations[0]) if dilations is not None else None
    pads = tuple(pads) if pads is not None else (0, 0, 0, 0)
    strides = tuple(strides) if strides is not None else (1, 1)
    dilations = tuple(dilations) if dilations is not None else (1, 1)
    N, C, H, W = x.shape
    M, Cg, kH, kW = w.shape
    assert C == Cg * group and M % group == 0
    OH = conv_output_size(H, kH, pads[0], pads[2], strides[0], dilations[0])
    OW = conv_output_size(W, kW, pads[1], pads[3], strides[1], dilations[1])
    if w_zero_point is None:
        zw = np.zeros(0, dtype=np.int32)
    else:
        zw = np.asarray(w_zero_point).reshape(-1).astype(np.int32)
    xs = _c(x, x.dtype)
    ws = _c(w, w.dtype)
    y = np.empty((N, M, OH, OW), dtype=np.int32)
    lib.oracle_conv_integer(N, C, H, W, _ptr(xs), _is_u8(xs), M, kH, kW, _ptr(ws), _is_u8(ws), group,
                            pads[0], pads[1], pads[2], pads[3], strides[0], strides[1], dilations[0], dilations[1],
                            int(x_zero_point), _ptr(zw) if zw.size else None, zw.size, _ptr(y))
    return y[:, :, 0, :] if rank3 else y

"""Exact pure-Python forms of the operators, for tiny inputs -- TEST INFRASTRUCTURE.

Independent of ``oracle.c``: Python integers (no width, no wrap until asked),
``fractions.Fraction`` for exact real arithmetic, and fp32 rounding emulated
through ``struct`` (a double-to-single store rounds to nearest even).  Used
only to pin the C oracle on small cases.
"""
import struct
from fractions import Fraction


def f32(x):
    """Round a Python float (double) to the nearest fp32 value, ties to even."""
    return struct.unpack("<f", struct.pack("<f", x))[0]


def wrap32(v):
    """Two's-complement wrap of an integer into int32."""
    v &= 0xFFFFFFFF
    return v - (1 << 32) if v >= (1 << 31) else v


def matmul_integer(A, B, za, zb):
    """Exact sum_k (A[m][k]-za)(B[k][n]-zb[n]) as Python ints (no wrap).

    A: list of M rows of K ints; B: list of K rows of N ints; zb: list of N.
    """
    M, K, N = len(A), len(B), len(B[0])
    return [[sum((A[m][k] - za) * (B[k][n] - zb[n]) for k in range(K))
             for n in range(N)] for m in range(M)]


def matmul_integer_rows(A, B, za, zb):
    """Exact sum_k (A[m][k]-za[m])(B[k][n]-zb[n]) as Python ints (no wrap)."""
    M, K, N = len(A), len(B), len(B[0])
    return [[sum((A[m][k] - za[m]) * (B[k][n] - zb[n]) for k in range(K))
             for n in range(N)] for m in range(M)]


def a8w8_acc(acc_in, A, W, act_scale, weight_scale):
    """A8W8 with an int32 accumulator input, each step exact or emulated
    fp32: acc = wrap32(acc_in + sum_k A W), then int -> fp32, *as, *ws."""
    M, K, N = len(A), len(W), len(W[0])
    out = []
    for m in range(M):
        row = []
        for n in range(N):
            acc = wrap32(acc_in[m][n] + sum(A[m][k] * W[k][n] for k in range(K)))
            f = f32(float(acc))
            f = f32(f * act_scale[m])
            f = f32(f * weight_scale[n])
            row.append((acc, f))
        out.append(row)
    return out


def a8w8(A, W, act_scale, weight_scale):
    """A8W8 with each fp32 step emulated exactly: int -> fp32, *as, *ws.

    The integer sum is exact; an int32 value converts to double exactly and
    the double -> fp32 store is the single RNE rounding of the cast.  A
    product of two fp32 values is exact in double (48 significant bits), so
    rounding it to fp32 is the fp32 multiply.
    """
    M, K, N = len(A), len(W), len(W[0])
    out = []
    for m in range(M):
        row = []
        for n in range(N):
            acc = wrap32(sum(A[m][k] * W[k][n] for k in range(K)))
            f = f32(float(acc))
            f = f32(f * act_scale[m])
            f = f32(f * weight_scale[n])
            row.append((acc, f))
        out.append(row)
    return out


def w8a32_exact(A, W, scale, zp):
    """Exact sum_k a (b - zp) scale, and sum_k |a| |b - zp| |scale|, as Fractions."""
    M, K, N = len(A), len(W), len(W[0])
    s = Fraction(scale)
    R, Bd = [], []
    for m in range(M):
        r, b = [], []
        for n in range(N):
            r.append(sum(Fraction(A[m][k]) * (W[k][n] - zp) for k in range(K)) * s)
            b.append(sum(abs(Fraction(A[m][k])) * abs(W[k][n] - zp) for k in range(K)) * abs(s))
        R.append(r)
        Bd.append(b)
    return R, Bd


def bf16_bits(x):
    """bfloat16 bits of a finite fp32 value by exact rational rounding.

    Finds the two bfloat16 neighbours of x by exact arithmetic on Fractions and
    keeps the nearer one, the even one on a tie.  Written independently of
    the bit trick in the C oracle.
    """
    bits = struct.unpack("<I", struct.pack("<f", x))[0]
    sign = bits >> 31
    mag = abs(Fraction(x))
    lo_bits = (bits & 0x7FFFFFFF) & 0xFFFF0000  # truncation toward zero
    hi_bits = lo_bits + 0x10000

    def val(b):
        return abs(Fraction(struct.unpack("<f", struct.pack("<I", b))[0])) \
            if (b & 0x7F800000) != 0x7F800000 else None

    lo = val(lo_bits)
    hi = val(hi_bits)
    if hi is None:  # rounding up would reach infinity: compare with the halfway point
        # largest finite bf16 is lo; the overflow threshold is lo + half an ulp
        ulp = lo - val(lo_bits - 0x10000)
        pick = hi_bits if mag >= lo + ulp / 2 else lo_bits
    elif mag - lo < hi - mag:
        pick = lo_bits
    elif mag - lo > hi - mag:
        pick = hi_bits
    else:
        pick = lo_bits if ((lo_bits >> 16) & 1) == 0 else hi_bits
    return (sign << 15) | (pick >> 16)


def dynamic_quantize_linear(xs):
    """DynamicQuantizeLinear on a list of fp32 values with every fp32 step
    emulated: a binary32 operation equals the double operation rounded to
    binary32 (double carries more than twice the bits, so the double
    rounding is innocuous for + - * /).  Python's round() is ties-to-even.
    The range includes 0; a zero scale becomes 1.  Returns (y, scale, zp)."""
    mn = min([0.0] + list(xs))
    mx = max([0.0] + list(xs))
    scale = f32(f32(mx - mn) / 255.0)
    if scale == 0.0:
        scale = 1.0
    zp = round(f32(0.0 - f32(mn / scale)))
    zp = min(255, max(0, zp))
    y = [min(255, max(0, round(f32(x / scale)) + zp)) for x in xs]
    return y, scale, zp


def conv_integer(x, w, x_zp, w_zp, pads, strides, dilations, group):
    """ConvInteger on nested lists with Python integers: x [N][C][H][W],
    w [M][C/group][kH][kW], w_zp a list of M values; pads (top, left,
    bottom, right).  Taps outside the input are skipped.  Returns y
    [N][M][OH][OW], each the exact sum wrapped to int32."""
    N, C, H, W = len(x), len(x[0]), len(x[0][0]), len(x[0][0][0])
    M, Cg, kH, kW = len(w), len(w[0]), len(w[0][0]), len(w[0][0][0])
    Mg = M // group
    OH = (H + pads[0] + pads[2] - dilations[0] * (kH - 1) - 1) // strides[0] + 1
    OW = (W + pads[1] + pads[3] - dilations[1] * (kW - 1) - 1) // strides[1] + 1
    y = [[[[0] * OW for _ in range(OH)] for _ in range(M)] for _ in range(N)]
    for n in range(N):
        for m in range(M):
            g = m // Mg
            for oh in range(OH):
                for ow in range(OW):
                    s = 0
                    for c in range(Cg):
                        for kh in range(kH):
                            for kw in range(kW):
                                ih = oh * strides[0] - pads[0] + kh * dilations[0]
                                iw = ow * strides[1] - pads[1] + kw * dilations[1]
                                if 0 <= ih < H and 0 <= iw < W:
                                    s += (x[n][g * Cg + c][ih][iw] - x_zp) * (w[m][c][kh][kw] - w_zp[m])
                    y[n][m][oh][ow] = wrap32(s)
    return y

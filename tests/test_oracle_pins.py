"""Pins for the CPU oracle: values the pages print, closed forms, brute force,
library routines on special cases.  CPU only; no HIP involved."""
import struct

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
import seeded_inputs as si
from golden_io import load



# ---------------------------------------------------------------------------
# MatMulInteger: accumulator bound and wrap (worked values on the hip-ep page)
# ---------------------------------------------------------------------------

def test_k259_worked_value_from_page():
    g = load("matmul_integer_accumulator.txt")
    a = np.full((1, 259), 255, np.uint8)
    b = np.full((259, 1), 255, np.uint8)
    assert oracle.matmul_integer(a, b, 0, None)[0, 0] == int(g["u8_all_255_k259"])
    assert 65025 * 259 == int(g["u8_all_255_k259"])


def test_f32_accumulator_exact_up_to_258_and_not_beyond():
    g = load("matmul_integer_accumulator.txt")
    kmax = int(g["f32_max_exact_k"])
    assert 65025 * kmax <= 2 ** 24 < 65025 * (kmax + 1)
    a = np.full(kmax, 255, np.uint8)
    assert oracle.dot_f32acc(a, a) == int(g["u8_all_255_k258"])
    a = np.full(kmax + 1, 255, np.uint8)
    exact = int(g["u8_all_255_k259"])
    f32_sum = oracle.dot_f32acc(a, a)
    # an independent sequential fp32 sum (numpy's cumsum is a running sum)
    running = np.cumsum(np.full(kmax + 1, 65025, np.float32), dtype=np.float32)[-1]
    assert f32_sum == int(running) == exact + 1


def test_f32_accumulator_agrees_with_int_when_k_at_most_258():
    g = si.rng(7)
    for K in (1, 17, 200, 258):
        for a_dt, b_dt, za, zb in ((np.uint8, np.uint8, 0, 255), (np.uint8, np.int8, 255, -128),
                                   (np.int8, np.int8, -128, 127), (np.int8, np.uint8, 127, 0)):
            a = si.randint(g, (K,), 0 if a_dt == np.uint8 else -128, 255 if a_dt == np.uint8 else 127, a_dt)
            b = si.randint(g, (K,), 0 if b_dt == np.uint8 else -128, 255 if b_dt == np.uint8 else 127, b_dt)
            y = oracle.matmul_integer(a.reshape(1, K), b.reshape(K, 1), za, zb)[0, 0]
            assert oracle.dot_f32acc(a, b, za, zb) == y


def test_wrap_to_int32():
    g = load("matmul_integer_accumulator.txt")
    K = 40000
    a = np.full((1, K), 255, np.uint8)
    b = np.full((K, 1), 255, np.uint8)
    assert oracle.matmul_integer(a, b)[0, 0] == int(g["u8_all_255_k40000_wrapped"])
    assert brute.wrap32(65025 * K) == int(g["u8_all_255_k40000_wrapped"])


# ---------------------------------------------------------------------------
# MatMulInteger: closed forms and brute force
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("a_dt,b_dt", [(np.uint8, np.uint8), (np.uint8, np.int8),
                                       (np.int8, np.int8), (np.int8, np.uint8)])
@pytest.mark.parametrize("za,zb", [(0, 0), (1, 127), (128, 255), (-128, -8), (127, 8)])
def test_product_table_k1(a_dt, b_dt, za, zb):
    """K = 1 with every 8-bit value on each side: Y is the outer product."""
    if a_dt == np.uint8 and za < 0 or a_dt == np.int8 and za > 127:
        pytest.skip("zero point outside the operand's range")
    if b_dt == np.uint8 and zb < 0 or b_dt == np.int8 and zb > 127:
        pytest.skip("zero point outside the operand's range")
    av = np.arange(256).astype(a_dt) if a_dt == np.uint8 else np.arange(-128, 128).astype(a_dt)
    bv = np.arange(256).astype(b_dt) if b_dt == np.uint8 else np.arange(-128, 128).astype(b_dt)
    Y = oracle.matmul_integer(av.reshape(256, 1), bv.reshape(1, 256), za, zb)
    expect = np.outer(av.astype(np.int64) - za, bv.astype(np.int64) - zb)
    np.testing.assert_array_equal(Y, expect)


def test_constant_fill_closed_form():
    for (av, za, bv, zb, K) in ((200, 3, -100, 7, 2048), (0, 255, 255, 0, 1000), (-128, 127, -128, 127, 333)):
        a_dt = np.uint8 if av >= 0 and za >= 0 and av <= 255 and za <= 255 and (av > 127 or za > 127) else np.int8
        b_dt = np.uint8 if bv >= 0 and bv > 127 else np.int8
        A = np.full((3, K), av).astype(a_dt)
        B = np.full((K, 5), bv).astype(b_dt)
        Y = oracle.matmul_integer(A, B, za, zb)
        assert (Y == brute.wrap32(K * (av - za) * (bv - zb))).all()


def test_one_hot_row_selects_centred_row_of_b():
    A, B, zb = si.matmul_integer_inputs(1, 1, 37, 53, seed=11)
    B = B.astype(np.int8)
    for j in (0, 9, 52):
        a = np.zeros((1, 53), np.uint8)
        a[0, j] = 1
        Y = oracle.matmul_integer(a, B, 0, zb)
        np.testing.assert_array_equal(Y[0], B[j].astype(np.int64) - zb.astype(np.int64))


def _rand8(g, shape, dt):
    return si.randint(g, shape, 0, 255, dt) if dt == np.uint8 else si.randint(g, shape, -128, 127, dt)


@pytest.mark.parametrize("seed", range(12))
def test_matmul_integer_brute_force(seed):
    g = si.rng(1000 + seed)
    M, N, K = (int(x) for x in g.integers(1, 10, size=3))
    a_dt = (np.uint8, np.int8)[seed % 2]
    b_dt = (np.uint8, np.int8)[(seed // 2) % 2]
    A = _rand8(g, (M, K), a_dt)
    B = _rand8(g, (K, N), b_dt)
    za = int(_rand8(g, (), a_dt))
    per_col = seed % 3 != 0
    zb = _rand8(g, (N,), b_dt) if per_col else np.array(int(_rand8(g, (), b_dt)))
    Y = oracle.matmul_integer(A, B, za, zb)
    zbl = [int(x) for x in np.broadcast_to(zb, (N,))]
    exact = brute.matmul_integer(A.astype(int).tolist(), B.astype(int).tolist(), za, zbl)
    assert Y.tolist() == [[brute.wrap32(v) for v in r] for r in exact]


def test_zero_point_identity_used_by_the_kernels():
    """sum (a-za)(b-zb) = sum a'b' + cb*sum a' + ca*sum b' + K*ca*cb with
    a' = a - 128 (u8) or a (i8), ca = 128 - za (u8) or -za (i8); same for b.
    Checked in exact integers against the oracle; this is the form the HIP
    kernels evaluate, so the oracle itself never uses it."""
    g = si.rng(99)
    for trial in range(40):
        M, N, K = (int(x) for x in g.integers(1, 12, size=3))
        a_dt = (np.uint8, np.int8)[trial % 2]
        b_dt = (np.uint8, np.int8)[(trial // 2) % 2]
        A = _rand8(g, (M, K), a_dt).astype(np.int64)
        B = _rand8(g, (K, N), b_dt).astype(np.int64)
        za = int(_rand8(g, (), a_dt))
        zb = _rand8(g, (N,), b_dt).astype(np.int64)
        sa = 128 if a_dt == np.uint8 else 0
        sb = 128 if b_dt == np.uint8 else 0
        A1, B1 = A - sa, B - sb
        ca, cb = sa - za, sb - zb
        ident = A1 @ B1 + np.outer(A1.sum(1), cb) + ca * B1.sum(0)[None, :] + K * ca * cb[None, :]
        Y = oracle.matmul_integer(A.astype(a_dt), B.astype(b_dt), za, zb.astype(b_dt))
        np.testing.assert_array_equal(Y, ident)


def test_shared_b_and_size1_batch_broadcast():
    g = si.rng(5)
    A = _rand8(g, (3, 4, 6, 9), np.uint8)
    B = _rand8(g, (9, 7), np.int8)
    zb = _rand8(g, (7,), np.int8)
    Y = oracle.matmul_integer(A, B, 100, zb)
    assert Y.shape == (3, 4, 6, 7)
    for i in range(3):
        for j in range(4):
            np.testing.assert_array_equal(Y[i, j], oracle.matmul_integer(A[i, j], B, 100, zb))
    # B whose batch dimensions are all 1 is the same shared matrix
    np.testing.assert_array_equal(oracle.matmul_integer(A, B.reshape(1, 1, 9, 7), 100, zb), Y)
    # a size-1 batch on A is repeated against a batched B
    A1 = _rand8(g, (1, 6, 9), np.int8)
    B3 = _rand8(g, (4, 9, 7), np.int8)
    Y3 = oracle.matmul_integer(A1, B3, -3, None)
    for i in range(4):
        np.testing.assert_array_equal(Y3[i], oracle.matmul_integer(A1[0], B3[i], -3, None))


def test_zero_point_zero_is_library_matmul():
    """With both zero points 0 the operator is the plain integer matmul."""
    A, B, _ = si.matmul_integer_inputs(2, 33, 45, 77, seed=3)
    Y = oracle.matmul_integer(A, B, 0, None)
    ref = np.matmul(A.astype(np.int64), B.astype(np.int64))
    np.testing.assert_array_equal(Y, ref)


def test_matmul_integer_at_matches_full():
    A, B, zb = si.matmul_integer_inputs(3, 20, 30, 70, seed=8)
    Y = oracle.matmul_integer(A, B, 128, zb)
    g = si.rng(1)
    bts, rows, cols = g.integers(0, 3, 50), g.integers(0, 20, 50), g.integers(0, 30, 50)
    y = oracle.matmul_integer_at(A, B, 128, zb, bts, rows, cols, b_shared=True)
    np.testing.assert_array_equal(y, Y[bts, rows, cols])


# ---------------------------------------------------------------------------
# A8W8 (pypto page): epilogue order, scale forms, torch expression
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(6))
def test_a8w8_brute_force(seed):
    g = si.rng(2000 + seed)
    M, N, K = (int(x) for x in g.integers(1, 9, size=3))
    A, W, s_a, s_w = si.a8w8_inputs(M, N, K, seed=seed, lo=-128, hi=127)
    r = oracle.a8w8(A, W, s_a, s_w)
    ref = brute.a8w8(A.astype(int).tolist(), W.astype(int).tolist(),
                     [float(x) for x in s_a], [float(x) for x in s_w])
    assert r["acc"].tolist() == [[c[0] for c in row] for row in ref]
    assert r["f32"].tolist() == [[c[1] for c in row] for row in ref]


def test_a8w8_unit_scales_give_the_rounded_accumulator():
    A, W, _, _ = si.a8w8_inputs(40, 50, 3000, seed=4, lo=-128, hi=127)
    r = oracle.a8w8(A, W, np.ones(1, np.float32), np.ones(1, np.float32))
    acc = np.matmul(A.astype(np.int64), W.astype(np.int64))
    np.testing.assert_array_equal(r["acc"], acc)
    np.testing.assert_array_equal(r["f32"], acc.astype(np.float32))


def test_a8w8_power_of_two_scales_are_exact():
    A, W, _, _ = si.a8w8_inputs(16, 24, 500, seed=6)
    s_a = np.array([2.0 ** -(i % 7) for i in range(16)], np.float32)
    s_w = np.array([2.0 ** (i % 5 - 2) for i in range(24)], np.float32)
    r = oracle.a8w8(A, W, s_a, s_w)
    acc = np.matmul(A.astype(np.int64), W.astype(np.int64)).astype(np.float64)
    np.testing.assert_array_equal(r["f32"].astype(np.float64), acc * s_a[:, None] * s_w[None, :])


def test_a8w8_rank1_act_scale_scales_rows_when_square():
    """With M == N a rank-1 act_scale must scale rows, not columns."""
    M = N = 12
    A, W, s_a, s_w = si.a8w8_inputs(M, N, 64, seed=12)
    s_a = np.arange(1, M + 1, dtype=np.float32)
    s_w = np.ones(N, np.float32)
    r = oracle.a8w8(A, W, s_a, s_w)
    acc = np.matmul(A.astype(np.int64), W.astype(np.int64)).astype(np.float32)
    np.testing.assert_array_equal(r["f32"], acc * s_a[:, None])
    assert not np.array_equal(r["f32"], acc * s_a[None, :])


def test_a8w8_scalar_scales_equal_broadcast_vectors():
    A, W, s_a, s_w = si.a8w8_inputs(9, 11, 100, seed=13)
    r1 = oracle.a8w8(A, W, s_a[:1], s_w[:1])
    r2 = oracle.a8w8(A, W, np.full(9, s_a[0]), np.full(11, s_w[0]))
    for k in ("acc", "f32", "bf16"):
        np.testing.assert_array_equal(r1[k], r2[k])


def test_a8w8_torch_expression_on_256x1024x1024():
    """The pypto page's torch reference, fp32 matmul then * act_scale[:, None]
    * weight_scale[None, :], is exact at K = 1024 with values in [-127, 127]
    (every partial sum is an integer below 2^24), so on the CPU it must equal
    the oracle bit for bit."""
    A, W, s_a, s_w = si.a8w8_inputs(256, 1024, 1024, seed=202)
    r = oracle.a8w8(A, W, s_a, s_w)
    t = torch.matmul(torch.from_numpy(A).float(), torch.from_numpy(W).float())
    t = t * torch.from_numpy(s_a)[:, None] * torch.from_numpy(s_w)[None, :]
    np.testing.assert_array_equal(r["f32"], t.numpy())
    np.testing.assert_array_equal(
        r["bf16"], t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


def test_a8w8_b_trans_equals_transposed_weight():
    A, W, s_a, s_w = si.a8w8_inputs(13, 29, 70, seed=14)
    r1 = oracle.a8w8(A, W, s_a, s_w)
    r2 = oracle.a8w8(A, np.ascontiguousarray(W.T), s_a, s_w, b_trans=True)
    np.testing.assert_array_equal(r1["f32"], r2["f32"])


def test_a8w8_at_matches_full():
    A, W, s_a, s_w = si.a8w8_inputs(30, 40, 200, seed=15)
    r = oracle.a8w8(A, W, s_a, s_w)
    g = si.rng(2)
    rows, cols = g.integers(0, 30, 64), g.integers(0, 40, 64)
    s = oracle.a8w8_at(A, W, s_a, s_w, rows, cols)
    for k in ("acc", "f32", "bf16"):
        np.testing.assert_array_equal(s[k], r[k][rows, cols])


# ---------------------------------------------------------------------------
# bfloat16 rounding
# ---------------------------------------------------------------------------

def test_bf16_matches_torch_and_exact_rounding():
    g = si.rng(21)
    x = np.concatenate([
        g.standard_normal(2000).astype(np.float32) * 1e3,
        g.uniform(-1e-3, 1e-3, 500).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 3.4e38, -3.4e38, 1e-40], np.float32),
    ])
    # exact ties: low 16 bits 0x8000 with even and odd kept parts
    ties = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0xC0418000, 0x47FF8000], np.uint32).view(np.float32)
    x = np.concatenate([x, ties])
    bits = oracle.f32_to_bf16(x)
    t = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, t)
    for v, b in zip(x[::17].tolist() + ties.tolist(), bits[::17].tolist() + bits[-5:].tolist()):
        assert brute.bf16_bits(v) == b
    assert bits[-5:].tolist() == [0x3F80, 0x3F82, 0xBF80, 0xC042, 0x4800]


# ---------------------------------------------------------------------------
# W8A32 (PULP page): dequantise-then-matmul in double
# ---------------------------------------------------------------------------

def test_w8a32_worked_example():
    gv = load("w8a32_identity.txt")
    a = np.array([[float(x) for x in gv["a"].split()]], np.float32)
    b = np.array([[int(x)] for x in gv["b"].split()], np.int8)
    R, B = oracle.w8a32(a, b, float(gv["scale"]), int(gv["zp"]))
    assert R[0, 0] == float(gv["result"])
    assert B[0, 0] == 0.5 * (1 * 1 + 2 * 2 + 3 * 9)


@pytest.mark.parametrize("seed", range(5))
def test_w8a32_brute_force_exact(seed):
    g = si.rng(3000 + seed)
    M, N, K = (int(x) for x in g.integers(1, 8, size=3))
    A, W = si.w8a32_inputs(M, N, K, seed=seed)
    scale, zp = float(np.float32(0.02)), int(g.integers(-9, 10))
    R, B = oracle.w8a32(A, W, scale, zp)
    Rx, Bx = brute.w8a32_exact(A.tolist(), W.astype(int).tolist(), scale, zp)
    for m in range(M):
        for n in range(N):
            assert abs(R[m, n] - float(Rx[m][n])) <= 1e-13 * float(Bx[m][n]) + 1e-300
            assert abs(B[m, n] - float(Bx[m][n])) <= 1e-13 * float(Bx[m][n])


def test_w8a32_integer_activations_are_exact():
    """Integer-valued A: every sum is an exact integer, so R must equal
    scale * (integer matmul of A with W - zp) exactly, and the factorised form
    scale * (S1 - zp * S2) gives the same number."""
    g = si.rng(31)
    A = g.integers(-3, 4, size=(64, 128)).astype(np.float32)
    W = si.randint(g, (128, 64), -128, 127, np.int8)
    scale = np.float32(0.02)
    for zp in (3, 0, -5):
        R, _ = oracle.w8a32(A, W, scale, zp)
        Ai = A.astype(np.int64)
        centred = Ai @ (W.astype(np.int64) - zp)
        np.testing.assert_array_equal(R, centred.astype(np.float64) * np.float64(scale))
        S1 = Ai @ W.astype(np.int64)
        S2 = Ai.sum(1)
        np.testing.assert_array_equal(centred, S1 - zp * S2[:, None])


def test_w8a32_zero_point_zero_is_the_plain_loop():
    """zp == 0 and scale == 1: the operator is A @ float(W)."""
    A, W = si.w8a32_inputs(64, 64, 128, seed=101)
    R, B = oracle.w8a32(A, W, 1.0, 0)
    ref = A.astype(np.float64) @ W.astype(np.float64)
    assert np.all(np.abs(R - ref) <= 1e-14 * B)


def test_w8a32_weight_equal_to_zero_point_gives_zero():
    A, _ = si.w8a32_inputs(8, 8, 50, seed=5)
    W = np.full((50, 8), -5, np.int8)
    R, B = oracle.w8a32(A, W, 0.01, -5)
    assert (R == 0).all() and (B == 0).all()


def test_w8a32_factorised_form_within_double_rounding():
    A, W = si.w8a32_inputs(64, 64, 128, seed=101)
    for zp in (3, 0):
        R, B = oracle.w8a32(A, W, 0.02, zp)
        A64 = A.astype(np.float64)
        fact = np.float64(np.float32(0.02)) * (A64 @ W.astype(np.float64) - zp * A64.sum(1)[:, None])
        assert np.all(np.abs(R - fact) <= 1e-12 * B)


# ---------------------------------------------------------------------------
# A8W8 with an int32 accumulator input (pypto page, matmul-dequant-acc op)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(6))
def test_a8w8_acc_brute_force(seed):
    """Independent pure-Python form, including accumulator inputs near the
    int32 limits so that the wrap is exercised."""
    g = si.rng(3000 + seed)
    M, N, K = (int(x) for x in g.integers(1, 9, size=3))
    A, W, s_a, s_w = si.a8w8_inputs(M, N, K, seed=seed, lo=-128, hi=127)
    edge = np.array([2**31 - 1, -2**31, 2**31 - 100, -2**31 + 7, 0], dtype=np.int64)
    acc_in = np.where(si.randint(g, (M, N), 0, 1, np.int64) == 1,
                      edge[si.randint(g, (M, N), 0, 4, np.int64)],
                      si.randint(g, (M, N), -2**31, 2**31 - 1, np.int64)).astype(np.int32)
    r = oracle.a8w8_acc(acc_in, A, W, s_a, s_w)
    ref = brute.a8w8_acc(acc_in.astype(int).tolist(), A.astype(int).tolist(), W.astype(int).tolist(),
                         [float(x) for x in s_a], [float(x) for x in s_w])
    assert r["acc"].tolist() == [[c[0] for c in row] for row in ref]
    assert r["f32"].tolist() == [[c[1] for c in row] for row in ref]


def test_a8w8_acc_with_zero_activations_is_the_scaled_input():
    """A = 0: the output is the fp32 chain applied to acc_in alone, computed
    here with numpy's IEEE float32 arithmetic (RNE per multiply)."""
    g = si.rng(17)
    M, N, K = 30, 40, 64
    A = np.zeros((M, K), np.int8)
    _, W, s_a, s_w = si.a8w8_inputs(M, N, K, seed=5)
    acc_in = si.randint(g, (M, N), -2**31, 2**31 - 1, np.int64).astype(np.int32)
    r = oracle.a8w8_acc(acc_in, A, W, s_a, s_w)
    f = (acc_in.astype(np.float32) * s_a[:, None]).astype(np.float32) * s_w[None, :]
    np.testing.assert_array_equal(r["acc"], acc_in)
    np.testing.assert_array_equal(r["f32"], f.astype(np.float32))


def test_a8w8_acc_chains_k_chunks():
    """Feeding the raw accumulator of one K chunk into the next gives the
    result over the whole K (the K-chunked use the op exists for)."""
    A, W, s_a, s_w = si.a8w8_inputs(20, 36, 300, seed=9, lo=-128, hi=127)
    first = oracle.a8w8(A[:, :128], W[:128], s_a, s_w)["acc"]
    r = oracle.a8w8_acc(first, A[:, 128:], W[128:], s_a, s_w)
    whole = oracle.a8w8(A, W, s_a, s_w)
    for key in ("acc", "f32", "bf16"):
        np.testing.assert_array_equal(r[key], whole[key])


# ---------------------------------------------------------------------------
# MatMulInteger with a per-row activation zero point (onnx-to-hip page)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(8))
def test_matmul_integer_row_zero_points_brute_force(seed):
    g = si.rng(4000 + seed)
    M, N, K = (int(x) for x in g.integers(1, 10, size=3))
    a_dt = (np.uint8, np.int8)[seed % 2]
    b_dt = (np.uint8, np.int8)[(seed // 2) % 2]
    A = _rand8(g, (M, K), a_dt)
    B = _rand8(g, (K, N), b_dt)
    za = _rand8(g, (M,), a_dt)
    zb = _rand8(g, (N,), b_dt)
    Y = oracle.matmul_integer(A, B, za, zb)
    exact = brute.matmul_integer_rows(A.astype(int).tolist(), B.astype(int).tolist(),
                                      [int(x) for x in za], [int(x) for x in zb])
    assert Y.tolist() == [[brute.wrap32(v) for v in r] for r in exact]


def test_matmul_integer_constant_row_zero_points_equal_the_scalar():
    A, B, zb = si.matmul_integer_inputs(3, 17, 23, 70, seed=12)
    Y = oracle.matmul_integer(A, B, np.full(17, 131, np.uint8), zb)
    np.testing.assert_array_equal(Y, oracle.matmul_integer(A, B, 131, zb))
    # [M, 1] is the same per-row form
    np.testing.assert_array_equal(oracle.matmul_integer(A, B, np.full((17, 1), 131, np.uint8), zb), Y)


def test_row_zero_point_identity_used_by_the_kernels():
    """With per-row ca[m]: sum (a-za[m])(b-zb[n]) = sum a'b' + cb[n] sum a'
    + ca[m] sum b'[:,n] + K ca[m] cb[n], in exact integers."""
    g = si.rng(98)
    for trial in range(30):
        M, N, K = (int(x) for x in g.integers(1, 12, size=3))
        a_dt = (np.uint8, np.int8)[trial % 2]
        b_dt = (np.uint8, np.int8)[(trial // 2) % 2]
        A = _rand8(g, (M, K), a_dt).astype(np.int64)
        B = _rand8(g, (K, N), b_dt).astype(np.int64)
        za = _rand8(g, (M,), a_dt).astype(np.int64)
        zb = _rand8(g, (N,), b_dt).astype(np.int64)
        sa = 128 if a_dt == np.uint8 else 0
        sb = 128 if b_dt == np.uint8 else 0
        A1, B1 = A - sa, B - sb
        ca, cb = sa - za, sb - zb
        ident = (A1 @ B1 + np.outer(A1.sum(1), cb) + np.outer(ca, B1.sum(0)) + K * np.outer(ca, cb))
        Y = oracle.matmul_integer(A.astype(a_dt), B.astype(b_dt), za.astype(a_dt), zb.astype(b_dt))
        np.testing.assert_array_equal(Y, ident)


# ---------------------------------------------------------------------------
# W8A32 input gradient (PULPOpen page intro; L3-sharing page intro)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(6))
def test_w8a32_input_grad_brute_force_exact(seed):
    """Exact rational arithmetic: the gradient is the forward operator applied
    to dC with the weight transposed."""
    g = si.rng(3100 + seed)
    M, N, K = (int(x) for x in g.integers(1, 8, size=3))
    dC, _ = si.w8a32_inputs(M, K, N, seed=seed)          # dC: [M, N] fp32
    _, W = si.w8a32_inputs(1, N, K, seed=seed + 50)       # W: [K, N] int8
    scale, zp = float(np.float32(0.03)), int(g.integers(-9, 10))
    R, B = oracle.w8a32_input_grad(dC, W, scale, zp)
    Rx, Bx = brute.w8a32_exact(dC.tolist(), W.T.astype(int).tolist(), scale, zp)
    for m in range(M):
        for k in range(K):
            assert abs(R[m, k] - float(Rx[m][k])) <= 1e-13 * float(Bx[m][k]) + 1e-300
            assert abs(B[m, k] - float(Bx[m][k])) <= 1e-13 * float(Bx[m][k])


def test_w8a32_input_grad_is_the_adjoint_of_the_forward():
    """<dC, A @ Wd> == <dC @ Wd^T, A> for any A and dC: the defining property
    of the input gradient (a wrong transpose or sign fails it)."""
    A, W = si.w8a32_inputs(37, 29, 53, seed=21)
    dC, _ = si.w8a32_inputs(37, 53, 29, seed=22)
    scale, zp = 0.017, -4
    fwd, fb = oracle.w8a32(A, W, scale, zp)
    grad, gb = oracle.w8a32_input_grad(dC, W, scale, zp)
    lhs = float((dC.astype(np.float64) * fwd).sum())
    rhs = float((grad * A.astype(np.float64)).sum())
    scale_of_terms = float((np.abs(dC.astype(np.float64)) * fb).sum())
    assert abs(lhs - rhs) <= 1e-12 * scale_of_terms


def test_w8a32_input_grad_matches_torch_autograd_in_double():
    A, W = si.w8a32_inputs(24, 31, 40, seed=23)
    dC, _ = si.w8a32_inputs(24, 40, 31, seed=24)
    scale, zp = 0.05, 3
    X = torch.from_numpy(A.astype(np.float64)).requires_grad_(True)
    Wd = (torch.from_numpy(W.astype(np.float64)) - zp) * scale
    (X @ Wd).backward(torch.from_numpy(dC.astype(np.float64)))
    R, B = oracle.w8a32_input_grad(dC, W, np.float32(scale), zp)
    # the oracle uses the fp32-rounded scale, torch the double one
    rel = abs(float(np.float32(scale)) - scale) / scale
    assert np.all(np.abs(R - X.grad.numpy()) <= (rel + 1e-13) * B + 1e-300)


# ---------------------------------------------------------------------------
# DynamicQuantizeLinear, uint8 (onnx-to-hip page)
# ---------------------------------------------------------------------------

def _floats(s):
    return np.array([float(t) for t in s.split()], dtype=np.float32)


def test_dynamic_quantize_all_zero_case_from_page():
    gv = load("dynamic_quantize_linear.txt")
    y, sc, zp = oracle.dynamic_quantize_linear(np.zeros(8, np.float32))
    assert sc == np.float32(float(gv["all_zero_scale"]))
    assert int(zp) == int(gv["all_zero_zero_point"])
    assert y.tolist() == [int(t) for t in gv["all_zero_output"].split()]


@pytest.mark.parametrize("case_name", ["ties_pos", "ties_neg", "unit_range", "sym_range"])
def test_dynamic_quantize_hand_worked_ties(case_name):
    gv = load("dynamic_quantize_linear.txt")
    y, sc, zp = oracle.dynamic_quantize_linear(_floats(gv[case_name + "_input"]))
    assert sc == np.float32(float(gv[case_name + "_scale"]))
    assert int(zp) == int(gv[case_name + "_zero_point"])
    assert y.tolist() == [int(t) for t in gv[case_name + "_output"].split()]


@pytest.mark.parametrize("seed", range(10))
def test_dynamic_quantize_brute_force(seed):
    g = si.rng(5000 + seed)
    n = int(g.integers(1, 300))
    kind = seed % 4
    if kind == 0:
        x = g.standard_normal(n).astype(np.float32)
    elif kind == 1:
        x = (g.standard_normal(n) * 1e3 + 5e3).astype(np.float32)      # all positive
    elif kind == 2:
        x = -np.abs(g.standard_normal(n)).astype(np.float32) * 1e-3    # all non-positive
    else:   # many exact ties: multiples of half a step
        x = (si.randint(g, (n,), -300, 300, np.int64) * 0.5).astype(np.float32)
    y, sc, zp = oracle.dynamic_quantize_linear(x)
    by, bsc, bzp = brute.dynamic_quantize_linear([float(v) for v in x])
    assert float(sc) == bsc and int(zp) == bzp
    assert y.tolist() == by


def test_dynamic_quantize_properties():
    """For any input: 0 quantizes to the zero point, the minimum (when
    negative) to 0, and every value dequantizes to within half a step."""
    for seed in range(6):
        g = si.rng(6000 + seed)
        x = (g.standard_normal(5000) * (10.0 ** (seed - 3)) + (seed - 2) * 10.0 ** (seed - 3)).astype(np.float32)
        x[17] = 0.0
        y, sc, zp = oracle.dynamic_quantize_linear(x)
        assert y[17] == zp
        if x.min() < 0:
            assert y[int(np.argmin(x))] == 0
        assert int(y[int(np.argmax(x))]) >= 254
        deq = (y.astype(np.float64) - int(zp)) * float(sc)
        assert np.all(np.abs(deq - x.astype(np.float64)) <= 0.5 * float(sc) * (1 + 1e-5))


# ---------------------------------------------------------------------------
# ConvInteger (onnx-to-hip page, "What" and its GPU numeric tests)
# ---------------------------------------------------------------------------

def _conv_case(seed, N, C, H, W, M, kH, kW, group, x_u8, w_u8, per_channel):
    g = si.rng(seed)
    xlo, xhi = (0, 255) if x_u8 else (-128, 127)
    wlo, whi = (0, 255) if w_u8 else (-128, 127)
    x = si.randint(g, (N, C, H, W), xlo, xhi, np.uint8 if x_u8 else np.int8)
    w = si.randint(g, (M, C // group, kH, kW), wlo, whi, np.uint8 if w_u8 else np.int8)
    x_zp = int(si.randint(g, (), xlo, xhi, np.int64))
    if per_channel:
        w_zp = si.randint(g, (M,), wlo, whi, np.int64)
    else:
        w_zp = np.full(M, int(si.randint(g, (), wlo, whi, np.int64)))
    return x, w, x_zp, w_zp


def _torch_conv_fp64(x, w, x_zp, w_zp, pads, strides, dilations, group):
    """The same convolution through torch's fp64 conv2d on the zero-point
    shifted operands, padded with 0 after the shift (exact: every partial sum
    is an integer far below 2^53)."""
    xf = torch.from_numpy(x.astype(np.float64) - x_zp)
    wf = torch.from_numpy(w.astype(np.float64) - np.asarray(w_zp, np.float64).reshape(-1, 1, 1, 1))
    xf = torch.nn.functional.pad(xf, (pads[1], pads[3], pads[0], pads[2]), value=0.0)
    y = torch.nn.functional.conv2d(xf, wf, stride=strides, dilation=dilations, groups=group)
    return y.numpy()


CONV_LIBRARY_CASES = [
    # N, C, H, W, M, kH, kW, group, pads, strides, dilations, x_u8, w_u8, per_channel
    (2, 6, 9, 11, 4, 3, 3, 1, (1, 1, 1, 1), (1, 1), (1, 1), True, False, True),
    (1, 58, 7, 7, 6, 3, 3, 2, (1, 1, 1, 1), (2, 2), (1, 1), True, False, True),   # reduction 261, stride 2, 2 groups
    (2, 8, 10, 6, 8, 3, 2, 4, (2, 0, 1, 3), (2, 1), (1, 2), False, True, False),
    (3, 5, 6, 13, 7, 1, 5, 1, (0, 2, 0, 2), (1, 3), (1, 1), False, False, True),
    (1, 4, 12, 12, 4, 3, 3, 4, (1, 1, 1, 1), (1, 1), (2, 2), True, True, True),    # depthwise, dilated
]


@pytest.mark.parametrize("case", CONV_LIBRARY_CASES)
def test_conv_integer_equals_torch_conv2d_fp64(case):
    N, C, H, W, M, kH, kW, group, pads, strides, dil, x_u8, w_u8, per_ch = case
    x, w, x_zp, w_zp = _conv_case(sum(case[:7]), N, C, H, W, M, kH, kW, group, x_u8, w_u8, per_ch)
    y = oracle.conv_integer(x, w, x_zp, w_zp, pads=pads, strides=strides, dilations=dil, group=group)
    ref = _torch_conv_fp64(x, w, x_zp, w_zp, pads, strides, dil, group)
    assert y.shape == ref.shape
    np.testing.assert_array_equal(y.astype(np.float64), ref)


@pytest.mark.parametrize("seed", range(8))
def test_conv_integer_brute_force(seed):
    g = si.rng(7000 + seed)
    group = int(g.choice([1, 2]))
    Cg, Mg = int(g.integers(1, 3)), int(g.integers(1, 3))
    kH, kW = int(g.integers(1, 4)), int(g.integers(1, 4))
    H, W = int(g.integers(kH, 6)), int(g.integers(kW, 6))
    pads = tuple(int(v) for v in g.integers(0, 3, size=4))
    strides = tuple(int(v) for v in g.integers(1, 3, size=2))
    dil = tuple(int(v) for v in g.integers(1, 3, size=2))
    if H + pads[0] + pads[2] < dil[0] * (kH - 1) + 1 or W + pads[1] + pads[3] < dil[1] * (kW - 1) + 1:
        dil = (1, 1)
    x, w, x_zp, w_zp = _conv_case(7100 + seed, 2, Cg * group, H, W, Mg * group, kH, kW, group,
                                  seed % 2 == 0, seed % 3 == 0, True)
    y = oracle.conv_integer(x, w, x_zp, w_zp, pads=pads, strides=strides, dilations=dil, group=group)
    by = brute.conv_integer(x.astype(np.int64).tolist(), w.astype(np.int64).tolist(), x_zp,
                            [int(v) for v in w_zp], pads, strides, dil, group)
    assert y.tolist() == by


def test_conv_integer_1x1_is_matmul_integer():
    """A 1x1, stride-1, unpadded convolution of image n is the MatMulInteger
    W [M, C] x X_n [C, H*W] with the weight zero points as per-row zero points
    of the left operand and the activation zero point as B's."""
    x, w, x_zp, w_zp = _conv_case(31, 3, 37, 5, 7, 9, 1, 1, 1, True, False, True)
    y = oracle.conv_integer(x, w, x_zp, w_zp)
    for n in range(3):
        ref = oracle.matmul_integer(w.reshape(9, 37), x[n].reshape(37, 35), w_zp.reshape(9), x_zp)
        np.testing.assert_array_equal(y[n].reshape(9, 35), ref)


def test_conv_integer_259_channel_1x1_worked_value_from_page():
    """The page's 259-channel 1x1 convolution; with every byte 255 and zero
    points 0 each output is the length-259 dot product the page works out."""
    gv = load("matmul_integer_accumulator.txt")
    x = np.full((1, 259, 2, 3), 255, np.uint8)
    w = np.full((2, 259, 1, 1), 255, np.uint8)
    y = oracle.conv_integer(x, w, 0, None)
    assert np.all(y == int(gv["u8_all_255_k259"]))


def test_conv_integer_constant_fill_counts_in_bounds_taps():
    """Constant operands: each output is (taps inside the input) * C/group *
    (a - za)(b - zb); with a 3x3 window and padding 1 that is 9 inside, 6 on
    an edge and 4 in a corner."""
    a, za, b, zb = 200, 13, -7, 5
    x = np.full((1, 4, 5, 6), a, np.uint8)
    w = np.full((4, 2, 3, 3), b, np.int8)
    y = oracle.conv_integer(x, w, za, np.full(4, zb), pads=(1, 1, 1, 1), group=2)[0]
    unit = 2 * (a - za) * (b - zb)
    taps = np.full((5, 6), 9)
    taps[0, :] = taps[-1, :] = 6
    taps[:, 0] = taps[:, -1] = 6
    taps[0, 0] = taps[0, -1] = taps[-1, 0] = taps[-1, -1] = 4
    for m in range(4):
        np.testing.assert_array_equal(y[m], taps * unit)


def test_conv_integer_wraps_like_matmul_integer():
    gv = load("matmul_integer_accumulator.txt")
    x = np.full((1, 40000, 1, 1), 255, np.uint8)
    w = np.full((1, 40000, 1, 1), 255, np.uint8)
    assert oracle.conv_integer(x, w, 0, None)[0, 0, 0, 0] == int(gv["u8_all_255_k40000_wrapped"])


def test_conv_integer_rank3_is_rank4_with_unit_height():
    x, w, x_zp, w_zp = _conv_case(41, 2, 6, 1, 17, 4, 1, 3, 2, False, False, True)
    y4 = oracle.conv_integer(x, w, x_zp, w_zp, pads=(0, 2, 0, 1), strides=(1, 2), dilations=(1, 2), group=2)
    y3 = oracle.conv_integer(x[:, :, 0, :], w[:, :, 0, :], x_zp, w_zp, pads=(2, 1), strides=(2,), dilations=(2,),
                             group=2)
    np.testing.assert_array_equal(y3, y4[:, :, 0, :])

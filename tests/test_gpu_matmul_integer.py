"""MatMulInteger on the GPU against the oracle: bit-exact int32."""
import numpy as np
import pytest
import torch

import oracle
import quantized_int8_gemm_amd as q
import seeded_inputs as si
from gpu_util import case, dev, env, to_dev

pytestmark = pytest.mark.gpu


def test_matmul_integer_batched_shared_b_8x512x2048x2048():
    """The full batched workload, every output compared."""
    case("matmul_integer 8x512x2048x2048 shared B")
    A, B, zb = si.matmul_integer_inputs(8, 512, 2048, 2048, seed=303)
    y = q.matmul_integer(to_dev(A), to_dev(B), 128, to_dev(zb)).cpu().numpy()
    np.testing.assert_array_equal(y, oracle.matmul_integer(A, B, 128, zb))


@pytest.mark.parametrize("a_dt,b_dt", [(np.uint8, np.int8), (np.uint8, np.uint8),
                                       (np.int8, np.int8), (np.int8, np.uint8)])
@pytest.mark.parametrize("za,zb_kind", [(0, "none"), ("mid", "scalar"), ("mid", "column"), ("edge", "column")])
@pytest.mark.parametrize("M,N,K", [(3, 5, 259), (40, 130, 261), (130, 256, 512)])
def test_matmul_integer_dtypes_and_zero_points(a_dt, b_dt, za, zb_kind, M, N, K):
    case(f"matmul_integer {np.dtype(a_dt)}x{np.dtype(b_dt)} za={za} zb={zb_kind} M={M} N={N} K={K}")
    g = si.rng(M * 1000 + N + K)
    A = si.randint(g, (M, K), 0, 255, a_dt) if a_dt == np.uint8 else si.randint(g, (M, K), -128, 127, a_dt)
    B = si.randint(g, (K, N), 0, 255, b_dt) if b_dt == np.uint8 else si.randint(g, (K, N), -128, 127, b_dt)
    if za == "mid":
        za = 128 if a_dt == np.uint8 else -3
    elif za == "edge":
        za = 255 if a_dt == np.uint8 else -128
    if zb_kind == "none":
        zb = None
    elif zb_kind == "scalar":
        zb = np.array([200 if b_dt == np.uint8 else 7], dtype=b_dt)
    else:
        zb = (si.randint(g, (N,), 0, 255, b_dt) if b_dt == np.uint8 else si.randint(g, (N,), -128, 127, b_dt))
    y = q.matmul_integer(to_dev(A), to_dev(B), za, None if zb is None else to_dev(zb)).cpu().numpy()
    np.testing.assert_array_equal(y, oracle.matmul_integer(A, B, za, zb))


@pytest.mark.parametrize("a_shape,b_shape", [
    ((2, 1, 2), (2, 3)),              # rank-3 A with a rank-2 B (batch stride 0)
    ((3, 70, 259), (259, 33)),        # shared B, contiguous A batches (folded into M)
    ((3, 70, 259), (1, 259, 33)),     # B with batch dims of 1 is shared too
    ((1, 40, 100), (4, 100, 50)),     # size-1 batch on A, batched B
    ((2, 3, 17, 64), (2, 3, 64, 24)), # rank 4, distinct per-batch weights
    ((4, 17, 259), (4, 259, 9)),      # length-259 reduction, distinct per-batch weights
])
def test_matmul_integer_batch_rules(a_shape, b_shape):
    case(f"matmul_integer batch A{a_shape} B{b_shape}")
    g = si.rng(sum(a_shape) + sum(b_shape))
    A = si.randint(g, a_shape, 0, 255, np.uint8)
    B = si.randint(g, b_shape, -128, 127, np.int8)
    zb = si.randint(g, (b_shape[-1],), -8, 8, np.int8)
    y = q.matmul_integer(to_dev(A), to_dev(B), 128, to_dev(zb)).cpu().numpy()
    ref = oracle.matmul_integer(A, B, 128, zb)
    assert y.shape == ref.shape
    np.testing.assert_array_equal(y, ref)


def test_matmul_integer_k259_all_255():
    """The worked value on the hip-ep page: a length-259 uint8 dot of 255s."""
    case("matmul_integer k259 all-255")
    A = np.full((4, 259), 255, np.uint8)
    B = np.full((259, 3), 255, np.uint8)
    y = q.matmul_integer(to_dev(A), to_dev(B)).cpu().numpy()
    assert (y == 16841475).all()


def test_matmul_integer_wraps_mod_2_32():
    """int8 x int8 sums past 2^31 store the two's-complement wrap (checks
    that the matrix-core int32 accumulation wraps rather than saturates)."""
    case("matmul_integer wrap K=131200 (-128 x -128)")
    K = 131200
    A = np.full((16, K), -128, np.int8)
    B = np.full((K, 16), -128, np.int8)
    y = q.matmul_integer(to_dev(A), to_dev(B)).cpu().numpy()
    ref = oracle.matmul_integer(A, B)
    assert ref[0, 0] == ((16384 * K + 2 ** 31) % 2 ** 32) - 2 ** 31
    np.testing.assert_array_equal(y, ref)
    # uint8 with zero point 0 on both sides: 65025 * 40000 wraps
    A = np.full((2, 40000), 255, np.uint8)
    B = np.full((40000, 2), 255, np.uint8)
    y = q.matmul_integer(to_dev(A), to_dev(B)).cpu().numpy()
    assert (y == -1693967296).all()


@pytest.mark.parametrize("stage", [0, 1, 2])
@pytest.mark.parametrize("tile", range(10))
def test_matmul_integer_every_tile_shape(tile, stage):
    """Every tile configuration, output straight from the fragments (stage 0)
    or through LDS (stage 1), with ragged M and N edges."""
    case(f"matmul_integer tile {tile} stage {stage} 2x300x528x640")
    A, B, zb = si.matmul_integer_inputs(2, 300, 528, 640, seed=31 + tile)
    with env(QGEMM_TILE=tile, QGEMM_STAGE=stage):
        y = q.matmul_integer(to_dev(A), to_dev(B), 100, to_dev(zb)).cpu().numpy()
        assert q.last_kernel().startswith("int8_dma"), q.last_kernel()
    np.testing.assert_array_equal(y, oracle.matmul_integer(A, B, 100, zb))


@pytest.mark.parametrize("family", ["dma", "staged"])
@pytest.mark.parametrize("a_dt,b_dt,za", [(np.uint8, np.int8, 128), (np.int8, np.uint8, -7), (np.uint8, np.uint8, 3)])
def test_matmul_integer_both_kernel_families(family, a_dt, b_dt, za):
    case(f"matmul_integer family={family} {np.dtype(a_dt)}x{np.dtype(b_dt)} za={za}")
    g = si.rng(77)
    A = si.randint(g, (3, 200, 512), 0, 255, a_dt) if a_dt == np.uint8 else si.randint(g, (3, 200, 512), -128, 127, a_dt)
    B = si.randint(g, (512, 384), 0, 255, b_dt) if b_dt == np.uint8 else si.randint(g, (512, 384), -128, 127, b_dt)
    zb = si.randint(g, (384,), 0, 255, b_dt) if b_dt == np.uint8 else si.randint(g, (384,), -8, 8, b_dt)
    with env(QGEMM_FAMILY=family):
        y = q.matmul_integer(to_dev(A), to_dev(B), za, to_dev(zb)).cpu().numpy()
        assert q.last_kernel().startswith("int8_dma" if family == "dma" else "int8_staged")
    np.testing.assert_array_equal(y, oracle.matmul_integer(A, B, za, zb))


@pytest.mark.parametrize("a_dt,b_dt", [(np.uint8, np.int8), (np.int8, np.uint8), (np.uint8, np.uint8)])
@pytest.mark.parametrize("tile", range(10))
def test_matmul_integer_row_zero_points_every_tile(tile, a_dt, b_dt):
    """Per-row activation zero points with a shared B (batch folded into M,
    so the row index wraps per batch), per-column b_zp, ragged edges."""
    case(f"matmul_integer row zp tile {tile} {np.dtype(a_dt)}x{np.dtype(b_dt)} 3x200x528x512")
    g = si.rng(500 + tile)
    A = si.randint(g, (3, 200, 512), 0, 255, a_dt) if a_dt == np.uint8 else si.randint(g, (3, 200, 512), -128, 127, a_dt)
    B = si.randint(g, (512, 528), 0, 255, b_dt) if b_dt == np.uint8 else si.randint(g, (512, 528), -128, 127, b_dt)
    za = si.randint(g, (200,), 0, 255, a_dt) if a_dt == np.uint8 else si.randint(g, (200,), -128, 127, a_dt)
    zb = si.randint(g, (528,), 0, 255, b_dt) if b_dt == np.uint8 else si.randint(g, (528,), -8, 8, b_dt)
    with env(QGEMM_TILE=tile):
        y = q.matmul_integer(to_dev(A), to_dev(B), to_dev(za), to_dev(zb)).cpu().numpy()
        assert q.last_kernel().startswith("int8_dma"), q.last_kernel()
    np.testing.assert_array_equal(y, oracle.matmul_integer(A, B, za, zb))


@pytest.mark.parametrize("family", ["dma", "staged"])
def test_matmul_integer_row_zero_points_families_and_forms(family):
    """[M, 1] zero points, a size-1 A batch broadcast against a batched B,
    and K = 259 (register-staged kernel: bytes past K are cleared)."""
    case(f"matmul_integer row zp family={family}")
    g = si.rng(77)
    A = si.randint(g, (1, 70, 512), 0, 255, np.uint8)
    B = si.randint(g, (4, 512, 96), -128, 127, np.int8)
    za = si.randint(g, (70, 1), 0, 255, np.uint8)
    with env(QGEMM_FAMILY=family):
        y = q.matmul_integer(to_dev(A), to_dev(B), to_dev(za), None).cpu().numpy()
    np.testing.assert_array_equal(y, oracle.matmul_integer(A, B, za, None))
    A2 = si.randint(g, (2, 33, 259), -128, 127, np.int8)
    B2 = si.randint(g, (259, 40), 0, 255, np.uint8)
    za2 = si.randint(g, (33,), -128, 127, np.int8)
    zb2 = si.randint(g, (40,), 0, 255, np.uint8)
    with env(QGEMM_FAMILY=family):
        y2 = q.matmul_integer_row_zp(to_dev(A2), to_dev(B2), to_dev(za2), to_dev(zb2)).cpu().numpy()
        assert q.last_kernel().startswith("int8_staged")   # K % 64 != 0 with sums
    np.testing.assert_array_equal(y2, oracle.matmul_integer(A2, B2, za2, zb2))


def test_matmul_integer_row_zero_points_full_size():
    """8 x 512 x 2048 x 2048 with per-row activation zero points and the
    per-column weight zero points: every output against the oracle."""
    case("matmul_integer row zp 8x512x2048x2048 every output")
    A, B, zb = si.matmul_integer_inputs(8, 512, 2048, 2048, seed=303)
    g = si.rng(9)
    za = si.randint(g, (512,), 0, 255, np.uint8)
    y = q.matmul_integer(to_dev(A), to_dev(B), to_dev(za), to_dev(zb)).cpu().numpy()
    assert q.last_kernel() == "int8_dma_128x128k128", q.last_kernel()
    np.testing.assert_array_equal(y, oracle.matmul_integer(A, B, za, zb))


@pytest.mark.parametrize("tile", [6, 7, 8])
def test_matmul_integer_k128_stages_fall_back_when_k_is_not_whole_stages(tile):
    """K = 576 is whole 64-byte stages but not 128-byte ones: a zero-point sum
    would see the bytes past K, so the 64-byte sibling of the tile runs."""
    case(f"matmul_integer k128 tile {tile} fallback 2x200x512x576")
    A, B, zb = si.matmul_integer_inputs(2, 200, 512, 576, seed=41 + tile)
    with env(QGEMM_TILE=tile):
        y = q.matmul_integer(to_dev(A), to_dev(B), 128, to_dev(zb)).cpu().numpy()
        assert q.last_kernel().startswith("int8_dma") and not q.last_kernel().endswith("k128"), q.last_kernel()
    np.testing.assert_array_equal(y, oracle.matmul_integer(A, B, 128, zb))

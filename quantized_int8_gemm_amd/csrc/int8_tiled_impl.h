// Tiled int8 x int8 -> int32 matrix-core kernel for gfx950, shared by the
// A8W8 matmul-dequant operator and MatMulInteger.  Included by one
// translation unit per tile shape.
//
// Operator sources (page titles and sections):
//  * "Feature/a8w8 matmul dequant fusion": int8 matmul into an INT32
//    accumulator, cast to FP32, multiply by act_scale per row, then by
//    weight_scale per column, cast to the output type (sequence diagram,
//    "What Changed").
//  * "feat(onnx-to-hip): lower quantized integer conv and matmul", "What":
//    MatMulInteger, Y = sum_k (A - a_zp)(B - b_zp), int32 result, shared B.
//
// One workgroup computes a BM x BN output tile, walking K in chunks of 128:
//  1. Global -> registers.  A rows are read as 16-byte vectors along K.  B
//     given as [K,N] (N contiguous) is read as blocks of 8 rows x 16 bytes,
//     each row a coalesced 16-byte vector; B given as [N,K] is read like A.
//     Loads go through buffer resources that end at the matrix edge, so rows
//     past M (A) or K (B) read as zero without a branch, and all of a chunk's
//     loads stay in flight together.
//  2. Registers -> LDS.  uint8 operands become int8 by flipping bit 7
//     (a - 128) and every byte outside the matrix becomes 0 after that shift,
//     so padding adds nothing to any sum.  A goes in as loaded.  B blocks are
//     transposed in registers with byte permutes so that LDS holds B^T (K
//     contiguous), the layout the matrix core reads; column n of the tile is
//     kept at LDS row (n % 16) * (BN / 16) + n / 16, which makes the
//     transposed writes as conflict-free as the reads.  Rows are 128 bytes
//     with XOR-swizzled 16-byte segments; two stages, so chunk k+1 is fetched
//     into registers while chunk k is multiplied.
//  3. LDS -> matrix cores: v_mfma_i32_16x16x64_i8 with int32 accumulators.
//     When the zero-point correction needs them, the same fragments feed row
//     sums of A and column sums of B through v_dot4 against ones.
//  4. Epilogue from the accumulators: the fp32 cast and the two scale
//     multiplies (each rounded, in that order) with an fp32 or bf16 store
//     (an int32 accumulator input, when given, is added first), or the
//     MatMulInteger correction in wrapping int32 with an int32 store.
#pragma once
#include "device_common.h"
#include "kernels.h"

namespace qg {
namespace tiled {

constexpr int BK = 128;    // K bytes per chunk (8 segments of 16)
constexpr int ROWB = 128;  // LDS row length in bytes
constexpr int GROUP_M = 8;

__device__ __forceinline__ u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

// 16 bytes of a row from column c onward, zero past `cols`, each byte flipped
// by `flip` first.  Byte-wise, for any alignment and leading dimension.
__device__ __forceinline__ u32x4 load16_bytes(const int8_t* rowp, int c, int cols, uint32_t flip) {
    uint32_t d[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        uint32_t w = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int cc = c + q * 4 + b;
            if (cc < cols) w |= (((uint32_t)(uint8_t)rowp[cc] ^ flip) & 0xffu) << (8 * b);
        }
        d[q] = w;
    }
    return u32x4{d[0], d[1], d[2], d[3]};
}

__device__ __forceinline__ u32x4 fix4(u32x4 v, bool valid, uint32_t flip) {
    v = u32x4{v.x ^ flip, v.y ^ flip, v.z ^ flip, v.w ^ flip};
    return valid ? v : zero4();
}

// Byte offset of segment `seg` of LDS row `r`.
__device__ __forceinline__ int lds_off(int r, int seg) { return r * ROWB + ((seg ^ swz(r)) << 4); }

template <int BM, int BN, int WM, int WN, bool B_KMAJOR>
struct Shape {
    static constexpr int WAVES_N = BN / WN;
    static constexpr int NT = (BM / WM) * (BN / WN) * 64;
    static constexpr int FM = WM / 16;
    static constexpr int FN = WN / 16;
    static constexpr int SEGS = BK / 16;
    static constexpr int A_VECS = BM * SEGS / NT;          // A vectors per thread
    static constexpr int B_VECS = BN * SEGS / NT;          // per thread, B as [N,K]
    static constexpr int B_BLOCKS = (BK / 8) * (BN / 16);  // 8x16 blocks, B as [K,N]
    static constexpr int B_BLK_PER_T = (B_BLOCKS + NT - 1) / NT;
    static constexpr int CB = BN / 16;                     // 16-column blocks
    static constexpr int CBH = BN / 128;
    static constexpr bool PERM = !B_KMAJOR;                // transposed B placement
    static_assert(BM * SEGS % NT == 0 && BN * SEGS % NT == 0, "tile/thread mismatch");
    static_assert(BN % 128 == 0, "BN must be a multiple of 128");
    static_assert((NT / SEGS) % 8 == 0, "row step must keep the swizzle");
    static constexpr int LDS_BYTES = 2 * (BM + BN) * ROWB;

    // Block index -> (group of 8 rows, block of 16 columns), ordered so that
    // the 16 lanes of one 8-byte LDS write pass hit 16 distinct bank slots
    // (eight column blocks x two row groups) while each group of 8 lanes
    // reads 128 contiguous bytes of one row from global memory.
    __device__ static void block_coords(int blk, int& rg, int& cb) {
        const int cb_lo = blk & 7;
        const int rg_lo = (blk >> 3) & 1;
        const int rest = blk >> 4;
        rg = (rest / CBH) * 2 + rg_lo;
        cb = (rest % CBH) * 8 + cb_lo;
    }
    // LDS row of B^T -> column of the tile.
    __device__ static int col_of_row(int rho) { return PERM ? (rho % CB) * 16 + rho / CB : rho; }
};

template <int BM, int BN, int WM, int WN, bool B_KMAJOR, bool VEC, int EPI, int ZP>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64)
void int8_tiled_kernel(Int8GemmArgs p) {
    using S = Shape<BM, BN, WM, WN, B_KMAJOR>;
    constexpr int NT = S::NT;
    constexpr bool ROWSUM = (ZP & 1) != 0;
    constexpr bool COLSUM = (ZP & 2) != 0;
    constexpr int NB_ST = B_KMAJOR ? S::B_VECS : 8 * S::B_BLK_PER_T;
    constexpr int STAGE = (BM + BN) * ROWB;
    __shared__ __attribute__((aligned(16))) uint8_t smem[S::LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / S::WAVES_N;
    const int wn = wave % S::WAVES_N;

    const int tiles_m = (p.M + BM - 1) / BM;
    const int tiles_n = (p.N + BN - 1) / BN;
    int tm, tn;
    tile_coords(xcd_remap(blockIdx.x, gridDim.x), tiles_m, tiles_n, GROUP_M, tm, tn);
    const int m0 = tm * BM;
    const int n0 = tn * BN;
    const int bz = blockIdx.y;
    const int rows_a = p.M - m0;  // rows of A inside the matrix, from this tile on
    const int cols_b = p.N - n0;  // columns of B inside the matrix
    const bool a_rows_full = rows_a >= BM;
    const bool b_cols_full = cols_b >= BN;
    const int lda = (int)p.lda, ldb = (int)p.ldb;

    const int8_t* A = p.A + (int64_t)bz * p.a_bstride + (int64_t)m0 * p.lda;
    const int8_t* B = B_KMAJOR ? p.B + (int64_t)bz * p.b_bstride + (int64_t)n0 * p.ldb
                               : p.B + (int64_t)bz * p.b_bstride + n0;
    // Buffer ranges end at the matrix edge (A: last valid row's K bytes; B as
    // [K,N]: row K-1's last column; B as [N,K]: like A).
    const int a_rows = a_rows_full ? BM : rows_a;
    const int b_rows = b_cols_full ? BN : cols_b;
    const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(A, (uint32_t)((a_rows - 1) * lda + p.K));
    const __amdgpu_buffer_rsrc_t b_rsrc = B_KMAJOR
        ? make_rsrc(B, (uint32_t)((b_rows - 1) * ldb + p.K))
        : make_rsrc(B, (uint32_t)((p.K - 1) * ldb + cols_b));

    // Per-thread parts of the load offsets; the rest is uniform.
    const int a_r0 = tid / S::SEGS, a_s = tid % S::SEGS;  // vector i: row a_r0 + i*NT/SEGS
    constexpr int A_RSTEP = NT / S::SEGS;
    const uint32_t a_voff = (uint32_t)(a_r0 * lda + a_s * 16);
    int b_rg = 0, b_cb = 0;
    uint32_t b_voff;
    if constexpr (B_KMAJOR) {
        b_voff = (uint32_t)(a_r0 * ldb + a_s * 16);
    } else {
        S::block_coords(tid, b_rg, b_cb);
        b_voff = (uint32_t)(b_rg * 8 * ldb + b_cb * 16);
    }
    const bool b_active = S::B_BLOCKS % NT == 0 || tid < S::B_BLOCKS;

    u32x4 a_st[S::A_VECS];
    u32x4 b_st[NB_ST];

    // Issue every global load of chunk k0 (no waits in between).
    auto fetch = [&](int k0) {
#pragma unroll
        for (int i = 0; i < S::A_VECS; ++i) {
            if constexpr (VEC) {
                a_st[i] = buffer_load16(a_rsrc, a_voff + (uint32_t)(i * A_RSTEP * lda + k0), 0u);
            } else {
                const int r = a_r0 + i * A_RSTEP;
                a_st[i] = r < rows_a ? load16_bytes(A + (int64_t)r * p.lda, k0 + a_s * 16, p.K, p.a_flip)
                                     : zero4();
            }
        }
        if constexpr (B_KMAJOR) {
#pragma unroll
            for (int i = 0; i < S::B_VECS; ++i) {
                if constexpr (VEC) {
                    b_st[i] = buffer_load16(b_rsrc, b_voff + (uint32_t)(i * A_RSTEP * ldb + k0), 0u);
                } else {
                    const int r = a_r0 + i * A_RSTEP;
                    b_st[i] = r < cols_b ? load16_bytes(B + (int64_t)r * p.ldb, k0 + a_s * 16, p.K, p.b_flip)
                                         : zero4();
                }
            }
        } else {
            static_assert(S::B_BLK_PER_T == 1, "one B block per thread");
            if (b_active) {
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    if constexpr (VEC) {
                        b_st[r] = buffer_load16(b_rsrc, b_voff + (uint32_t)((k0 + r) * ldb), 0u);
                    } else {
                        const int gk = k0 + b_rg * 8 + r;
                        b_st[r] = gk < p.K ? load16_bytes(B + (int64_t)gk * p.ldb, b_cb * 16, cols_b, p.b_flip)
                                           : zero4();
                    }
                }
            }
        }
    };

    // Write the fetched chunk k0 into LDS stage `buf`, applying the uint8
    // shift and zeroing everything outside the matrix.
    auto stash = [&](int buf, int k0) {
        uint8_t* As = smem + buf * STAGE;
        uint8_t* Bs = As + BM * ROWB;
        const bool k_full = k0 + BK <= p.K;
        const bool a_fix = VEC && (!(a_rows_full && k_full) || p.a_flip != 0);
        const bool b_fix = VEC && (!(b_cols_full && k_full) || p.b_flip != 0);
        const bool k_ok = k0 + a_s * 16 < p.K;
#pragma unroll
        for (int i = 0; i < S::A_VECS; ++i) {
            const int r = a_r0 + i * A_RSTEP;
            u32x4 x = a_st[i];
            if (a_fix) x = fix4(x, r < rows_a && k_ok, p.a_flip);
            *reinterpret_cast<u32x4*>(As + lds_off(r, a_s)) = x;
        }
        if constexpr (B_KMAJOR) {
#pragma unroll
            for (int i = 0; i < S::B_VECS; ++i) {
                const int r = a_r0 + i * A_RSTEP;
                u32x4 x = b_st[i];
                if (b_fix) x = fix4(x, r < cols_b && k_ok, p.b_flip);
                *reinterpret_cast<u32x4*>(Bs + lds_off(r, a_s)) = x;
            }
        } else if (b_active) {
            if (b_fix) {
                const bool c_ok = b_cb * 16 < cols_b;
#pragma unroll
                for (int r = 0; r < 8; ++r) b_st[r] = fix4(b_st[r], c_ok && k0 + b_rg * 8 + r < p.K, p.b_flip);
            }
            // Column d*4+c of the block: k bytes rg*8 .. rg*8+7 as (lo, hi),
            // written to LDS row (d*4+c)*CB + cb.
            const int seg = b_rg >> 1, half = b_rg & 1;
            uint8_t* wbase = Bs + b_cb * ROWB + ((seg ^ (b_cb & 7)) << 4) + half * 8;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                uint32_t x[4], lo[4], hi[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) x[i] = (&b_st[i].x)[d];
                transpose4x4_bytes(x, lo);
#pragma unroll
                for (int i = 0; i < 4; ++i) x[i] = (&b_st[4 + i].x)[d];
                transpose4x4_bytes(x, hi);
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    *reinterpret_cast<uint2*>(wbase + (d * 4 + c) * S::CB * ROWB) = make_uint2(lo[c], hi[c]);
            }
        }
    };

    v4i acc[S::FM][S::FN];
#pragma unroll
    for (int i = 0; i < S::FM; ++i)
#pragma unroll
        for (int j = 0; j < S::FN; ++j) acc[i][j] = v4i{0, 0, 0, 0};
    int rs[S::FM];
    int cs[S::FN];
#pragma unroll
    for (int i = 0; i < S::FM; ++i) rs[i] = 0;
#pragma unroll
    for (int j = 0; j < S::FN; ++j) cs[j] = 0;

    const int nk = (p.K + BK - 1) / BK;
    fetch(0);
    stash(0, 0);
    __syncthreads();

    const int l16 = lane & 15;
    // Multiply the chunk held in LDS stage `buf`.
    auto compute = [&](int buf) {
        const uint8_t* As = smem + buf * STAGE + wm * WM * ROWB;
        const uint8_t* Bs = smem + buf * STAGE + BM * ROWB + wn * WN * ROWB;
#pragma unroll
        for (int ks = 0; ks < BK / 64; ++ks) {
            const int off = lds_off(l16, ks * 4 + (lane >> 4));  // same for A and B fragments
            u32x4 bf[S::FN];
#pragma unroll
            for (int j = 0; j < S::FN; ++j) bf[j] = *reinterpret_cast<const u32x4*>(Bs + j * 16 * ROWB + off);
            if constexpr (COLSUM) {
#pragma unroll
                for (int j = 0; j < S::FN; ++j)
                    cs[j] = sum_i8x4(bf[j].w, sum_i8x4(bf[j].z, sum_i8x4(bf[j].y, sum_i8x4(bf[j].x, cs[j]))));
            }
#pragma unroll
            for (int i = 0; i < S::FM; ++i) {
                const u32x4 af = *reinterpret_cast<const u32x4*>(As + i * 16 * ROWB + off);
                if constexpr (ROWSUM)
                    rs[i] = sum_i8x4(af.w, sum_i8x4(af.z, sum_i8x4(af.y, sum_i8x4(af.x, rs[i]))));
#pragma unroll
                for (int j = 0; j < S::FN; ++j) acc[i][j] = mfma_i8_16x16x64(af, bf[j], acc[i][j]);
            }
        }
    };

    // Steady state: fetch chunk kt+1 into registers, multiply chunk kt, then
    // move chunk kt+1 into the other LDS stage.  The last chunk is peeled so
    // the loop body carries no conditionals.
    for (int kt = 0; kt + 1 < nk; ++kt) {
        fetch((kt + 1) * BK);
        compute(kt & 1);
        stash((kt + 1) & 1, (kt + 1) * BK);
        __syncthreads();
    }
    compute((nk - 1) & 1);

    // Complete row / column sums: add the four lane groups (k segments).
    if constexpr (ROWSUM) {
#pragma unroll
        for (int i = 0; i < S::FM; ++i) {
            rs[i] += __shfl_xor(rs[i], 16);
            rs[i] += __shfl_xor(rs[i], 32);
        }
    }
    if constexpr (COLSUM) {
#pragma unroll
        for (int j = 0; j < S::FN; ++j) {
            cs[j] += __shfl_xor(cs[j], 16);
            cs[j] += __shfl_xor(cs[j], 32);
        }
    }

    const int row_base = m0 + wm * WM + 4 * (lane >> 4);
    constexpr int OUT_BYTES = EPI == EPI_BF16 ? 2 : 4;
    char* out = reinterpret_cast<char*>(p.out) + (int64_t)bz * p.o_bstride * OUT_BYTES;

#pragma unroll
    for (int j = 0; j < S::FN; ++j) {
        const int n = n0 + S::col_of_row(wn * WN + j * 16 + l16);
        const bool n_ok = n < p.N;
        float ws = 0.f;
        uint32_t cbn = 0, colt = 0;
        if constexpr (EPI == EPI_I32) {
            int32_t zb = 0;
            if (p.b_zp != nullptr && n_ok) {
                const int idx = n * p.b_zp_stride;
                zb = p.b_zp_u8 ? (int32_t) reinterpret_cast<const uint8_t*>(p.b_zp)[idx]
                               : (int32_t) reinterpret_cast<const int8_t*>(p.b_zp)[idx];
            }
            cbn = (uint32_t)(p.sb - zb);
            colt = (uint32_t)p.K * cbn;
            if constexpr (COLSUM) colt += (uint32_t)cs[j];
        } else {
            if (n_ok) ws = p.weight_scale[n * p.ws_stride];
        }
#pragma unroll
        for (int i = 0; i < S::FM; ++i) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = row_base + i * 16 + r;
                int rsum = 0;
                if constexpr (ROWSUM) rsum = __shfl(rs[i], 4 * (lane >> 4) + r);
                if (!(n_ok && m < p.M)) continue;
                const int64_t o = (int64_t)m * p.ldo + n;
                if constexpr (EPI == EPI_I32) {
                    uint32_t y = (uint32_t)acc[i][j][r];
                    if constexpr (COLSUM) {
                        // ca[m]: per row when a_zp is given, else the scalar
                        uint32_t ca_m = (uint32_t)p.ca;
                        if (p.a_zp != nullptr) {
                            const int idx = (m % p.a_zp_rows) * p.a_zp_stride;
                            const int32_t za = p.a_zp_u8 ? (int32_t) reinterpret_cast<const uint8_t*>(p.a_zp)[idx]
                                                         : (int32_t) reinterpret_cast<const int8_t*>(p.a_zp)[idx];
                            ca_m = (uint32_t)(p.sa - za);
                        }
                        y += ca_m * colt;
                    }
                    if constexpr (ROWSUM) y += cbn * (uint32_t)rsum;
                    reinterpret_cast<int32_t*>(out)[o] = (int32_t)y;
                } else {
                    int32_t v = acc[i][j][r];
                    if (p.acc_in != nullptr)
                        v = (int32_t)((uint32_t)v + (uint32_t)p.acc_in[(int64_t)m * p.ld_acc + n]);
                    float f = (float)v;
                    f = f * p.act_scale[m * p.as_stride];
                    f = f * ws;
                    if constexpr (EPI == EPI_F32) reinterpret_cast<float*>(out)[o] = f;
                    else reinterpret_cast<uint16_t*>(out)[o] = f32_to_bf16_rne(f);
                }
            }
        }
    }
}

template <int BM, int BN, int WM, int WN, bool BKM, bool VEC, int EPI, int ZP>
hipError_t launch_one(const Int8GemmArgs& a, hipStream_t s) {
    const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    dim3 grid(tiles, a.batch);
    hipLaunchKernelGGL((int8_tiled_kernel<BM, BN, WM, WN, BKM, VEC, EPI, ZP>), grid,
                       dim3(Shape<BM, BN, WM, WN, BKM>::NT), 0, s, a);
    return hipGetLastError();
}

// Every variant of one tile shape.  WITH_BYTEWISE: also instantiate the
// byte-wise (any alignment) variants.
template <int BM, int BN, int WM, int WN, bool WITH_BYTEWISE>
hipError_t launch_shape(const Int8GemmArgs& a, bool bkm, bool vec, int epi, int zp, hipStream_t s) {
    if (epi == EPI_I32) {
        if (vec) {
            switch (zp) {
                case 0: return launch_one<BM, BN, WM, WN, false, true, EPI_I32, 0>(a, s);
                case 1: return launch_one<BM, BN, WM, WN, false, true, EPI_I32, 1>(a, s);
                case 2: return launch_one<BM, BN, WM, WN, false, true, EPI_I32, 2>(a, s);
                default: return launch_one<BM, BN, WM, WN, false, true, EPI_I32, 3>(a, s);
            }
        }
        if constexpr (WITH_BYTEWISE) return launch_one<BM, BN, WM, WN, false, false, EPI_I32, 3>(a, s);
        return hipErrorInvalidValue;
    }
    if (vec) {
        if (bkm) return epi == EPI_F32 ? launch_one<BM, BN, WM, WN, true, true, EPI_F32, 0>(a, s)
                                       : launch_one<BM, BN, WM, WN, true, true, EPI_BF16, 0>(a, s);
        return epi == EPI_F32 ? launch_one<BM, BN, WM, WN, false, true, EPI_F32, 0>(a, s)
                              : launch_one<BM, BN, WM, WN, false, true, EPI_BF16, 0>(a, s);
    }
    if constexpr (WITH_BYTEWISE) {
        if (bkm) return epi == EPI_F32 ? launch_one<BM, BN, WM, WN, true, false, EPI_F32, 0>(a, s)
                                       : launch_one<BM, BN, WM, WN, true, false, EPI_BF16, 0>(a, s);
        return epi == EPI_F32 ? launch_one<BM, BN, WM, WN, false, false, EPI_F32, 0>(a, s)
                              : launch_one<BM, BN, WM, WN, false, false, EPI_BF16, 0>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace tiled

}  // namespace qg

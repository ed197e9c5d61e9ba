// Multi-stage int8 x int8 -> int32 matrix-core kernel for gfx950, fed by
// direct global-to-LDS loads.  Shared by the A8W8 matmul-dequant operator
// and MatMulInteger; included by one translation unit per tile shape.
//
// Operator sources (page titles and sections):
//  * "Feature/a8w8 matmul dequant fusion": int8 matmul into an INT32
//    accumulator, cast to FP32, multiply by act_scale per row, then by
//    weight_scale per column, cast to the output type (sequence diagram,
//    "What Changed").
//  * "feat(onnx-to-hip): lower quantized integer conv and matmul", "What":
//    MatMulInteger, Y = sum_k (A - a_zp)(B - b_zp), int32 result, shared B.
//
// One workgroup (four or eight waves) computes a BM x BN output tile, K in
// chunks of 64 bytes held in a ring of STAGES LDS stages:
//  * Loads go global -> LDS directly (buffer_load_dwordx4 ... lds), STAGES-1
//    chunks ahead of the one being multiplied, so that many chunks of
//    memory latency are covered and no register holds staged data.  Each
//    lane's 16 bytes land at consecutive LDS addresses, so the lane picks the
//    global segment whose swizzled home is that address.  Rows past M (A) or
//    K (B) read as zero through the buffer range check.
//  * A fragments (K contiguous) come from ds_read_b128.  B stays as stored,
//    [K rows][N bytes], and its fragments come from ds_read_b64_tr_b8: within
//    each 16-lane group, lanes 2j and 2j+1 point at the two 8-byte halves of
//    k-row j of a 16-column block and lane i receives column i of those eight
//    rows, which is the matrix core's B layout.  Two such reads give a lane
//    its 16 k-bytes.  B given as [N,K] is stored and read like A.
//  * v_mfma_i32_16x16x64_i8 accumulates; uint8 operands are shifted to int8
//    by flipping bit 7 as fragments are read, and the row / column sums the
//    MatMulInteger correction needs come from the same fragments.
//  * Epilogue as in the register-staged kernel, written out through LDS in
//    whole rows.
// This kernel needs K % 64 == 0 whenever an operand is flipped or a row or
// column sum is taken (bytes past K are not cleared); the host routes other
// shapes to the register-staged kernel.
#pragma once
#include "device_common.h"
#include "kernels.h"

namespace qg {
namespace dma {

constexpr int GROUP_M = 8;

// Epilogue codes of this kernel beyond Int8Epilogue: fp32 / bf16 output with
// an int32 accumulator input, so that the plain A8W8 kernels carry no code
// for it.
constexpr int EPI_F32_ACC = 3, EPI_BF16_ACC = 4;

typedef int v2i __attribute__((ext_vector_type(2)));

// Buffer descriptor words for [base, base + bytes); loads past the end give 0.
__device__ __forceinline__ v4i rsrc_words(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    v4i r;
    r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r.y = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
    r.z = __builtin_amdgcn_readfirstlane((int)bytes);
    r.w = 0x00020000;
    return r;
}

// 16 bytes per lane from buffer offset `voff` into LDS at lds_base + 16*lane.
// Written as inline assembly so that the compiler does not wait for these
// loads before every LDS read; the kernel waits for them explicitly.  The
// block sets M0 (the LDS destination) itself, so M0 is declared clobbered:
// the compiler then treats it as redefined here.  M0 is a reserved register,
// which the compiler never saves around an asm statement (hence the
// suppressed warning); in these kernels nothing else uses M0 at all -- every
// M0 reference in their compiled code is this block's own s_mov_b32.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(v4i rsrc, uint32_t voff, uint32_t lds_base) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_base);  // wave-uniform
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :: "v"(voff), "s"(rsrc), "s"(m0) : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt with vmcnt = n and the other counters unconstrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ u32x4 xor4(u32x4 v, uint32_t f) {
    return u32x4{v.x ^ f, v.y ^ f, v.z ^ f, v.w ^ f};
}

// K-contiguous tile (A, or B as [N,K]), rows of BK bytes.
//  * BK = 64 (4 segments of 16): segment s of row r at slot s ^ f(r) with
//    f(r) = bits (r1 ^ r3, r2).  Rows r, r+2, r+4, r+6 then take four
//    distinct slots, and so do rows r, r+4, r+8, r+12.
//  * BK = 128 (8 segments): slot s ^ ((r >> 1) & 7); the 16 rows of a
//    fragment read take 16 distinct (row parity, slot) pairs.
// Adding a multiple of 16 to r leaves the slot unchanged, so fragment blocks
// 16 rows apart share one swizzle.
template <int BK>
__device__ __forceinline__ int kc_slot(int r, int s) {
    if constexpr (BK == 64) return s ^ ((((r >> 1) ^ (r >> 3)) & 1) | ((r >> 1) & 2));
    else return s ^ ((r >> 1) & 7);
}

// [K,N] tile: rows of BN bytes; segment s of k-row r at slot
// s ^ (r & 7) ^ t(r), where t flips bit 3 (BN >= 256) or bit 0 (BN = 128)
// for rows 16..31 of each 32.  A transposed read touches rows 16g+8h+0..7
// for two lane groups g at once; the flip keeps those 16 rows apart.
template <int BN>
__device__ __forceinline__ int kn_slot(int r, int s) {
    const int t = (r >> 4) & 1;
    return s ^ (r & 7) ^ (BN >= 256 ? (t << 3) : t);
}

// SK: split-K.  blockIdx.z is the split; each split multiplies
// p.split_steps * 64 rows of K (whole stages) and leaves its exact int32
// partial tile, with its partial row / column sums when the MatMulInteger
// correction needs them, in the workspace; the split that takes the last
// ticket of its tile adds the others' partials to its own and runs the
// epilogue.  Exchange as in the decode kernel: device-coherent 16-byte stores
// and loads, one atomic ticket per tile in the fixed header, reset by the
// last split.
template <int BM, int BN, int WM, int WN, int STAGES, bool B_KMAJOR, int EPI, int ZP, int FLIP, int BK, bool SK = false>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) void int8_dma_kernel(Int8GemmArgs p) {
    static_assert(BK == 64 || BK == 128, "64 or 128 k-bytes per stage");
    constexpr int KB = BK / 64;                     // 64-k matrix-core blocks per stage
    constexpr int NT = (BM / WM) * (BN / WN) * 64;
    constexpr int ROUND = NT * 16;                  // bytes one load round moves
    constexpr int WAVES_N = BN / WN, WAVES_M = BM / WM;
    constexpr int FM = WM / 16, FN = WN / 16;
    constexpr int A_BYTES = BM * BK, B_BYTES = BN * BK;
    constexpr int STAGE = A_BYTES + B_BYTES;
    constexpr int A_ROUNDS = A_BYTES / ROUND, B_ROUNDS = B_BYTES / ROUND;
    constexpr int LOADS = A_ROUNDS + B_ROUNDS;      // per thread per chunk
    constexpr bool ACC = EPI == EPI_F32_ACC || EPI == EPI_BF16_ACC;   // int32 accumulator input
    constexpr int OUT = ACC ? EPI - EPI_F32_ACC : EPI;                 // EPI_F32, EPI_BF16 or EPI_I32
    constexpr bool ROWSUM = (ZP & 1) != 0, COLSUM = (ZP & 2) != 0;
    constexpr bool FLIP_A = (FLIP & 1) != 0, FLIP_B = (FLIP & 2) != 0;
    static_assert(NT == 256 || NT == 512, "four or eight waves");
    static_assert(A_BYTES % ROUND == 0 && B_BYTES % ROUND == 0, "whole load rounds");
    static_assert(LOADS * (STAGES - 2) < 64, "vmcnt range");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * STAGE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int wm_s = __builtin_amdgcn_readfirstlane(wm);   // the same, known wave-uniform
    const int wn_s = __builtin_amdgcn_readfirstlane(wn);
    const int g = lane >> 4, i16 = lane & 15;

    const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    int tm, tn;
    tile_coords(xcd_remap(blockIdx.x, gridDim.x), tiles_m, tiles_n, GROUP_M, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN, bz = blockIdx.y;
    const int rows_a = p.M - m0 < BM ? p.M - m0 : BM;
    const int cols_b = p.N - n0 < BN ? p.N - n0 : BN;
    const int lda = (int)p.lda, ldb = (int)p.ldb;
    // This workgroup's rows of K: [kbeg, kbeg + Kl).
    const int kbeg = SK ? (int)blockIdx.z * p.split_steps * 64 : 0;
    const int Kl = SK ? (p.K - kbeg < p.split_steps * 64 ? p.K - kbeg : p.split_steps * 64) : p.K;
    const int8_t* A = p.A + (int64_t)bz * p.a_bstride + (int64_t)m0 * p.lda + kbeg;
    const int8_t* B = B_KMAJOR ? p.B + (int64_t)bz * p.b_bstride + (int64_t)n0 * p.ldb + kbeg
                               : p.B + (int64_t)bz * p.b_bstride + (int64_t)kbeg * p.ldb + n0;
    const v4i a_rsrc = rsrc_words(A, (uint32_t)((rows_a - 1) * lda + Kl));
    const v4i b_rsrc = B_KMAJOR ? rsrc_words(B, (uint32_t)((cols_b - 1) * ldb + Kl))
                                : rsrc_words(B, (uint32_t)((Kl - 1) * ldb + (p.N - n0)));
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

    // Per-lane global offsets (chunk 0) of each load round.  Round q of a
    // stage covers LDS bytes [q*ROUND, (q+1)*ROUND); this lane writes the 16
    // bytes at q*ROUND + wave*1024 + lane*16.
    uint32_t a_off[A_ROUNDS], b_off[B_ROUNDS];
#pragma unroll
    for (int q = 0; q < A_ROUNDS; ++q) {
        const int o = q * ROUND + wave * 1024 + lane * 16;
        const int r = o / BK, slot = (o % BK) / 16;
        a_off[q] = (uint32_t)(r * lda + 16 * kc_slot<BK>(r, slot));
    }
#pragma unroll
    for (int q = 0; q < B_ROUNDS; ++q) {
        const int o = q * ROUND + wave * 1024 + lane * 16;
        if constexpr (B_KMAJOR) {
            const int r = o / BK, slot = (o % BK) / 16;
            b_off[q] = (uint32_t)(r * ldb + 16 * kc_slot<BK>(r, slot));
        } else {
            const int r = o / BN, slot = (o % BN) / 16;
            b_off[q] = (uint32_t)(r * ldb + 16 * kn_slot<BN>(r, slot));
        }
    }

    auto issue = [&](int kt, int stage) {
        const uint32_t sbase = lds0 + stage * STAGE + wave * 1024;
        const uint32_t ka = (uint32_t)(kt * BK);
#pragma unroll
        for (int q = 0; q < A_ROUNDS; ++q) dma16(a_rsrc, a_off[q] + ka, sbase + q * ROUND);
        const uint32_t kb = B_KMAJOR ? ka : (uint32_t)(kt * BK * ldb);
#pragma unroll
        for (int q = 0; q < B_ROUNDS; ++q) dma16(b_rsrc, b_off[q] + kb, sbase + A_BYTES + q * ROUND);
    };

    v4i acc[FM][FN];
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int b = 0; b < FN; ++b) acc[a][b] = v4i{0, 0, 0, 0};
    // Row sums of A and column sums of B (after the flips) for the
    // MatMulInteger correction.  The waves that share a row (column) block
    // take turns by k-block, and their partial sums are added through LDS
    // after the loop, so each sum is taken once per tile instead of once per
    // wave.  With 64 x 64 wave tiles, or when only row sums are needed
    // (SUM_MFMA), the row sums run on the matrix cores, as products with an
    // all-ones operand, which leaves the sum of row 16a + i in every register
    // of lane (g, i); elsewhere, and for every column sum, they are per-lane
    // v_dot4 sums completed by shuffles (on the matrix cores they would need
    // more registers than the workgroups per CU allow).  MatMulInteger
    // 8x512x2048x2048 with per-column weight zero points: 26.0 -> 24.1 us;
    // with per-row activation zero points too: 29.2 -> 26.7 us; 8192^3 with
    // per-column weight zero points: 551.7 -> 514.6 us.  All of it wraps mod
    // 2^32 alike.
    constexpr bool SUM_MFMA = FM * FN <= 16 || (ROWSUM && !COLSUM);
    const u32x4 ones = u32x4{0x01010101u, 0x01010101u, 0x01010101u, 0x01010101u};
    int rs[FM], cs[FN];
    v4i rs4[SUM_MFMA && ROWSUM ? FM : 1];
#pragma unroll
    for (int a = 0; a < FM; ++a) rs[a] = 0;
#pragma unroll
    for (int b = 0; b < FN; ++b) cs[b] = 0;
    if constexpr (SUM_MFMA && ROWSUM) {
#pragma unroll
        for (int a = 0; a < FM; ++a) rs4[a] = v4i{0, 0, 0, 0};
    }


    // Fragment read offsets within a stage (per lane; the block index adds an
    // immediate).
    // k-block kb of a stage: A segment 4*kb + g of row i16.
    auto a_rd_at = [&](int kb) { return (wm * WM + i16) * BK + (kc_slot<BK>(i16, 4 * kb + g) << 4); };
    int b_rd = 0;
    if constexpr (B_KMAJOR) {
        b_rd = A_BYTES + (wn * WN + i16) * BK;
    } else {
        // ds_read_b64_tr_b8: lane (g, i) addresses k-row 16g + 8h + i/2,
        // bytes 8*(i&1) .. of the fragment's 16-column segment.
        b_rd = A_BYTES + (16 * g + (i16 >> 1)) * BN + 8 * (i16 & 1);
    }
    // slot = seg ^ b_x for this lane's transposed-read rows (16g + 8h + i/2)
    const int b_x = (i16 >> 1) ^ (BN >= 256 ? ((g & 1) << 3) : (g & 1));

    // B fragments of k-block kb of a stage.
    auto read_b = [&](const uint8_t* S, int kb, u32x4* bf) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            if constexpr (B_KMAJOR) {
                bf[j] = *reinterpret_cast<const u32x4*>(S + b_rd + j * 16 * BK + (kc_slot<BK>(i16, 4 * kb + g) << 4));
            } else {
                const int seg = (wn * WN) / 16 + j;
                const uint8_t* base = S + b_rd + kb * 64 * BN + ((seg ^ b_x) << 4);
                const v2i lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (__attribute__((address_space(3))) v2i*)(base));
                const v2i hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (__attribute__((address_space(3))) v2i*)(base + 8 * BN));
                bf[j] = u32x4{(uint32_t)lo.x, (uint32_t)lo.y, (uint32_t)hi.x, (uint32_t)hi.y};
            }
        }
    };

    // Every k-block's B fragments are read at the start of the stage (the
    // first k-block's, then its first A fragment, then the rest), and the A
    // fragments one block ahead run on across the k-block boundary, so no
    // k-block waits for reads issued just before its first multiply.
    // The next chunk's global->LDS loads (next_kt >= 0) are issued right
    // after this stage's first fragment reads, so those reads start as soon
    // as the stage is ready.
    auto compute = [&](int stage, int next_kt, int kt) {
        const uint8_t* S = smem + stage * STAGE;
        u32x4 bfs[KB][FN];
        read_b(S, 0, bfs[0]);
        u32x4 af_next = *reinterpret_cast<const u32x4*>(S + a_rd_at(0));
#pragma unroll
        for (int kb = 1; kb < KB; ++kb) read_b(S, kb, bfs[kb]);
        __builtin_amdgcn_sched_barrier(0);
        if (next_kt >= 0) issue(next_kt, next_kt % STAGES);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            u32x4* bf = bfs[kb];
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                if constexpr (FLIP_B) bf[j] = xor4(bf[j], 0x80808080u);
                if constexpr (COLSUM) {
                    if ((kt * KB + kb) % WAVES_M == wm_s)
                        cs[j] = sum_i8x4(bf[j].w, sum_i8x4(bf[j].z, sum_i8x4(bf[j].y, sum_i8x4(bf[j].x, cs[j]))));
                }
            }
            const int a_rd = a_rd_at(kb);
#pragma unroll
            for (int a = 0; a < FM; ++a) {
                u32x4 af = af_next;
                if (a + 1 < FM) af_next = *reinterpret_cast<const u32x4*>(S + a_rd + (a + 1) * 16 * BK);
                else if (kb + 1 < KB) af_next = *reinterpret_cast<const u32x4*>(S + a_rd_at(kb + 1));
                __builtin_amdgcn_sched_barrier(0);  // keep the next read ahead of this block's MFMAs
                if constexpr (FLIP_A) af = xor4(af, 0x80808080u);
                if constexpr (ROWSUM) {
                    // wn_s is wave-uniform in a scalar register, so this is a
                    // scalar branch around the sum: a matrix instruction under
                    // an EXEC mask alone would still run
                    if ((kt * KB + kb) % WAVES_N == wn_s) {
                        if constexpr (SUM_MFMA) rs4[a] = mfma_i8_16x16x64(ones, af, rs4[a]);
                        else rs[a] = sum_i8x4(af.w, sum_i8x4(af.z, sum_i8x4(af.y, sum_i8x4(af.x, rs[a]))));
                    }
                }
#pragma unroll
                for (int b = 0; b < FN; ++b) acc[a][b] = mfma_i8_16x16x64(bf[b], af, acc[a][b]);
            }
        }
    };

    // The A8W8 epilogue's scales, loaded now so their latency hides behind
    // the main loop: rows wm*WM + 16a + i16 and columns wn*WN + 16b + i16
    // (each lane fetches the column scales its neighbours need).
    float as_r[OUT == EPI_I32 ? 1 : FM], ws_c[OUT == EPI_I32 ? 1 : FN];
    // MatMulInteger: cb for column wn*WN + 16b + i16 (sb - b_zp[n]), likewise.
    int32_t cb_c[OUT == EPI_I32 ? FN : 1];
    if constexpr (OUT == EPI_I32) {
#pragma unroll
        for (int b = 0; b < FN; ++b) {
            const int n = n0 + wn * WN + b * 16 + i16;
            int32_t zb = 0;
            if (p.b_zp != nullptr && n < p.N) {
                const int idx = n * p.b_zp_stride;
                zb = p.b_zp_u8 ? (int32_t) reinterpret_cast<const uint8_t*>(p.b_zp)[idx]
                               : (int32_t) reinterpret_cast<const int8_t*>(p.b_zp)[idx];
            }
            cb_c[b] = p.sb - zb;
        }
    }
    if constexpr (OUT != EPI_I32) {
#pragma unroll
        for (int a = 0; a < FM; ++a) {
            const int m = m0 + wm * WM + a * 16 + i16;
            as_r[a] = m < p.M ? p.act_scale[m * p.as_stride] : 0.f;
        }
#pragma unroll
        for (int b = 0; b < FN; ++b) {
            const int n = n0 + wn * WN + b * 16 + i16;
            ws_c[b] = n < p.N ? p.weight_scale[n * p.ws_stride] : 0.f;
        }
    }

    const int nk = (Kl + BK - 1) / BK;
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
        if (s < nk) issue(s, s);
    for (int kt = 0; kt < nk; ++kt) {
        // chunk kt has landed once at most the later chunks are outstanding
        if (kt + STAGES - 2 < nk) wait_vmcnt<LOADS * (STAGES - 2)>();
        else if (kt + 1 < nk) wait_vmcnt<LOADS>();
        else wait_vmcnt<0>();
        __syncthreads();
        compute(kt % STAGES, kt + STAGES - 1 < nk ? kt + STAGES - 1 : -1, kt);
    }

    // Complete row / column sums: add the four lane groups (k segments) of
    // the v_dot4 sums, then the partial sums of the waves that took turns on
    // a row or column block, through LDS.
    if constexpr (ROWSUM && !SUM_MFMA) {
#pragma unroll
        for (int a = 0; a < FM; ++a) {
            rs[a] += __shfl_xor(rs[a], 16);
            rs[a] += __shfl_xor(rs[a], 32);
        }
    }
    if constexpr (COLSUM) {
#pragma unroll
        for (int b = 0; b < FN; ++b) {
            cs[b] += __shfl_xor(cs[b], 16);
            cs[b] += __shfl_xor(cs[b], 32);
        }
    }
    if constexpr (ROWSUM || COLSUM) {
        __shared__ int rs_part[ROWSUM ? WAVES_N : 1][BM];
        __shared__ int cs_part[COLSUM ? WAVES_M : 1][BN];
        if (g == 0) {
            if constexpr (ROWSUM) {
#pragma unroll
                for (int a = 0; a < FM; ++a) rs_part[wn][wm * WM + 16 * a + i16] = SUM_MFMA ? rs4[a][0] : rs[a];
            }
            if constexpr (COLSUM) {
#pragma unroll
                for (int b = 0; b < FN; ++b) cs_part[wm][wn * WN + 16 * b + i16] = cs[b];
            }
        }
        __syncthreads();
        if constexpr (ROWSUM) {
#pragma unroll
            for (int a = 0; a < FM; ++a) {
                uint32_t t = 0u;
#pragma unroll
                for (int w = 0; w < WAVES_N; ++w) t += (uint32_t)rs_part[w][wm * WM + 16 * a + i16];
                rs[a] = (int)t;
            }
        }
        if constexpr (COLSUM) {
#pragma unroll
            for (int b = 0; b < FN; ++b) {
                uint32_t t = 0u;
#pragma unroll
                for (int w = 0; w < WAVES_M; ++w) t += (uint32_t)cs_part[w][wn * WN + 16 * b + i16];
                cs[b] = (int)t;
            }
        }
    }

    // Split-K exchange (after the row / column sums of this split's K range
    // are complete): each split stores its accumulators and sums, lane-major;
    // the split that takes its tile's last ticket adds the others' into its
    // own registers and runs the epilogue.
    if constexpr (SK) {
        const int S = (int)gridDim.z, sk = (int)blockIdx.z;
        if (S > 1) {
            constexpr int COHERENT = 16;   // sc1: device scope
            constexpr int NWV = (BM / WM) * (BN / WN);
            constexpr int TILE_BYTES = BM * BN * 4;
            constexpr int SUMS = (ROWSUM ? FM : 0) + (COLSUM ? FN : 0);
            constexpr int SUMS_V4 = (SUMS + 3) / 4;
            constexpr int SLOT = TILE_BYTES + SUMS_V4 * NWV * 64 * 16;
            const int tile = tm * tiles_n + tn;   // < SKINNY_MAX_TICKETS (host plan)
            int* tickets = reinterpret_cast<int*>(p.workspace);
            char* part = reinterpret_cast<char*>(p.workspace) + SKINNY_TICKET_BYTES + (size_t)tile * S * SLOT;
            const __amdgpu_buffer_rsrc_t p_rsrc = make_rsrc(part, (uint32_t)(S * SLOT));
            // fragment (a, b) of wave w at ((w * FM + a) * FN + b) * 1024 + 16 * lane; sum vector q
            // at TILE_BYTES + ((q * NWV + w) * 64 + lane) * 16
            auto frag_off = [&](int s2, int a, int b) {
                return (uint32_t)(s2 * SLOT + ((wave * FM + a) * FN + b) * 1024 + 16 * lane);
            };
            auto sums_off = [&](int s2, int q) {
                return (uint32_t)(s2 * SLOT + TILE_BYTES + ((q * NWV + wave) * 64 + lane) * 16);
            };
            int sv[SUMS_V4 * 4 > 0 ? SUMS_V4 * 4 : 1];
#pragma unroll
            for (int i = 0; i < SUMS_V4 * 4; ++i) sv[i] = 0;
            if constexpr (ROWSUM) {
#pragma unroll
                for (int a = 0; a < FM; ++a) sv[a] = rs[a];
            }
            if constexpr (COLSUM) {
#pragma unroll
                for (int b = 0; b < FN; ++b) sv[(ROWSUM ? FM : 0) + b] = cs[b];
            }
#pragma unroll
            for (int a = 0; a < FM; ++a)
#pragma unroll
                for (int b = 0; b < FN; ++b)
                    __builtin_amdgcn_raw_buffer_store_b128(acc[a][b], p_rsrc, frag_off(sk, a, b), 0, COHERENT);
#pragma unroll
            for (int q = 0; q < SUMS_V4; ++q)
                __builtin_amdgcn_raw_buffer_store_b128(v4i{sv[4 * q], sv[4 * q + 1], sv[4 * q + 2], sv[4 * q + 3]},
                                                       p_rsrc, sums_off(sk, q), 0, COHERENT);
            __builtin_amdgcn_s_waitcnt(0);
            __shared__ int ticket;
            __syncthreads();
            if (tid == 0) ticket = __hip_atomic_fetch_add(&tickets[tile], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __syncthreads();
            if (ticket != S - 1) return;
            for (int s2 = 0; s2 < S; ++s2) {
                if (s2 == sk) continue;
                v4i v[FM][FN];
#pragma unroll
                for (int a = 0; a < FM; ++a)
#pragma unroll
                    for (int b = 0; b < FN; ++b)
                        v[a][b] = __builtin_bit_cast(
                            v4i, __builtin_amdgcn_raw_buffer_load_b128(p_rsrc, frag_off(s2, a, b), 0, COHERENT));
                v4i w[SUMS_V4 > 0 ? SUMS_V4 : 1];
#pragma unroll
                for (int q = 0; q < SUMS_V4; ++q)
                    w[q] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(p_rsrc, sums_off(s2, q), 0, COHERENT));
#pragma unroll
                for (int a = 0; a < FM; ++a)
#pragma unroll
                    for (int b = 0; b < FN; ++b)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            acc[a][b][r] = (int)((uint32_t)acc[a][b][r] + (uint32_t)v[a][b][r]);
#pragma unroll
                for (int i = 0; i < SUMS_V4 * 4; ++i) sv[i] = (int)((uint32_t)sv[i] + (uint32_t)w[i / 4][i % 4]);
            }
            if constexpr (ROWSUM) {
#pragma unroll
                for (int a = 0; a < FM; ++a) rs[a] = sv[a];
            }
            if constexpr (COLSUM) {
#pragma unroll
                for (int b = 0; b < FN; ++b) cs[b] = sv[(ROWSUM ? FM : 0) + b];
            }
            if (tid == 0) __hip_atomic_store(&tickets[tile], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }

    // With the operands swapped in the MFMA, register r of block (a, b) in
    // lane (g, i) holds row 16a + i, column 16b + 4g + r of the wave's tile:
    // four consecutive columns.  Stored straight to memory these leave as 32-
    // or 64-byte pieces of rows; with stage_out set the finished values go
    // through LDS (free once the last chunk is multiplied) and leave as whole
    // rows, 16 bytes per lane: plain stores (stage_out 1) for grids of several
    // rounds, whose lines L2 merges long before the end, or non-temporal ones
    // (stage_out 2) for single-round grids that write everything at once.  The direct stores are non-temporal: small
    // grids finish all their tiles at once, and an output left in L2 would be
    // written back in one burst when the kernel ends (MatMulInteger
    // 4096x2048x2048: 32 -> 25 us).  The staged path serves large grids whose
    // earlier tiles' lines leave L2 long before the end; there plain stores
    // measured 1% faster.  Staging row pitch is BN outputs; the 16-byte chunk c of
    // staged row r sits at chunk c ^ (r & 15), so the 16 rows one fragment
    // store touches fall in distinct banks, and so do the chunks of a row read
    // back.  A tile larger than the stage ring is staged in passes of whole
    // wave rows.
    constexpr int OUT_BYTES = OUT == EPI_BF16 ? 2 : 4;
    constexpr int ROW_BYTES = BN * OUT_BYTES;
    constexpr int CPR = ROW_BYTES / 16;              // 16-byte chunks per row
    constexpr int PER_CHUNK = 16 / OUT_BYTES;        // outputs per chunk
    constexpr int PASSES = (BM * ROW_BYTES + STAGES * STAGE - 1) / (STAGES * STAGE);
    static_assert(CPR >= 16, "staging swizzle spans 16 chunks");
    static_assert(WAVES_M % PASSES == 0, "passes of whole wave rows");
    constexpr int PASS_ROWS = BM / PASSES, PASS_WAVE_ROWS = WAVES_M / PASSES;
    static_assert((PASS_ROWS * CPR) % NT == 0, "whole store rounds");
    constexpr int STORE_ROUNDS = PASS_ROWS * CPR / NT;

    char* out = reinterpret_cast<char*>(p.out) + (int64_t)bz * p.o_bstride * OUT_BYTES;
    const bool vec_out = ((p.ldo * OUT_BYTES) % 16 == 0) && ((reinterpret_cast<uintptr_t>(out) & 15) == 0);

    // ca[m] of the MatMulInteger correction: per row when a_zp is given.
    auto row_ca = [&](int m) -> uint32_t {
        if (p.a_zp == nullptr) return (uint32_t)p.ca;
        const int idx = (m % p.a_zp_rows) * p.a_zp_stride;
        const int32_t za = p.a_zp_u8 ? (int32_t) reinterpret_cast<const uint8_t*>(p.a_zp)[idx]
                                     : (int32_t) reinterpret_cast<const int8_t*>(p.a_zp)[idx];
        return (uint32_t)(p.sa - za);
    };
    // A8W8 accumulator input at row m, columns n .. n+3 (zero past N).
    const bool acc_vec = p.acc_in != nullptr && p.ld_acc % 4 == 0 &&
                         (reinterpret_cast<uintptr_t>(p.acc_in) & 15) == 0;
    auto acc_in4 = [&](int m, int n) -> v4i {
        const int32_t* src = p.acc_in + (int64_t)m * p.ld_acc + n;
        if (acc_vec && n + 4 <= p.N) return __builtin_nontemporal_load(reinterpret_cast<const v4i*>(src));
        v4i r = v4i{0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (n + e < p.N) r[e] = src[e];
        return r;
    };

    if (!p.stage_out) {
        // Direct stores from the fragments (small grids, where the staging
        // round trip costs more latency than the wider stores save).
        const bool vec4 = (p.ldo % 4 == 0) && ((reinterpret_cast<uintptr_t>(out) & 15) == 0);
#pragma unroll
        for (int b = 0; b < FN; ++b) {
            const int nq = n0 + wn * WN + b * 16 + 4 * g;   // first of this lane's four columns
            uint32_t colt[4] = {0u, 0u, 0u, 0u}, cbn[4] = {0u, 0u, 0u, 0u};
            float ws[4] = {0.f, 0.f, 0.f, 0.f};
            if constexpr (OUT == EPI_I32) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    cbn[r] = (uint32_t)__shfl(cb_c[b], 4 * g + r);
                    colt[r] = (uint32_t)p.K * cbn[r];
                    if constexpr (COLSUM) colt[r] += (uint32_t)__shfl(cs[b], 4 * g + r);
                }
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) ws[r] = __shfl(ws_c[b], 4 * g + r);
            }
#pragma unroll
            for (int a = 0; a < FM; ++a) {
                const int m = m0 + wm * WM + a * 16 + i16;
                if (m >= p.M || nq >= p.N) continue;
                const int64_t o = (int64_t)m * p.ldo + nq;
                const bool full = nq + 4 <= p.N && vec4;
                if constexpr (OUT == EPI_I32) {
                    const uint32_t ca_m = COLSUM ? row_ca(m) : 0u;
                    uint32_t y[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        y[r] = (uint32_t)acc[a][b][r];
                        if constexpr (COLSUM) y[r] += ca_m * colt[r];
                        if constexpr (ROWSUM) y[r] += cbn[r] * (uint32_t)rs[a];
                    }
                    int32_t* dst = reinterpret_cast<int32_t*>(out) + o;
                    if (full) {
                        __builtin_nontemporal_store(v4i{(int)y[0], (int)y[1], (int)y[2], (int)y[3]}, reinterpret_cast<v4i*>(dst));
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (nq + r < p.N) dst[r] = (int32_t)y[r];
                    }
                } else {
                    const float as = as_r[a];
                    v4i v = acc[a][b];
                    if constexpr (ACC) {
                        const v4i ai = acc_in4(m, nq);
#pragma unroll
                        for (int r = 0; r < 4; ++r) v[r] = (int)((uint32_t)v[r] + (uint32_t)ai[r]);
                    }
                    float f[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        f[r] = (float)v[r];
                        f[r] = f[r] * as;
                        f[r] = f[r] * ws[r];
                    }
                    if constexpr (OUT == EPI_F32) {
                        float* dst = reinterpret_cast<float*>(out) + o;
                        if (full) {
                            __builtin_nontemporal_store(v4f{f[0], f[1], f[2], f[3]}, reinterpret_cast<v4f*>(dst));
                        } else {
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                if (nq + r < p.N) dst[r] = f[r];
                        }
                    } else {
                        uint16_t h[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r) h[r] = f32_to_bf16_rne(f[r]);
                        uint16_t* dst = reinterpret_cast<uint16_t*>(out) + o;
                        if (full) {
                            __builtin_nontemporal_store(
                                v2i{(int)((uint32_t)h[0] | ((uint32_t)h[1] << 16)), (int)((uint32_t)h[2] | ((uint32_t)h[3] << 16))},
                                reinterpret_cast<v2i*>(dst));
                        } else {
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                if (nq + r < p.N) dst[r] = h[r];
                        }
                    }
                }
            }
        }
        return;
    }

    // Per-column epilogue terms for fragment column block b.
    uint32_t colt[FN][OUT == EPI_I32 ? 4 : 1], cbn[FN][OUT == EPI_I32 ? 4 : 1];
    float ws[FN][OUT == EPI_I32 ? 1 : 4];
#pragma unroll
    for (int b = 0; b < FN; ++b) {
        // this lane's four columns are wn*WN + 16b + 4g + r
        if constexpr (OUT == EPI_I32) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                cbn[b][r] = (uint32_t)__shfl(cb_c[b], 4 * g + r);
                colt[b][r] = (uint32_t)p.K * cbn[b][r];
                if constexpr (COLSUM) colt[b][r] += (uint32_t)__shfl(cs[b], 4 * g + r);
            }
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) ws[b][r] = __shfl(ws_c[b], 4 * g + r);
        }
    }

    // Accumulator input (A8W8 _acc) with 16-byte rows: the four vectors of
    // fragment row a are loaded together before any is used, so a wave waits
    // for one load latency per row instead of one per fragment (8192^3 bf16:
    // 498 -> 491 us; loading them a row ahead measured the same).  The loads
    // go through a buffer window over rows [m0, m0 + rows_a) from column n0,
    // with no per-element checks: the window ends at the tile's last element
    // the caller must provide (row m0 + rows_a - 1, column N - 1), so rows
    // past M and columns past N of the last row read 0 and nothing outside
    // the (M-1)*ld_acc + N elements of acc_in is touched.  With N a multiple
    // of 4 (and ld_acc too) no vector straddles that end; columns past N are
    // never stored.  Other accumulator layouts load per fragment, as the
    // direct path does.
    const bool acc_win = ACC && acc_vec && p.N % 4 == 0 && (int64_t)BM * p.ld_acc * 4 < ((int64_t)1 << 32) - 64;
    const __amdgpu_buffer_rsrc_t acc_rsrc =
        make_rsrc(acc_win ? p.acc_in + (int64_t)m0 * p.ld_acc + n0 : p.acc_in,
                  acc_win ? (uint32_t)(((int64_t)(rows_a - 1) * p.ld_acc + (p.N - n0)) * 4) : 0u);
    v4i ai_buf[ACC ? FN : 1];
    auto load_acc_row = [&](int a, v4i* dst) {
        const uint32_t r = (uint32_t)(wm * WM + a * 16 + i16);
#pragma unroll
        for (int b = 0; b < FN; ++b) {
            const uint32_t c = (uint32_t)(wn * WN + b * 16 + 4 * g);
            // non-temporal: each accumulator is read once, and cached reads
            // of them evict weight panels (8192^3 bf16: 482.2 -> 452.2 us)
            dst[b] = __builtin_bit_cast(v4i, buffer_load16_nt(acc_rsrc, (r * (uint32_t)p.ld_acc + c) * 4u));
        }
    };

    __syncthreads();   // every wave is done reading the stage ring
#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
        if (pass > 0) __syncthreads();   // previous pass has been read back
        if (wm / PASS_WAVE_ROWS == pass) {
#pragma unroll
            for (int a = 0; a < FM; ++a) {
                const int row = (wm % PASS_WAVE_ROWS) * WM + a * 16 + i16;
                const int m = m0 + wm * WM + a * 16 + i16;   // output row (may be >= M)
                uint8_t* srow = smem + row * ROW_BYTES;
                uint32_t ca_m = 0u;
                if constexpr (OUT == EPI_I32 && COLSUM) ca_m = m < p.M ? row_ca(m) : 0u;
                if constexpr (ACC)
                    if (acc_win) load_acc_row(a, ai_buf);
                (void)m;
#pragma unroll
                for (int b = 0; b < FN; ++b) {
                    const int col = wn * WN + b * 16 + 4 * g;
                    if constexpr (OUT == EPI_I32) {
                        uint32_t y[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            y[r] = (uint32_t)acc[a][b][r];
                            if constexpr (COLSUM) y[r] += ca_m * colt[b][r];
                            if constexpr (ROWSUM) y[r] += cbn[b][r] * (uint32_t)rs[a];
                        }
                        const int c = col / 4;
                        *reinterpret_cast<u32x4*>(srow + ((c ^ (row & 15)) << 4)) = u32x4{y[0], y[1], y[2], y[3]};
                    } else {
                        const float as = as_r[a];
                        v4i v = acc[a][b];
                        if constexpr (ACC) {
                            if (acc_win) {
                                const v4i ai = ai_buf[b];
#pragma unroll
                                for (int r = 0; r < 4; ++r) v[r] = (int)((uint32_t)v[r] + (uint32_t)ai[r]);
                            } else if (m < p.M && n0 + col < p.N) {
                                const v4i ai = acc_in4(m, n0 + col);
#pragma unroll
                                for (int r = 0; r < 4; ++r) v[r] = (int)((uint32_t)v[r] + (uint32_t)ai[r]);
                            }
                        }
                        float f[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            f[r] = (float)v[r];
                            f[r] = f[r] * as;
                            f[r] = f[r] * ws[b][r];
                        }
                        if constexpr (OUT == EPI_F32) {
                            const int c = col / 4;
                            *reinterpret_cast<u32x4*>(srow + ((c ^ (row & 15)) << 4)) =
                                u32x4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                                      __float_as_uint(f[3])};
                        } else {
                            const int c = col / 8, half = (col / 4) & 1;
                            uint16_t h[4];
#pragma unroll
                            for (int r = 0; r < 4; ++r) h[r] = f32_to_bf16_rne(f[r]);
                            *reinterpret_cast<uint2*>(srow + ((c ^ (row & 15)) << 4) + 8 * half) =
                                make_uint2((uint32_t)h[0] | ((uint32_t)h[1] << 16),
                                           (uint32_t)h[2] | ((uint32_t)h[3] << 16));
                        }
                    }
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < STORE_ROUNDS; ++q) {
            const int idx = q * NT + tid;
            const int row = idx / CPR, c = idx % CPR;
            const int m = m0 + pass * PASS_ROWS + row, n = n0 + c * PER_CHUNK;
            const u32x4 v = *reinterpret_cast<const u32x4*>(smem + row * ROW_BYTES + ((c ^ (row & 15)) << 4));
            if (m >= p.M || n >= p.N) continue;
            char* dst = out + ((int64_t)m * p.ldo + n) * OUT_BYTES;
            if (vec_out && n + PER_CHUNK <= p.N) {
                if (p.stage_out == 2)
                    __builtin_nontemporal_store(v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w}, reinterpret_cast<v4i*>(dst));
                else
                    *reinterpret_cast<u32x4*>(dst) = v;
            } else {
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < PER_CHUNK; ++e) {
                    if (n + e >= p.N) break;
                    if constexpr (OUT_BYTES == 4)
                        reinterpret_cast<uint32_t*>(dst)[e] = w[e];
                    else
                        reinterpret_cast<uint16_t*>(dst)[e] = (uint16_t)(w[e / 2] >> (16 * (e & 1)));
                }
            }
        }
    }
}

template <int BM, int BN, int WM, int WN, int ST, bool BKM, int EPI, int ZP, int FLIP, int BK, bool SK = false>
hipError_t launch_one(const Int8GemmArgs& a, hipStream_t s) {
    const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    hipLaunchKernelGGL((int8_dma_kernel<BM, BN, WM, WN, ST, BKM, EPI, ZP, FLIP, BK, SK>),
                       dim3(tiles, a.batch, SK ? a.splits : 1), dim3((BM / WM) * (BN / WN) * 64), 0, s, a);
    return hipGetLastError();
}

// The three-stage kernel, split over K when a.splits > 1 (a.split_steps
// 64-row steps per split, a whole number of stages; batch 1; a.workspace as
// the host plan sized it): A8W8 (B as [K,N] or [N,K]) or MatMulInteger.
template <int BM, int BN, int WM, int WN, int ST, int BK>
hipError_t launch_split(const Int8GemmArgs& a, bool bkm, int epi, int zp, hipStream_t s) {
    if (a.batch != 1 || (a.splits > 1 && a.workspace == nullptr) || (a.split_steps * 64) % BK != 0 ||
        ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN) > SKINNY_MAX_TICKETS)
        return hipErrorInvalidValue;
    if (epi == EPI_I32) {   // MatMulInteger: B as [K,N], any flips and sums
        const int flip = (a.a_flip ? 1 : 0) | (a.b_flip ? 2 : 0);
        switch (zp * 4 + flip) {
#define QG_SPLIT_I32(Z, F) \
    case Z * 4 + F: return launch_one<BM, BN, WM, WN, ST, false, EPI_I32, Z, F, BK, true>(a, s);
            QG_SPLIT_I32(0, 0) QG_SPLIT_I32(0, 1) QG_SPLIT_I32(0, 2) QG_SPLIT_I32(0, 3)
            QG_SPLIT_I32(1, 0) QG_SPLIT_I32(1, 1) QG_SPLIT_I32(1, 2) QG_SPLIT_I32(1, 3)
            QG_SPLIT_I32(2, 0) QG_SPLIT_I32(2, 1) QG_SPLIT_I32(2, 2) QG_SPLIT_I32(2, 3)
            QG_SPLIT_I32(3, 0) QG_SPLIT_I32(3, 1) QG_SPLIT_I32(3, 2) QG_SPLIT_I32(3, 3)
#undef QG_SPLIT_I32
            default: return hipErrorInvalidValue;
        }
    }
    const bool f32 = epi == EPI_F32;
    if (a.acc_in != nullptr) {
        if (bkm) return f32 ? launch_one<BM, BN, WM, WN, ST, true, EPI_F32_ACC, 0, 0, BK, true>(a, s)
                            : launch_one<BM, BN, WM, WN, ST, true, EPI_BF16_ACC, 0, 0, BK, true>(a, s);
        return f32 ? launch_one<BM, BN, WM, WN, ST, false, EPI_F32_ACC, 0, 0, BK, true>(a, s)
                   : launch_one<BM, BN, WM, WN, ST, false, EPI_BF16_ACC, 0, 0, BK, true>(a, s);
    }
    if (bkm) return f32 ? launch_one<BM, BN, WM, WN, ST, true, EPI_F32, 0, 0, BK, true>(a, s)
                        : launch_one<BM, BN, WM, WN, ST, true, EPI_BF16, 0, 0, BK, true>(a, s);
    return f32 ? launch_one<BM, BN, WM, WN, ST, false, EPI_F32, 0, 0, BK, true>(a, s)
               : launch_one<BM, BN, WM, WN, ST, false, EPI_BF16, 0, 0, BK, true>(a, s);
}

template <int BM, int BN, int WM, int WN, int ST, int EPI, int ZP, int BK>
hipError_t by_flip(const Int8GemmArgs& a, int flip, hipStream_t s) {
    switch (flip) {
        case 0: return launch_one<BM, BN, WM, WN, ST, false, EPI, ZP, 0, BK>(a, s);
        case 1: return launch_one<BM, BN, WM, WN, ST, false, EPI, ZP, 1, BK>(a, s);
        case 2: return launch_one<BM, BN, WM, WN, ST, false, EPI, ZP, 2, BK>(a, s);
        default: return launch_one<BM, BN, WM, WN, ST, false, EPI, ZP, 3, BK>(a, s);
    }
}

// Every variant of one tile configuration: A8W8 (fp32 / bf16 out, B as
// [K,N] or [N,K]) and MatMulInteger (B as [K,N], any flips and sums).
template <int BM, int BN, int WM, int WN, int ST, int BK = 64>
hipError_t launch_shape(const Int8GemmArgs& a, bool bkm, int epi, int zp, hipStream_t s) {
    const int flip = (a.a_flip ? 1 : 0) | (a.b_flip ? 2 : 0);
    if (epi == EPI_I32) {
        switch (zp) {
            case 0: return by_flip<BM, BN, WM, WN, ST, EPI_I32, 0, BK>(a, flip, s);
            case 1: return by_flip<BM, BN, WM, WN, ST, EPI_I32, 1, BK>(a, flip, s);
            case 2: return by_flip<BM, BN, WM, WN, ST, EPI_I32, 2, BK>(a, flip, s);
            default: return by_flip<BM, BN, WM, WN, ST, EPI_I32, 3, BK>(a, flip, s);
        }
    }
    if (a.acc_in != nullptr) {
        if (bkm) return epi == EPI_F32 ? launch_one<BM, BN, WM, WN, ST, true, EPI_F32_ACC, 0, 0, BK>(a, s)
                                       : launch_one<BM, BN, WM, WN, ST, true, EPI_BF16_ACC, 0, 0, BK>(a, s);
        return epi == EPI_F32 ? launch_one<BM, BN, WM, WN, ST, false, EPI_F32_ACC, 0, 0, BK>(a, s)
                              : launch_one<BM, BN, WM, WN, ST, false, EPI_BF16_ACC, 0, 0, BK>(a, s);
    }
    if (bkm) return epi == EPI_F32 ? launch_one<BM, BN, WM, WN, ST, true, EPI_F32, 0, 0, BK>(a, s)
                                   : launch_one<BM, BN, WM, WN, ST, true, EPI_BF16, 0, 0, BK>(a, s);
    return epi == EPI_F32 ? launch_one<BM, BN, WM, WN, ST, false, EPI_F32, 0, 0, BK>(a, s)
                          : launch_one<BM, BN, WM, WN, ST, false, EPI_BF16, 0, 0, BK>(a, s);
}

}  // namespace dma
}  // namespace qg

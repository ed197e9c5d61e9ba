// W8A32 on the bf16 matrix cores of gfx950: the fp32 operand is split
// exactly into three bfloat16 parts, a = hi + lo + lo2, and the int8 weight
// is exact in bfloat16, so every product a_k * b_k is formed without error
// and only the fp32 accumulation rounds.
//
// Operator: "feat(PULPOpen): matmul that dequantises an int8 weight
// in-kernel", section "The kernel": sum_k a_k (b_k - zp) scale equals
// scale (sum_k a_k b_k - zp sum_k a_k).  S1 = sum_k a_k b_k runs on
// v_mfma_f32_16x16x32_bf16 as three products per k-block (one per part of A)
// into the same fp32 accumulators; S2 = sum_k a_k is taken in fp32 from the
// staged values; the epilogue is scale * (S1 - zp * S2), or scale * S1 when
// zp == 0.  The dequantised weight is never formed.
//
// Why the split is exact: hi keeps the top 8 significant bits of a (its bit
// pattern with the low 16 bits cleared), the remainder a - hi is exact in
// fp32 and has at most 16 significant bits, lo keeps its top 8, and what is
// left (at most 8 bits) is lo2.  This holds while every part is a normal
// number, i.e. for a = 0 and |a| >= 2^-103 (a's lowest bit at or above
// 2^-126); below that, bits under 2^-126 may be lost.  A bf16 part times an
// int8 weight has at most 16 significant bits, so the matrix core forms it
// exactly.  The accumulation rounds once per 32-k block and part, where the
// fp32 matrix-core form (v_mfma_f32_16x16x4_f32) rounds once per 4 k.  An
// infinite activation makes its row's outputs NaN (a - hi is NaN), as the
// factorised form already does for any nonzero zero point.
//
// Tiles: BM x BN outputs, waves of WM x WN, K in chunks of 32 (one matrix-
// core k-block per part).  A chunk of A (fp32) is loaded into registers,
// split, and written to LDS as three bf16 planes [BM][32 k]; the chunk of W
// (int8) is widened to bf16 in registers and written as [BN][32 k] (the
// [K,N] weight is transposed 4x4 bytes at a time on the way).  Every LDS row
// is 64 bytes, four 16-byte segments.  In the A planes segment c of row r
// sits at slot c ^ (r >> 1) ^ (r >> 3) (two bits); the W tile, whose staging
// writes touch rows 4 apart ([K,N]) or two lanes per row (WT), also permutes
// its rows within groups of four (row n at (n & ~3) | ((n ^ (n >> 2)) & 3))
// and places segment c at c ^ (n >> 1) ^ (n >> 2) ^ (n >> 3).  Fragment reads
// (16 rows, one segment) and every staging write then hit distinct banks,
// for 32 or 64 banks of 4 bytes (an exhaustive check of the access patterns;
// the first W layout, the A one, had 4-way conflicts on the [K,N] writes).
// A lane's B fragments (16 k of column 16j + l16) stay in registers for the
// three planes.
//
// SK: the contraction split across workgroups (blockIdx.y is the split, each
// takes p.split_k values of it).  Every split leaves its fp32 partial tile
// (the fragments holding rows below M) and its partial S2 in the workspace,
// with device-coherent stores, and takes a ticket; the split that takes the
// last ticket adds the partials of all splits in split order (its own
// included, read back), so the sum does not depend on which split finished
// last and the result is the same on every run, then runs the epilogue and
// resets the ticket.
//
// With WT = true the same kernel is the gradient with respect to the
// activations: dA[m,k] = scale * (sum_n dC[m,n] W[k,n] - zp * sum_n dC[m,n]),
// the contraction over W's contiguous dimension, whose rows are already the
// [outputs][contraction] layout the LDS tile wants.
#include <algorithm>

#include "device_common.h"
#include "kernels.h"

namespace qg {
namespace {

constexpr int BKF = 32;
constexpr int GROUP_M = 8;

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int seg3(int r, int c) { return (c ^ (r >> 1) ^ (r >> 3)) & 3; }

// Byte offset of segment c of row n in the W tile.
__device__ __forceinline__ int wslot(int n, int c) {
    return (((n & ~3) | ((n ^ (n >> 2)) & 3)) << 6) + (((c ^ (n >> 1) ^ (n >> 2) ^ (n >> 3)) & 3) << 4);
}

// Two bf16 held in the high halves of a and b, packed a first.
__device__ __forceinline__ uint32_t pk_hi(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

// Four consecutive fp32 values as their three bf16 parts, two words each.
__device__ __forceinline__ void split4(const u32x4& v, uint2& h, uint2& l, uint2& q) {
    const uint32_t x[4] = {v.x, v.y, v.z, v.w};
    uint32_t hh[4], ll[4], qq[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        hh[e] = x[e] & 0xffff0000u;
        const float r1 = __uint_as_float(x[e]) - __uint_as_float(hh[e]);
        ll[e] = __float_as_uint(r1) & 0xffff0000u;
        qq[e] = __float_as_uint(r1 - __uint_as_float(ll[e]));
    }
    h = make_uint2(pk_hi(hh[0], hh[1]), pk_hi(hh[2], hh[3]));
    l = make_uint2(pk_hi(ll[0], ll[1]), pk_hi(ll[2], ll[3]));
    q = make_uint2(pk_hi(qq[0], qq[1]), pk_hi(qq[2], qq[3]));
}

// Four int8 (one word) as four bf16 (two words), exactly.
__device__ __forceinline__ uint2 i8x4_to_bf16(uint32_t w) {
    const uint32_t f0 = __float_as_uint((float)(int8_t)(w & 0xffu));
    const uint32_t f1 = __float_as_uint((float)(int8_t)((w >> 8) & 0xffu));
    const uint32_t f2 = __float_as_uint((float)(int8_t)((w >> 16) & 0xffu));
    const uint32_t f3 = __float_as_uint((float)(int8_t)(w >> 24));
    return make_uint2(pk_hi(f0, f1), pk_hi(f2, f3));
}

// WT == false: W is [K,N]; true: W is [N,K] rows of the contraction (p.N
// outputs, p.K contraction bytes per row).
template <int BM, int BN, int WM, int WN, bool VEC, bool WT, bool ZP, bool SK = false>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) void w8a32_split_kernel(W8A32Args p) {
    constexpr int WAVES_N = BN / WN;
    constexpr int NT = (BM / WM) * WAVES_N * 64;
    constexpr int FM = WM / 16, FN = WN / 16;
    constexpr int PLANE = BM * 64;                 // bytes of one bf16 plane of A
    constexpr int A_STAGE = 3 * PLANE;
    constexpr int STAGE = A_STAGE + BN * 64;
    constexpr int A_ROWS = NT / 8;                 // A rows one load round covers
    constexpr int A_ITERS = BM / A_ROWS;
    static_assert(BN * 2 == NT, "one 16-byte piece of the W chunk per lane");
    static_assert(BM % A_ROWS == 0, "whole A load rounds");
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];
    __shared__ float s2_rows[ZP ? BM : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int l16 = lane & 15, g = lane >> 4;

    const int tiles_m = (p.M + BM - 1) / BM;
    const int tiles_n = (p.N + BN - 1) / BN;
    int tm, tn;
    tile_coords(xcd_remap(blockIdx.x, gridDim.x), tiles_m, tiles_n, GROUP_M, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int rows = p.M - m0 < BM ? p.M - m0 : BM;
    const int cols = p.N - n0 < BN ? p.N - n0 : BN;
    const int lda = (int)p.lda, ldw = (int)p.ldw;
    // This workgroup's range of the contraction: [kbeg, kbeg + K).
    const int kbeg = SK ? (int)blockIdx.y * p.split_k : 0;
    const int K = SK ? (p.K - kbeg < p.split_k ? p.K - kbeg : p.split_k) : p.K;
    const float* A = p.A + (int64_t)m0 * p.lda + kbeg;
    const int8_t* W = WT ? p.W + (int64_t)n0 * p.ldw + kbeg : p.W + (int64_t)kbeg * p.ldw + n0;
    const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(A, (uint32_t)(((rows - 1) * lda + K) * 4));
    const __amdgpu_buffer_rsrc_t w_rsrc = WT ? make_rsrc(W, (uint32_t)((cols - 1) * ldw + K))
                                             : make_rsrc(W, (uint32_t)((K - 1) * ldw + (p.N - n0)));

    // A: lane -> rows ar + A_ROWS*i, floats 4*ac .. 4*ac+3 of the chunk.
    const int ar = tid >> 3, ac = tid & 7;
    // W: k rows 4*wr .. 4*wr+3, columns 4*wc .. 4*wc+3; with WT, output row
    // tr, contraction bytes 16*th .. 16*th+15.
    const int wr = tid & 7, wc = tid >> 3;
    const int tr = tid >> 1, th = tid & 1;

    u32x4 a_st[A_ITERS];
    uint32_t w_st[4];
    auto fetch = [&](int k0) {
#pragma unroll
        for (int i = 0; i < A_ITERS; ++i) {
            const int r = ar + A_ROWS * i;
            if constexpr (VEC) {
                a_st[i] = buffer_load16(a_rsrc, (uint32_t)((r * lda + ac * 4 + k0) * 4), 0u);
            } else {
                uint32_t d[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int k = k0 + ac * 4 + e;
                    d[e] = (r < rows && k < K) ? __float_as_uint(A[(int64_t)r * p.lda + k]) : 0u;
                }
                a_st[i] = u32x4{d[0], d[1], d[2], d[3]};
            }
        }
        if constexpr (WT) {
            if constexpr (VEC) {
                const u32x4 v = buffer_load16(w_rsrc, (uint32_t)(tr * ldw + k0 + 16 * th), 0u);
                w_st[0] = v.x; w_st[1] = v.y; w_st[2] = v.z; w_st[3] = v.w;
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    uint32_t d = 0;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int k = k0 + 16 * th + 4 * i + e;
                        if (tr < cols && k < K) d |= (uint32_t)(uint8_t)W[(int64_t)tr * p.ldw + k] << (8 * e);
                    }
                    w_st[i] = d;
                }
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k = k0 + wr * 4 + i;
            if constexpr (VEC) {
                w_st[i] = __builtin_amdgcn_raw_buffer_load_b32(w_rsrc, (int)(k * ldw + wc * 4), 0, 0);
            } else {
                uint32_t d = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int n = wc * 4 + e;
                    if (k < K && n < cols) d |= (uint32_t)(uint8_t)W[(int64_t)k * p.ldw + n] << (8 * e);
                }
                w_st[i] = d;
            }
        }
    };

    float rs[A_ITERS];   // this lane's share of S2 for rows ar + A_ROWS*i
#pragma unroll
    for (int i = 0; i < A_ITERS; ++i) rs[i] = 0.f;

    // Registers -> LDS: A split into its three planes, W widened to bf16.
    // Columns of A past K read as zero (the values past K in a 16-byte load
    // belong to the next row); W's rows past K are zero through its buffer
    // range, and its bytes past K in a WT row meet those zero columns of A.
    auto stash = [&](int buf, int k0) {
        uint8_t* S = smem + buf * STAGE;
        const bool k_full = k0 + BKF <= K;
#pragma unroll
        for (int i = 0; i < A_ITERS; ++i) {
            u32x4 v = a_st[i];
            if (VEC && !k_full) {
                const int k = k0 + ac * 4;
                if (k + 0 >= K) v.x = 0u;
                if (k + 1 >= K) v.y = 0u;
                if (k + 2 >= K) v.z = 0u;
                if (k + 3 >= K) v.w = 0u;
            }
            if constexpr (ZP)
                rs[i] += (__uint_as_float(v.x) + __uint_as_float(v.y)) + (__uint_as_float(v.z) + __uint_as_float(v.w));
            uint2 h, l, q;
            split4(v, h, l, q);
            const int r = ar + A_ROWS * i;
            const int off = r * 64 + (seg3(r, ac >> 1) << 4) + 8 * (ac & 1);
            *reinterpret_cast<uint2*>(S + off) = h;
            *reinterpret_cast<uint2*>(S + PLANE + off) = l;
            *reinterpret_cast<uint2*>(S + 2 * PLANE + off) = q;
        }
        uint8_t* Ws = S + A_STAGE;
        if constexpr (WT) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint2 d0 = i8x4_to_bf16(w_st[2 * h]), d1 = i8x4_to_bf16(w_st[2 * h + 1]);
                *reinterpret_cast<u32x4*>(Ws + wslot(tr, 2 * th + h)) = u32x4{d0.x, d0.y, d1.x, d1.y};
            }
        } else {
            uint32_t y[4];
            transpose4x4_bytes(w_st, y);   // y[c]: k rows 4wr .. 4wr+3 of column 4wc + c
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int n = wc * 4 + c;
                *reinterpret_cast<uint2*>(Ws + wslot(n, wr >> 1) + 8 * (wr & 1)) = i8x4_to_bf16(y[c]);
            }
        }
    };

    v4f acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int buf) {
        const uint8_t* S = smem + buf * STAGE;
        v8bf bfr[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int n = wn * WN + j * 16 + l16;
            bfr[j] = __builtin_bit_cast(v8bf, *reinterpret_cast<const u32x4*>(S + A_STAGE + wslot(n, g)));
        }
#pragma unroll
        for (int pl = 0; pl < 3; ++pl) {
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int r = wm * WM + i * 16 + l16;
                const v8bf af =
                    __builtin_bit_cast(v8bf, *reinterpret_cast<const u32x4*>(S + pl * PLANE + r * 64 + (seg3(r, g) << 4)));
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bfr[j], acc[i][j], 0, 0, 0);
            }
        }
    };

    // Ping-pong (eight-wave tiles): a SIMD runs one wave of each half of the
    // workgroup (wave w on SIMD w % 4).  The first half loads chunk kt+1,
    // multiplies chunk kt, then splits and stores chunk kt+1; the second half
    // splits and stores chunk kt+1 (loaded one chunk earlier) before its
    // multiplies and loads chunk kt+2 in between.  The two waves of a SIMD
    // are then in opposite phases, so one's vector work runs beside the
    // other's multiplies (4096^3: 339 -> 313 us forward, 331 -> 300 us
    // gradient, identical bits).  Each half still writes only its own share
    // of chunk kt+1, into the buffer nobody reads until the barrier.
    const int nk = (K + BKF - 1) / BKF;
    const bool early = NT == 512 && __builtin_amdgcn_readfirstlane(wave) >= 4;
    fetch(0);
    stash(0, 0);
    if (early && nk > 1) fetch(BKF);
    __syncthreads();
    for (int kt = 0; kt + 1 < nk; ++kt) {
        if (early) stash((kt + 1) & 1, (kt + 1) * BKF);
        const int fk = kt + (early ? 2 : 1);
        if (fk < nk) fetch(fk * BKF);
        compute(kt & 1);
        if (!early) stash((kt + 1) & 1, (kt + 1) * BKF);
        __syncthreads();
    }
    compute((nk - 1) & 1);

    // S2 of row ar + A_ROWS*i is spread over the eight lanes ac = 0..7.
    if constexpr (ZP) {
#pragma unroll
        for (int i = 0; i < A_ITERS; ++i) {
            rs[i] += __shfl_xor(rs[i], 1);
            rs[i] += __shfl_xor(rs[i], 2);
            rs[i] += __shfl_xor(rs[i], 4);
        }
        if (ac == 0) {
#pragma unroll
            for (int i = 0; i < A_ITERS; ++i) s2_rows[ar + A_ROWS * i] = rs[i];
        }
        __syncthreads();
    }

    if constexpr (SK) {
        const int S = (int)gridDim.y, sk = (int)blockIdx.y;
        if (S > 1) {
            constexpr int COHERENT = 16;   // sc1: device scope
            constexpr int SLOT = BM * BN * 4 + BM * 4;
            const int tile = tm * tiles_n + tn;   // < W8A32_MAX_TICKETS (host plan)
            int* tickets = reinterpret_cast<int*>(p.workspace);
            char* part = reinterpret_cast<char*>(p.workspace) + SKINNY_TICKET_BYTES + (size_t)tile * S * SLOT;
            const __amdgpu_buffer_rsrc_t p_rsrc = make_rsrc(part, (uint32_t)(S * SLOT));
            // fragment (i, j) of wave w at ((w * FM + i) * FN + j) * 1024 + 16 * lane;
            // only fragments with a row below M travel (lane group g holds
            // rows 16i + 4g .. 16i + 4g + 3 of the wave's tile)
            auto frag_off = [&](int s2, int i, int j) {
                return (uint32_t)(s2 * SLOT + ((wave * FM + i) * FN + j) * 1024 + 16 * lane);
            };
            auto live = [&](int i) { return wm * WM + i * 16 + 4 * g < rows; };
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                if (!live(i)) continue;
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, acc[i][j]), p_rsrc, frag_off(sk, i, j), 0,
                                                           COHERENT);
            }
            if (ZP && tid < BM / 4)
                __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const v4i*>(&s2_rows[4 * tid]), p_rsrc,
                                                       (uint32_t)(sk * SLOT + BM * BN * 4 + 16 * tid), 0, COHERENT);
            __builtin_amdgcn_s_waitcnt(0);
            __shared__ int ticket;
            __syncthreads();
            if (tid == 0) ticket = __hip_atomic_fetch_add(&tickets[tile], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __syncthreads();
            if (ticket != S - 1) return;
            // The sum of all splits' partials, in split order.
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
            v4f s2v = v4f{0.f, 0.f, 0.f, 0.f};
            for (int s2 = 0; s2 < S; ++s2) {
                v4f v[FM][FN];
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        v[i][j] = live(i) ? __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(p_rsrc, frag_off(s2, i, j), 0,
                                                                                                          COHERENT))
                                          : v4f{0.f, 0.f, 0.f, 0.f};
                v4f w = v4f{0.f, 0.f, 0.f, 0.f};
                if (ZP && tid < BM / 4)
                    w = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(
                                                    p_rsrc, (uint32_t)(s2 * SLOT + BM * BN * 4 + 16 * tid), 0, COHERENT));
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[i][j][r] = acc[i][j][r] + v[i][j][r];
#pragma unroll
                for (int r = 0; r < 4; ++r) s2v[r] = s2v[r] + w[r];
            }
            if constexpr (ZP) {
                __syncthreads();   // every thread has read its own split's S2 from LDS
                if (tid < BM / 4) *reinterpret_cast<v4f*>(&s2_rows[4 * tid]) = s2v;
                __syncthreads();
            }
            if (tid == 0) __hip_atomic_store(&tickets[tile], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }

    // Register r of block (i, j) in lane (g, l16) holds row 16i + 4g + r,
    // column 16j + l16 of the wave's tile.
    const float zp = (float)p.zp;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int lr = wm * WM + i * 16 + 4 * g + r;
            const int m = m0 + lr;
            const float s2 = ZP ? s2_rows[lr] : 0.f;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int n = n0 + wn * WN + j * 16 + l16;
                if (m < p.M && n < p.N) {
                    float v = acc[i][j][r];
                    if constexpr (ZP) v = v - zp * s2;
                    p.C[(int64_t)m * p.ldc + n] = p.scale * v;
                }
            }
        }
    }
}

// The 128 x 128 tiles split over the contraction (a.splits > 1, a.split_k
// values per split, a multiple of 32; at most SKINNY_MAX_TICKETS tiles; the
// workspace as the host plan sized it).
template <int BM, int BN, int WM, int WN>
void launch_tile_split(const W8A32Args& a, bool vec, bool wt, hipStream_t s) {
    const dim3 grid(((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN), a.splits), block((BM / WM) * (BN / WN) * 64);
    const bool zp = a.zp != 0;
    const int v = (vec ? 4 : 0) | (wt ? 2 : 0) | (zp ? 1 : 0);
    switch (v) {
        case 7: hipLaunchKernelGGL((w8a32_split_kernel<BM, BN, WM, WN, true, true, true, true>), grid, block, 0, s, a); break;
        case 6: hipLaunchKernelGGL((w8a32_split_kernel<BM, BN, WM, WN, true, true, false, true>), grid, block, 0, s, a); break;
        case 5: hipLaunchKernelGGL((w8a32_split_kernel<BM, BN, WM, WN, true, false, true, true>), grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL((w8a32_split_kernel<BM, BN, WM, WN, true, false, false, true>), grid, block, 0, s, a); break;
        case 3: hipLaunchKernelGGL((w8a32_split_kernel<BM, BN, WM, WN, false, true, true, true>), grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL((w8a32_split_kernel<BM, BN, WM, WN, false, true, false, true>), grid, block, 0, s, a); break;
        case 1: hipLaunchKernelGGL((w8a32_split_kernel<BM, BN, WM, WN, false, false, true, true>), grid, block, 0, s, a); break;
        default: hipLaunchKernelGGL((w8a32_split_kernel<BM, BN, WM, WN, false, false, false, true>), grid, block, 0, s, a); break;
    }
}

template <int BM, int BN, int WM, int WN>
void launch_tile(const W8A32Args& a, bool vec, bool wt, hipStream_t s) {
    const dim3 grid(((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN)), block((BM / WM) * (BN / WN) * 64);
    const bool zp = a.zp != 0;
    const int v = (vec ? 4 : 0) | (wt ? 2 : 0) | (zp ? 1 : 0);
    switch (v) {
        case 7: hipLaunchKernelGGL((w8a32_split_kernel<BM, BN, WM, WN, true, true, true>), grid, block, 0, s, a); break;
        case 6: hipLaunchKernelGGL((w8a32_split_kernel<BM, BN, WM, WN, true, true, false>), grid, block, 0, s, a); break;
        case 5: hipLaunchKernelGGL((w8a32_split_kernel<BM, BN, WM, WN, true, false, true>), grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL((w8a32_split_kernel<BM, BN, WM, WN, true, false, false>), grid, block, 0, s, a); break;
        case 3: hipLaunchKernelGGL((w8a32_split_kernel<BM, BN, WM, WN, false, true, true>), grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL((w8a32_split_kernel<BM, BN, WM, WN, false, true, false>), grid, block, 0, s, a); break;
        case 1: hipLaunchKernelGGL((w8a32_split_kernel<BM, BN, WM, WN, false, false, true>), grid, block, 0, s, a); break;
        default: hipLaunchKernelGGL((w8a32_split_kernel<BM, BN, WM, WN, false, false, false>), grid, block, 0, s, a); break;
    }
}

}  // namespace

// Whether a call takes the 256 x 256 tiles (see launch_w8a32_split).
static bool big_tiles(int64_t M, int64_t N, int64_t K, int64_t lda) {
    const int64_t big = ((M + 255) / 256) * ((N + 255) / 256);
    return big > 128 && (256 * lda + K + 64) * 4 < ((int64_t)1 << 31);
}

void w8a32_split_plan(int64_t M, int64_t N, int64_t K, int64_t lda, int forced, int* splits, int* split_k) {
    *splits = 1;
    *split_k = 0;
    if (big_tiles(M, N, K, lda)) return;
    // About two workgroups per CU (the 128x128 tiles run two per CU):
    // graph-timed at N = K = 8192, 64 tiles (M = 80 / 128) take 70.3 / 77.1
    // us with 8 splits against 98.7 / 102.9 with 4, and 128 tiles (M = 256)
    // 128.7 with 4 against 181.9 with 2; at 4096^2, M = 256 / 384 / 512
    // (64 / 96 / 128 tiles) 48.5 / 68.1 / 70.7 against 58.6 / 98.0 / 97.8.
    const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
    if (tiles > SKINNY_MAX_TICKETS) return;
    int64_t S = forced > 0 ? forced : std::min<int64_t>(std::min<int64_t>(512 / tiles, K / 512), 8);
    if (S < 2) return;
    const int64_t chunks = (K + BKF - 1) / BKF;
    const int64_t per = (chunks + S - 1) / S;
    const int64_t n = (chunks + per - 1) / per;
    if (n < 2) return;
    *splits = (int)n;
    *split_k = (int)(per * BKF);
}

size_t w8a32_split_bytes(int64_t M, int64_t N, int splits) {
    if (splits <= 1) return 0;
    const size_t tiles = (size_t)((M + 127) / 128) * (size_t)((N + 127) / 128);
    return SKINNY_TICKET_BYTES + tiles * (size_t)splits * (128 * 128 * 4 + 128 * 4);
}

hipError_t launch_w8a32_split(const W8A32Args& a, bool vec_a, bool vec_w, bool wt, hipStream_t s,
                              const char** name) {
    const bool vec = vec_a && vec_w;
    if (a.splits > 1) {
        const int64_t tiles = ((int64_t)(a.M + 127) / 128) * ((a.N + 127) / 128);
        if (big_tiles(a.M, a.N, a.K, a.lda) || a.workspace == nullptr || tiles > SKINNY_MAX_TICKETS ||
            a.split_k % BKF != 0 || (int64_t)a.split_k * a.splits < a.K || (int64_t)a.split_k * (a.splits - 1) >= a.K)
            return hipErrorInvalidValue;
        *name = wt ? "w8a32_input_grad_bf16x3_128x128_splitk" : "w8a32_bf16x3_128x128_splitk";
        launch_tile_split<128, 128, 64, 64>(a, vec, wt, s);
        return hipGetLastError();
    }
    // 256 x 256 tiles (eight waves of 64 x 128, one workgroup per CU) when
    // there are more than 128 of them and 256 rows of A stay within the
    // 32-bit buffer offsets; 128 x 128 otherwise.  The small tiles run more
    // workgroups per CU but take two rounds from 129 large-tile counts on:
    // 3072^3 201.1 against 283.4 us, 2560x4096x4096 260.7 / 358.4,
    // 3584x4096x4096 281.5 / 440.0; at 128 (2048x4096x4096, one round of
    // small tiles) they win, 237.7 against 268.9.
    if (big_tiles(a.M, a.N, a.K, a.lda)) {
        *name = wt ? "w8a32_input_grad_bf16x3_256x256" : "w8a32_bf16x3_256x256";
        launch_tile<256, 256, 64, 128>(a, vec, wt, s);
    } else {
        *name = wt ? "w8a32_input_grad_bf16x3_128x128" : "w8a32_bf16x3_128x128";
        launch_tile<128, 128, 64, 64>(a, vec, wt, s);
    }
    return hipGetLastError();
}

}  // namespace qg

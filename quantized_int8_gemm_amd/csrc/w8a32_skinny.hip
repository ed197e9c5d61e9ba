// Decode-shaped W8A32 (M <= 16) and its input gradient on the bf16 matrix
// cores of gfx950, bound by reading the int8 weight once.
//
// Operator: "feat(PULPOpen): matmul that dequantises an int8 weight
// in-kernel", section "The kernel": C = scale * (S1 - zp * S2) with
// S1 = sum_k a_k b_k and S2 = sum_k a_k, the dequantised weight never
// formed.  As in the tiled split kernel, every fp32 activation is split
// exactly into three bf16 parts (hi + lo + lo2) and the int8 weight is exact
// in bf16, so the matrix cores form every product exactly and only the fp32
// accumulation rounds.
//
// Grid: (N / 256 column tiles) x (S splits of K) x (blocks of 16 rows: up to
// SKINNY_W8A32_MAX_M rows, each block streaming the weight again, mostly
// from the Infinity Cache), four waves taking 64-row
// steps of K round robin, two steps in flight, the weight read with the
// non-temporal policy (as the int8 decode kernel reads it):
//  * lane (g = lane/16, c = lane%16) loads rows 16g .. 16g+15 of the step at
//    columns 16c .. 16c+15 (16-byte vectors), and the 16 fp32 values of
//    activation row c at the same 16 k;
//  * the activation values become three bf16 planes, 8 k per half; for
//    output column 16c + j, byte j of the lane's rows 8h .. 8h+7 widens to
//    the matching 8 bf16, so v_mfma_f32_16x16x32_bf16 number (j, h, part)
//    adds the products of those k for rows 0..15 and columns {16c + j}
//    (96 multiplies per step, no LDS in the loop);
//  * the waves' fp32 tiles are added through LDS in wave order; with S > 1
//    each split leaves its partial (rows < M, and its 16 partial row sums
//    S2) in the workspace with device-coherent stores and takes a ticket; the
//    split that takes the last ticket adds all S partials in split order (so
//    the sum does not depend on which split finished last), runs the
//    epilogue and resets the ticket.
// Values of A past K (the next row's, or beyond the buffer) are cleared
// before they reach a product or S2; weight rows past K read as zero.
//
// WT: the input gradient, dA = scale * (dC W^T - zp * rowsum(dC)), whose
// contraction runs along W's rows (the outputs are W's rows).  Lane (g, c)
// then loads, for j = 0..15, bytes 16g .. 16g+15 of the step from W row
// 16c + j, which already hold 16 contraction values of output 16c + j in
// order: they widen to the same bf16 fragments without a transpose, and
// everything else is the forward kernel's.
#include <algorithm>

#include "device_common.h"
#include "kernels.h"

namespace qg {
namespace {

constexpr int NT = 256;     // threads (four waves)
constexpr int TN = 256;     // columns per workgroup
constexpr int KS = 64;      // k rows per wave step
constexpr int WAVES = 4;
constexpr int SLOT_ROWS = 17;   // a split's partial: 16 tile rows, then the 16 row sums

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// Two bf16 held in the high halves of a and b, packed a first.
__device__ __forceinline__ uint32_t pk_hi(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

// Eight fp32 values as their three bf16 parts (exact: see the tiled kernel).
__device__ __forceinline__ void split8(const float* v, v8bf& hi, v8bf& lo, v8bf& lo2) {
    uint32_t h[8], l[8], q[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t x = __float_as_uint(v[e]);
        h[e] = x & 0xffff0000u;
        const float r1 = v[e] - __uint_as_float(h[e]);
        l[e] = __float_as_uint(r1) & 0xffff0000u;
        q[e] = __float_as_uint(r1 - __uint_as_float(l[e]));
    }
    u32x4 H, L, Q;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        (&H.x)[e] = pk_hi(h[2 * e], h[2 * e + 1]);
        (&L.x)[e] = pk_hi(l[2 * e], l[2 * e + 1]);
        (&Q.x)[e] = pk_hi(q[2 * e], q[2 * e + 1]);
    }
    hi = __builtin_bit_cast(v8bf, H);
    lo = __builtin_bit_cast(v8bf, L);
    lo2 = __builtin_bit_cast(v8bf, Q);
}

// Bytes 8h .. 8h+7 of a 16-byte vector as eight bf16 (exact for int8).
__device__ __forceinline__ v8bf half8(const u32x4& v, int h) {
    uint32_t f[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const uint32_t w = (&v.x)[2 * h + (t >> 2)];
        f[t] = __float_as_uint((float)(int8_t)(uint8_t)(w >> (8 * (t & 3))));
    }
    return __builtin_bit_cast(v8bf, u32x4{pk_hi(f[0], f[1]), pk_hi(f[2], f[3]), pk_hi(f[4], f[5]), pk_hi(f[6], f[7])});
}

// Byte j of eight 16-byte rows as eight bf16 (exact for int8).
__device__ __forceinline__ v8bf column8(const u32x4* rows, int j) {
    uint32_t f[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const uint32_t w = (&rows[t].x)[j >> 2];
        f[t] = __float_as_uint((float)(int8_t)(uint8_t)(w >> (8 * (j & 3))));
    }
    return __builtin_bit_cast(v8bf, u32x4{pk_hi(f[0], f[1]), pk_hi(f[2], f[3]), pk_hi(f[4], f[5]), pk_hi(f[6], f[7])});
}

// WV waves taking steps of KSZ k-rows: the forward runs eight waves of
// 32-row steps (two waves per SIMD, so one wave's widening and splitting
// runs beside another's loads and multiplies).  The gradient takes 64-row
// steps (its 16-byte loads cover 16 contraction values of a row) with four
// waves, or with eight as two halves of four: both halves walk the same
// steps, each over 128 of the tile's 256 outputs (lane c16 then holds rows
// 128 half + 8 c16 + j, j < 8), which halves a wave's weight registers and
// again puts two waves on each SIMD; only the first half adds S2.
template <bool ZP, bool WT, int WV = WAVES, int KSZ = KS>
__global__ __launch_bounds__(64 * WV) __attribute__((amdgpu_waves_per_eu(WV == 8 ? 2 : 1))) void w8a32_skinny_kernel(W8A32Args p) {
    constexpr int NTW = 64 * WV;
    constexpr int RPL = KSZ / 4;    // k-rows per lane per step (forward)
    constexpr int H = RPL / 8;      // 8-row halves of them
    // The gradient with eight waves: two halves of four, each half covering
    // 128 of the tile's 256 outputs over the same steps (SW waves share the
    // steps; JN column blocks of 16 per wave).
    constexpr bool HALVES = WT && WV == 8;
    constexpr int SW = HALVES ? 4 : WV;
    constexpr int JN = HALVES ? 8 : 16;
    static_assert(!WT || (KSZ == 64 && (WV == 4 || WV == 8)), "the gradient's loads take 64-row steps");
    static_assert(RPL % 8 == 0 && SW * KSZ == 256, "steps of 512 rows per wave pair");
    __shared__ __attribute__((aligned(16))) float red[SW][16][TN];
    __shared__ float s2_red[SW][16];
    __shared__ __attribute__((aligned(16))) float s2_tot[16];
    __shared__ int ticket;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    const int half = HALVES ? wave / SW : 0, swave = HALVES ? wave % SW : wave;
    const int tn = blockIdx.x, split = blockIdx.y, S = gridDim.y;
    const int n0 = tn * TN;
    const int cols = p.N - n0;
    // blockIdx.z: the block of 16 rows (p.M up to 16 * gridDim.z)
    const int rb = blockIdx.z;
    const int M = p.M - 16 * rb < 16 ? p.M - 16 * rb : 16, K = p.K;
    const float* Ab = p.A + (int64_t)16 * rb * p.lda;
    float* Cb = p.C + (int64_t)16 * rb * p.ldc;
    const int unit = rb * (int)gridDim.x + tn;   // this (row block, column tile)'s ticket

    // K range of this split: `per` steps of KSZ rows, a multiple of 2*WV.
    const int per = p.split_k / KSZ;
    const int s_begin = split * per;

    const int ldw = (int)p.ldw, lda = (int)p.lda;
    const __amdgpu_buffer_rsrc_t w_rsrc = WT ? make_rsrc(p.W + (int64_t)n0 * ldw, (uint32_t)(((cols < TN ? cols : TN) - 1) * ldw + K))
                                             : make_rsrc(p.W + n0, (uint32_t)((K - 1) * ldw + cols));
    const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(Ab, (uint32_t)(((M - 1) * lda + K) * 4));
    const uint32_t w_voff = WT ? (uint32_t)((128 * half + JN * c16) * ldw + 16 * g) : (uint32_t)(RPL * g * ldw + 16 * c16);
    const uint32_t a_voff = (uint32_t)((c16 * lda + RPL * g) * 4);

    u32x4 wbuf[2][WT ? JN : RPL];
    u32x4 abuf[2][RPL / 4];
    // Loads of one step into buffer b; a step past this split's range reads
    // rows that are never multiplied (or zeros past K), so no branch
    // separates the loads.
    auto fetch = [&](int step, int b) {
        const int k0 = step * KSZ;
        if constexpr (WT) {   // W row 16 c16 + j, contraction bytes k0 + 16g ..
            // cached: a step reads half of each 128-byte line, the other half
            // is the next step's (1x8192x8192: 22.3 against 22.6 us; 64
            // rows: 50.3 against 56.0)
#pragma unroll
            for (int j = 0; j < JN; ++j) wbuf[b][j] = buffer_load16(w_rsrc, w_voff + (uint32_t)(j * ldw + k0), 0u);
        } else {   // non-temporal even for several row blocks (M = 64: 37.0 against 43.9 us cached)
#pragma unroll
            for (int r = 0; r < RPL; ++r) wbuf[b][r] = buffer_load16_nt(w_rsrc, w_voff + (uint32_t)((k0 + r) * ldw));
        }
#pragma unroll
        for (int q = 0; q < RPL / 4; ++q) abuf[b][q] = buffer_load16(a_rsrc, a_voff + (uint32_t)((k0 + 4 * q) * 4), 0u);
    };

    v4f acc[JN];
#pragma unroll
    for (int j = 0; j < JN; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
    float s2 = 0.f;   // this lane's share of S2 for row c16

    auto consume = [&](int b, int step) {
        const int k0 = step * KSZ + RPL * g;
        float a[RPL];
#pragma unroll
        for (int q = 0; q < RPL / 4; ++q) {
            a[4 * q] = __uint_as_float(abuf[b][q].x);
            a[4 * q + 1] = __uint_as_float(abuf[b][q].y);
            a[4 * q + 2] = __uint_as_float(abuf[b][q].z);
            a[4 * q + 3] = __uint_as_float(abuf[b][q].w);
        }
        if (step * KSZ + KSZ > K) {   // a step reaching past K: clear those values
#pragma unroll
            for (int e = 0; e < RPL; ++e)
                if (k0 + e >= K) a[e] = 0.f;
        }
        if constexpr (ZP) {
            const float t = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
            if constexpr (H == 2)
                s2 += t + (((a[8] + a[9]) + (a[10] + a[11])) + ((a[12] + a[13]) + (a[14] + a[15])));
            else
                s2 += t;
        }
        v8bf pa[H][3];
#pragma unroll
        for (int h = 0; h < H; ++h) split8(a + 8 * h, pa[h][0], pa[h][1], pa[h][2]);
#pragma unroll
        for (int j = 0; j < JN; ++j) {
#pragma unroll
            for (int h = 0; h < H; ++h) {
                const v8bf bw = WT ? half8(wbuf[b][j], h) : column8(&wbuf[b][8 * h], j);
#pragma unroll
                for (int pl = 0; pl < 3; ++pl)
                    acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[h][pl], bw, acc[j], 0, 0, 0);
            }
        }
    };

    // This wave's steps: s_begin + wave + WV*i, i < n_my (even, the same
    // for all waves); two in flight, the last pair peeled.
    const int first = s_begin + swave;
    const int n_my = per / SW;
    fetch(first, 0);
    __builtin_amdgcn_sched_barrier(0);
    fetch(first + SW, 1);
    __builtin_amdgcn_sched_barrier(0);
    int i = 0;
    for (; i + 2 < n_my; i += 2) {
        consume(0, first + SW * i);
        __builtin_amdgcn_sched_barrier(0);
        fetch(first + SW * (i + 2), 0);
        __builtin_amdgcn_sched_barrier(0);
        consume(1, first + SW * (i + 1));
        __builtin_amdgcn_sched_barrier(0);
        fetch(first + SW * (i + 3), 1);
        __builtin_amdgcn_sched_barrier(0);
    }
    consume(0, first + SW * i);
    consume(1, first + SW * (i + 1));

    // Register r of block j holds row 4g + r, column 16*c16 + j: four
    // 16-byte chunks per row, placed as in the int8 decode kernel.
    auto chunk = [](int ch) { return (ch & ~3) | ((ch ^ (ch >> 4)) & 3); };
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        if (4 * g + r >= M) continue;
#pragma unroll
        for (int q = 0; q < JN / 4; ++q) {
            const v4f v = v4f{acc[4 * q][r], acc[4 * q + 1][r], acc[4 * q + 2][r], acc[4 * q + 3][r]};
            *reinterpret_cast<v4f*>(&red[swave][4 * g + r][4 * chunk(32 * half + (JN / 4) * c16 + q)]) = v;
        }
    }
    if constexpr (ZP) {
        // lane groups held different k: (g0 + g1) + (g2 + g3) in every lane
        s2 += __shfl_xor(s2, 16);
        s2 += __shfl_xor(s2, 32);
        if (g == 0 && half == 0) s2_red[swave][c16] = s2;
    }
    __syncthreads();
    if (ZP && tid < 16) {
        float t = s2_red[0][tid];
#pragma unroll
        for (int w = 1; w < SW; ++w) t = t + s2_red[w][tid];
        s2_tot[tid] = t;
    }

    // Items: (row m < M, group of 4 columns); the waves' tiles in wave order.
    auto tile_sum = [&](int m, int cg) -> v4f {
        const int at = 4 * chunk(cg);
        v4f s = *reinterpret_cast<const v4f*>(&red[0][m][at]);
#pragma unroll
        for (int w = 1; w < SW; ++w) s = s + *reinterpret_cast<const v4f*>(&red[w][m][at]);
        return s;
    };
    const float zp = (float)p.zp;
    const bool vec_out = (p.ldc % 4 == 0) && ((reinterpret_cast<uintptr_t>(Cb) & 15) == 0);
    auto epilogue = [&](int m, int n, v4f v) {
        if (n >= p.N) return;
        float f[4] = {v[0], v[1], v[2], v[3]};
        const float s2m = ZP ? s2_tot[m] : 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if constexpr (ZP) f[e] = f[e] - zp * s2m;
            f[e] = p.scale * f[e];
        }
        float* dst = Cb + (int64_t)m * p.ldc + n;
        if (vec_out && n + 4 <= p.N) {
            *reinterpret_cast<float4*>(dst) = make_float4(f[0], f[1], f[2], f[3]);
            return;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (n + e < p.N) dst[e] = f[e];
    };
    const int items = M * (TN / 4);

    if (S == 1) {
        if constexpr (ZP) __syncthreads();   // s2_tot
        for (int it = tid; it < items; it += NTW) {
            const int m = it / (TN / 4), cg = it % (TN / 4);
            epilogue(m, n0 + cg * 4, tile_sum(m, cg));
        }
        return;
    }

    // Split-K exchange (workspace: the fixed ticket header, one int per
    // column tile, then per column tile S partials of SLOT_ROWS x TN fp32).
    int* tickets = reinterpret_cast<int*>(p.workspace);
    constexpr int SLOT = SLOT_ROWS * TN * 4;
    char* part = reinterpret_cast<char*>(p.workspace) + SKINNY_TICKET_BYTES + (size_t)unit * S * SLOT;
    const __amdgpu_buffer_rsrc_t p_rsrc = make_rsrc(part, (uint32_t)(S * SLOT));
    constexpr int COHERENT = 16;   // sc1: device scope
    for (int it = tid; it < items; it += NTW) {
        const int m = it / (TN / 4), cg = it % (TN / 4);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, tile_sum(m, cg)), p_rsrc,
                                               (uint32_t)(split * SLOT + (m * TN + cg * 4) * 4), 0, COHERENT);
    }
    if constexpr (ZP) {
        __syncthreads();   // s2_tot
        if (tid < 4)
            __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const v4i*>(&s2_tot[4 * tid]), p_rsrc,
                                                   (uint32_t)(split * SLOT + (16 * TN + 4 * tid) * 4), 0, COHERENT);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) ticket = __hip_atomic_fetch_add(&tickets[unit], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (ticket != S - 1) return;

    // Every split's partial, added in split order, SU splits per round with
    // their loads in flight together; loads past split S - 1 read zeros.
    constexpr int SU = 8, IPT = 16 * (TN / 4) / NTW;
    v4f sum[IPT];
    uint32_t off[IPT];
#pragma unroll
    for (int q = 0; q < IPT; ++q) {
        const int it = tid + q * NTW;
        const int m = it / (TN / 4), cg = it % (TN / 4);
        sum[q] = v4f{0.f, 0.f, 0.f, 0.f};
        off[q] = it < items ? (uint32_t)((m * TN + cg * 4) * 4) : 0xFFFFFFF0u;
    }
    v4f ssum = v4f{0.f, 0.f, 0.f, 0.f};
    const uint32_t soff = (ZP && tid < 4) ? (uint32_t)((16 * TN + 4 * tid) * 4) : 0xFFFFFFF0u;
    for (int s0 = 0; s0 < S; s0 += SU) {
        v4f v[IPT][SU];
        v4f w[ZP ? SU : 1];
#pragma unroll
        for (int q = 0; q < IPT; ++q)
#pragma unroll
            for (int u = 0; u < SU; ++u) {
                const uint32_t o = off[q] == 0xFFFFFFF0u ? off[q] : off[q] + (uint32_t)((s0 + u) * SLOT);
                v[q][u] = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(p_rsrc, o, 0, COHERENT));
            }
        if constexpr (ZP) {
#pragma unroll
            for (int u = 0; u < SU; ++u) {
                const uint32_t o = soff == 0xFFFFFFF0u ? soff : soff + (uint32_t)((s0 + u) * SLOT);
                w[u] = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(p_rsrc, o, 0, COHERENT));
            }
        }
        // splits past S - 1 read zeros: adding them changes nothing
#pragma unroll
        for (int q = 0; q < IPT; ++q)
#pragma unroll
            for (int u = 0; u < SU; ++u) sum[q] = sum[q] + v[q][u];
        if constexpr (ZP) {
#pragma unroll
            for (int u = 0; u < SU; ++u) ssum = ssum + w[u];
        }
    }
    if constexpr (ZP) {
        if (tid < 4) *reinterpret_cast<v4f*>(&s2_tot[4 * tid]) = ssum;
        __syncthreads();
    }
#pragma unroll
    for (int q = 0; q < IPT; ++q) {
        const int it = tid + q * NTW;
        if (it >= items) continue;
        const int m = it / (TN / 4), cg = it % (TN / 4);
        epilogue(m, n0 + cg * 4, sum[q]);
    }
    if (tid == 0) __hip_atomic_store(&tickets[unit], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Slab form of the input gradient for at most 16 rows: the contraction
// runs along W's rows, so a workgroup that owns TN = 16 NF outputs (W rows
// n0 .. n0 + TN - 1) streams those rows whole, every 128-byte line used by
// itself, over ALL of the contraction: N / TN workgroups occupy the chip and
// nothing crosses workgroups (no partials, no ticket, no workspace).  Eight
// waves take steps of 64 KB contraction values round robin, NB in flight.
// Every workgroup reads and splits all of dC, which costs more than the
// split form's exchange from about 16 rows on.
// Lane (i16, g) loads 16 bytes of W row n0 + 16c + i16 at contraction bytes
// 64kb + 16g (the B fragments of two v_mfma_f32_16x16x32_bf16, halves h = 0
// and 1, once widened) and the 16 fp32 values of dC row i16 at the same
// contraction indices, split into three bf16 planes; every product is exact
// and only the fp32 accumulation rounds, as in the split form.  The waves'
// tiles and row sums S2 are added through LDS in wave order and the epilogue
// scale * (S1 - zp * S2) runs once per output.  Contraction values past K
// are cleared before they reach a product or S2 (the weight bytes there are
// the next row's).
constexpr int GS_WAVES = 8;
constexpr int GS_NT = 64 * GS_WAVES;

template <bool ZP, int NF, int KB, int NB>
__global__ __launch_bounds__(GS_NT) __attribute__((amdgpu_waves_per_eu(2))) void w8a32_grad_slab_kernel(W8A32Args p) {
    constexpr int TS = 16 * NF;     // outputs per workgroup
    constexpr int SK = 64 * KB;     // contraction values per wave step
    __shared__ __attribute__((aligned(16))) float red[GS_WAVES][16][TS];
    __shared__ float s2_red[GS_WAVES][16];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, i16 = lane & 15;
    const int n0 = blockIdx.x * TS;
    const int cols = p.N - n0;
    const int M = p.M, K = p.K;
    const int ldw = (int)p.ldw, lda = (int)p.lda;
    const __amdgpu_buffer_rsrc_t w_rsrc = make_rsrc(p.W + (int64_t)n0 * ldw, (uint32_t)(((cols < TS ? cols : TS) - 1) * ldw + K));
    const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(p.A, (uint32_t)(((M - 1) * lda + K) * 4));
    const uint32_t w_voff = (uint32_t)(i16 * ldw + 16 * g);
    const uint32_t a_voff = (uint32_t)((i16 * lda + 16 * g) * 4);
    const int nsteps = (K + SK - 1) / SK;

    u32x4 wbuf[NB][KB][NF];
    u32x4 abuf[NB][KB][4];
    // Loads of one step into buffer b; a step past K (a wave's last round)
    // loads from past the buffer ends: zeros, no memory touched.
    auto fetch = [&](int step, int b) {
        const bool live = step < nsteps;
        const uint32_t wo = live ? w_voff + (uint32_t)(step * SK) : 0x80000000u;
        const uint32_t ao = live ? a_voff + (uint32_t)(step * SK * 4) : 0x80000000u;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
            for (int c = 0; c < NF; ++c)
                wbuf[b][kb][c] = buffer_load16(w_rsrc, wo + (uint32_t)(16 * c * ldw + 64 * kb), 0u);
#pragma unroll
            for (int q = 0; q < 4; ++q) abuf[b][kb][q] = buffer_load16(a_rsrc, ao + (uint32_t)((64 * kb + 4 * q) * 4), 0u);
        }
    };

    v4f acc[NF];
#pragma unroll
    for (int c = 0; c < NF; ++c) acc[c] = v4f{0.f, 0.f, 0.f, 0.f};
    float s2 = 0.f;   // this lane's share of S2 for row i16

    auto consume = [&](int b, int step) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int k0 = step * SK + 64 * kb + 16 * g;
            float a[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                a[4 * q] = __uint_as_float(abuf[b][kb][q].x);
                a[4 * q + 1] = __uint_as_float(abuf[b][kb][q].y);
                a[4 * q + 2] = __uint_as_float(abuf[b][kb][q].z);
                a[4 * q + 3] = __uint_as_float(abuf[b][kb][q].w);
            }
            if (k0 + 16 > K) {   // values reaching past K: cleared
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    if (k0 + e >= K) a[e] = 0.f;
            }
            if constexpr (ZP) {
                s2 += ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7])) +
                      (((a[8] + a[9]) + (a[10] + a[11])) + ((a[12] + a[13]) + (a[14] + a[15])));
            }
            v8bf pa[2][3];
            split8(a, pa[0][0], pa[0][1], pa[0][2]);
            split8(a + 8, pa[1][0], pa[1][1], pa[1][2]);
#pragma unroll
            for (int c = 0; c < NF; ++c)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const v8bf bw = half8(wbuf[b][kb][c], h);
#pragma unroll
                    for (int pl = 0; pl < 3; ++pl)
                        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[h][pl], bw, acc[c], 0, 0, 0);
                }
        }
    };

    // This wave's steps: wave + GS_WAVES * i, i < n_my (a multiple of NB, the
    // same for every wave; steps past K add nothing), NB in flight.
    const int n_my = (((nsteps + GS_WAVES - 1) / GS_WAVES) + NB - 1) / NB * NB;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        fetch(wave + GS_WAVES * b, b);
        __builtin_amdgcn_sched_barrier(0);
    }
    int i = 0;
    for (; i + NB < n_my; i += NB) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            consume(b, wave + GS_WAVES * (i + b));
            __builtin_amdgcn_sched_barrier(0);
            fetch(wave + GS_WAVES * (i + NB + b), b);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) consume(b, wave + GS_WAVES * (i + b));

    // Register r of fragment c holds row 4g + r, output 16c + i16.
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        if (4 * g + r >= M) continue;
#pragma unroll
        for (int c = 0; c < NF; ++c) red[wave][4 * g + r][16 * c + i16] = acc[c][r];
    }
    if constexpr (ZP) {
        s2 += __shfl_xor(s2, 16);
        s2 += __shfl_xor(s2, 32);
        if (g == 0) s2_red[wave][i16] = s2;
    }
    __syncthreads();

    const float zp = (float)p.zp;
    const bool vec_out = (p.ldc % 4 == 0) && ((reinterpret_cast<uintptr_t>(p.C) & 15) == 0);
    const int items = M * (TS / 4);
    for (int it = tid; it < items; it += GS_NT) {
        const int m = it / (TS / 4), cg = it % (TS / 4);
        const int n = n0 + 4 * cg;
        if (n >= p.N) continue;
        v4f v = *reinterpret_cast<const v4f*>(&red[0][m][4 * cg]);
#pragma unroll
        for (int w = 1; w < GS_WAVES; ++w) v = v + *reinterpret_cast<const v4f*>(&red[w][m][4 * cg]);
        float s2m = 0.f;
        if constexpr (ZP) {
            s2m = s2_red[0][m];
#pragma unroll
            for (int w = 1; w < GS_WAVES; ++w) s2m = s2m + s2_red[w][m];
        }
        float f[4] = {v[0], v[1], v[2], v[3]};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if constexpr (ZP) f[e] = f[e] - zp * s2m;
            f[e] = p.scale * f[e];
        }
        float* dst = p.C + (int64_t)m * p.ldc + n;
        if (vec_out && n + 4 <= p.N) {
            *reinterpret_cast<float4*>(dst) = make_float4(f[0], f[1], f[2], f[3]);
            continue;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (n + e < p.N) dst[e] = f[e];
    }
}

template <int NF, int KB, int NB>
hipError_t launch_grad_slab_cfg(const W8A32Args& a, hipStream_t s) {
    const dim3 grid((a.N + 16 * NF - 1) / (16 * NF));
    if (a.zp != 0) hipLaunchKernelGGL((w8a32_grad_slab_kernel<true, NF, KB, NB>), grid, dim3(GS_NT), 0, s, a);
    else hipLaunchKernelGGL((w8a32_grad_slab_kernel<false, NF, KB, NB>), grid, dim3(GS_NT), 0, s, a);
    return hipGetLastError();
}

}  // namespace

void w8a32_skinny_plan(int64_t M, int64_t N, int64_t K, int forced, int* splits, int* split_k) {
    const int64_t tiles_n = ((M + 15) / 16) * ((N + TN - 1) / TN);   // (row block, column tile) units
    const int64_t steps = (K + KS - 1) / KS;
    int64_t per;
    if (forced > 0) {
        per = (steps + forced - 1) / forced;
    } else {
        // at most one workgroup per CU (the kernel holds a CU alone): 96
        // units would otherwise give 3 splits, 288 workgroups, two rounds
        const int64_t want = std::max<int64_t>(1, 256 / tiles_n);
        per = (steps + want - 1) / want;
    }
    per = ((per + 2 * WAVES - 1) / (2 * WAVES)) * (2 * WAVES);
    int64_t n = (steps + per - 1) / per;
    // more column tiles than the fixed ticket header holds: one split
    if (n > 1 && tiles_n > SKINNY_MAX_TICKETS) {
        per = ((steps + 2 * WAVES - 1) / (2 * WAVES)) * (2 * WAVES);
        n = 1;
    }
    *splits = (int)n;
    *split_k = (int)(per * KS);
}

size_t w8a32_skinny_bytes(int64_t M, int64_t N, int splits) {
    if (splits <= 1) return 0;
    const size_t tiles_n = (size_t)((M + 15) / 16) * (size_t)((N + TN - 1) / TN);
    return SKINNY_TICKET_BYTES + tiles_n * (size_t)splits * SLOT_ROWS * TN * 4;
}

hipError_t launch_w8a32_skinny(const W8A32Args& a, bool wt, hipStream_t s, const char** name) {
    *name = wt ? "w8a32_input_grad_skinny" : "w8a32_skinny";
    const dim3 grid((a.N + TN - 1) / TN, a.splits > 1 ? a.splits : 1, (a.M + 15) / 16);
    if (a.M < 1 || a.M > SKINNY_W8A32_MAX_M || a.split_k % (KS * 2 * WAVES) != 0 ||
        (int64_t)a.split_k * grid.y < a.K ||
        (grid.y > 1 && (a.workspace == nullptr || (int)(grid.x * grid.z) > SKINNY_MAX_TICKETS)))
        return hipErrorInvalidValue;
    if (wt) {
        // eight waves for one block of rows (graph-timed at N = K = 8192,
        // identical bits: M = 1 22.5 -> 20.8 us, M = 16 24.1 -> 23.1), four
        // for several (M = 40: 49.1 against 51.7 with eight)
        if (grid.z == 1) {
            if (a.zp != 0) hipLaunchKernelGGL((w8a32_skinny_kernel<true, true, 8, 64>), grid, dim3(512), 0, s, a);
            else hipLaunchKernelGGL((w8a32_skinny_kernel<false, true, 8, 64>), grid, dim3(512), 0, s, a);
        } else {
            if (a.zp != 0) hipLaunchKernelGGL((w8a32_skinny_kernel<true, true>), grid, dim3(NT), 0, s, a);
            else hipLaunchKernelGGL((w8a32_skinny_kernel<false, true>), grid, dim3(NT), 0, s, a);
        }
    } else {
        if (a.zp != 0) hipLaunchKernelGGL((w8a32_skinny_kernel<true, false, 8, 32>), grid, dim3(512), 0, s, a);
        else hipLaunchKernelGGL((w8a32_skinny_kernel<false, false, 8, 32>), grid, dim3(512), 0, s, a);
    }
    return hipGetLastError();
}

bool w8a32_grad_slab_ok(const W8A32Args& a) {
    const uintptr_t al = reinterpret_cast<uintptr_t>(a.A) | reinterpret_cast<uintptr_t>(a.W);
    if ((al & 15) != 0 || a.lda % 4 != 0 || a.ldw % 16 != 0 || a.K % 4 != 0) return false;
    if (a.M < 1 || a.M > 16 || a.N < 1 || a.K < 1) return false;
    // 32-bit buffer offsets: a live step reads below K + 512 in a row
    return (int64_t)48 * a.ldw + a.K + 512 < ((int64_t)1 << 31) &&
           ((int64_t)16 * a.lda + a.K + 512) * 4 < ((int64_t)1 << 31);
}

// Steps: 64 contraction values two deep for one or two rows, 128 two deep
// above (32 outputs per workgroup; 16-output slabs and four-deep forms
// measured slower at N = K = 8192).
hipError_t launch_w8a32_grad_slab(const W8A32Args& a, hipStream_t s, const char** name) {
    *name = "w8a32_input_grad_slab";
    if (!w8a32_grad_slab_ok(a)) return hipErrorInvalidValue;
    if (a.M <= 2) return launch_grad_slab_cfg<2, 1, 2>(a, s);
    return launch_grad_slab_cfg<2, 2, 2>(a, s);
}

}  // namespace qg

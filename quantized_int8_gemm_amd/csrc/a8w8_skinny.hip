// Skinny (decode-shaped) A8W8 kernel for M <= 16 on gfx950.
//
// Operator: "Feature/a8w8 matmul dequant fusion" -- int8 matmul into an
// INT32 accumulator (optionally one given as input, the page's
// matmul-dequant-acc op), cast to FP32, times act_scale[m], times
// weight_scale[n], cast to the output type.  That page lowers logical M == 1
// to a separate GEMV; here every M up to 16 takes this path, which is bound by
// reading the weight once from HBM.
//
// Grid: (N / 256 column tiles) x (S splits of K).  Each workgroup streams a
// [K/S x 256] slab of W once; its four waves take 64-row steps round robin.
//  * A lane (g = lane/16, c = lane%16) loads rows 16g .. 16g+15 of the step
//    as 16-byte vectors at columns 16c .. 16c+15 (16 lanes cover 256
//    contiguous bytes of a row), two steps ahead of the one being multiplied,
//    with the non-temporal cache policy (every weight byte is read once).
//  * The lane's 16 x 16 byte block is transposed in registers; column j of it
//    is then exactly a matrix-core B fragment (16 k-bytes of column 16c + j),
//    and row c of A is the matching A fragment, so v_mfma_i32_16x16x64_i8
//    number j accumulates output columns {16c + j}.  No LDS in the hot loop.
//  * The four waves' int32 tiles are added through LDS in natural column
//    order.  With S == 1 the epilogue runs there.  With S > 1 each split
//    stores its exact int32 partial (rows < M) and takes a ticket; the last
//    split of a column tile adds the S partials (integer addition: any order
//    gives the same bits), runs the epilogue once and resets the ticket.
// Rows past M and bytes past K read as zero through the buffer range checks
// (or meet zero weight rows), so they add nothing.
//
// The same kernel computes MatMulInteger ("feat(onnx-to-hip): lower quantized
// integer conv and matmul", section "What", MatMulInteger) for M <= 16 with B
// as [K,N] and K a multiple of 64 (EPI_I32): uint8 operands are flipped to
// int8 - 128 as they are multiplied, each lane also takes the row sums of its
// A fragments and the column sums of its transposed weight block (v_dot4),
// those sums travel with the partial tiles, and the epilogue applies
// Y = acc + cb[n] * rowsum[m] + ca[m] * (colsum[n] + K * cb[n]) in wrapping
// int32 arithmetic.  Steps past K are masked (their flips and A bytes
// zeroed), so only the K rows of both operands reach the sums.
#include <mutex>

#include "device_common.h"
#include "kernels.h"

namespace qg {
namespace {

constexpr int TN = 256;     // columns per workgroup
constexpr int KS = 64;      // k rows per wave step
constexpr int WAVES = 4;    // the fewest waves of a workgroup: steps per split are a multiple of 2 * WAVES

// In-place 16 x 16 byte transpose: on entry v[r] holds row r (16 bytes); on
// exit v[c] holds column c (16 bytes, rows 0..15 in order).  Block (q, d) of
// 4 x 4 bytes (rows 4q.., bytes 4d..) moves to block (d, q), so the two are
// transposed together.
__device__ __forceinline__ void transpose16x16_inplace(u32x4 v[16]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int d = q; d < 4; ++d) {
            uint32_t x[4], y[4], xs[4], ys[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] = (&v[4 * q + i].x)[d];
#pragma unroll
            for (int i = 0; i < 4; ++i) xs[i] = (&v[4 * d + i].x)[q];
            transpose4x4_bytes(x, y);
            transpose4x4_bytes(xs, ys);
#pragma unroll
            for (int c = 0; c < 4; ++c) (&v[4 * d + c].x)[q] = y[c];
#pragma unroll
            for (int c = 0; c < 4; ++c) (&v[4 * q + c].x)[d] = ys[c];
        }
    }
}

// MatMulInteger's sums do not fit beside two waves per SIMD; its grid gives
// one workgroup per CU anyway.
// WV waves: eight (two per SIMD, so one wave's transposes run beside
// another's loads; 8192^2 at M = 1 / 4 / 16: 14.8 / 15.5 / 17.5 -> 14.4 /
// 15.0 / 16.8 us) when each split spans a multiple of 16 steps, else four;
// MatMulInteger four when it takes the weight's column sums (they need the
// registers of one wave per SIMD).  CS: MatMulInteger takes the column sums,
// which only multiply ca[m]; with no activation correction (ca = 0, e.g.
// uint8 activations at zero point 128) it skips them.
template <bool VEC, int EPI, bool BKM = false, int WV = 4, bool CS = true>
__global__ __launch_bounds__(64 * WV) __attribute__((amdgpu_waves_per_eu(EPI == EPI_I32 ? 1 : 2))) void a8w8_skinny_kernel(Int8GemmArgs p) {
    constexpr bool I32 = EPI == EPI_I32;
    static_assert(!I32 || WV == 4, "MatMulInteger's sums take four waves");
    constexpr int NTW = 64 * WV;
    // A split's partial: 16 rows of the tile, then (MatMulInteger) a row of
    // column sums and a row whose first 16 entries are the row sums.
    constexpr int SLOT_ROWS = I32 ? 18 : 16;
    __shared__ __attribute__((aligned(16))) int32_t red[WV][16][TN];
    __shared__ float ws_tile[I32 ? 1 : TN];
    __shared__ float as_rows[I32 ? 1 : 16];
    // MatMulInteger: per-wave sums, the tile's totals, cb[n] and ca[m]
    __shared__ __attribute__((aligned(16))) int32_t cs_red[I32 ? WV : 1][I32 ? TN : 4];
    __shared__ int32_t rs_red[I32 ? WV : 1][16];
    __shared__ __attribute__((aligned(16))) int32_t cs_tot[I32 ? TN : 4];
    __shared__ __attribute__((aligned(16))) int32_t rs_tot[16];
    __shared__ int32_t cb_tile[I32 ? TN : 1];
    __shared__ int32_t ca_rows[I32 ? 16 : 1];
    __shared__ int ticket;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    const int tn = blockIdx.x, split = blockIdx.y, S = gridDim.y;
    const int n0 = tn * TN;
    const int cols = p.N - n0;

    // K range of this split: `per` 64-row steps, a multiple of 2*WV.
    const int per = p.split_steps;
    const int s_begin = split * per;

    const int ldb = (int)p.ldb, lda = (int)p.lda;
    const int8_t* Wt = BKM ? p.B + (int64_t)n0 * ldb : p.B + n0;
    // [N,K]: the tile's own rows only (the whole weight may span 2^31 bytes)
    const __amdgpu_buffer_rsrc_t w_rsrc = BKM ? make_rsrc(Wt, (uint32_t)(((cols < TN ? cols : TN) - 1) * ldb + p.K))
                                              : make_rsrc(Wt, (uint32_t)((p.K - 1) * ldb + cols));
    const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(p.A, (uint32_t)((p.M - 1) * lda + p.K));
    const uint32_t w_voff = BKM ? (uint32_t)(16 * c16 * ldb + 16 * g) : (uint32_t)(16 * g * ldb + 16 * c16);
    const uint32_t a_voff = (uint32_t)(c16 * lda + 16 * g);

    // The epilogue's scales (MatMulInteger: zero-point terms), loaded now so
    // their latency hides behind the weight stream.
    if constexpr (I32) {
        if (tid < TN) {
            const int n = n0 + tid;
            int zb = 0;
            if (p.b_zp != nullptr && n < p.N)
                zb = p.b_zp_u8 ? (int)static_cast<const uint8_t*>(p.b_zp)[n * p.b_zp_stride]
                               : (int)static_cast<const int8_t*>(p.b_zp)[n * p.b_zp_stride];
            cb_tile[tid] = n < p.N ? p.sb - zb : 0;
        }
        if (tid < 16) {
            int ca = p.ca;
            if (p.a_zp != nullptr) {
                const int i = (tid % p.a_zp_rows) * p.a_zp_stride;
                ca = p.sa - (p.a_zp_u8 ? (int)static_cast<const uint8_t*>(p.a_zp)[i]
                                       : (int)static_cast<const int8_t*>(p.a_zp)[i]);
            }
            ca_rows[tid] = tid < p.M ? ca : 0;
        }
    } else {
        if (tid < TN) ws_tile[tid] = (n0 + tid < p.N) ? p.weight_scale[(n0 + tid) * p.ws_stride] : 0.f;
        if (tid < 16) as_rows[tid] = (tid < p.M) ? p.act_scale[tid * p.as_stride] : 0.f;
    }

    u32x4 wbuf[2][16];
    u32x4 abuf[2];
    // Loads of one step into buffer b.  Unconditional: a step past this
    // split's range reads rows of the matrix (or zeros past K) that are never
    // multiplied, so no branch separates the loads and all stay in flight.
    auto fetch = [&](int step, int b) {
        const int k0 = step * KS;
        if constexpr (VEC) {
            if constexpr (BKM) {
                // W as [N,K]: row 16 c16 + j, k-bytes k0 + 16g ..  is already
                // the B fragment of column 16 c16 + j (cached: each step
                // reads half of every 128-byte line)
#pragma unroll
                for (int j = 0; j < 16; ++j) wbuf[b][j] = buffer_load16(w_rsrc, w_voff + (uint32_t)(j * ldb + k0), 0u);
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) wbuf[b][r] = buffer_load16_nt(w_rsrc, w_voff + (uint32_t)((k0 + r) * ldb));
            }
            abuf[b] = buffer_load16(a_rsrc, a_voff + (uint32_t)k0, 0u);
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int gk = k0 + 16 * g + r;
                uint32_t d[4] = {0u, 0u, 0u, 0u};
                if (gk < p.K) {
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int cc = 16 * c16 + e;
                        if (cc < cols) d[e >> 2] |= (uint32_t)(uint8_t)Wt[(int64_t)gk * p.ldb + cc] << (8 * (e & 3));
                    }
                }
                wbuf[b][r] = u32x4{d[0], d[1], d[2], d[3]};
            }
            uint32_t d[4] = {0u, 0u, 0u, 0u};
            if (c16 < p.M) {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int kk = k0 + 16 * g + e;
                    if (kk < p.K) d[e >> 2] |= (uint32_t)(uint8_t)p.A[(int64_t)c16 * p.lda + kk] << (8 * (e & 3));
                }
            }
            abuf[b] = u32x4{d[0], d[1], d[2], d[3]};
        }
    };

    v4i acc[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = v4i{0, 0, 0, 0};
    // MatMulInteger: this lane's sums of A row c16 and of weight columns
    // 16 c16 + j over the k rows it multiplies (after the flips).
    int rs = 0;
    int cs[I32 ? 16 : 1];
#pragma unroll
    for (int j = 0; j < (I32 ? 16 : 1); ++j) cs[j] = 0;
    const int nsteps = (p.K + KS - 1) / KS;

    // This wave's steps: s_begin + wave + WV*i, i < n_my.  Every split
    // spans a multiple of 2*WV steps (steps past K read as zeros and add
    // nothing), so n_my is even and the same for all waves, and no branch
    // sits between the loads.  Two steps are in flight; the loop is unrolled
    // by two so both register buffers have fixed homes, and the last pair is
    // peeled so that nothing is fetched past the wave's range.
    const int first = s_begin + wave;
    const int n_my = per / WV;
    auto consume = [&](int b, int step) {
        if constexpr (I32) {
            // a step past K multiplies nothing: no flips, A bytes cleared
            // (those of rows < M - 1 would be the next row's)
            const bool live = step < nsteps;
            const uint32_t fa = live ? p.a_flip : 0u, fb = live ? p.b_flip : 0u;
            if (!live) abuf[b] = u32x4{0u, 0u, 0u, 0u};
            abuf[b] = u32x4{abuf[b].x ^ fa, abuf[b].y ^ fa, abuf[b].z ^ fa, abuf[b].w ^ fa};
#pragma unroll
            for (int r = 0; r < 16; ++r)
                wbuf[b][r] = u32x4{wbuf[b][r].x ^ fb, wbuf[b][r].y ^ fb, wbuf[b][r].z ^ fb, wbuf[b][r].w ^ fb};
            rs = sum_i8x4(abuf[b].w, sum_i8x4(abuf[b].z, sum_i8x4(abuf[b].y, sum_i8x4(abuf[b].x, rs))));
        }
        if constexpr (BKM) {
            // bytes past K in a row of either operand are the next row's:
            // a 16-byte piece there (K % 16 == 0) multiplies nothing
            if (step * KS + 16 * g >= p.K) abuf[b] = u32x4{0u, 0u, 0u, 0u};
        } else {
            transpose16x16_inplace(wbuf[b]);
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[j] = mfma_i8_16x16x64(abuf[b], wbuf[b][j], acc[j]);
        if constexpr (I32 && CS) {
#pragma unroll
            for (int j = 0; j < 16; ++j)
                cs[j] = sum_i8x4(wbuf[b][j].w, sum_i8x4(wbuf[b][j].z, sum_i8x4(wbuf[b][j].y, sum_i8x4(wbuf[b][j].x, cs[j]))));
        }
    };
    // Scheduling barriers keep each fetch's loads together, so that waiting
    // for one buffer never waits for the other buffer's loads.
    fetch(first, 0);
    __builtin_amdgcn_sched_barrier(0);
    fetch(first + WV, 1);
    __builtin_amdgcn_sched_barrier(0);
    int i = 0;
    for (; i + 2 < n_my; i += 2) {
        consume(0, first + WV * i);
        __builtin_amdgcn_sched_barrier(0);
        fetch(first + WV * (i + 2), 0);
        __builtin_amdgcn_sched_barrier(0);
        consume(1, first + WV * (i + 1));
        __builtin_amdgcn_sched_barrier(0);
        fetch(first + WV * (i + 3), 1);
        __builtin_amdgcn_sched_barrier(0);
    }
    consume(0, first + WV * i);
    consume(1, first + WV * (i + 1));

    // Add the four waves' tiles through LDS.  Register r of MFMA j holds
    // row 4g + r, column 16*c16 + j, so for each r a lane owns 16 consecutive
    // columns and writes them as four 16-byte chunks.  Chunk 4*c16 + q of a
    // staged row sits at 4*c16 + (q ^ ((c16 >> 2) & 3)): the 16 lanes of a
    // group then hit 16 distinct chunks of a 256-byte bank line.
    const int M = p.M;
    auto chunk = [](int ch) { return (ch & ~3) | ((ch ^ (ch >> 4)) & 3); };
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        if (4 * g + r >= M) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const v4i v = v4i{acc[4 * q][r], acc[4 * q + 1][r], acc[4 * q + 2][r], acc[4 * q + 3][r]};
            *reinterpret_cast<v4i*>(&red[wave][4 * g + r][4 * chunk(4 * c16 + q)]) = v;
        }
    }
    if constexpr (I32) {
        // the four lane groups held different k rows: add them, then each
        // wave leaves its sums in LDS
        rs += __shfl_xor(rs, 16);
        rs += __shfl_xor(rs, 32);
        if constexpr (CS) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                cs[j] += __shfl_xor(cs[j], 16);
                cs[j] += __shfl_xor(cs[j], 32);
            }
        }
        if (g == 0) {
            rs_red[wave][c16] = rs;
            if constexpr (CS) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *reinterpret_cast<v4i*>(&cs_red[wave][16 * c16 + 4 * q]) =
                        v4i{cs[4 * q], cs[4 * q + 1], cs[4 * q + 2], cs[4 * q + 3]};
            }
        }
    }
    __syncthreads();
    if constexpr (I32) {
        // this workgroup's sums over its k range
        if (tid < TN) {
            uint32_t t = 0u;
            if constexpr (CS) {
#pragma unroll
                for (int w = 0; w < WV; ++w) t += (uint32_t)cs_red[w][tid];
            }
            cs_tot[tid] = (int)t;   // without CS: zero, and ca = 0 multiplies it
        }
        if (tid < 16) {
            uint32_t t = 0u;
#pragma unroll
            for (int w = 0; w < WV; ++w) t += (uint32_t)rs_red[w][tid];
            rs_tot[tid] = (int)t;
        }
        __syncthreads();
    }

    // Items: (row m < M, group of 4 columns); each thread takes some.
    auto tile_sum = [&](int m, int cg) -> int4 {
        const int at = 4 * chunk(cg);
        int4 s = *reinterpret_cast<const int4*>(&red[0][m][at]);
#pragma unroll
        for (int w = 1; w < WV; ++w) {
            const int4 v = *reinterpret_cast<const int4*>(&red[w][m][at]);
            s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
        }
        return s;
    };
    // Output row m, columns n .. n+3 (those < N): scales, then one vector
    // store when the four are in range and aligned.
    const bool vec_out = (p.ldo % 4 == 0) && ((reinterpret_cast<uintptr_t>(p.out) & 15) == 0);
    const bool acc_vec = p.acc_in != nullptr && p.ld_acc % 4 == 0 &&
                         (reinterpret_cast<uintptr_t>(p.acc_in) & 15) == 0;
    // The accumulator input of row m, columns n .. n+3 (zeros past N).
    auto load_acc = [&](int m, int n) -> v4i {
        const int32_t* src = p.acc_in + (int64_t)m * p.ld_acc + n;
        if (acc_vec && n + 4 <= p.N) return __builtin_bit_cast(v4i, *reinterpret_cast<const int4*>(src));
        v4i t = v4i{0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (n + e < p.N) t[e] = src[e];
        return t;
    };
    // add_acc: the accumulator input is still to be added (the reducing
    // split folds it into its sum instead).
    auto epilogue = [&](int m, int n, int4 v, bool add_acc) {
        if (n >= p.N) return;
        int32_t vi[4] = {v.x, v.y, v.z, v.w};
        if (add_acc && p.acc_in != nullptr) {   // accumulator input, added before the cast (wrapping)
            const v4i ai = load_acc(m, n);
#pragma unroll
            for (int e = 0; e < 4; ++e) vi[e] = (int32_t)((uint32_t)vi[e] + (uint32_t)ai[e]);
        }
        float f[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            f[e] = (float)vi[e];
            f[e] = f[e] * as_rows[m];
            f[e] = f[e] * ws_tile[(n - n0 + e) & (TN - 1)];
        }
        const int64_t o = (int64_t)m * p.ldo + n;
        if (vec_out && n + 4 <= p.N) {
            if constexpr (EPI == EPI_F32) {
                *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + o) = make_float4(f[0], f[1], f[2], f[3]);
            } else {
                *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + o) =
                    make_uint2(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]));
            }
            return;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (n + e >= p.N) break;
            if constexpr (EPI == EPI_F32) reinterpret_cast<float*>(p.out)[o + e] = f[e];
            else reinterpret_cast<uint16_t*>(p.out)[o + e] = f32_to_bf16_rne(f[e]);
        }
    };
    // MatMulInteger: Y = acc + cb[n] * rowsum[m] + ca[m] * (colsum[n] + K * cb[n]),
    // wrapping, from the tile's totals in LDS.
    const bool vec_y = (p.ldo % 4 == 0) && ((reinterpret_cast<uintptr_t>(p.out) & 15) == 0);
    auto epilogue_i32 = [&](int m, int n, int4 v) {
        if (n >= p.N) return;
        const uint32_t ca = (uint32_t)ca_rows[m], rsm = (uint32_t)rs_tot[m];
        const int32_t vi[4] = {v.x, v.y, v.z, v.w};
        int32_t y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int c = (n - n0 + e) & (TN - 1);
            const uint32_t cb = (uint32_t)cb_tile[c];
            y[e] = (int32_t)((uint32_t)vi[e] + cb * rsm + ca * ((uint32_t)cs_tot[c] + (uint32_t)p.K * cb));
        }
        int32_t* dst = reinterpret_cast<int32_t*>(p.out) + (int64_t)m * p.ldo + n;
        if (vec_y && n + 4 <= p.N) {
            *reinterpret_cast<int4*>(dst) = int4{y[0], y[1], y[2], y[3]};
            return;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (n + e < p.N) dst[e] = y[e];
    };
    auto finish = [&](int m, int n, int4 v, bool add_acc = true) {
        if constexpr (I32) epilogue_i32(m, n, v);
        else epilogue(m, n, v, add_acc);
    };
    const int items = M * (TN / 4);

    if (S == 1) {
        for (int it = tid; it < items; it += NTW) {
            const int m = it / (TN / 4), cg = it % (TN / 4);
            finish(m, n0 + cg * 4, tile_sum(m, cg));
        }
        return;
    }

    // Split-K: workspace = [tickets: one int per column tile, a fixed
    //                       SKINNY_TICKET_BYTES header whatever the shape]
    //                      [partials: per column tile, S x 16 x TN int32]
    // The header's size does not depend on N, so a workspace left by a call
    // of one shape (tickets back at zero, partials arbitrary) serves a call
    // of any other shape: its tickets never overlap old partials.
    // Partials and tickets cross workgroups (and XCDs, whose L2s are not
    // coherent with each other), so every access to them is device-coherent:
    // stores and loads with the device-scope cache policy (they bypass the
    // XCD-private cache level) and an atomic ticket.  Waiting for all
    // outstanding memory operations orders each thread's partial stores
    // before the barrier, and the barrier orders them before thread 0's
    // ticket; no cache-wide writeback or invalidate is needed.
    int* tickets = reinterpret_cast<int*>(p.workspace);
    constexpr int SLOT = SLOT_ROWS * TN * 4;
    char* part = reinterpret_cast<char*>(p.workspace) + SKINNY_TICKET_BYTES + (size_t)tn * S * SLOT;
    // Partial of split s: rows m < M of [16][TN] int32 (MatMulInteger: then
    // the column sums and the row sums), as 16-byte vectors through a buffer
    // resource with device-coherent cache policy.
    const __amdgpu_buffer_rsrc_t p_rsrc = make_rsrc(part, (uint32_t)(S * SLOT));
    constexpr int COHERENT = 16;  // sc1: device scope, bypass the XCD-private cache level
    for (int it = tid; it < items; it += NTW) {
        const int m = it / (TN / 4), cg = it % (TN / 4);
        const int4 s4 = tile_sum(m, cg);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, s4), p_rsrc,
                                               (uint32_t)(split * SLOT + (m * TN + cg * 4) * 4), 0, COHERENT);
    }
    // MatMulInteger sums: 64 vectors of column sums (row 16), 4 of row sums (row 17)
    constexpr int SUM_ITEMS = TN / 4 + 4;
    auto sums_off = [&](int it) { return (uint32_t)((it < TN / 4 ? 16 * TN + 4 * it : 17 * TN + 4 * (it - TN / 4)) * 4); };
    if constexpr (I32) {
        if (tid < SUM_ITEMS) {
            const int32_t* src = tid < TN / 4 ? &cs_tot[4 * tid] : &rs_tot[4 * (tid - TN / 4)];
            __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const v4i*>(src), p_rsrc,
                                                   (uint32_t)(split * SLOT) + sums_off(tid), 0, COHERENT);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) ticket = __hip_atomic_fetch_add(&tickets[tn], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (ticket != S - 1) return;
    // Each thread owns up to four (row, column group) items and keeps all of
    // their partial loads in flight at once: SU splits per round, loads past
    // split S - 1 fall outside the buffer range and read as zero.
    constexpr int SU = 8, IPT = 16 * (TN / 4) / NTW;   // items per thread at M = 16
    static_assert(IPT * NTW == 16 * (TN / 4), "whole items");
    v4i sum[IPT];
    uint32_t off[IPT];
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
        const int it = tid + i * NTW;
        const int m = it / (TN / 4), cg = it % (TN / 4);
        sum[i] = v4i{0, 0, 0, 0};
        // an item past M reads past the buffer (zeros) and is not stored
        off[i] = it < items ? (uint32_t)((m * TN + cg * 4) * 4) : 0xFFFFFFF0u;
        // the accumulator input starts the sum (wrapping, so the order does
        // not matter), its loads in flight with the partials'
        if (!I32 && p.acc_in != nullptr && it < items && n0 + cg * 4 < p.N) sum[i] = load_acc(m, n0 + cg * 4);
    }
    // MatMulInteger: threads below SUM_ITEMS also add one vector of sums
    v4i ssum = v4i{0, 0, 0, 0};
    const uint32_t soff = (I32 && tid < SUM_ITEMS) ? sums_off(tid) : 0xFFFFFFF0u;
    auto add4 = [](v4i a, v4i b) {
        return v4i{(int)((uint32_t)a.x + (uint32_t)b.x), (int)((uint32_t)a.y + (uint32_t)b.y),
                   (int)((uint32_t)a.z + (uint32_t)b.z), (int)((uint32_t)a.w + (uint32_t)b.w)};
    };
    for (int s0 = 0; s0 < S; s0 += SU) {
        v4i v[IPT][SU];
#pragma unroll
        for (int i = 0; i < IPT; ++i)
#pragma unroll
            for (int u = 0; u < SU; ++u) {
                const uint32_t o = off[i] == 0xFFFFFFF0u ? off[i] : off[i] + (uint32_t)((s0 + u) * SLOT);
                v[i][u] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(p_rsrc, o, 0, COHERENT));
            }
        v4i w[I32 ? SU : 1];
        if constexpr (I32) {
#pragma unroll
            for (int u = 0; u < SU; ++u) {
                const uint32_t o = soff == 0xFFFFFFF0u ? soff : soff + (uint32_t)((s0 + u) * SLOT);
                w[u] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(p_rsrc, o, 0, COHERENT));
            }
        }
#pragma unroll
        for (int i = 0; i < IPT; ++i)
#pragma unroll
            for (int u = 0; u < SU; ++u) sum[i] = add4(sum[i], v[i][u]);
        if constexpr (I32) {
#pragma unroll
            for (int u = 0; u < SU; ++u) ssum = add4(ssum, w[u]);
        }
    }
    if constexpr (I32) {
        // the totals over all splits replace this split's own in LDS
        if (tid < SUM_ITEMS) *reinterpret_cast<v4i*>(tid < TN / 4 ? &cs_tot[4 * tid] : &rs_tot[4 * (tid - TN / 4)]) = ssum;
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
        const int it = tid + i * NTW;
        if (it >= items) continue;
        const int m = it / (TN / 4), cg = it % (TN / 4);
        finish(m, n0 + cg * 4, int4{sum[i].x, sum[i].y, sum[i].z, sum[i].w}, false);
    }
    if (tid == 0) __hip_atomic_store(&tickets[tn], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Ticket words to zero: one thread per ticket of the fixed header.
__global__ __launch_bounds__(SKINNY_MAX_TICKETS) void clear_tickets_kernel(int* tickets) {
    tickets[threadIdx.x] = 0;
}

// Split-K scratch held by the library for callers that cannot allocate (the
// workspace-free A8W8 entry point): one copy per GPU, kept until the process
// ends.  Host code never passes `scratch` itself to a kernel (its host-side
// name is no device address); it uses the address hipGetSymbolAddress gives
// for the current device.
__device__ __attribute__((aligned(256))) uint8_t scratch[SKINNY_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex scratch_mutex;
void* scratch_ptr[MAX_DEVICES];

}  // namespace

hipError_t skinny_scratch(hipStream_t s, void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (scratch_ptr[dev] == nullptr) {
        // Set-up, once per device with that device current: look up this
        // device's copy of the array, then clear its tickets on the caller's
        // stream ahead of the first kernel that uses them (a fill kernel, not
        // a memset, so that a captured first call records a kernel node).
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        hipLaunchKernelGGL(clear_tickets_kernel, dim3(1), dim3(SKINNY_MAX_TICKETS), 0, s, reinterpret_cast<int*>(p));
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        scratch_ptr[dev] = p;
    }
    *ptr = scratch_ptr[dev];
    return hipSuccess;
}

size_t skinny_workspace_bytes(int M, int N, int splits, bool sums) {
    (void)M;
    if (splits <= 1) return 0;
    const size_t tiles_n = (size_t)(N + TN - 1) / TN;
    return SKINNY_TICKET_BYTES + tiles_n * (size_t)splits * (sums ? 18 : 16) * TN * 4;
}

// Steps (64 k-rows) per split: a multiple of 2*WAVES, chosen so that about
// one workgroup runs per compute unit (256 CUs).
int skinny_split_steps(int N, int K) {
    const int tiles_n = (N + TN - 1) / TN;
    const int steps = (K + KS - 1) / KS;
    const int want = (256 + tiles_n - 1) / tiles_n;        // splits wanted
    int per = (steps + want - 1) / want;
    per = ((per + 2 * WAVES - 1) / (2 * WAVES)) * (2 * WAVES);
    return per;
}

int skinny_splits_for(int N, int K, int per) {
    const int steps = (K + KS - 1) / KS;
    return (steps + per - 1) / per;
}

int skinny_splits(int M, int N, int K) {
    (void)M;
    return skinny_splits_for(N, K, skinny_split_steps(N, K));
}

namespace {
// One A8W8 decode launch with WV waves per workgroup.
template <bool VEC, int EPI, bool BKM, int WV>
void launch_waves(const Int8GemmArgs& a, dim3 grid, hipStream_t s) {
    hipLaunchKernelGGL((a8w8_skinny_kernel<VEC, EPI, BKM, WV>), grid, dim3(64 * WV), 0, s, a);
}
template <bool VEC, int EPI, bool BKM>
void launch_a8w8(const Int8GemmArgs& a, dim3 grid, hipStream_t s) {
    if (a.split_steps % 16 == 0) launch_waves<VEC, EPI, BKM, 8>(a, grid, s);
    else launch_waves<VEC, EPI, BKM, 4>(a, grid, s);
}
}  // namespace

hipError_t launch_a8w8_skinny(const Int8GemmArgs& a, bool vec, int epi, hipStream_t s, const char** name, bool bkm) {
    dim3 grid((a.N + TN - 1) / TN, a.splits > 1 ? a.splits : 1);
    *name = epi == EPI_I32 ? "matmul_integer_skinny" : "a8w8_skinny";
    if (a.split_steps % (2 * WAVES) != 0 || (int64_t)a.split_steps * grid.y * KS < a.K) return hipErrorInvalidValue;
    if (grid.y > 1 && (a.workspace == nullptr || (int)grid.x > SKINNY_MAX_TICKETS)) return hipErrorInvalidValue;
    if (a.M > 16 || a.batch != 1) return hipErrorInvalidValue;
    if (bkm) {   // A8W8 with W as [N,K]: 16-byte rows, K % 16 == 0
        if (!vec || epi == EPI_I32 || a.K % 16 != 0) return hipErrorInvalidValue;
        if (epi == EPI_F32) launch_a8w8<true, EPI_F32, true>(a, grid, s);
        else launch_a8w8<true, EPI_BF16, true>(a, grid, s);
    } else if (epi == EPI_I32) {   // 16-byte rows, B as [K,N], whole 64-row steps
        if (!vec || a.K % KS != 0 || (a.a_zp != nullptr && a.a_zp_rows < 1)) return hipErrorInvalidValue;
        if (a.ca != 0 || a.a_zp != nullptr) launch_waves<true, EPI_I32, false, 4>(a, grid, s);
        else hipLaunchKernelGGL((a8w8_skinny_kernel<true, EPI_I32, false, 4, false>), grid, dim3(256), 0, s, a);
    } else if (vec) {
        if (epi == EPI_F32) launch_a8w8<true, EPI_F32, false>(a, grid, s);
        else launch_a8w8<true, EPI_BF16, false>(a, grid, s);
    } else {
        if (epi == EPI_F32) launch_a8w8<false, EPI_F32, false>(a, grid, s);
        else launch_a8w8<false, EPI_BF16, false>(a, grid, s);
    }
    return hipGetLastError();
}

}  // namespace qg

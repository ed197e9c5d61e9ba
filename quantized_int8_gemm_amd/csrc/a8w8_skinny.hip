// Skinny (decode-shaped) A8W8 kernel for M <= 16 on gfx950.
//
// Operator: "Feature/a8w8 matmul dequant fusion" -- int8 matmul into an
// INT32 accumulator, cast to FP32, times act_scale[m], times
// weight_scale[n], cast to the output type.  That page lowers logical M == 1
// to a separate GEMV; here every M up to 16 takes this path, which is bound by
// reading the weight once from HBM.
//
// Grid: (N / 256 column tiles) x (S splits of K).  Each workgroup streams a
// [K/S x 256] slab of W exactly once:
//  * every thread reads a 16-row x 16-byte block per 256-row chunk (16
//    consecutive lanes cover 256 contiguous bytes of a row), transposes it in
//    registers, and writes 16 k-contiguous column segments to LDS, so W^T is
//    ready for the matrix cores;
//  * A (at most 16 rows, resident in L2) is loaded straight into matrix-core
//    fragments; rows past M and bytes past K read as zero or meet zero
//    weight rows, so they add nothing;
//  * v_mfma_i32_16x16x64_i8 accumulates the 16 x 256 int32 partial tile.
// With S == 1 the epilogue runs directly.  With S > 1 each split stores its
// exact int32 partial in the workspace and takes a ticket; the last split of a
// column tile adds the S partials (integer addition, so the order does not
// matter) and runs the epilogue once, then resets the ticket to zero.
#include "device_common.h"
#include "kernels.h"

namespace qg {
namespace {

constexpr int NT = 256;     // threads
constexpr int TN = 256;     // columns per workgroup
constexpr int KC = 256;     // k rows per chunk
constexpr int ROW = KC;     // LDS row bytes (one column of W^T per row)

// LDS row of W^T that holds tile column n (16x16 block transposed: column
// cb*16 + c goes to row c*16 + cb) and the swizzled offset of segment s.
__device__ __forceinline__ int sk_off(int row, int seg) { return row * ROW + ((seg ^ (row & 15)) << 4); }
__device__ __forceinline__ int sk_col_of_row(int row) { return (row & 15) * 16 + (row >> 4); }

__device__ __forceinline__ void transpose16x16(const u32x4 in[16], u32x4 out[16]) {
    // out[c] word q = bytes (rows 4q..4q+3, column c)
#pragma unroll
    for (int d = 0; d < 4; ++d) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t x[4], y[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] = (&in[q * 4 + i].x)[d];
            transpose4x4_bytes(x, y);
#pragma unroll
            for (int c = 0; c < 4; ++c) (&out[d * 4 + c].x)[q] = y[c];
        }
    }
}

template <bool VEC, int EPI>
__global__ __launch_bounds__(NT) void a8w8_skinny_kernel(Int8GemmArgs p) {
    __shared__ __attribute__((aligned(16))) uint8_t Ws[TN * ROW];
    __shared__ int ticket;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l16 = lane & 15;
    const int tn = blockIdx.x;
    const int split = blockIdx.y;
    const int S = gridDim.y;
    const int n0 = tn * TN;
    const int cols = p.N - n0;

    // K range of this split, whole chunks except possibly the last split.
    const int chunks = (p.K + KC - 1) / KC;
    const int per = (chunks + S - 1) / S;
    const int c_begin = split * per;
    int c_end = c_begin + per;
    if (c_end > chunks) c_end = chunks;

    const int ldb = (int)p.ldb, lda = (int)p.lda;
    const int8_t* Wt = p.B + n0;
    const __amdgpu_buffer_rsrc_t w_rsrc = make_rsrc(Wt, (uint32_t)((p.K - 1) * ldb + cols));
    const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(p.A, (uint32_t)((p.M - 1) * lda + p.K));

    const int cb = tid & 15, rg = tid >> 4;           // this thread's 16x16 block
    const uint32_t w_voff = (uint32_t)(rg * 16 * ldb + cb * 16);
    const uint32_t a_voff = (uint32_t)(l16 * lda + (lane >> 4) * 16);

    u32x4 wst[16];
    u32x4 ast[KC / 64];
    auto load_a = [&](int k) -> u32x4 {   // 16 bytes of row l16 from k + 16*(lane/16) on
        if constexpr (VEC) {
            return buffer_load16(a_rsrc, a_voff + (uint32_t)k, 0u);
        } else {
            uint32_t d[4] = {0u, 0u, 0u, 0u};
            if (l16 < p.M) {
                const int kk = k + (lane >> 4) * 16;
#pragma unroll
                for (int b = 0; b < 16; ++b)
                    if (kk + b < p.K)
                        d[b >> 2] |= (uint32_t)(uint8_t)p.A[(int64_t)l16 * p.lda + kk + b] << (8 * (b & 3));
            }
            return u32x4{d[0], d[1], d[2], d[3]};
        }
    };
    // Issue the loads of chunk c: this thread's 16 x 16 W block and its A
    // fragments (A is small and L2 resident).
    auto fetch = [&](int c) {
        const int k0 = c * KC;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            if constexpr (VEC) {
                wst[r] = buffer_load16(w_rsrc, w_voff + (uint32_t)((k0 + r) * ldb), 0u);
            } else {
                const int gk = k0 + rg * 16 + r;
                uint32_t d[4] = {0u, 0u, 0u, 0u};
                if (gk < p.K) {
#pragma unroll
                    for (int b = 0; b < 16; ++b) {
                        const int cc = cb * 16 + b;
                        if (cc < cols) d[b >> 2] |= (uint32_t)(uint8_t)Wt[(int64_t)gk * p.ldb + cc] << (8 * (b & 3));
                    }
                }
                wst[r] = u32x4{d[0], d[1], d[2], d[3]};
            }
        }
#pragma unroll
        for (int ks = 0; ks < KC / 64; ++ks) ast[ks] = load_a(k0 + ks * 64);
    };

    v4i acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = v4i{0, 0, 0, 0};

    if (c_begin < c_end) fetch(c_begin);
    for (int c = c_begin; c < c_end; ++c) {
        // registers -> LDS (W^T), then prefetch the next chunk
        u32x4 t[16];
        transpose16x16(wst, t);
        u32x4 af[KC / 64];
#pragma unroll
        for (int ks = 0; ks < KC / 64; ++ks) af[ks] = ast[ks];
        __syncthreads();  // previous chunk's reads are done
#pragma unroll
        for (int i = 0; i < 16; ++i) *reinterpret_cast<u32x4*>(Ws + sk_off(i * 16 + cb, rg)) = t[i];
        __syncthreads();
        if (c + 1 < c_end) fetch(c + 1);
#pragma unroll
        for (int ks = 0; ks < KC / 64; ++ks) {
            const int seg = ks * 4 + (lane >> 4);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const u32x4 bf = *reinterpret_cast<const u32x4*>(Ws + sk_off(wave * 64 + j * 16 + l16, seg));
                acc[j] = mfma_i8_16x16x64(af[ks], bf, acc[j]);
            }
        }
    }

    // Row 4*(lane/16)+r, column col_of_row(wave*64 + j*16 + l16) of the tile.
    const int row0 = 4 * (lane >> 4);
    auto epilogue = [&](int j, int r, int32_t v) {
        const int m = row0 + r;
        const int n = n0 + sk_col_of_row(wave * 64 + j * 16 + l16);
        if (m >= p.M || n >= p.N) return;
        float f = (float)v;
        f = f * p.act_scale[m * p.as_stride];
        f = f * p.weight_scale[n * p.ws_stride];
        const int64_t o = (int64_t)m * p.ldo + n;
        if constexpr (EPI == EPI_F32) reinterpret_cast<float*>(p.out)[o] = f;
        else reinterpret_cast<uint16_t*>(p.out)[o] = f32_to_bf16_rne(f);
    };

    if (S == 1) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) epilogue(j, r, acc[j][r]);
        return;
    }

    // Split-K: workspace = [tickets: one int per column tile, padded to 256 B]
    //                      [partials: S x 16 x TN int32 per column tile]
    const int tiles_n = gridDim.x;
    int* tickets = reinterpret_cast<int*>(p.workspace);
    int32_t* part = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(p.workspace) +
                                               ((tiles_n * 4 + 255) / 256) * 256) +
                    (int64_t)tn * S * 16 * TN;
    // Partials and tickets cross workgroups (and XCDs, whose L2s are not
    // coherent with each other), so every access to them is a device-scope
    // coherent access: stores and loads that bypass the non-coherent cache
    // level, and an atomic ticket.  The wait on all outstanding memory
    // operations orders each thread's partial stores before the barrier,
    // and the barrier orders them before thread 0's ticket.  No cache-wide
    // writeback or invalidate is needed.
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            __hip_atomic_store(&part[(split * 16 + row0 + r) * TN + wave * 64 + j * 16 + l16], acc[j][r],
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) ticket = __hip_atomic_fetch_add(&tickets[tn], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (ticket != S - 1) return;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            uint32_t sum = 0;
            const int idx = (row0 + r) * TN + wave * 64 + j * 16 + l16;
            for (int s = 0; s < S; ++s)
                sum += (uint32_t)__hip_atomic_load(&part[s * 16 * TN + idx], __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
            epilogue(j, r, (int32_t)sum);
        }
    }
    if (tid == 0) __hip_atomic_store(&tickets[tn], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

size_t skinny_workspace_bytes(int M, int N, int splits) {
    (void)M;
    if (splits <= 1) return 0;
    const size_t tiles_n = (size_t)(N + TN - 1) / TN;
    return ((tiles_n * 4 + 255) / 256) * 256 + tiles_n * (size_t)splits * 16 * TN * 4;
}

int skinny_splits(int M, int N, int K) {
    (void)M;
    const int tiles_n = (N + TN - 1) / TN;
    const int chunks = (K + KC - 1) / KC;
    // aim at about two workgroups per compute unit (256 CUs)
    int s = (512 + tiles_n - 1) / tiles_n;
    if (s > chunks) s = chunks;
    if (s < 1) s = 1;
    // every split must own at least one chunk
    const int per = (chunks + s - 1) / s;
    s = (chunks + per - 1) / per;
    return s;
}

hipError_t launch_a8w8_skinny(const Int8GemmArgs& a, bool vec, int epi, hipStream_t s, const char** name) {
    dim3 grid((a.N + TN - 1) / TN, a.splits > 1 ? a.splits : 1);
    *name = "a8w8_skinny";
    if (vec) {
        if (epi == EPI_F32) hipLaunchKernelGGL((a8w8_skinny_kernel<true, EPI_F32>), grid, dim3(NT), 0, s, a);
        else hipLaunchKernelGGL((a8w8_skinny_kernel<true, EPI_BF16>), grid, dim3(NT), 0, s, a);
    } else {
        if (epi == EPI_F32) hipLaunchKernelGGL((a8w8_skinny_kernel<false, EPI_F32>), grid, dim3(NT), 0, s, a);
        else hipLaunchKernelGGL((a8w8_skinny_kernel<false, EPI_BF16>), grid, dim3(NT), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace qg

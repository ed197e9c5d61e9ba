// W8A32 matmul on gfx950: fp32 activations times an int8 weight with a
// per-tensor scale and zero point, dequantisation folded into the epilogue.
//
// Operator: "feat(PULPOpen): matmul that dequantises an int8 weight
// in-kernel", section "The kernel": sum_k a_k (b_k - zp) scale equals
// scale (sum_k a_k b_k - zp sum_k a_k), so the dequantised weight is never
// formed and the correction costs one multiply per output element; with
// zp == 0 the correction vanishes and the loop is the fp32 loop with an int8
// load.
//
// One workgroup computes a 128 x 128 tile with four waves of 64 x 64, walking
// K in chunks of 32:
//  * A (fp32) and W (int8, [K,N]) tiles are read through buffer resources
//    ending at the matrix edge (rows past M or K read as zero), A as 16-byte
//    vectors, W as 4-byte words; the next chunk is in flight while the
//    current one is multiplied.  W stays int8 in LDS, transposed 4x4 bytes
//    at a time so each k-quad of a column is one word.
//  * Each lane widens its W bytes to fp32 in registers and feeds
//    v_mfma_f32_16x16x4_f32.  When zp != 0, the same A values are summed
//    into the row sum S2 (per lane, then across the four lane groups); with
//    zp == 0 the kernel is compiled without it.  Both waves of a row block
//    take the same sum (12 adds per 64 matrix-core multiplies): splitting it
//    between them by k-group needs 192 VGPRs instead of 160, which leaves
//    two workgroups per CU instead of three.
//  * Epilogue: C = scale * (S1 - zp * S2), or scale * S1 when zp == 0.
//
// The same kernel with WT = true is the gradient with respect to the
// activations (the frozen weight's second consumer: "feat(PULPOpen): matmul
// that dequantises an int8 weight in-kernel", intro; "perf(pulpopen/gap9):
// share L3 storage between byte-identical constants", intro):
//   dA[m,k] = scale * (sum_n dC[m,n] W[k,n] - zp * sum_n dC[m,n]),
// the same factorisation with the contraction over W's contiguous
// dimension.  The kernel then sees W as [outputs][contraction] rows, which
// is already the layout its LDS tile wants: each row segment is copied
// as is, with no byte transpose.
#include "device_common.h"
#include "kernels.h"

namespace qg {
namespace {

constexpr int NT = 256;
constexpr int BM = 128, BN = 128, BKF = 32;
constexpr int WMT = 64, WNT = 64;
constexpr int AROW = BKF + 4;   // floats per LDS row of A (16 B pad)
constexpr int WROW = BKF + 4;   // bytes per LDS row of W^T
constexpr int A_STAGE = BM * AROW * 4;
constexpr int W_STAGE = BN * WROW;
constexpr int GROUP_M = 8;

// WT == false: W is [K,N] (contraction over rows); true: W is [N,K] rows of
// the contraction (p.N outputs, p.K contraction bytes per row).
template <bool VEC, bool WT, bool ZP>
__global__ __launch_bounds__(NT) void w8a32_kernel(W8A32Args p) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * (A_STAGE + W_STAGE)];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int l16 = lane & 15, g = lane >> 4;

    const int tiles_m = (p.M + BM - 1) / BM;
    const int tiles_n = (p.N + BN - 1) / BN;
    int tm, tn;
    tile_coords(xcd_remap(blockIdx.x, gridDim.x), tiles_m, tiles_n, GROUP_M, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int rows = p.M - m0 < BM ? p.M - m0 : BM;
    const int cols = p.N - n0 < BN ? p.N - n0 : BN;
    const int lda = (int)p.lda, ldw = (int)p.ldw;
    const float* A = p.A + (int64_t)m0 * p.lda;
    const int8_t* W = WT ? p.W + (int64_t)n0 * p.ldw : p.W + n0;
    const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(A, (uint32_t)(((rows - 1) * lda + p.K) * 4));
    const __amdgpu_buffer_rsrc_t w_rsrc = WT ? make_rsrc(W, (uint32_t)((cols - 1) * ldw + p.K))
                                             : make_rsrc(W, (uint32_t)((p.K - 1) * ldw + (p.N - n0)));

    // A: thread -> rows ar + 32*i, floats 4*ac .. 4*ac+3 of the chunk
    const int ar = tid >> 3, ac = tid & 7;
    // W: thread -> rows 4*wr .. 4*wr+3 of the chunk, columns 4*wc .. 4*wc+3;
    // with WT, output row tr, contraction bytes 16*th .. 16*th+15.
    const int wr = tid & 7, wc = tid >> 3;
    const int tr = tid >> 1, th = tid & 1;

    u32x4 a_st[4];
    uint32_t w_st[4];
    auto fetch = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = ar + 32 * i;
            if constexpr (VEC) {
                a_st[i] = buffer_load16(a_rsrc, (uint32_t)((r * lda + ac * 4 + k0) * 4), 0u);
            } else {
                uint32_t d[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int k = k0 + ac * 4 + e;
                    d[e] = (r < rows && k < p.K) ? __float_as_uint(A[(int64_t)r * p.lda + k]) : 0u;
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
                        if (tr < cols && k < p.K) d |= (uint32_t)(uint8_t)W[(int64_t)tr * p.ldw + k] << (8 * e);
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
                w_st[i] = __builtin_amdgcn_raw_buffer_load_b32(w_rsrc, (int)((k0 + wr * 4 + i) * ldw + wc * 4), 0, 0);
            } else {
                uint32_t d = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int n = wc * 4 + e;
                    if (k < p.K && n < cols) d |= (uint32_t)(uint8_t)W[(int64_t)k * p.ldw + n] << (8 * e);
                }
                w_st[i] = d;
            }
        }
    };
    auto stash = [&](int buf, int k0) {
        float* As = reinterpret_cast<float*>(smem + buf * (A_STAGE + W_STAGE));
        uint8_t* Ws = smem + buf * (A_STAGE + W_STAGE) + A_STAGE;
        const bool k_full = k0 + BKF <= p.K;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            u32x4 v = a_st[i];
            if (VEC && !k_full) {
                const int k = k0 + ac * 4;
                if (k + 0 >= p.K) v.x = 0u;
                if (k + 1 >= p.K) v.y = 0u;
                if (k + 2 >= p.K) v.z = 0u;
                if (k + 3 >= p.K) v.w = 0u;
            }
            *reinterpret_cast<u32x4*>(As + (ar + 32 * i) * AROW + ac * 4) = v;
        }
        if constexpr (WT) {
#pragma unroll
            for (int i = 0; i < 4; ++i) *reinterpret_cast<uint32_t*>(Ws + tr * WROW + 16 * th + 4 * i) = w_st[i];
        } else {
            uint32_t y[4];
            transpose4x4_bytes(w_st, y);
#pragma unroll
            for (int c = 0; c < 4; ++c) *reinterpret_cast<uint32_t*>(Ws + (wc * 4 + c) * WROW + wr * 4) = y[c];
        }
    };

    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    float rsum[4] = {0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int buf) {
        const float* As = reinterpret_cast<const float*>(smem + buf * (A_STAGE + W_STAGE)) + wm * WMT * AROW;
        const uint8_t* Ws = smem + buf * (A_STAGE + W_STAGE) + A_STAGE + wn * WNT * WROW;
#pragma unroll
        for (int kg = 0; kg < BKF / 16; ++kg) {
            // lane group g holds k = kg*16 + 4g + t for MFMA t = 0..3
            v4f af[4];
            float wf[4][4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                af[i] = *reinterpret_cast<const v4f*>(As + (i * 16 + l16) * AROW + kg * 16 + 4 * g);
                if constexpr (ZP) rsum[i] += (af[i].x + af[i].y) + (af[i].z + af[i].w);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t w = *reinterpret_cast<const uint32_t*>(Ws + (j * 16 + l16) * WROW + kg * 16 + 4 * g);
#pragma unroll
                for (int t = 0; t < 4; ++t) wf[j][t] = (float)(int8_t)(w >> (8 * t));
            }
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[i][j] = mfma_f32_16x16x4(af[i][t], wf[j][t], acc[i][j]);
        }
    };

    const int nk = (p.K + BKF - 1) / BKF;
    fetch(0);
    stash(0, 0);
    __syncthreads();
    for (int kt = 0; kt + 1 < nk; ++kt) {
        fetch((kt + 1) * BKF);
        compute(kt & 1);
        stash((kt + 1) & 1, (kt + 1) * BKF);
        __syncthreads();
    }
    compute((nk - 1) & 1);

    // Row sums over the whole K: add the four lane groups.
    if constexpr (ZP) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            rsum[i] += __shfl_xor(rsum[i], 16);
            rsum[i] += __shfl_xor(rsum[i], 32);
        }
    }
    const float zp = (float)p.zp;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = m0 + wm * WMT + i * 16 + 4 * g + r;
            const float s2 = __shfl(rsum[i], 4 * g + r);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = n0 + wn * WNT + j * 16 + l16;
                if (m < p.M && n < p.N) {
                    float v = acc[i][j][r];
                    if constexpr (ZP) v = v - zp * s2;
                    p.C[(int64_t)m * p.ldc + n] = p.scale * v;
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_w8a32(const W8A32Args& a, bool vec_a, bool vec_w, bool wt, hipStream_t s, const char** name) {
    const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    const bool vec = vec_a && vec_w;
    const bool zp = a.zp != 0;
    *name = wt ? "w8a32_input_grad_128x128" : "w8a32_tiled_128x128";
    const dim3 grid(tiles), block(NT);
    const int v = (vec ? 4 : 0) | (wt ? 2 : 0) | (zp ? 1 : 0);
    switch (v) {
        case 7: hipLaunchKernelGGL((w8a32_kernel<true, true, true>), grid, block, 0, s, a); break;
        case 6: hipLaunchKernelGGL((w8a32_kernel<true, true, false>), grid, block, 0, s, a); break;
        case 5: hipLaunchKernelGGL((w8a32_kernel<true, false, true>), grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL((w8a32_kernel<true, false, false>), grid, block, 0, s, a); break;
        case 3: hipLaunchKernelGGL((w8a32_kernel<false, true, true>), grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL((w8a32_kernel<false, true, false>), grid, block, 0, s, a); break;
        case 1: hipLaunchKernelGGL((w8a32_kernel<false, false, true>), grid, block, 0, s, a); break;
        default: hipLaunchKernelGGL((w8a32_kernel<false, false, false>), grid, block, 0, s, a); break;
    }
    return hipGetLastError();
}

}  // namespace qg

// Column-slab A8W8 kernel for few rows with the weight given as [N,K] on
// gfx950: each workgroup owns TN output columns over ALL of K, so nothing
// crosses workgroups -- no split partials, no tickets, no workspace.
//
// Operator: "Feature/a8w8 matmul dequant fusion" -- int8 matmul into an INT32
// accumulator (optionally one given as input, the page's matmul-dequant-acc
// op), cast to FP32, times act_scale[m], times weight_scale[n], cast to the
// output type; the op takes the weight transposed (b_trans), and logical
// M == 1 goes to a GEMV of its own on that page.
//
// A decode-shaped product reads the int8 weight once and little else, so it
// is bound by streaming the weight from HBM.  With W as [N,K], output column
// n's k-bytes are one contiguous row, so a workgroup that owns TN columns
// streams TN whole rows: every 128-byte line it fetches is used entirely by
// itself.  The chip is occupied by cutting N (N / TN workgroups: 256 at
// N = 8192, TN = 32), not K, so the split-K exchange of the [K,N] decode
// kernel (device-coherent partial stores, a ticket, the last split's reload)
// is not needed.
//  * Eight waves take steps of SK k-bytes round robin, NB steps in flight
//    per wave (128 KiB per CU).  Lane (i16, g) loads 16 bytes of weight row
//    n0 + 16c + i16 at k-bytes 64kb + 16g of the step: exactly the matrix
//    core's B fragment of column 16c + i16 for k-block kb, with the A
//    fragment (row i16 of A, same k-bytes) from one more 16-byte load.  The
//    two k-blocks of a 128-byte line are loaded back to back (cached, so the
//    second load of a line meets the first one's fill).
//  * v_mfma_i32_16x16x64_i8 accumulates per wave; the eight waves' tiles are
//    added through LDS at the end and the epilogue runs once per output.
// Weight rows past N read as zero through the buffer range check.  Bytes of
// a row past K are the next row's, so a 16-byte piece there (K % 16 == 0)
// has its A fragment cleared and multiplies nothing.
#include "device_common.h"
#include "kernels.h"

namespace qg {
namespace {

constexpr int SL_WAVES = 8;
constexpr int SL_NT = 64 * SL_WAVES;

// TN output columns per workgroup; SK k-bytes per wave step, NB steps in
// flight per wave; CONTIG: each wave takes one contiguous range of steps
// instead of every eighth step.  At most 16 rows (one fragment of A).
template <int TN, int EPI, int SK, int NB, bool CONTIG>
__global__ __launch_bounds__(SL_NT) __attribute__((amdgpu_waves_per_eu(2))) void a8w8_slab_kernel(Int8GemmArgs p) {
    constexpr int NF = TN / 16;   // 16-column fragments of the slab
    constexpr int KB = SK / 64;   // 64-byte k-blocks per step

    __shared__ __attribute__((aligned(16))) int32_t red[SL_WAVES][16][TN];
    __shared__ float ws_tile[TN];
    __shared__ float as_rows[16];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, i16 = lane & 15;
    const int n0 = blockIdx.x * TN;
    const int cols = p.N - n0;
    const int ldb = (int)p.ldb, lda = (int)p.lda;
    // the slab's own rows only (a whole [N,K] weight may span 2^31 bytes)
    const int rows_w = cols < TN ? cols : TN;
    const __amdgpu_buffer_rsrc_t w_rsrc = make_rsrc(p.B + (int64_t)n0 * ldb, (uint32_t)((rows_w - 1) * ldb + p.K));
    const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(p.A, (uint32_t)((p.M - 1) * lda + p.K));
    const uint32_t w_voff = (uint32_t)(i16 * ldb + 16 * g);
    const uint32_t a_voff = (uint32_t)(i16 * lda + 16 * g);

    // Epilogue scales, loaded now so that their latency hides behind the
    // weight stream.
    if (tid < TN) ws_tile[tid] = (n0 + tid < p.N) ? p.weight_scale[(n0 + tid) * p.ws_stride] : 0.f;
    if (tid < 16) as_rows[tid] = (tid < p.M) ? p.act_scale[tid * p.as_stride] : 0.f;

    const int nsteps = (p.K + SK - 1) / SK;
    u32x4 wbuf[NB][KB][NF];
    u32x4 abuf[NB][KB];
    // Loads of one step into buffer b.  A step past K (the last round of a
    // wave) loads from past the buffer ends, which reads zeros and touches no
    // memory; bytes past K within a live step are cleared in consume.
    auto fetch = [&](int step, int b) {
        const uint32_t k0 = (uint32_t)step * SK;
        const uint32_t wo = step < nsteps ? w_voff + k0 : 0x80000000u;
        const uint32_t ao = step < nsteps ? a_voff + k0 : 0x80000000u;
#pragma unroll
        for (int c = 0; c < NF; ++c)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
                wbuf[b][kb][c] = buffer_load16(w_rsrc, wo + (uint32_t)(16 * c * ldb + 64 * kb), 0u);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) abuf[b][kb] = buffer_load16(a_rsrc, ao + (uint32_t)(64 * kb), 0u);
    };

    v4i acc[NF];
#pragma unroll
    for (int c = 0; c < NF; ++c) acc[c] = v4i{0, 0, 0, 0};

    auto consume = [&](int b, int step) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            // a 16-byte piece past K belongs to the next row of both operands
            const bool live = step * SK + 64 * kb + 16 * g < p.K;
            const u32x4 a = live ? abuf[b][kb] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int c = 0; c < NF; ++c) acc[c] = mfma_i8_16x16x64(a, wbuf[b][kb][c], acc[c]);
        }
    };

    // This wave's steps: step_of(i), i < n_my, with n_my a multiple of NB and
    // the same for every wave (steps past K add nothing), NB in flight, the
    // loop unrolled by NB so that the register buffers have fixed homes.
    const int n_my = (((nsteps + SL_WAVES - 1) / SL_WAVES) + NB - 1) / NB * NB;
    auto step_of = [&](int i) { return CONTIG ? wave * n_my + i : wave + SL_WAVES * i; };
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        fetch(step_of(b), b);
        __builtin_amdgcn_sched_barrier(0);
    }
    int i = 0;
    for (; i + NB < n_my; i += NB) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            consume(b, step_of(i + b));
            __builtin_amdgcn_sched_barrier(0);
            fetch(step_of(i + NB + b), b);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) consume(b, step_of(i + b));

    // The waves' tiles through LDS: register r of fragment c holds row
    // 4g + r, column 16c + i16.
    const int M = p.M;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int m = 4 * g + r;
        if (m >= M) continue;
#pragma unroll
        for (int c = 0; c < NF; ++c) red[wave][m][16 * c + i16] = acc[c][r];
    }
    __syncthreads();

    // Output row m, columns n .. n+3 (those < N): the waves' sum, the
    // accumulator input, the scales, then one vector store when the four are
    // in range and aligned.
    const bool vec_out = (p.ldo % 4 == 0) && ((reinterpret_cast<uintptr_t>(p.out) & 15) == 0);
    const bool acc_vec = p.acc_in != nullptr && p.ld_acc % 4 == 0 &&
                         (reinterpret_cast<uintptr_t>(p.acc_in) & 15) == 0;
    const int items = M * (TN / 4);
    for (int it = tid; it < items; it += SL_NT) {
        const int m = it / (TN / 4), cg = it % (TN / 4);
        const int n = n0 + 4 * cg;
        if (n >= p.N) continue;
        int32_t vi[4] = {0, 0, 0, 0};
#pragma unroll
        for (int w = 0; w < SL_WAVES; ++w) {
            const int4 t = *reinterpret_cast<const int4*>(&red[w][m][4 * cg]);
            vi[0] = (int32_t)((uint32_t)vi[0] + (uint32_t)t.x);
            vi[1] = (int32_t)((uint32_t)vi[1] + (uint32_t)t.y);
            vi[2] = (int32_t)((uint32_t)vi[2] + (uint32_t)t.z);
            vi[3] = (int32_t)((uint32_t)vi[3] + (uint32_t)t.w);
        }
        if (p.acc_in != nullptr) {   // accumulator input, added before the cast (wrapping)
            const int32_t* src = p.acc_in + (int64_t)m * p.ld_acc + n;
            int32_t ai[4] = {0, 0, 0, 0};
            if (acc_vec && n + 4 <= p.N) {
                const int4 t = *reinterpret_cast<const int4*>(src);
                ai[0] = t.x; ai[1] = t.y; ai[2] = t.z; ai[3] = t.w;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (n + e < p.N) ai[e] = src[e];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) vi[e] = (int32_t)((uint32_t)vi[e] + (uint32_t)ai[e]);
        }
        float f[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            f[e] = (float)vi[e];
            f[e] = f[e] * as_rows[m];
            f[e] = f[e] * ws_tile[4 * cg + e];
        }
        const int64_t o = (int64_t)m * p.ldo + n;
        if (vec_out && n + 4 <= p.N) {
            if constexpr (EPI == EPI_F32) {
                *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + o) = make_float4(f[0], f[1], f[2], f[3]);
            } else {
                *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + o) =
                    make_uint2(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]));
            }
            continue;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (n + e >= p.N) break;
            if constexpr (EPI == EPI_F32) reinterpret_cast<float*>(p.out)[o + e] = f[e];
            else reinterpret_cast<uint16_t*>(p.out)[o + e] = f32_to_bf16_rne(f[e]);
        }
    }
}

template <int TN, int SK, int NB, bool CONTIG>
hipError_t launch_cfg(const Int8GemmArgs& a, int epi, hipStream_t s) {
    const dim3 grid((a.N + TN - 1) / TN), block(SL_NT);
    if (epi == EPI_F32) hipLaunchKernelGGL((a8w8_slab_kernel<TN, EPI_F32, SK, NB, CONTIG>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((a8w8_slab_kernel<TN, EPI_BF16, SK, NB, CONTIG>), grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace

bool slab_shape_ok(const Int8GemmArgs& a, int tn) {
    const uintptr_t al = reinterpret_cast<uintptr_t>(a.A) | reinterpret_cast<uintptr_t>(a.B);
    if ((al & 15) != 0 || a.lda % 16 != 0 || a.ldb % 16 != 0 || a.K % 16 != 0) return false;
    if (a.batch != 1 || a.M < 1 || a.M > SLAB_MAX_M || a.K < 1 || a.N < 1) return false;
    if (tn != 16 && tn != 32) return false;
    // 32-bit buffer offsets: a live step reads below K + 256 in a row
    return (int64_t)(tn + 16) * a.ldb + a.K + 256 < ((int64_t)1 << 31) &&
           (int64_t)16 * a.lda + a.K + 256 < ((int64_t)1 << 31);
}

// Steps: a 16-column slab takes 128-byte steps four deep, each wave one
// contiguous range of them (13.4 -> 13.1 us at M = 1), a 32-column slab
// 256-byte steps two deep, every eighth per wave (8 KiB per wave either way;
// measured fastest of the 16/32-column, 128/256/512-byte, two/three/four-deep
// forms at N = K = 8192: M = 1 13.9 us, M = 16 16.7 us).
hipError_t launch_a8w8_slab(const Int8GemmArgs& a, int tn, int epi, hipStream_t s, const char** name) {
    *name = "a8w8_slab";
    if (!slab_shape_ok(a, tn) || (epi != EPI_F32 && epi != EPI_BF16)) return hipErrorInvalidValue;
    if (tn == 16) return launch_cfg<16, 128, 4, true>(a, epi, s);
    return launch_cfg<32, 256, 2, false>(a, epi, s);
}

}  // namespace qg

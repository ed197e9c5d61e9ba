// Calibration kernels for the roofline figures: a streaming read and
// matrix-core loops.  They implement no part of the quantised matmuls; they
// measure, on the machine at hand, the ceilings those kernels are held to
// (HBM read bandwidth for the decode kernel, int8, fp32 and bf16 matrix-core
// rates under data-dependent clocks for the tiled kernels).
#include "device_common.h"
#include "kernels.h"

namespace qg {
namespace {

constexpr int CAL_NT = 256;

// Each workgroup reads one contiguous chunk of the buffer, 16-byte vectors
// with the non-temporal cache policy, eight in flight per thread, and xors
// them; one word per wave goes to `sink` so the reads are kept.  Of the read
// shapes tried (grid-stride or chunked, 4/8/16 loads in flight, cached or
// non-temporal, 256..4096 workgroups), this one streamed fastest: about
// 7.0 TB/s over 1 GiB against 5.3 TB/s for a cached grid-stride read.
__global__ __launch_bounds__(CAL_NT) void calib_read_kernel(const v4i* __restrict__ p, size_t n_vec, uint32_t* sink) {
    const size_t per = (n_vec + gridDim.x - 1) / gridDim.x;
    const size_t b0 = (size_t)blockIdx.x * per;
    const size_t e = b0 + per < n_vec ? b0 + per : n_vec;
    size_t i = b0 + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 7 * CAL_NT < e; i += 8 * CAL_NT) {
        v4i v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(&p[i + u * CAL_NT]);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc ^= (uint32_t)(v[u].x ^ v[u].y ^ v[u].z ^ v[u].w);
    }
    for (; i < e; i += CAL_NT) {
        const v4i v = p[i];
        acc ^= (uint32_t)(v.x ^ v.y ^ v.z ^ v.w);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o);
    if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (CAL_NT / 64) + (threadIdx.x >> 6)] = acc;
}

// Each wave runs `iters` rounds of 16 independent v_mfma_i32_16x16x64_i8 on
// operands taken from `ops` (256 16-byte vectors); no memory traffic in the
// loop.  The operand bytes decide how much the data paths toggle, and with
// that the clock the chip can hold.
__global__ __launch_bounds__(CAL_NT) void calib_mfma_kernel(const u32x4* __restrict__ ops, int iters, uint32_t* sink) {
    const int l = threadIdx.x & 63;
    u32x4 a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[i] = ops[(l + 64 * i) & 255];
        b[i] = ops[(l + 64 * i + 7) & 255];
    }
    v4i acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = v4i{0, 0, 0, 0};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = mfma_i8_16x16x64(a[i & 3], b[i >> 2], acc[i]);
    }
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) s ^= (uint32_t)(acc[i].x ^ acc[i].y ^ acc[i].z ^ acc[i].w);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s ^= (uint32_t)__shfl_xor((int)s, o);
    if (l == 0) sink[blockIdx.x * (CAL_NT / 64) + (threadIdx.x >> 6)] = s;
}

// The same int8 work with v_mfma_i32_32x32x32_i8: eight independent 32x32
// accumulators per wave (16 registers each), each multiply twice the
// operations of a 16x16x64 one for the same operand bytes, so a round does
// the same 16 * 32768 operations per wave with half the operand reads.
typedef int v16i __attribute__((ext_vector_type(16)));
__global__ __launch_bounds__(CAL_NT) void calib_mfma32_kernel(const u32x4* __restrict__ ops, int iters, uint32_t* sink) {
    const int l = threadIdx.x & 63;
    v4i a[4], b[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const u32x4 t = ops[(l + 64 * i) & 255];
        a[i] = v4i{(int)t.x, (int)t.y, (int)t.z, (int)t.w};
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const u32x4 t = ops[(l + 64 * i + 7) & 255];
        b[i] = v4i{(int)t.x, (int)t.y, (int)t.z, (int)t.w};
    }
    v16i acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[i][j] = 0;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i & 3], b[i >> 2], acc[i], 0, 0, 0);
    }
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) s ^= (uint32_t)acc[i][j];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s ^= (uint32_t)__shfl_xor((int)s, o);
    if (l == 0) sink[blockIdx.x * (CAL_NT / 64) + (threadIdx.x >> 6)] = s;
}

// The same loop with v_mfma_f32_16x16x4_f32, the W8A32 kernels' instruction,
// on fp32 operands from `ops` (1024 floats).  With operands in [-1, 1] an
// accumulator grows by at most 4 per round, so it stays finite.
__global__ __launch_bounds__(CAL_NT) void calib_mfma_f32_kernel(const float* __restrict__ ops, int iters,
                                                                uint32_t* sink) {
    const int l = threadIdx.x & 63;
    float a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[i] = ops[(l + 64 * i) & 1023];
        b[i] = ops[(l + 64 * i + 7) & 1023];
    }
    v4f acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = mfma_f32_16x16x4(a[i & 3], b[i >> 2], acc[i]);
    }
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        s ^= __float_as_uint(acc[i].x) ^ __float_as_uint(acc[i].y) ^ __float_as_uint(acc[i].z) ^
             __float_as_uint(acc[i].w);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s ^= (uint32_t)__shfl_xor((int)s, o);
    if (l == 0) sink[blockIdx.x * (CAL_NT / 64) + (threadIdx.x >> 6)] = s;
}

// The same loop with v_mfma_f32_16x16x32_bf16, the instruction of the
// W8A32 kernels' exact bf16 split, on bf16 operands from `ops` (2048
// values).  With operands in [-1, 1] an accumulator grows by at most 32 per
// round, so it stays finite.
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
__global__ __launch_bounds__(CAL_NT) void calib_mfma_bf16_kernel(const u32x4* __restrict__ ops, int iters,
                                                                 uint32_t* sink) {
    const int l = threadIdx.x & 63;
    v8bf a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[i] = __builtin_bit_cast(v8bf, ops[(l + 64 * i) & 255]);
        b[i] = __builtin_bit_cast(v8bf, ops[(l + 64 * i + 7) & 255]);
    }
    v4f acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i & 3], b[i >> 2], acc[i], 0, 0, 0);
    }
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        s ^= __float_as_uint(acc[i].x) ^ __float_as_uint(acc[i].y) ^ __float_as_uint(acc[i].z) ^
             __float_as_uint(acc[i].w);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s ^= (uint32_t)__shfl_xor((int)s, o);
    if (l == 0) sink[blockIdx.x * (CAL_NT / 64) + (threadIdx.x >> 6)] = s;
}

}  // namespace

hipError_t launch_calib_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t s) {
    hipLaunchKernelGGL(calib_read_kernel, dim3(CALIB_READ_BLOCKS), dim3(CAL_NT), 0, s,
                       reinterpret_cast<const v4i*>(buf), bytes / 16, sink);
    return hipGetLastError();
}

hipError_t launch_calib_mfma(const void* ops, int iters, uint32_t* sink, hipStream_t s) {
    hipLaunchKernelGGL(calib_mfma_kernel, dim3(CALIB_MFMA_BLOCKS), dim3(CAL_NT), 0, s,
                       reinterpret_cast<const u32x4*>(ops), iters, sink);
    return hipGetLastError();
}

hipError_t launch_calib_mfma32(const void* ops, int iters, uint32_t* sink, hipStream_t s) {
    hipLaunchKernelGGL(calib_mfma32_kernel, dim3(CALIB_MFMA_BLOCKS), dim3(CAL_NT), 0, s,
                       reinterpret_cast<const u32x4*>(ops), iters, sink);
    return hipGetLastError();
}

hipError_t launch_calib_mfma_f32(const void* ops, int iters, uint32_t* sink, hipStream_t s) {
    hipLaunchKernelGGL(calib_mfma_f32_kernel, dim3(CALIB_MFMA_BLOCKS), dim3(CAL_NT), 0, s,
                       reinterpret_cast<const float*>(ops), iters, sink);
    return hipGetLastError();
}

hipError_t launch_calib_mfma_bf16(const void* ops, int iters, uint32_t* sink, hipStream_t s) {
    hipLaunchKernelGGL(calib_mfma_bf16_kernel, dim3(CALIB_MFMA_BLOCKS), dim3(CAL_NT), 0, s,
                       reinterpret_cast<const u32x4*>(ops), iters, sink);
    return hipGetLastError();
}

}  // namespace qg

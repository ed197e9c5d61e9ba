// DynamicQuantizeLinear to uint8 on gfx950.
//
// Operator: "feat(onnx-to-hip): lower quantized integer conv and matmul",
// section "What", DynamicQuantizeLinear paragraph: reduce the fp32 input to
// its minimum and maximum, scale = (max - min) / 255 with a zero range
// selecting scale 1, a zero point rounded with ties to even, then quantize
// every element.  Readings of the points the page leaves open: the range is
// widened to include 0 (the ONNX operator's definition, so a real 0 maps
// exactly to the zero point); every step is fp32 with correctly rounded
// division; a scale that underflows to 0 also takes the value 1; quantizing
// rounds x / scale to the nearest integer, ties to even, adds the zero point
// and saturates to [0, 255].
//
// Two launches, both bound by HBM:
//  1. dql_minmax: each workgroup reduces a contiguous share of x to one
//     (min, max) pair, 16-byte loads eight deep, and writes it to the
//     workspace slot of its own index.  No atomics, so the workspace needs no
//     clearing and no state survives the call.
//  2. dql_quantize: each workgroup first folds all the pairs (min and max are
//     exact, so every workgroup reaches the same two values), derives scale
//     and zero point, then quantizes its contiguous share 16 elements per
//     lane per step: four 16-byte loads, one 16-byte store.  Workgroup 0 also writes scale and
//     zero point.
// x is read twice (the second read is served by the 256 MB Infinity Cache
// when x fits in it); y is written once.
#include "device_common.h"
#include "kernels.h"

namespace qg {
namespace {

constexpr int NT = 256;            // quantize pass
constexpr int NT_MM = 512;         // min/max pass
constexpr int MM_UNROLL = 16;      // 16-byte loads in flight per lane in the min/max pass
constexpr int MAX_WAVES = NT_MM / 64;

// Range includes 0: start both ends at +0 and move only on a strict
// comparison, so -0 never replaces +0 and NaN never enters.
__device__ __forceinline__ void take(float v, float& mn, float& mx) {
    mn = v < mn ? v : mn;
    mx = v > mx ? v : mx;
}

// Min and max over the workgroup; every thread receives both.
template <int WAVES>
__device__ __forceinline__ void block_minmax(float& mn, float& mx, float* red) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        take(__shfl_xor(mn, off), mn, mx);
        take(__shfl_xor(mx, off), mn, mx);
    }
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        red[2 * wave] = mn;
        red[2 * wave + 1] = mx;
    }
    __syncthreads();
    mn = red[0];
    mx = red[1];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) {
        take(red[2 * w], mn, mx);
        take(red[2 * w + 1], mn, mx);
    }
}

// Contiguous share [lo, hi) of `total` items for workgroup `b` of `nb`.
__device__ __forceinline__ void chunk_of(int64_t total, int b, int nb, int64_t& lo, int64_t& hi) {
    const int64_t per = (total + nb - 1) / nb;
    lo = (int64_t)b * per;
    hi = lo + per < total ? lo + per : total;
}

template <bool VEC>
__global__ __launch_bounds__(NT_MM) void dql_minmax(const float* __restrict__ x, int64_t n,
                                                    float2* __restrict__ part) {
    __shared__ float red[2 * MAX_WAVES];
    float mn = 0.0f, mx = 0.0f;
    if constexpr (VEC) {
        // This workgroup's contiguous share of the whole float4 vectors,
        // MM_UNROLL per lane in flight (cached: the quantize pass reads x
        // again), then the last n % 4 values in workgroup 0.
        const v4f* xv = reinterpret_cast<const v4f*>(x);
        int64_t lo, hi;
        chunk_of(n >> 2, blockIdx.x, gridDim.x, lo, hi);
        int64_t i = lo + threadIdx.x;
        for (; i + (MM_UNROLL - 1) * NT_MM < hi; i += MM_UNROLL * NT_MM) {
            v4f v[MM_UNROLL];
#pragma unroll
            for (int u = 0; u < MM_UNROLL; ++u) v[u] = xv[i + u * NT_MM];
#pragma unroll
            for (int u = 0; u < MM_UNROLL; ++u) {
                take(v[u].x, mn, mx); take(v[u].y, mn, mx);
                take(v[u].z, mn, mx); take(v[u].w, mn, mx);
            }
        }
        for (; i < hi; i += NT_MM) {
            const v4f v = xv[i];
            take(v.x, mn, mx); take(v.y, mn, mx); take(v.z, mn, mx); take(v.w, mn, mx);
        }
        if (blockIdx.x == 0 && threadIdx.x < (n & 3)) take(x[((n >> 2) << 2) + threadIdx.x], mn, mx);
    } else {
        const int64_t stride = (int64_t)gridDim.x * NT_MM;
        for (int64_t i = (int64_t)blockIdx.x * NT_MM + threadIdx.x; i < n; i += stride) take(x[i], mn, mx);
    }
    block_minmax<NT_MM / 64>(mn, mx, red);
    if (threadIdx.x == 0) part[blockIdx.x] = make_float2(mn, mx);
}

__device__ __forceinline__ uint32_t quant1(float v, float scale, int zp) {
    int q = (int)rintf(v / scale) + zp;   // correctly rounded division; rint: ties to even
    q = q < 0 ? 0 : (q > 255 ? 255 : q);
    return (uint32_t)q;
}

template <bool VEC>
__global__ __launch_bounds__(NT) void dql_quantize(const float* __restrict__ x, int64_t n,
                                                   const float2* __restrict__ part, int parts,
                                                   uint8_t* __restrict__ y, float* __restrict__ y_scale,
                                                   uint8_t* __restrict__ y_zp) {
    __shared__ float red[2 * MAX_WAVES];
    // This workgroup's contiguous share of the 16-element chunks (VEC), or a
    // grid stride of single elements.  The first chunk's loads go out before
    // the partials are read, so the two latencies overlap.
    const v4f* xv = reinterpret_cast<const v4f*>(x);
    int64_t lo = 0, hi = 0;
    if constexpr (VEC) chunk_of(n >> 4, blockIdx.x, gridDim.x, lo, hi);
    int64_t c = lo + threadIdx.x;
    v4f v[4];
    if constexpr (VEC) {
        if (c < hi) {
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(&xv[4 * c + u]);
        }
    }
    float mn = 0.0f, mx = 0.0f;
    for (int i = threadIdx.x; i < parts; i += NT) {
        const float2 p = part[i];
        take(p.x, mn, mx);
        take(p.y, mn, mx);
    }
    block_minmax<NT / 64>(mn, mx, red);
    // The page's scalar steps, each a single fp32 operation rounded to nearest.
    const float range = mx - mn;
    float scale = range / 255.0f;
    if (scale == 0.0f) scale = 1.0f;
    const float q0 = mn / scale;
    int zp = (int)rintf(0.0f - q0);
    zp = zp < 0 ? 0 : (zp > 255 ? 255 : zp);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        *y_scale = scale;
        *y_zp = (uint8_t)zp;
    }

    if constexpr (VEC) {
        // Four non-temporal float4 loads and one 16-byte store per chunk; the
        // last n % 16 values in workgroup 0.
        v4i* yv = reinterpret_cast<v4i*>(y);
        while (c < hi) {
            uint32_t w[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                w[u] = quant1(v[u].x, scale, zp) | (quant1(v[u].y, scale, zp) << 8) |
                       (quant1(v[u].z, scale, zp) << 16) | (quant1(v[u].w, scale, zp) << 24);
            __builtin_nontemporal_store(v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]}, &yv[c]);
            c += NT;
            if (c < hi) {
#pragma unroll
                for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(&xv[4 * c + u]);
            }
        }
        const int64_t tail = (n >> 4) << 4;
        if (blockIdx.x == 0 && threadIdx.x < n - tail) y[tail + threadIdx.x] = (uint8_t)quant1(x[tail + threadIdx.x], scale, zp);
    } else {
        const int64_t stride = (int64_t)gridDim.x * NT;
        for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n; i += stride)
            y[i] = (uint8_t)quant1(x[i], scale, zp);
    }
}

}  // namespace

int dql_partials(int64_t n) {
    // One min/max workgroup per 128 KiB of x (a single round of MM_UNROLL
    // loads per lane), at most DQL_MAX_PARTIALS (one per compute unit).
    const int64_t per_block = (int64_t)NT_MM * MM_UNROLL * 4;
    const int64_t want = (n + per_block - 1) / per_block;
    return (int)(want < 1 ? 1 : (want > DQL_MAX_PARTIALS ? DQL_MAX_PARTIALS : want));
}

hipError_t launch_dynamic_quantize(const float* x, int64_t n, uint8_t* y, float* y_scale, uint8_t* y_zp,
                                   void* workspace, bool vec, hipStream_t s) {
    const int parts = dql_partials(n);
    float2* part = reinterpret_cast<float2*>(workspace);
    // Quantize grid: 16-element chunks, at most 1024 workgroups (four per
    // compute unit; [8, 512, 2048] fp32: 18.7 us with 2048, 17.4 with 1024,
    // 19.4 with 768, 19.9 with 1536), so that each lane quantizes a couple of
    // chunks and the partials are folded by fewer workgroups.
    int64_t qblocks = (n + 16 * NT - 1) / (16 * NT);
    if (qblocks < 1) qblocks = 1;
    if (qblocks > 1024) qblocks = 1024;
    if (vec) {
        hipLaunchKernelGGL(dql_minmax<true>, dim3(parts), dim3(NT_MM), 0, s, x, n, part);
        hipLaunchKernelGGL(dql_quantize<true>, dim3((unsigned)qblocks), dim3(NT), 0, s, x, n, part, parts, y,
                           y_scale, y_zp);
    } else {
        hipLaunchKernelGGL(dql_minmax<false>, dim3(parts), dim3(NT_MM), 0, s, x, n, part);
        hipLaunchKernelGGL(dql_quantize<false>, dim3((unsigned)qblocks), dim3(NT), 0, s, x, n, part, parts, y,
                           y_scale, y_zp);
    }
    return hipGetLastError();
}

}  // namespace qg

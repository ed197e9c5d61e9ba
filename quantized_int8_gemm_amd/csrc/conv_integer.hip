// ConvInteger on gfx950: the operand-staging kernels.  The contraction itself
// runs on the int8 matrix-core GEMM of the MatMulInteger operator.
//
// Operator: "feat(onnx-to-hip): lower quantized integer conv and matmul",
// section "What", ConvInteger paragraph: an integer convolution of x [N, C,
// H, W] (or NCL) with w [M, C/group, kH, kW], the activation minus its scalar
// zero point, the weight minus its scalar or per-output-channel zero point,
// summed exactly into a wrapping int32 [N, M, OH, OW].  A tap outside the
// input contributes nothing (the input is padded with its own zero point).
//
// For image n and group g the convolution is the matrix product
//   y[n, g*Mg + m, p] = sum_k (Wg[m, k] - w_zp[m]) * (col[n, g][k, p] - x_zp)
// with k = (c, kh, kw) over the group's Cg = C/group channels and
// p = (oh, ow).  So:
//  * conv_pack_weight copies w into [group][Mg][Kp] rows, K padded to a
//    multiple of 64 with each row's own zero point;
//  * conv_im2col_lds writes col[n][g][Kp][Pp] (P = OH*OW padded to 16): one
//    workgroup stages an input plane in LDS and writes the kH*kW column rows
//    it feeds, each lane gathering 16 consecutive output positions from LDS
//    and storing them as one 16-byte vector (conv_im2col gathers straight
//    from memory for planes larger than 64 KiB); taps outside the input,
//    k >= Kg and p >= P hold the activation zero point.
// Padded entries equal their operand's zero point, so they add exactly 0 to
// every sum; the GEMM then runs with A = packed w (per-row zero points) and
// B = col (scalar zero point), batch = images, and writes y in NCHW order.
#include "device_common.h"
#include "kernels.h"

namespace qg {
namespace {

constexpr int NT = 256;

__global__ __launch_bounds__(NT) void conv_pack_weight(ConvGeom c, const uint8_t* __restrict__ w,
                                                       const uint8_t* __restrict__ w_zp, int w_zp_len,
                                                       uint8_t* __restrict__ wp) {
    const int64_t total = (int64_t)c.group * c.Mg * c.Kp;
    const int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x;
    if (i >= total) return;
    const int64_t k = i % c.Kp;
    const int64_t mm = i / c.Kp;   // output channel g*Mg + m
    uint8_t v;
    if (k < c.Kg) {
        v = w[mm * c.Kg + k];
    } else {
        v = w_zp == nullptr ? (uint8_t)0 : w_zp[w_zp_len == 1 ? 0 : mm];
    }
    wp[i] = v;
}

__global__ __launch_bounds__(NT) void conv_im2col(ConvGeom c, const uint8_t* __restrict__ x,
                                                  uint8_t x_zp, uint8_t* __restrict__ col) {
    const int64_t chunks_p = c.Pp / 16;
    const int64_t total = (int64_t)c.N * c.group * c.Kp * chunks_p;
    const int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x;
    if (i >= total) return;
    const int64_t pc = i % chunks_p;
    int64_t r = i / chunks_p;
    const int k = (int)(r % c.Kp);
    r /= c.Kp;
    const int g = (int)(r % c.group);
    const int64_t n = r / c.group;

    uint32_t d[4] = {0u, 0u, 0u, 0u};
    const uint32_t zfill = x_zp;
    if (k >= c.Kg) {
        const uint32_t z4 = zfill * 0x01010101u;
        d[0] = d[1] = d[2] = d[3] = z4;
    } else {
        const int ci = k / (c.kH * c.kW);
        const int kh = (k / c.kW) % c.kH;
        const int kw = k % c.kW;
        const uint8_t* plane = x + ((n * c.C + (int64_t)g * c.Cg + ci) * c.H) * c.W;
        int p = (int)(pc * 16);
        int oh = p / c.OW, ow = p % c.OW;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            uint32_t v = zfill;
            if (p + e < c.P) {
                const int ih = oh * c.sh - c.pt + kh * c.dh;
                const int iw = ow * c.sw - c.pl + kw * c.dw;
                if (ih >= 0 && ih < c.H && iw >= 0 && iw < c.W) v = plane[(int64_t)ih * c.W + iw];
            }
            d[e >> 2] |= v << (8 * (e & 3));
            if (++ow == c.OW) { ow = 0; ++oh; }
        }
    }
    uint8_t* dst = col + ((n * c.group + g) * c.Kp + k) * c.Pp + pc * 16;
    *reinterpret_cast<v4i*>(dst) = v4i{(int)d[0], (int)d[1], (int)d[2], (int)d[3]};
}

// LDS bytes conv_im2col_lds may use for its staged planes (guards included).
constexpr int PLANE_LDS_MAX = 65536;
constexpr int PPW_MAX = 1;           // planes per workgroup (1 measured fastest of 1..8)

constexpr int GUARD = 16;

__device__ __forceinline__ uint32_t lds_u32(const uint8_t* base, int off) {
    return *reinterpret_cast<const uint32_t*>(base + off);
}

// q = x / d and r = x % d for 0 <= x, d < 2^22 with inv = 1.0f / d.  The
// float quotient is within one of the true one there (x is exact in fp32 and
// the product's relative error is below 2^-22), and one correction step
// restores it; the launcher checks the bound.
__device__ __forceinline__ void divmod_small(int x, int d, float inv, int& q, int& r) {
    q = (int)((float)x * inv);
    r = x - q * d;
    if (r < 0) { --q; r += d; }
    else if (r >= d) { ++q; r -= d; }
}

// Byte mask of the 4 bytes 4j..4j+3 selected by bits 4j..4j+3 of `bits16`.
__device__ __forceinline__ uint32_t byte_mask(uint32_t bits16, int j) {
    const uint32_t nib = (bits16 >> (4 * j)) & 0xFu;
    return ((nib * 0x00204081u) & 0x01010101u) * 0xFFu;
}

// Workgroups [0, plane_blocks) each stage `ppw` consecutive (image, channel)
// planes in LDS, every plane behind a 16-byte guard, loaded together so that
// one memory latency covers them all; the workgroups after them fill the
// padding rows k >= Kg, one per (image, group).  Then every column row the
// staged planes feed -- k = ci*kH*kW + kh*kW + kw for the kH*kW taps -- is
// written 16 positions per lane, one 16-byte store each.
//  * Fast path (horizontal stride 1, the 16 positions inside one output row):
//    they read the contiguous bytes iw0 .. iw0+15 of input row ih, fetched as
//    five aligned LDS dwords and shifted into place with alignbyte; bytes of
//    columns outside [0, W) are replaced by the zero point through a mask.
//    Reads may touch the guard or a neighbouring row, always inside the
//    plane's LDS slot, and those bytes are masked.
//  * Otherwise each of the 16 positions is gathered on its own.
__global__ __launch_bounds__(NT) void conv_im2col_lds(ConvGeom c, const uint8_t* __restrict__ x,
                                                      uint8_t x_zp, uint8_t* __restrict__ col, int ppw,
                                                      int plane_blocks, int slot) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    __shared__ int64_t row_base[PPW_MAX];   // first column row each staged plane feeds
    const int chunks = c.Pp / 16;
    const uint32_t z4 = (uint32_t)x_zp * 0x01010101u;
    if ((int)blockIdx.x >= plane_blocks) {
        // padding rows of one (image, group)
        const int ng = blockIdx.x - plane_blocks;
        const int rows = c.Kp - c.Kg;
        uint8_t* base = col + ((int64_t)ng * c.Kp + c.Kg) * c.Pp;
        for (int i = threadIdx.x; i < rows * chunks; i += NT)
            *reinterpret_cast<v4i*>(base + (int64_t)(i / chunks) * c.Pp + (i % chunks) * 16) =
                v4i{(int)z4, (int)z4, (int)z4, (int)z4};
        return;
    }
    const int hw = c.H * c.W;
    const int64_t planes = (int64_t)c.N * c.C;
    const int64_t q0 = (int64_t)blockIdx.x * ppw;
    const int np = (int)(planes - q0 < ppw ? planes - q0 : ppw);
    // planes q0 .. q0+np-1 are consecutive in memory: one contiguous span
    const uint8_t* src = x + q0 * hw;
    if ((hw & 15) == 0 && (reinterpret_cast<uintptr_t>(src) & 15) == 0) {
        const int vpp = hw / 16;   // vectors per plane
        for (int pi = 0; pi < np; ++pi)
            for (int v = threadIdx.x; v < vpp; v += NT)
                *reinterpret_cast<v4i*>(lds + pi * slot + GUARD + 16 * v) =
                    *reinterpret_cast<const v4i*>(src + (int64_t)pi * hw + 16 * v);
    } else {
        for (int pi = 0; pi < np; ++pi)
            for (int v = threadIdx.x; v < hw; v += NT) lds[pi * slot + GUARD + v] = src[(int64_t)pi * hw + v];
    }
    const int taps = c.kH * c.kW;
    if ((int)threadIdx.x < np) {
        const int64_t q = q0 + threadIdx.x;
        const int64_t n = q / c.C;
        const int cc = (int)(q - n * c.C);
        const int g = cc / c.Cg, ci = cc - g * c.Cg;
        row_base[threadIdx.x] = (n * c.group + g) * c.Kp + (int64_t)ci * taps;
    }
    __syncthreads();
    const int per_plane = taps * chunks;
    const float inv_pp = 1.0f / (float)per_plane, inv_chunks = 1.0f / (float)chunks;
    const float inv_kw = 1.0f / (float)c.kW, inv_ow = 1.0f / (float)c.OW;
    for (int i = threadIdx.x; i < np * per_plane; i += NT) {
        int pi, rest, t, pc, kh, kw, oh, ow0;
        divmod_small(i, per_plane, inv_pp, pi, rest);
        divmod_small(rest, chunks, inv_chunks, t, pc);
        divmod_small(t, c.kW, inv_kw, kh, kw);
        const int p0 = pc * 16;
        divmod_small(p0, c.OW, inv_ow, oh, ow0);
        const uint8_t* plane = lds + pi * slot + GUARD;
        uint32_t d[4];
        if (c.sw == 1 && ow0 + 16 <= c.OW) {
            const int ih = oh * c.sh - c.pt + kh * c.dh;
            const int iw0 = ow0 - c.pl + kw * c.dw;
            // valid bytes e in [lo, hi): columns iw0 + e inside [0, W)
            const int lo = iw0 >= 0 ? 0 : (-iw0 < 16 ? -iw0 : 16);
            const int hi = c.W - iw0 >= 16 ? 16 : (c.W - iw0 > 0 ? c.W - iw0 : 0);
            if (ih < 0 || ih >= c.H || lo >= hi) {
                d[0] = d[1] = d[2] = d[3] = z4;
            } else {
                const int a = ih * c.W + iw0;          // >= -15: within the guard
                const int a0 = a & ~3, sh = a & 3;
                uint32_t wv[5];
#pragma unroll
                for (int j = 0; j < 5; ++j) wv[j] = lds_u32(plane, a0 + 4 * j);
                // bit e set: byte e is column iw0 + e inside [0, W)
                const uint32_t valid = ((1u << hi) - 1u) & ~((1u << lo) - 1u);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t v = __builtin_amdgcn_alignbyte(wv[j + 1], wv[j], sh);
                    const uint32_t keep = byte_mask(valid, j);
                    d[j] = (v & keep) | (z4 & ~keep);
                }
            }
        } else {
            d[0] = d[1] = d[2] = d[3] = 0u;
            int oh_e = oh, ow = ow0;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                uint32_t v = x_zp;
                if (p0 + e < c.P) {
                    const int ih = oh_e * c.sh - c.pt + kh * c.dh;
                    const int iw = ow * c.sw - c.pl + kw * c.dw;
                    if (ih >= 0 && ih < c.H && iw >= 0 && iw < c.W) v = plane[ih * c.W + iw];
                }
                d[e >> 2] |= v << (8 * (e & 3));
                if (++ow == c.OW) { ow = 0; ++oh_e; }
            }
        }
        uint8_t* dst = col + (row_base[pi] + t) * c.Pp + p0;
        *reinterpret_cast<v4i*>(dst) = v4i{(int)d[0], (int)d[1], (int)d[2], (int)d[3]};
    }
}

}  // namespace

hipError_t launch_conv_stage(const ConvGeom& c, const void* x, uint8_t x_zp, const void* w, const void* w_zp,
                             int w_zp_len, uint8_t* wp, uint8_t* col, hipStream_t s) {
    const int64_t wtotal = (int64_t)c.group * c.Mg * c.Kp;
    hipLaunchKernelGGL(conv_pack_weight, dim3((unsigned)((wtotal + NT - 1) / NT)), dim3(NT), 0, s, c,
                       reinterpret_cast<const uint8_t*>(w), reinterpret_cast<const uint8_t*>(w_zp), w_zp_len, wp);
    const int64_t hw = (int64_t)c.H * c.W;
    // the LDS kernel's index arithmetic needs every divided value below 2^22
    const int64_t lim = (int64_t)1 << 22;
    const int64_t slot = GUARD + (hw + 15) / 16 * 16 + 32;   // guard, plane, room for the last window
    const int64_t per_plane = (int64_t)c.kH * c.kW * (c.Pp / 16);
    if (slot <= PLANE_LDS_MAX && per_plane * PPW_MAX < lim && c.Pp < lim) {
        int ppw = (int)(PLANE_LDS_MAX / slot);
        if (ppw > PPW_MAX) ppw = PPW_MAX;
        const int64_t planes = (int64_t)c.N * c.C;
        const int plane_blocks = (int)((planes + ppw - 1) / ppw);
        const int blocks = plane_blocks + c.N * c.group;
        hipLaunchKernelGGL(conv_im2col_lds, dim3((unsigned)blocks), dim3(NT), (size_t)(ppw * slot), s, c,
                           reinterpret_cast<const uint8_t*>(x), x_zp, col, ppw, plane_blocks, (int)slot);
    } else {
        const int64_t ctotal = (int64_t)c.N * c.group * c.Kp * (c.Pp / 16);
        hipLaunchKernelGGL(conv_im2col, dim3((unsigned)((ctotal + NT - 1) / NT)), dim3(NT), 0, s, c,
                           reinterpret_cast<const uint8_t*>(x), x_zp, col);
    }
    return hipGetLastError();
}

}  // namespace qg

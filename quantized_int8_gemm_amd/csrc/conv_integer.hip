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

// Planes of up to this many bytes are staged in LDS by conv_im2col_lds.
constexpr int PLANE_LDS_MAX = 65536 - 64;

// One workgroup per (image n, input channel cc) plane, plus `group` extra
// workgroups per image that fill the padding rows k >= Kg of each group.  The
// plane is read once from memory into LDS (16-byte loads when its rows allow),
// behind a 16-byte guard, then every column row the plane feeds --
// k = ci*kH*kW + kh*kW + kw for the kH*kW taps -- is written 16 positions per
// lane, one 16-byte store each.
//  * Fast path (horizontal stride 1, the 16 positions inside one output row):
//    they read the contiguous bytes iw0 .. iw0+15 of input row ih, fetched as
//    five aligned LDS dwords and shifted into place with alignbyte; bytes of
//    columns outside [0, W) are replaced by the zero point through a mask.
//    Reads may touch the guard or a neighbouring row, always inside the LDS
//    allocation, and those bytes are masked.
//  * Otherwise each of the 16 positions is gathered on its own.
constexpr int GUARD = 16;

__device__ __forceinline__ uint32_t lds_u32(const uint8_t* base, int off) {
    return *reinterpret_cast<const uint32_t*>(base + off);
}

__global__ __launch_bounds__(NT) void conv_im2col_lds(ConvGeom c, const uint8_t* __restrict__ x,
                                                      uint8_t x_zp, uint8_t* __restrict__ col) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    uint8_t* plane = lds + GUARD;
    const int per_img = c.C + c.group;
    const int64_t n = blockIdx.x / per_img;
    const int cc = blockIdx.x % per_img;
    const int chunks = c.Pp / 16;
    const uint32_t z4 = (uint32_t)x_zp * 0x01010101u;
    if (cc >= c.C) {
        // padding rows of group cc - C
        const int g = cc - c.C;
        const int rows = c.Kp - c.Kg;
        uint8_t* base = col + ((n * c.group + g) * c.Kp + c.Kg) * c.Pp;
        for (int i = threadIdx.x; i < rows * chunks; i += NT)
            *reinterpret_cast<v4i*>(base + (int64_t)(i / chunks) * c.Pp + (i % chunks) * 16) =
                v4i{(int)z4, (int)z4, (int)z4, (int)z4};
        return;
    }
    const int g = cc / c.Cg, ci = cc % c.Cg;
    const int hw = c.H * c.W;
    const uint8_t* src = x + (n * c.C + cc) * (int64_t)hw;
    if ((hw & 15) == 0 && (reinterpret_cast<uintptr_t>(src) & 15) == 0) {
        for (int i = threadIdx.x; i < hw / 16; i += NT)
            *reinterpret_cast<v4i*>(plane + 16 * i) = *reinterpret_cast<const v4i*>(src + 16 * i);
    } else {
        for (int i = threadIdx.x; i < hw; i += NT) plane[i] = src[i];
    }
    __syncthreads();
    const int taps = c.kH * c.kW;
    uint8_t* rows = col + ((n * c.group + g) * c.Kp + (int64_t)ci * taps) * c.Pp;
    for (int i = threadIdx.x; i < taps * chunks; i += NT) {
        const int t = i / chunks, pc = i % chunks;
        const int kh = t / c.kW, kw = t % c.kW;
        const int p0 = pc * 16;
        const int oh = p0 / c.OW, ow0 = p0 % c.OW;
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
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t v = __builtin_amdgcn_alignbyte(wv[j + 1], wv[j], sh);
                    // byte e = 4j + b is kept when lo <= e < hi
                    uint32_t keep = 0u;
#pragma unroll
                    for (int b = 0; b < 4; ++b)
                        keep |= (4 * j + b >= lo && 4 * j + b < hi) ? (0xffu << (8 * b)) : 0u;
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
        *reinterpret_cast<v4i*>(rows + (int64_t)t * c.Pp + p0) = v4i{(int)d[0], (int)d[1], (int)d[2], (int)d[3]};
    }
}

}  // namespace

hipError_t launch_conv_stage(const ConvGeom& c, const void* x, uint8_t x_zp, const void* w, const void* w_zp,
                             int w_zp_len, uint8_t* wp, uint8_t* col, hipStream_t s) {
    const int64_t wtotal = (int64_t)c.group * c.Mg * c.Kp;
    hipLaunchKernelGGL(conv_pack_weight, dim3((unsigned)((wtotal + NT - 1) / NT)), dim3(NT), 0, s, c,
                       reinterpret_cast<const uint8_t*>(w), reinterpret_cast<const uint8_t*>(w_zp), w_zp_len, wp);
    const int64_t hw = (int64_t)c.H * c.W;
    if (hw <= PLANE_LDS_MAX) {
        // the plane behind a 16-byte guard, and room after it for the last
        // row's five-dword window (at most 19 bytes past the plane)
        const size_t lds = (size_t)(GUARD + (hw + 15) / 16 * 16 + 32);
        hipLaunchKernelGGL(conv_im2col_lds, dim3((unsigned)((int64_t)c.N * (c.C + c.group))), dim3(NT), lds, s, c,
                           reinterpret_cast<const uint8_t*>(x), x_zp, col);
    } else {
        const int64_t ctotal = (int64_t)c.N * c.group * c.Kp * (c.Pp / 16);
        hipLaunchKernelGGL(conv_im2col, dim3((unsigned)((ctotal + NT - 1) / NT)), dim3(NT), 0, s, c,
                           reinterpret_cast<const uint8_t*>(x), x_zp, col);
    }
    return hipGetLastError();
}

}  // namespace qg

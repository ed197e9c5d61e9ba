// Device helpers shared by the gfx950 kernels of the quantised matmul library.
//
// Operand layout for the int8 matrix cores (v_mfma_i32_16x16x64_i8): lane l
// supplies 16 bytes of row (l % 16) of the 16x64 left operand and 16 bytes of
// column (l % 16) of the 64x16 right operand, both covering the same 16 values
// of the contraction index (group l / 16).  The 16x16 int32 result lives in
// four registers per lane: register r of lane l holds row 4*(l/16)+r, column
// l % 16.  Because the contraction is an exact integer sum, any assignment of
// k values to (lane group, byte) works as long as both operands use the same
// one; the kernels always read both operands through the same k-segment index.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

// 16 bytes as four dwords.
struct u32x4 { uint32_t x, y, z, w; };

__device__ __forceinline__ v4i mfma_i8_16x16x64(const u32x4& a, const u32x4& b, v4i c) {
    v4i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w};
    v4i bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w};
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bv, c, 0, 0, 0);
}

__device__ __forceinline__ v4f mfma_f32_16x16x4(float a, float b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Sum of the four signed bytes of x added to c (v_dot4 against ones).
__device__ __forceinline__ int sum_i8x4(uint32_t x, int c) {
    return __builtin_amdgcn_sdot4((int)x, 0x01010101, c, false);
}

// 4x4 byte transpose: x[i] holds bytes (row i, cols 0..3); y[c] receives
// bytes (rows 0..3, col c).  Two rounds of byte permutes.
__device__ __forceinline__ void transpose4x4_bytes(const uint32_t x[4], uint32_t y[4]) {
    uint32_t t0 = __builtin_amdgcn_perm(x[1], x[0], 0x05010400u);
    uint32_t t1 = __builtin_amdgcn_perm(x[1], x[0], 0x07030602u);
    uint32_t t2 = __builtin_amdgcn_perm(x[3], x[2], 0x05010400u);
    uint32_t t3 = __builtin_amdgcn_perm(x[3], x[2], 0x07030602u);
    y[0] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
    y[1] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
    y[2] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
    y[3] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
}

// Row swizzle of the 16-byte segments of an LDS tile whose rows are 128 bytes
// (eight segments): segment s of row r is stored at slot s ^ (r & 7).  Eight
// consecutive rows then cover all eight slots for any one segment, so a
// fragment read (16 consecutive rows, one segment) is free of bank conflicts,
// and so is a row written as eight segments by eight lanes.
__device__ __forceinline__ int swz(int r) { return r & 7; }

// IEEE binary32 -> bfloat16 bits, round to nearest, ties to even, two
// values at once (lo in bits 0..15) by the hardware's packed conversion
// (v_cvt_pk_bf16_f32 in the default rounding mode, fp32 denormals kept):
// one instruction where the integer rounding sequence takes about six per
// value.  On every non-NaN input it equals the textbook rounding
// (b + 0x7fff + ((b >> 16) & 1)) >> 16 of the bit pattern b; all 2^32
// patterns were compared on the device.  A NaN becomes a quiet NaN.
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){lo, hi}, v2bf));
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    return (uint16_t)pack_bf16x2(f, 0.f);
}

// Workgroups are handed to the eight XCDs round robin (id % 8).  Renumber so
// that consecutive tile ids run on the same XCD and share its L2: the first
// nb/8 ids go to XCD 0, the next nb/8 to XCD 1, and so on.  Ids past the last
// full round keep their number.
__device__ __forceinline__ int xcd_remap(int bid, int nb) {
    const int per = nb / 8;
    if (bid >= per * 8) return bid;
    return (bid % 8) * per + bid / 8;
}

// Grouped tile order: walk GROUP_M tile rows down before moving one tile
// column right, so concurrently running tiles share A rows and B columns.
__device__ __forceinline__ void tile_coords(int t, int tiles_m, int tiles_n, int group_m,
                                            int& tm, int& tn) {
    const int per_group = group_m * tiles_n;
    const int g = t / per_group;
    const int first_m = g * group_m;
    int gsz = tiles_m - first_m;
    if (gsz > group_m) gsz = group_m;
    const int in_g = t - g * per_group;
    tm = first_m + in_g % gsz;
    tn = in_g / gsz;
}

}  // namespace qg

namespace qg {

// Raw buffer resource over [base, base + bytes): loads at offsets past
// `bytes` return zeros instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// The whole offset must be in `voff`: the range check that turns loads past
// the end into zeros applies to the per-lane offset, and callers pass soff = 0.
__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    v4i v = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
    return u32x4{(uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w};
}

// The same load with the non-temporal cache policy, for data read exactly
// once (a streamed weight): it does not displace reused lines, and a 64 MiB
// stream of such loads measured about 14% faster than cached loads.
constexpr int CPOL_NT = 2;
__device__ __forceinline__ u32x4 buffer_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    v4i v = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, CPOL_NT));
    return u32x4{(uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w};
}

}  // namespace qg

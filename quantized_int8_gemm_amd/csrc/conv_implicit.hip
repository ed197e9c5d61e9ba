// ConvInteger on gfx950 as an implicit GEMM: no column matrix is written.
//
// Operator: "feat(onnx-to-hip): lower quantized integer conv and matmul",
// section "What", ConvInteger paragraph: y[n, m, oh, ow] is the exact int32
// sum over the group's channels c and the taps (kh, kw) of
// (w[m, c, kh, kw] - w_zp[m]) * (x[n, g*Cg + c, ih, iw] - x_zp), with
// ih = oh*sh - pt + kh*dh, iw = ow*sw - pl + kw*dw, and taps outside the
// input counting as x_zp (they add nothing).
//
// Three kernels:
//  * conv_pack_weight_taps writes each output channel's weights as one row
//    in (channel block of 64, tap, channel) order, channels past Cg padded
//    with the channel's zero point, uint8 turned into int8 - 128 by flipping
//    bit 7, and the row's sum of those int8 values.
//  * conv_pad_input writes x as xp[n][g][hp][wp][Cgp]: the group's channels
//    innermost (padded to a multiple of 64), the input framed by the pads
//    and by enough further rows and columns that every output tile reads
//    inside xp; every position outside the input holds x_zp; flipped like w.
//  * conv_implicit_kernel: one workgroup computes 128 output channels x a
//    BH x BW block of output positions of one image and group.  Per block of
//    64 channels it copies the block's halo (the xp positions its taps read,
//    64 bytes each) and its 128 weight rows straight into LDS
//    (buffer_load ... lds), then for every tap multiplies the shifted halo
//    against that tap's weights on the int8 matrix cores: a B fragment is
//    16 channels of one position, read with ds_read_b128 at the position the
//    tap moves it to, so no data is reordered per tap.
// FUSED (one launch, no workspace): where x's rows are 16-byte aligned
// (W % 16 == 0), the main kernel stages the halo straight from x: a lane
// loads 16 columns of 4 channels (four 16-byte vectors), regroups them into
// one 4-channel word per column with byte permutes and writes each word to
// the position's 16-byte slot in LDS; halo positions outside the input get
// x_zp.  Its weight rows come straight from w the same way (4 channels x the
// taps of one output channel per lane, each tap's 4 bytes one word), their
// row sums added into LDS.  The multiplies and the epilogue are the same.
//
// With a' = w - sa and b' = x - sb the flipped values (sa, sb = 128 for
// uint8, else 0), ca[m] = sa - w_zp[m] and cb = sb - x_zp:
//   sum (w - w_zp)(x - x_zp) = sum a'b' + cb*rowsum'(m) + ca[m]*colsum'(p)
//                              + Keff*ca[m]*cb
// over Keff = taps * Cgp terms (padded terms are zero on one side of the
// first form); every step wraps mod 2^32 like the int32 result.
#include <cstdlib>

#include "device_common.h"
#include "int8_dma_impl.h"
#include "kernels.h"

namespace qg {
namespace {

constexpr int CI_NT = 256;
constexpr int CONV_FUSED_MAX_DYN_LDS = 159 * 1024;

struct ConvPrepArgs {
    ConvGeom c;
    int cgp, hp_rows, wp_cols, cblocks, w_pitch;   // w_pitch: LDS bytes per staged channel row
    int rpb;                                       // padded rows per workgroup
    int64_t kt;
    const uint8_t* x; uint8_t x_zp; uint32_t x_flip;
    const uint8_t* w; const uint8_t* w_zp; int w_zp_len; uint32_t w_flip;
    int8_t* wp; int32_t* rowsum; uint8_t* xp;
};

// One launch for both operands.  Workgroups [0, M) pack one output channel's
// weights each: the row in (channel block of 64, tap, channel) order,
// channels past Cg padded with the channel's zero point, flipped, and the
// row's sum of its int8 values.  The others each write `rpb` consecutive
// padded rows xp[n][g][hp][*][64-channel block]: the block's input rows
// (64 channels each, at ih = hp - pt) are read whole into LDS (16-byte loads
// where rows are 16-byte aligned, all issued before any is used), then every
// lane writes 16 channels of one position as one 16-byte vector, x_zp
// (flipped) outside the input.
__global__ __launch_bounds__(CI_NT) void conv_prep(ConvPrepArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t rows[];
    __shared__ int part[CI_NT / 64];
    const ConvGeom& c = a.c;
    const int tid = threadIdx.x;
    // Consecutive workgroup numbers go to one XCD, so the workgroups of
    // neighbouring padded rows (which read the same 128-byte lines of x)
    // share an L2.
    const int bid = xcd_remap((int)blockIdx.x, (int)gridDim.x);
    if (bid < c.M) {
        const int mm = bid;                        // output channel g*Mg + m
        const int taps = c.kH * c.kW;
        const int zw = a.w_zp == nullptr ? 0 : a.w_zp[a.w_zp_len == 1 ? 0 : mm];
        const uint8_t* wrow = a.w + (int64_t)mm * c.Cg * taps;
        int sum = 0;
        // PK elements per thread per pass, all loads issued before any store
        constexpr int PK = 4;
        for (int64_t k0 = tid; k0 < a.kt; k0 += PK * CI_NT) {
            int v[PK];
#pragma unroll
            for (int j = 0; j < PK; ++j) {
                const int64_t k = k0 + j * CI_NT;
                v[j] = zw;
                if (k < a.kt) {
                    const int blk = (int)(k / (taps * 64));
                    const int rem = (int)(k - (int64_t)blk * taps * 64);
                    const int tap = rem >> 6, ch = blk * 64 + (rem & 63);
                    if (ch < c.Cg) v[j] = wrow[(int64_t)ch * taps + tap];
                }
            }
#pragma unroll
            for (int j = 0; j < PK; ++j) {
                const int64_t k = k0 + j * CI_NT;
                if (k >= a.kt) break;
                const int8_t b = (int8_t)(uint8_t)((uint32_t)v[j] ^ a.w_flip);
                a.wp[(int64_t)mm * a.kt + k] = b;
                sum += b;
            }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
        if ((tid & 63) == 0) part[tid >> 6] = sum;
        __syncthreads();
        if (tid == 0) a.rowsum[mm] = part[0] + part[1] + part[2] + part[3];
        return;
    }
    int64_t b = (int64_t)bid - c.M;
    const int row_blocks = (a.hp_rows + a.rpb - 1) / a.rpb;
    const int cb = (int)(b % a.cblocks); b /= a.cblocks;
    const int hb = (int)(b % row_blocks); b /= row_blocks;
    const int64_t ng = b;                      // n * group + g
    const int64_t n = ng / c.group;
    const int g = (int)(ng - n * c.group);
    const int hp0 = hb * a.rpb;
    const int nrows = a.hp_rows - hp0 < a.rpb ? a.hp_rows - hp0 : a.rpb;
    const int ch0 = cb * 64;
    const int nch = c.Cg - ch0 < 64 ? c.Cg - ch0 : 64;
    const int64_t plane = (int64_t)c.H * c.W;
    const uint8_t* src0 = a.x + (n * c.C + (int64_t)g * c.Cg + ch0) * plane;
    const int row_bytes = 64 * a.w_pitch;      // one staged row: 64 channels
    const bool vec = (c.W & 15) == 0 && (reinterpret_cast<uintptr_t>(a.x) & 15) == 0;
    // every load of the block's input rows is issued before any is used
    for (int rr = 0; rr < nrows; ++rr) {
        const int ih = hp0 + rr - c.pt;
        if (ih < 0 || ih >= c.H) continue;
        const uint8_t* src = src0 + (int64_t)ih * c.W;
        uint8_t* dst = rows + rr * row_bytes;
        if (vec) {
            const int vpr = c.W / 16;          // vectors per row
            for (int i = tid; i < nch * vpr; i += CI_NT) {
                const int ch = i / vpr, v = i - ch * vpr;
                *reinterpret_cast<v4i*>(dst + ch * a.w_pitch + 16 * v) =
                    *reinterpret_cast<const v4i*>(src + ch * plane + 16 * v);
            }
        } else {
            for (int i = tid; i < nch * c.W; i += CI_NT) {
                const int ch = i / c.W, col = i - ch * c.W;
                dst[ch * a.w_pitch + col] = src[ch * plane + col];
            }
        }
    }
    __syncthreads();
    const uint32_t zf = ((uint32_t)a.x_zp ^ a.x_flip) & 0xffu;
    for (int rr = 0; rr < nrows; ++rr) {
        const int hp = hp0 + rr, ih = hp - c.pt;
        const bool row_in = ih >= 0 && ih < c.H;
        const uint8_t* srow = rows + rr * row_bytes;
        uint8_t* dst_row = a.xp + ((ng * a.hp_rows + hp) * (int64_t)a.wp_cols) * a.cgp + ch0;
        // lane -> (channel quarter q, position wq), positions fastest: a
        // wave's byte reads then walk one staged row (no bank conflicts)
        for (int i = tid; i < a.wp_cols * 4; i += CI_NT) {
            const int q = i / a.wp_cols, wq = i - q * a.wp_cols;
            const int iw = wq - c.pl;
            const bool in = row_in && iw >= 0 && iw < c.W;
            uint32_t d[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint32_t word = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int ch = q * 16 + 4 * j + e;
                    const uint32_t v = (in && ch < nch) ? (((uint32_t)srow[ch * a.w_pitch + iw] ^ a.x_flip) & 0xffu) : zf;
                    word |= v << (8 * e);
                }
                d[j] = word;
            }
            *reinterpret_cast<v4i*>(dst_row + (int64_t)wq * a.cgp + 16 * q) =
                v4i{(int)d[0], (int)d[1], (int)d[2], (int)d[3]};
        }
    }
}

struct ConvImplicitArgs {
    ConvGeom c;
    int bh, th, tw, hp_rows, wp_cols, cgp, taps, cblocks, hr, hc, a_pitch, a_rounds, h_rounds;
    int a_dq, a_dr;       // 256 weight units = a_dq rows + a_dr units (a_pitch / 16 units per row)
    int h_dq, h_dr;       // 64 halo positions = h_dq rows + h_dr columns
    int64_t kt;
    const int8_t* wp; const int32_t* rowsum; const int8_t* xp;
    const uint8_t* w_zp; int w_zp_len; int w_u8;  // ca[m] = sa - w_zp[m]
    int32_t sa, cb;                               // cb = sb - x_zp
    int32_t* y;
    // FUSED: the operands themselves, their flips, x_zp (flipped) in every byte
    const uint8_t* x; const uint8_t* w; uint32_t x_flip, w_flip, zf4;
};

// FUSED weight staging: output channel m's 4 channels c .. c+3 of the block,
// all T taps (4*T consecutive bytes of w, already loaded as T words), as one
// word per tap at the tap's slot of row r; returns the sum of the 4*T
// flipped int8 values.
template <int T>
__device__ __forceinline__ int stage_w_quad(const uint32_t* wd, uint32_t flip, uint8_t* row, int r, int cq) {
    int sum = 0;
#pragma unroll
    for (int t = 0; t < T; ++t) {
        uint32_t d = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int idx = e * T + t;   // channel c + e, tap t
            const uint32_t b = ((wd[idx >> 2] >> (8 * (idx & 3))) & 0xffu) ^ flip;
            d |= b << (8 * e);
            sum += (int)(int8_t)(uint8_t)b;
        }
        *reinterpret_cast<uint32_t*>(row + ((4 * t + ((cq >> 2) ^ ((r >> 2) & 3))) << 4) + 4 * (cq & 3)) = d;
    }
    return sum;
}

// 16-byte slot of channel group j at halo column col: j ^ ((col >> 2) & 3),
// so the 16 positions of a fragment read (16 consecutive columns) fall in 16
// distinct 16-byte bank groups.
__device__ __forceinline__ int halo_slot(int col, int j) { return j ^ ((col >> 2) & 3); }
// Weight row r, tap t, channel group j at slot 4t + (j ^ ((r >> 2) & 3)):
// with the row pitch 64 mod 256 the 16 rows of a fragment read take 16
// distinct bank groups.
__device__ __forceinline__ int w_slot(int r, int t, int j) { return 4 * t + (j ^ ((r >> 2) & 3)); }

// BM output channels (64 or 128) x 128 positions per workgroup; four waves,
// each 64 channels x (128 / (4 / (BM / 64))) positions.
template <int BW, int BM, int NPOS, bool FUSED>
__global__ __launch_bounds__(CI_NT) void conv_implicit_kernel(ConvImplicitArgs p) {
    constexpr int WAVES_M = BM / 64, WAVES_N = 4 / WAVES_M;
    constexpr int WNP = NPOS / WAVES_N;              // positions per wave
    constexpr int FN = WNP / 16, FM = 4;
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    const ConvGeom& c = p.c;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int g16 = lane >> 4, i16 = lane & 15;

    // tile: (m tile, output row block, output column block); image and group
    // Consecutive workgroup numbers (over the whole grid) go to one XCD, so
    // the channel tiles and neighbouring row tiles of an image, which read
    // the same padded input, share an L2.
    const int m_tiles = (c.Mg + BM - 1) / BM;
    const int lin = xcd_remap((int)(blockIdx.y * gridDim.x + blockIdx.x), (int)(gridDim.x * gridDim.y));
    int t = lin % (int)gridDim.x;
    const int mt = t % m_tiles; t /= m_tiles;
    const int tcol = t % p.tw; t /= p.tw;
    const int trow = t;
    const int ng = lin / (int)gridDim.x;
    const int n = ng / c.group, g = ng - (ng / c.group) * c.group;
    const int m0 = mt * BM;
    const int oh0 = trow * p.bh, ow0 = tcol * BW;

    // The epilogue's per-channel terms, loaded now so that their latency
    // hides behind the staging: ca[m] = sa - w_zp[m] and cb*rowsum'(m).
    uint32_t ca_r[FM], rs_r[FM];
#pragma unroll
    for (int a = 0; a < FM; ++a) {
        const int m = m0 + wm * 64 + 16 * a + i16;
        const int mm = g * c.Mg + (m < c.Mg ? m : c.Mg - 1);
        int zw = 0;
        if (p.w_zp != nullptr) {
            const int idx = p.w_zp_len == 1 ? 0 : mm;
            zw = p.w_u8 ? (int)p.w_zp[idx] : (int)(int8_t)p.w_zp[idx];
        }
        ca_r[a] = (uint32_t)(p.sa - zw);
        rs_r[a] = FUSED ? 0u : (uint32_t)p.rowsum[mm];
    }
    // FUSED: the row sums of this tile's flipped weights, built while staging
    __shared__ int rs_lds[FUSED ? BM : 1];
    if constexpr (FUSED) {
        if (tid < BM) rs_lds[tid] = 0;
        __syncthreads();
    }

    const int a_bytes = BM * p.a_pitch;
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
    const uint32_t lds_h = lds0 + a_bytes;

    // operand windows: this group's packed weights, this tile's part of xp
    const int8_t* wbase = p.wp + (int64_t)g * c.Mg * p.kt;
    const v4i w_rsrc = dma::rsrc_words(wbase, (uint32_t)((int64_t)c.Mg * p.kt));
    const int64_t img = (int64_t)p.hp_rows * p.wp_cols * p.cgp;
    const int64_t tile_off = ((int64_t)oh0 * c.sh * p.wp_cols + (int64_t)ow0 * c.sw) * p.cgp;
    const int8_t* xbase = p.xp + (int64_t)ng * img + tile_off;
    const v4i x_rsrc = dma::rsrc_words(xbase, (uint32_t)(img - tile_off));

    // Position wn*WNP + 16b + i16 of the tile sits at halo row rr[b], column
    // cc[b] for tap (0, 0).
    int rr[FN], cc[FN];
#pragma unroll
    for (int b = 0; b < FN; ++b) {
        const int pl = wn * WNP + 16 * b + i16;
        rr[b] = (pl / BW) * c.sh;
        cc[b] = (pl % BW) * c.sw;
    }

    v4i acc[FM][FN];
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int b = 0; b < FN; ++b) acc[a][b] = v4i{0, 0, 0, 0};
    int cs[FN];
#pragma unroll
    for (int b = 0; b < FN; ++b) cs[b] = 0;

    const uint32_t OUT = 0xFFFFFFF0u;   // past every buffer: the load returns zeros
    const int a_upr = p.a_pitch / 16;   // weight units per row
    const int h_slot = tid & 3;
    // first unit of this lane: weight row / unit, halo row / column
    const int a_r0 = tid / a_upr, a_s0 = tid - a_r0 * a_upr;
    const int h_p0 = tid >> 2;
    const int h_r0 = h_p0 / p.hc, h_c0 = h_p0 - h_r0 * p.hc;
    for (int blk = 0; blk < p.cblocks; ++blk) {
        if (blk > 0) __syncthreads();   // every wave is done with the previous block
        if constexpr (FUSED) {
            // weights: unit u = q * 256 + tid is row r = u / 16, channels
            // 4 (u % 16) .. + 3; every unit's loads are issued before any is
            // used (rows past Mg multiply into outputs never stored: skipped)
            const bool need_rs = p.cb != 0;
            constexpr int WU = BM * 16 / CI_NT;
            auto wsrc = [&](int r, int cq) {
                return p.w + ((int64_t)(g * c.Mg + m0 + r) * c.Cg + blk * 64 + 4 * cq) * p.taps;
            };
            if (p.taps == 9 || p.taps == 1) {
                uint32_t wd[WU][9];
#pragma unroll
                for (int q = 0; q < WU; ++q) {
                    const int u = q * CI_NT + tid, r = u >> 4, cq = u & 15;
                    if (m0 + r >= c.Mg) continue;
                    const uint8_t* src = wsrc(r, cq);
                    if (p.taps == 9) {
#pragma unroll
                        for (int i = 0; i < 9; ++i) wd[q][i] = *reinterpret_cast<const uint32_t*>(src + 4 * i);
                    } else {
                        wd[q][0] = *reinterpret_cast<const uint32_t*>(src);
                    }
                }
#pragma unroll
                for (int q = 0; q < WU; ++q) {
                    const int u = q * CI_NT + tid, r = u >> 4, cq = u & 15;
                    if (m0 + r >= c.Mg) continue;
                    uint8_t* row = smem + r * p.a_pitch;
                    const int sum = p.taps == 9 ? stage_w_quad<9>(wd[q], p.w_flip, row, r, cq)
                                                : stage_w_quad<1>(wd[q], p.w_flip, row, r, cq);
                    if (need_rs) atomicAdd(&rs_lds[r], sum);
                }
            } else for (int u = tid; u < BM * 16; u += CI_NT) {
                const int r = u >> 4, cq = u & 15;
                if (m0 + r >= c.Mg) continue;
                const uint8_t* src = wsrc(r, cq);
                uint8_t* row = smem + r * p.a_pitch;
                int sum;
                {
                    sum = 0;
                    for (int t = 0; t < p.taps; ++t) {
                        uint32_t d = 0;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const uint32_t b = (uint32_t)src[e * p.taps + t] ^ p.w_flip;
                            d |= b << (8 * e);
                            sum += (int)(int8_t)(uint8_t)b;
                        }
                        *reinterpret_cast<uint32_t*>(row + ((4 * t + ((cq >> 2) ^ ((r >> 2) & 3))) << 4) + 4 * (cq & 3)) = d;
                    }
                }
                if (need_rs) atomicAdd(&rs_lds[r], sum);
            }
            // halo from x: positions inside the input, as units of 4 channels x
            // one aligned 16-column piece of one halo row
            uint8_t* Hd = smem + a_bytes;
            const int ih0 = oh0 * c.sh - c.pt, iw0 = ow0 * c.sw - c.pl;
            const int c_lo = iw0 > 0 ? iw0 : 0;
            const int c_hi = iw0 + p.hc < c.W ? iw0 + p.hc : c.W;
            const int cs0 = c_lo & ~15;
            const int nchunks = c_hi > c_lo ? (c_hi - cs0 + 15) >> 4 : 0;
            const int64_t plane = (int64_t)c.H * c.W;
            const uint8_t* xblk = p.x + ((int64_t)n * c.C + (int64_t)g * c.Cg + blk * 64) * plane;
            const int units = 16 * p.hr * nchunks;
            // XU units per lane per round, their loads issued together
            constexpr int XU = 2;
            for (int u0 = tid; u0 < units; u0 += XU * CI_NT) {
                u32x4 v[XU][4];
                int rr_[XU], cs_[XU];
                bool ok[XU];
#pragma unroll
                for (int q = 0; q < XU; ++q) {
                    const int u = u0 + q * CI_NT;
                    const int cq = u & 15, rk = u >> 4;
                    const int r = rk / nchunks, k = rk - r * nchunks;
                    const int ih = ih0 + r;
                    rr_[q] = r;
                    cs_[q] = cs0 + 16 * k;
                    ok[q] = u < units && ih >= 0 && ih < c.H;
                    if (!ok[q]) continue;
                    const uint8_t* src = xblk + (int64_t)(4 * cq) * plane + (int64_t)ih * c.W + cs_[q];
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[q][e] = *reinterpret_cast<const u32x4*>(src + (int64_t)e * plane);
                }
#pragma unroll
                for (int q = 0; q < XU; ++q) {
                    if (!ok[q]) continue;
                    const int cq = (u0 + q * CI_NT) & 15, r = rr_[q], cs = cs_[q];
#pragma unroll
                    for (int k4 = 0; k4 < 4; ++k4) {
                        // columns cs + 4 k4 .. + 3: a 4x4 byte transpose turns the
                        // four channels' words into one word per column
                        uint32_t xin[4], col4[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) xin[e] = (&v[q][e].x)[k4];
                        transpose4x4_bytes(xin, col4);
#pragma unroll
                        for (int i4 = 0; i4 < 4; ++i4) {
                            const int iw = cs + 4 * k4 + i4;
                            if (iw < c_lo || iw >= c_hi) continue;
                            const int col = iw - iw0;
                            *reinterpret_cast<uint32_t*>(Hd + 16 * (((r * p.hc + col) << 2) + halo_slot(col, cq >> 2)) +
                                                         4 * (cq & 3)) = col4[i4] ^ (p.x_flip * 0x01010101u);
                        }
                    }
                }
            }
            // positions outside the input hold x_zp
            for (int pidx = tid; pidx < p.hr * p.hc; pidx += CI_NT) {
                const int r = pidx / p.hc, col = pidx - r * p.hc;
                const int ih = ih0 + r, iw = iw0 + col;
                if (ih >= 0 && ih < c.H && iw >= 0 && iw < c.W) continue;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *reinterpret_cast<u32x4*>(Hd + 16 * ((pidx << 2) + j)) = u32x4{p.zf4, p.zf4, p.zf4, p.zf4};
            }
        } else {
            {   // weights: unit q*256 + tid of the A region is row ar, unit as
                int ar = a_r0, as = a_s0;
                const int64_t kblk = (int64_t)blk * p.taps * 64;
                for (int q = 0; q < p.a_rounds; ++q) {
                    uint32_t off = OUT;
                    if (as < 4 * p.taps && m0 + ar < c.Mg) {
                        const int tp = as >> 2, j = (as & 3) ^ ((ar >> 2) & 3);
                        off = (uint32_t)((int64_t)(m0 + ar) * p.kt + kblk + 64 * tp + 16 * j);
                    }
                    dma::dma16(w_rsrc, off, lds0 + (uint32_t)(q * CI_NT + wave * 64) * 16u);
                    as += p.a_dr; ar += p.a_dq;
                    if (as >= a_upr) { as -= a_upr; ++ar; }
                }
            }
            {   // halo: unit q*256 + tid is position (hr_, hc_) of the halo, slot h_slot
                int hr_ = h_r0, hc_ = h_c0;
                for (int q = 0; q < p.h_rounds; ++q) {
                    uint32_t off = OUT;
                    if (hr_ < p.hr)
                        off = (uint32_t)(((int64_t)hr_ * p.wp_cols + hc_) * p.cgp + blk * 64 + 16 * halo_slot(hc_, h_slot));
                    dma::dma16(x_rsrc, off, lds_h + (uint32_t)(q * CI_NT + wave * 64) * 16u);
                    hc_ += p.h_dr; hr_ += p.h_dq;
                    if (hc_ >= p.hc) { hc_ -= p.hc; ++hr_; }
                }
            }
        }
        dma::wait_vmcnt<0>();
        __syncthreads();

        const uint8_t* A = smem;
        const uint8_t* Hs = smem + a_bytes;
        int kh = 0, kw = 0;
        for (int tp = 0; tp < p.taps; ++tp) {
            u32x4 bf[FN], af[FM];
#pragma unroll
            for (int b = 0; b < FN; ++b) {
                const int r = rr[b] + kh * c.dh, col = cc[b] + kw * c.dw;
                bf[b] = *reinterpret_cast<const u32x4*>(Hs + (((r * p.hc + col) << 2) + halo_slot(col, g16)) * 16);
            }
#pragma unroll
            for (int a = 0; a < FM; ++a) {
                const int row = wm * 64 + 16 * a + i16;
                af[a] = *reinterpret_cast<const u32x4*>(A + ((row * a_upr + w_slot(row, tp, g16)) << 4));
            }
#pragma unroll
            for (int b = 0; b < FN; ++b)
                cs[b] = sum_i8x4(bf[b].w, sum_i8x4(bf[b].z, sum_i8x4(bf[b].y, sum_i8x4(bf[b].x, cs[b]))));
#pragma unroll
            for (int a = 0; a < FM; ++a)
#pragma unroll
                for (int b = 0; b < FN; ++b) acc[a][b] = mfma_i8_16x16x64(bf[b], af[a], acc[a][b]);
            if (++kw == c.kW) { kw = 0; ++kh; }
        }
    }

    if constexpr (FUSED) {
#pragma unroll
        for (int a = 0; a < FM; ++a) rs_r[a] = (uint32_t)rs_lds[wm * 64 + 16 * a + i16];
    }
    // column sums over the four lane groups (channel groups)
#pragma unroll
    for (int b = 0; b < FN; ++b) {
        cs[b] += __shfl_xor(cs[b], 16);
        cs[b] += __shfl_xor(cs[b], 32);
    }
    // lane (g16, i16) holds channel m = wm*64 + 16a + i16 at positions
    // wn*WNP + 16b + 4*g16 + r, r = 0..3 (four consecutive columns of one
    // output row, BW being a multiple of 16)
    const uint32_t cbv = (uint32_t)p.cb;
    const uint32_t keff = (uint32_t)(p.taps * p.cgp);
    const bool vec = (c.OW & 3) == 0 && ((reinterpret_cast<uintptr_t>(p.y) & 15) == 0);
    // column sums of this lane's output positions, gathered while every lane
    // is active
    uint32_t colv[FN][4];
#pragma unroll
    for (int b = 0; b < FN; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) colv[b][r] = (uint32_t)__shfl(cs[b], 4 * g16 + r);
#pragma unroll
    for (int a = 0; a < FM; ++a) {
        const int m = m0 + wm * 64 + 16 * a + i16;
        if (m >= c.Mg) continue;
        const int mm = g * c.Mg + m;
        const uint32_t ca = ca_r[a];
        const uint32_t rowt = cbv * rs_r[a] + keff * ca * cbv;
        int32_t* yrow = p.y + ((int64_t)n * c.M + mm) * c.OH * c.OW;
#pragma unroll
        for (int b = 0; b < FN; ++b) {
            const int pl = wn * WNP + 16 * b + 4 * g16;
            const int oh = oh0 + pl / BW, ow = ow0 + pl % BW;
            uint32_t v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                v[r] = (uint32_t)acc[a][b][r] + rowt + ca * colv[b][r];
            if (oh >= c.OH || ow >= c.OW) continue;
            int32_t* dst = yrow + (int64_t)oh * c.OW + ow;
            if (vec && ow + 4 <= c.OW) {
                *reinterpret_cast<v4i*>(dst) = v4i{(int)v[0], (int)v[1], (int)v[2], (int)v[3]};
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (ow + r < c.OW) dst[r] = (int32_t)v[r];
            }
        }
    }
}

}  // namespace

bool conv_implicit_plan(const ConvGeom& c, ConvImplicitPlan* p) {
    if (c.Cg % 64 != 0) return false;
    const int taps = c.kH * c.kW;
    if (taps > 9) return false;
    if (c.W > 1024) return false;                    // the copy kernel stages 64 input rows in LDS
    // 64-channel tiles (three workgroups per compute unit) unless
    // QGEMM_CONV_BM=128 asks for 128
    const char* bm_env = std::getenv("QGEMM_CONV_BM");
    const int bm = (bm_env != nullptr && std::atoi(bm_env) == 128) ? 128 : 64;
    const int bw = c.OW > 16 ? 32 : 16;
    // weight rows of taps*64 bytes, pitch 64 mod 256
    int64_t pitch = (int64_t)taps * 64;
    pitch += (64 - pitch % 256 + 256) % 256;
    // 256 positions per tile (twice the multiplies per weight slice staged,
    // half the workgroups) for 64-channel tiles whenever the output has a
    // full tile of rows and two workgroups still fit a compute unit's LDS
    // (64x64x32x32 3x3 layer: 25.1 -> 23.3 us); else 128
    int npos = 128, bh = 0;
    int64_t hr = 0, hc = 0, h_rounds = 0, lds = 0;
    for (const int cand : {256, 128}) {
        if (cand == 256 && (bm != 64 || c.OH < cand / bw)) continue;
        const int cbh = cand / bw;
        const int64_t chr = (int64_t)(cbh - 1) * c.sh + (int64_t)(c.kH - 1) * c.dh + 1;
        const int64_t chc = (int64_t)(bw - 1) * c.sw + (int64_t)(c.kW - 1) * c.dw + 1;
        const int64_t crounds = (chr * chc * 4 + CI_NT - 1) / CI_NT;
        const int64_t clds = bm * pitch + crounds * CI_NT * 16;
        if (cand == 256 && clds > 80 * 1024) continue;
        npos = cand; bh = cbh; hr = chr; hc = chc; h_rounds = crounds; lds = clds;
        break;
    }
    if (lds > 160 * 1024) return false;
    const int64_t th = (c.OH + bh - 1) / bh, tw = (c.OW + bw - 1) / bw;
    // padded rows / columns: exactly the ones the output tiles read (input
    // rows a stride skips at the end are not copied)
    const int64_t HPr = (th * bh - 1) * c.sh + (int64_t)(c.kH - 1) * c.dh + 1;
    const int64_t WPc = (tw * bw - 1) * c.sw + (int64_t)(c.kW - 1) * c.dw + 1;
    const int64_t cgp = c.Cg;
    const int64_t img = HPr * WPc * cgp;
    if (img >= ((int64_t)1 << 31) - 256) return false;           // 32-bit offsets in one image
    if ((int64_t)c.Mg * cgp * taps >= ((int64_t)1 << 31) - 256) return false;
    const int64_t tiles = (int64_t)((c.Mg + bm - 1) / bm) * th * tw;
    if (tiles >= ((int64_t)1 << 31) || (int64_t)c.N * c.group >= 65536) return false;
    if (tiles * c.N * c.group >= ((int64_t)1 << 31)) return false;    // workgroup numbers fit an int
    const int64_t prep_blocks = (int64_t)c.M + (int64_t)c.N * c.group * HPr * (cgp / 64);
    if (prep_blocks >= ((int64_t)1 << 31)) return false;
    p->BM = bm; p->BW = bw; p->BH = bh; p->NPOS = npos; p->TH = (int)th; p->TWt = (int)tw;
    p->HP = (int)HPr; p->WP = (int)WPc; p->Cgp = (int)cgp; p->taps = taps; p->cblks = (int)(cgp / 64);
    p->HR = (int)hr; p->HC = (int)hc; p->a_pitch = (int)pitch; p->h_rounds = (int)h_rounds;
    p->lds_bytes = (int)lds;
    p->Kt = cgp * taps;
    const size_t wp_bytes = (size_t)c.group * c.Mg * p->Kt;
    p->wp_off = 0;
    p->rs_off = (wp_bytes + 255) / 256 * 256;
    p->xp_off = (p->rs_off + (size_t)c.M * 4 + 255) / 256 * 256;
    p->total = p->xp_off + (size_t)c.N * c.group * img;
    return true;
}

namespace {

// LDS beyond 64 KiB per workgroup is granted per kernel (160 KiB on gfx950).
template <int BW, int BM, int NPOS, bool FUSED>
hipError_t launch_main(const dim3& grid, const ConvImplicitArgs& a, int lds, hipStream_t s) {
    static bool granted = false;
    if (!granted) {
        // the fused form's row sums take 1 KiB of static LDS (the dynamic
        // region is 1 KiB aligned)
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(conv_implicit_kernel<BW, BM, NPOS, FUSED>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 FUSED ? CONV_FUSED_MAX_DYN_LDS : 160 * 1024);
        if (e != hipSuccess) return e;
        granted = true;
    }
    hipLaunchKernelGGL((conv_implicit_kernel<BW, BM, NPOS, FUSED>), grid, dim3(CI_NT), (size_t)lds, s, a);
    return hipGetLastError();
}

template <bool FUSED>
hipError_t launch_main_cfg(const ConvImplicitPlan& p, const dim3& grid, const ConvImplicitArgs& a, hipStream_t s) {
    if (p.BM == 128) return p.BW == 32 ? launch_main<32, 128, 128, FUSED>(grid, a, p.lds_bytes, s)
                                       : launch_main<16, 128, 128, FUSED>(grid, a, p.lds_bytes, s);
    if (p.NPOS == 256) return p.BW == 32 ? launch_main<32, 64, 256, FUSED>(grid, a, p.lds_bytes, s)
                                         : launch_main<16, 64, 256, FUSED>(grid, a, p.lds_bytes, s);
    return p.BW == 32 ? launch_main<32, 64, 128, FUSED>(grid, a, p.lds_bytes, s)
                      : launch_main<16, 64, 128, FUSED>(grid, a, p.lds_bytes, s);
}

}  // namespace

bool conv_fused_ok(const ConvGeom& c, const ConvImplicitPlan& p, const void* x, const void* w) {
    return c.W % 16 == 0 && (reinterpret_cast<uintptr_t>(x) & 15u) == 0 && (reinterpret_cast<uintptr_t>(w) & 3u) == 0 &&
           p.lds_bytes <= CONV_FUSED_MAX_DYN_LDS;
}

hipError_t launch_conv_implicit(const ConvGeom& c, const ConvImplicitPlan& p, const void* x, bool x_u8, int x_zp,
                                const void* w, bool w_u8, const void* w_zp, int w_zp_len, void* ws, int32_t* y,
                                bool fused, hipStream_t s) {
    if (fused) {
        if (!conv_fused_ok(c, p, x, w)) return hipErrorInvalidValue;
        ConvImplicitArgs a{};
        a.c = c;
        a.bh = p.BH; a.th = p.TH; a.tw = p.TWt; a.hp_rows = p.HP; a.wp_cols = p.WP; a.cgp = p.Cgp; a.taps = p.taps;
        a.cblocks = p.cblks; a.hr = p.HR; a.hc = p.HC; a.a_pitch = p.a_pitch;
        a.a_rounds = p.BM * p.a_pitch / 16 / CI_NT; a.h_rounds = p.h_rounds;
        a.a_dq = CI_NT / (p.a_pitch / 16); a.a_dr = CI_NT % (p.a_pitch / 16);
        a.h_dq = 64 / p.HC; a.h_dr = 64 % p.HC;
        a.kt = p.Kt;
        a.w_zp = reinterpret_cast<const uint8_t*>(w_zp); a.w_zp_len = w_zp_len; a.w_u8 = w_u8 ? 1 : 0;
        a.sa = w_u8 ? 128 : 0;
        a.cb = (x_u8 ? 128 : 0) - x_zp;
        a.y = y;
        a.x = reinterpret_cast<const uint8_t*>(x);
        a.w = reinterpret_cast<const uint8_t*>(w);
        a.x_flip = x_u8 ? 0x80u : 0u;
        a.w_flip = w_u8 ? 0x80u : 0u;
        a.zf4 = (((uint32_t)x_zp ^ a.x_flip) & 0xffu) * 0x01010101u;
        const int m_tiles = (c.Mg + p.BM - 1) / p.BM;
        const dim3 grid((unsigned)(m_tiles * p.TH * p.TWt), (unsigned)(c.N * c.group));
        return launch_main_cfg<true>(p, grid, a, s);
    }
    uint8_t* base = reinterpret_cast<uint8_t*>(ws);
    int8_t* wp = reinterpret_cast<int8_t*>(base + p.wp_off);
    int32_t* rowsum = reinterpret_cast<int32_t*>(base + p.rs_off);
    uint8_t* xp = base + p.xp_off;

    ConvPrepArgs pa{};
    pa.c = c;
    pa.cgp = p.Cgp; pa.hp_rows = p.HP; pa.wp_cols = p.WP; pa.cblocks = p.cblks;
    pa.w_pitch = (c.W + 15) / 16 * 16;
    // two padded rows per workgroup where their staged input rows fit the
    // default 64 KiB of LDS (25.4 -> 25.0 us on a 64x64x32x32 3x3 layer;
    // four rows measured slower), else one
    pa.rpb = 2 * 64 * pa.w_pitch <= 64 * 1024 ? 2 : 1;
    pa.kt = p.Kt;
    pa.x = reinterpret_cast<const uint8_t*>(x); pa.x_zp = (uint8_t)(x_zp & 0xff); pa.x_flip = x_u8 ? 0x80u : 0u;
    pa.w = reinterpret_cast<const uint8_t*>(w); pa.w_zp = reinterpret_cast<const uint8_t*>(w_zp);
    pa.w_zp_len = w_zp_len; pa.w_flip = w_u8 ? 0x80u : 0u;
    pa.wp = wp; pa.rowsum = rowsum; pa.xp = xp;
    const int64_t prep_blocks = (int64_t)c.M + (int64_t)c.N * c.group * ((p.HP + pa.rpb - 1) / pa.rpb) * p.cblks;
    hipLaunchKernelGGL(conv_prep, dim3((unsigned)prep_blocks), dim3(CI_NT), (size_t)(pa.rpb * 64 * pa.w_pitch), s, pa);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    ConvImplicitArgs a{};
    a.c = c;
    a.bh = p.BH; a.th = p.TH; a.tw = p.TWt; a.hp_rows = p.HP; a.wp_cols = p.WP; a.cgp = p.Cgp; a.taps = p.taps;
    a.cblocks = p.cblks; a.hr = p.HR; a.hc = p.HC; a.a_pitch = p.a_pitch;
    a.a_rounds = p.BM * p.a_pitch / 16 / CI_NT; a.h_rounds = p.h_rounds;
    a.a_dq = CI_NT / (p.a_pitch / 16); a.a_dr = CI_NT % (p.a_pitch / 16);
    a.h_dq = 64 / p.HC; a.h_dr = 64 % p.HC;
    a.kt = p.Kt;
    a.wp = wp; a.rowsum = rowsum; a.xp = reinterpret_cast<const int8_t*>(xp);
    a.w_zp = reinterpret_cast<const uint8_t*>(w_zp); a.w_zp_len = w_zp_len; a.w_u8 = w_u8 ? 1 : 0;
    a.sa = w_u8 ? 128 : 0;
    a.cb = (x_u8 ? 128 : 0) - x_zp;
    a.y = y;
    const int m_tiles = (c.Mg + p.BM - 1) / p.BM;
    const dim3 grid((unsigned)(m_tiles * p.TH * p.TWt), (unsigned)(c.N * c.group));
    return launch_main_cfg<false>(p, grid, a, s);
}

}  // namespace qg

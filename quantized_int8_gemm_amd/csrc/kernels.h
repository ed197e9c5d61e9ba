// Launchers for the gfx950 kernels and the argument blocks they take.
// Host code (the C-ABI entry points) fills these blocks after validation.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

// Epilogue selector of the int8 tiled kernel.
enum Int8Epilogue { EPI_F32 = 0, EPI_BF16 = 1, EPI_I32 = 2 };

// Arguments of the int8 x int8 -> int32 tiled matrix-core kernel and of the
// skinny (decode) kernel.  One block describes one problem of `batch`
// independent [M,K] x [K,N] products (batch strides may be 0 for a shared
// operand).
struct Int8GemmArgs {
    int M, N, K, batch;
    const int8_t* A; int64_t lda; int64_t a_bstride;
    const int8_t* B; int64_t ldb; int64_t b_bstride;  // [K,N] rows, or [N,K] if k-major
    uint32_t a_flip, b_flip;                          // 0x80808080 turns uint8 into int8 - 128
    void* out; int64_t ldo; int64_t o_bstride;
    // A8W8 epilogue: scales indexed by row / column (stride 0 = one value)
    const float* act_scale; int as_stride;
    const float* weight_scale; int ws_stride;
    // A8W8 accumulator input: acc += acc_in[m*ld_acc + n] before the cast
    // (NULL: none); int32, wrapping.
    const int32_t* acc_in; int64_t ld_acc;
    // MatMulInteger epilogue: Y = acc + cb[n]*rowsum[m] + ca[m]*(colsum[n] + K*cb[n])
    const void* b_zp; int b_zp_stride; int b_zp_u8;  // NULL means zero
    int32_t ca;   // (128 if A is uint8 else 0) - a_zero_point, when a_zp is NULL
    int32_t sb;   // 128 if B is uint8 else 0; cb[n] = sb - b_zp[n]
    // Per-row activation zero points (NULL: the scalar ca above):
    // ca[m] = sa - a_zp[(m % a_zp_rows) * a_zp_stride]
    const void* a_zp; int a_zp_stride; int a_zp_rows; int a_zp_u8; int32_t sa;
    // split-K workspace (skinny kernel): counters then int32 partials
    void* workspace;
    int splits;
    int split_steps;   // skinny kernel: 64-row steps per split (multiple of 8)
    int stage_out;     // tiled kernel: 0 stores from the fragments; 1 / 2 writes the
                       // output tile through LDS in whole rows, plain / non-temporal
};

// Tile configurations of the int8 GEMM kernels.
enum TileCfg {
    TILE_256x256 = 0,     // four waves of 128x128, four LDS stages
    TILE_256x128_S3 = 1,  // four waves of 128x64, three stages (two workgroups per CU)
    TILE_128x128 = 2,     // four waves of 64x64, four stages (two workgroups per CU)
    TILE_128x128_S3 = 3,  // four waves of 64x64, three stages (three workgroups per CU)
    TILE_256x256_W8 = 4,  // eight waves of 128x64, four stages
    TILE_256x128_W8 = 5,  // eight waves of 64x64, four stages
    TILE_128x128_K128 = 6,     // four waves of 64x64, 128-byte k stages, two stages
    TILE_256x128_W8_K128 = 7,  // eight waves of 64x64, 128-byte k stages, three stages
    TILE_256x256_W8_K128 = 8,  // eight waves of 128x64, 128-byte k stages, two stages
    TILE_64x128_K128 = 9,      // four waves of 32x64, 128-byte k stages, two stages
    NUM_TILE_CFGS = 10
};

// Register-staged kernel, one launcher per tile shape.  bkm: B is [N,K];
// vec: 16-byte vector loads allowed (only the 128x128 shape has byte-wise
// variants); epi: Int8Epilogue; zp bit 0: row sums of A, bit 1: column sums.
hipError_t launch_tiled_256x256(const Int8GemmArgs& a, bool bkm, bool vec, int epi, int zp, hipStream_t s);
hipError_t launch_tiled_256x128(const Int8GemmArgs& a, bool bkm, bool vec, int epi, int zp, hipStream_t s);
hipError_t launch_tiled_128x128(const Int8GemmArgs& a, bool bkm, bool vec, int epi, int zp, hipStream_t s);

// Multi-stage kernel fed by direct global-to-LDS loads, one launcher per
// configuration.  Needs 16-byte aligned rows; K a multiple of the stage's
// k-bytes (64, or 128 for the *_K128 configurations) when an operand is uint8
// or a zero-point sum is taken, or when B is [N,K].
hipError_t launch_dma_256x256(const Int8GemmArgs& a, bool bkm, int epi, int zp, hipStream_t s);
hipError_t launch_dma_256x128s3(const Int8GemmArgs& a, bool bkm, int epi, int zp, hipStream_t s);
hipError_t launch_dma_128x128(const Int8GemmArgs& a, bool bkm, int epi, int zp, hipStream_t s);
hipError_t launch_dma_128x128s3(const Int8GemmArgs& a, bool bkm, int epi, int zp, hipStream_t s);
hipError_t launch_dma_256x256w8(const Int8GemmArgs& a, bool bkm, int epi, int zp, hipStream_t s);
hipError_t launch_dma_256x128w8(const Int8GemmArgs& a, bool bkm, int epi, int zp, hipStream_t s);
hipError_t launch_dma_128x128k128(const Int8GemmArgs& a, bool bkm, int epi, int zp, hipStream_t s);
// The same tile with three stages, split over K when a.splits > 1 (a.splits,
// a.split_steps, a.workspace): A8W8, or MatMulInteger (epi EPI_I32, zp sums).
hipError_t launch_dma_128x128k128_split(const Int8GemmArgs& a, bool bkm, int epi, int zp, hipStream_t s);
hipError_t launch_dma_256x128w8k128(const Int8GemmArgs& a, bool bkm, int epi, int zp, hipStream_t s);
hipError_t launch_dma_256x256w8k128(const Int8GemmArgs& a, bool bkm, int epi, int zp, hipStream_t s);
hipError_t launch_dma_64x128k128(const Int8GemmArgs& a, bool bkm, int epi, int zp, hipStream_t s);
// Three stages of it, split over K when a.splits > 1 (at most 64 rows: the
// 128x128 split plan's tile count and workspace hold).
hipError_t launch_dma_64x128k128_split(const Int8GemmArgs& a, bool bkm, int epi, int zp, hipStream_t s);

// Skinny kernel for M <= 16 (A8W8 only, B is [K,N]); splits > 1 needs workspace.
// The split-K workspace starts with a ticket header of fixed size (one int
// per 256-column tile, at most SKINNY_MAX_TICKETS tiles); shapes with more
// column tiles run one split (they fill the chip without splitting K).
constexpr int SKINNY_MAX_TICKETS = 256;
constexpr size_t SKINNY_TICKET_BYTES = SKINNY_MAX_TICKETS * 4;
// Library-held split-K scratch for the workspace-free entry point: the ticket
// header plus 8 MiB of partial sums (every shape the default plan splits
// needs at most 510 column-tile slabs of 16 KiB: 8,356,864 bytes in all).
constexpr size_t SKINNY_SCRATCH_BYTES = SKINNY_TICKET_BYTES + ((size_t)8 << 20);
// The current device's copy of that scratch; the first call on a device
// looks it up and clears its tickets with a kernel on `s`.
hipError_t skinny_scratch(hipStream_t s, void** ptr);
// epi EPI_F32 / EPI_BF16: A8W8; EPI_I32: MatMulInteger (16-byte rows, K a
// multiple of 64, flips and zero points as in the tiled kernels).
// bkm: A8W8 with W as [N,K] (vec only).
hipError_t launch_a8w8_skinny(const Int8GemmArgs& a, bool vec, int epi, hipStream_t s,
                              const char** name, bool bkm = false);
// sums: MatMulInteger partials, which carry row and column sums too
size_t skinny_workspace_bytes(int M, int N, int splits, bool sums = false);

// Column-slab A8W8 kernel for decode rows with W as [N,K] (each workgroup
// owns tn output columns over all of K, no workspace): M <= SLAB_MAX_M,
// 16-byte aligned rows, K % 16 == 0; tn is 16 or 32.
constexpr int SLAB_MAX_M = 16;
bool slab_shape_ok(const Int8GemmArgs& a, int tn);
hipError_t launch_a8w8_slab(const Int8GemmArgs& a, int tn, int epi, hipStream_t s, const char** name);
int skinny_splits(int M, int N, int K);
int skinny_split_steps(int N, int K);
int skinny_splits_for(int N, int K, int split_steps);

// W8A32: C = scale * (A @ W - zp * rowsum(A)) with fp32 matrix cores.
struct W8A32Args {
    int M, N, K;
    const float* A; int64_t lda;
    const int8_t* W; int64_t ldw;
    float scale; int32_t zp;
    float* C; int64_t ldc;
    // split of the contraction (bf16 split kernel, 128x128 tiles): `splits`
    // ranges of split_k values (a multiple of 32), partials in `workspace`
    void* workspace; int splits; int split_k;
};
// wt: W is [N,K] (rows of the contraction), the input-gradient form.
hipError_t launch_w8a32(const W8A32Args& a, bool vec_a, bool vec_w, bool wt, hipStream_t s,
                        const char** name);
// The same operation on the bf16 matrix cores, with the fp32 operand split
// exactly into three bf16 parts.
// Split of the contraction for the 128x128 tiles of the bf16 split kernel
// (splits = 1: none): outputs of at most 256 such tiles, up to 8 splits of at
// least 512 values, about two workgroups per CU; forced > 0 asks for that
// many.  M x N outputs, K the contraction, lda the row stride of the fp32
// operand.
void w8a32_split_plan(int64_t M, int64_t N, int64_t K, int64_t lda, int forced, int* splits, int* split_k);
size_t w8a32_split_bytes(int64_t M, int64_t N, int splits);
// Decode-shaped W8A32 (M <= SKINNY_W8A32_MAX_M in blocks of 16 rows, 16-byte
// aligned rows, K % 4 == 0; wt: the
// input gradient, W as [outputs][contraction]): 256-output tiles x splits of
// the contraction (split_k a multiple of 512); the plan gives about one
// workgroup per CU (forced > 0: that many splits).
constexpr int SKINNY_W8A32_MAX_M = 64;   // blocks of 16 rows on the grid's third dimension
void w8a32_skinny_plan(int64_t M, int64_t N, int64_t K, int forced, int* splits, int* split_k);
size_t w8a32_skinny_bytes(int64_t M, int64_t N, int splits);
hipError_t launch_w8a32_skinny(const W8A32Args& a, bool wt, hipStream_t s, const char** name);
// Slab form of the W8A32 input gradient (kernel view: M <= 16 rows, N
// outputs = W's rows, contraction K along them; each workgroup owns 16 or 32
// outputs over all of K, no workspace): 16-byte aligned rows, lda % 4 == 0,
// ldw % 16 == 0, K % 4 == 0.
bool w8a32_grad_slab_ok(const W8A32Args& a);
hipError_t launch_w8a32_grad_slab(const W8A32Args& a, hipStream_t s, const char** name);
hipError_t launch_w8a32_split(const W8A32Args& a, bool vec_a, bool vec_w, bool wt, hipStream_t s,
                              const char** name);

// ConvInteger staging: geometry of one call (validated on the host).
// Kg = Cg*kH*kW, Kp = Kg rounded up to 64, P = OH*OW, Pp = P rounded up to 16.
struct ConvGeom {
    int N, C, H, W, M, kH, kW, group, Cg, Mg, Kg, Kp, OH, OW, P, Pp;
    int pt, pl, sh, sw, dh, dw;
};
// Packs w into [group][Mg][Kp] at wp and writes the column matrices
// [N][group][Kp][Pp] at col (both in the caller's workspace).
hipError_t launch_conv_stage(const ConvGeom& c, const void* x, uint8_t x_zp, const void* w, const void* w_zp,
                             int w_zp_len, uint8_t* wp, uint8_t* col, hipStream_t s);

// ConvInteger as an implicit GEMM (no column matrix): the tiling and the
// workspace layout of one call.  Eligible when Cg is a multiple of 64, there
// are at most 9 taps and a tile's weights and input halo fit in LDS.
struct ConvImplicitPlan {
    int BM;              // output channels per tile (64 or 128)
    int BW, BH;          // output tile: BH rows x BW columns (NPOS positions)
    int NPOS;            // positions per tile: 128 or 256
    int TH, TWt;         // output tiles down / across
    int HP, WP;          // rows / columns of the padded input xp
    int Cgp, taps, cblks;
    int HR, HC;          // halo rows / columns one tile reads
    int a_pitch;         // LDS bytes per weight row (taps*64, padded to 64 mod 256)
    int h_rounds;        // 4 KiB load rounds of the halo
    int lds_bytes;
    int64_t Kt;          // packed weight row bytes: Cgp * taps
    size_t wp_off, rs_off, xp_off, total;   // packed weights, row sums, xp
};
bool conv_implicit_plan(const ConvGeom& c, ConvImplicitPlan* p);
// fused: one launch that stages x and w itself (no workspace used); needs
// conv_fused_ok (rows of x 16-byte aligned, w 4-byte aligned).
bool conv_fused_ok(const ConvGeom& c, const ConvImplicitPlan& p, const void* x, const void* w);
hipError_t launch_conv_implicit(const ConvGeom& c, const ConvImplicitPlan& p, const void* x, bool x_u8, int x_zp,
                                const void* w, bool w_u8, const void* w_zp, int w_zp_len, void* ws, int32_t* y,
                                bool fused, hipStream_t s);

// DynamicQuantizeLinear (uint8): a min/max pass writing one (min, max)
// float pair per workgroup into the workspace, then a quantize pass.
constexpr int DQL_MAX_PARTIALS = 256;
int dql_partials(int64_t n);
hipError_t launch_dynamic_quantize(const float* x, int64_t n, uint8_t* y, float* y_scale, uint8_t* y_zp,
                                   void* workspace, bool vec, hipStream_t s);

// Calibration kernels (roofline ceilings; no part of the method).  Each
// writes one word per wave: CALIB_*_BLOCKS * 4 words of sink.
constexpr int CALIB_READ_BLOCKS = 2048;
constexpr int CALIB_MFMA_BLOCKS = 2048;
hipError_t launch_calib_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t s);
hipError_t launch_calib_mfma(const void* ops, int iters, uint32_t* sink, hipStream_t s);
hipError_t launch_calib_mfma_f32(const void* ops, int iters, uint32_t* sink, hipStream_t s);
hipError_t launch_calib_mfma_bf16(const void* ops, int iters, uint32_t* sink, hipStream_t s);
hipError_t launch_calib_mfma32(const void* ops, int iters, uint32_t* sink, hipStream_t s);

}  // namespace qg

// C-ABI entry points: argument validation (before any HIP call), kernel
// selection, launch, and the launch-status convention of
// "feat(onnx-to-hip): lower quantized integer conv and matmul" ("What", last
// paragraph): clear the pending HIP error, launch, return hipGetLastError().
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include <hip/hip_runtime.h>

#include "../../include/qgemm.h"
#include "kernels.h"

namespace {

thread_local const char* g_last_kernel = "";

constexpr int64_t SPAN_LIMIT = (int64_t)1 << 31;  // 32-bit buffer offsets
constexpr int SKINNY_MAX_M = 16;

bool env_is(const char* name, const char* value) {
    const char* v = std::getenv(name);
    return v != nullptr && std::strcmp(v, value) == 0;
}

int env_int(const char* name, int dflt) {
    const char* v = std::getenv(name);
    return v != nullptr && *v ? std::atoi(v) : dflt;
}

// W8A32 runs on the bf16 matrix cores with the exact three-way split of its
// fp32 operand unless QGEMM_W8A32=fp32 asks for the fp32 matrix cores.
bool w8a32_split() { return !env_is("QGEMM_W8A32", "fp32"); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

void log_dispatch(const char* op, const char* kernel, int64_t batch, int64_t M, int64_t N, int64_t K,
                  int extra) {
    if (env_is("QGEMM_LOG_DISPATCH", "1"))
        std::fprintf(stderr, "[qgemm] %s -> %s batch=%lld M=%lld N=%lld K=%lld splits=%d\n", op, kernel,
                     (long long)batch, (long long)M, (long long)N, (long long)K, extra);
}

bool dims_ok(int64_t M, int64_t N, int64_t K) {
    const int64_t lim = (int64_t)1 << 30;
    return M >= 1 && N >= 1 && K >= 1 && M < lim && N < lim && K < lim;
}

// An output with no elements (rows, cols or batch zero, none negative or
// past the limits): the call has nothing to compute, launches nothing and
// returns QG_OK; its pointers may be NULL.
bool empty_output(int64_t rows, int64_t cols, int64_t inner, int64_t batch = 1) {
    const int64_t lim = (int64_t)1 << 30;
    if (rows < 0 || cols < 0 || inner < 0 || batch < 0) return false;
    if (rows >= lim || cols >= lim || inner >= lim || batch >= 65536) return false;
    return rows == 0 || cols == 0 || batch == 0;
}

// Tile configuration of the int8 GEMM for an (effective) problem shape:
// large tiles when there are enough of them to fill the chip, smaller tiles
// (several workgroups per compute unit) otherwise.  QGEMM_TILE forces one.
int pick_tile(int64_t batch, int64_t M, int64_t N, int64_t K) {
    const int forced = env_int("QGEMM_TILE", -1);
    if (forced >= 0 && forced < qg::NUM_TILE_CFGS) return forced;
    // 256x256 tiles (eight waves, 128-byte k stages, one workgroup per
    // compute unit) from 160 of them on; measured best for 8192^3 (3-4 %
    // ahead of the same tile with 64-byte stages) and, A8W8 bf16 event-timed,
    // for one round of 160-256 tiles (2560x4096x4096 47.6 against 54.1 us on
    // 128x128 tiles, 4096^3 59.3 / 73.1, 2048x8192x8192 109.2 / 135.5,
    // 4096x4096x1024 22.1 / 23.4) and for 384-511 (6144x4096x4096 100.2 /
    // 108.1).  A second round at most 3/8 full loses (5120x4096x4096, 320
    // tiles: 97.1 against 92.6 us), as does a first round of at most 128
    // tiles (2048x4096x4096: 48.0 / 38.2).  Otherwise 128x128 tiles with
    // 128-byte k stages, two workgroups per compute unit (best for
    // 4096x2048x2048 and smaller).  Either falls back to its 64-byte-stage
    // sibling where K is not whole 128-byte stages and bytes past K would
    // reach a sum.
    const int64_t t256 = batch * ((M + 255) / 256) * ((N + 255) / 256);
    if (t256 >= 512 || (t256 >= 160 && !(t256 > 256 && t256 <= 352))) return qg::TILE_256x256_W8_K128;
    // At most 256 tiles of 128 x 128 over K <= 2048: 64x128 tiles, twice the
    // workgroups with half the multiplies each between first load and last
    // store.  A8W8 bf16, graph-timed with the operands cached: 256 / 1024 /
    // 2048 x 1024 x 1024 6.2 / 6.3 / 6.7 against 8.0 / 8.1 / 8.2 us, 256 /
    // 1024 / 2048 x 2048 x 2048 9.0 / 9.4 / 12.6 against 11.8 / 13.7 / 14.2
    // (split or three-stage 128x128 tiles); from 512 tiles or a longer K it
    // loses (4096x2048x2048 26.6 against 19.3, 64x8192x8192 39.9 against
    // 19.9 split).
    const int64_t t128 = batch * ((M + 127) / 128) * ((N + 127) / 128);
    if (K <= 2048 && t128 <= 256) return qg::TILE_64x128_K128;
    return qg::TILE_128x128_K128;
}

// How the multi-stage kernel writes its output tile: 0 straight from the
// fragments (less latency), 1 through LDS in whole rows with plain stores
// (large grids), 2 through LDS with non-temporal stores (single-round
// grids).  QGEMM_STAGE=0/1/2 forces the choice.
int stage_output(int cfg, int64_t K, int epi) {
    const int forced = env_int("QGEMM_STAGE", -1);
    if (forced >= 0 && forced <= 2) return forced;
    // 256x256 tiles: plain row stores for bf16 output (8192^3: 407.7 us
    // against 414.0 non-temporal), non-temporal ones for fp32, whose output
    // is twice the bytes (447.6 -> 427.8 us).
    if (cfg == qg::TILE_256x256 || cfg == qg::TILE_256x256_W8 || cfg == qg::TILE_256x256_W8_K128)
        return epi == qg::EPI_F32 ? 2 : 1;
    // Smaller tiles: staged non-temporal rows once the main loop is long
    // enough to absorb the staging barriers (MatMulInteger 8x512x2048x2048:
    // 29.5 -> 27.6 us; A8W8 4096x2048x2048 bf16: 28.9 -> 22.9 us); straight
    // fragment stores for short K (a K = 576 convolution: 37.8 us against 39.3).
    return K >= 1024 ? 2 : 0;
}

qg_status empty_call() {
    g_last_kernel = "none";
    return QG_OK;
}

qg_status finish_launch(hipError_t e, const char* name) {
    if (e != hipSuccess) return QG_ERR_HIP;
    g_last_kernel = name;
    return QG_OK;
}

// The multi-stage direct-to-LDS kernel takes every 16-byte-aligned shape
// except those whose bytes past K would reach a sum: uint8 flips, zero-point
// sums and a k-major B need K % 64 == 0.  Everything else runs the
// register-staged kernel, which clears bytes past K itself.
bool dma_ok(const qg::Int8GemmArgs& a, bool bkm, bool vec, int epi, int bk) {
    if (!vec || env_is("QGEMM_FAMILY", "staged")) return false;
    const bool needs_whole_chunks = bkm || epi == qg::EPI_I32;
    return !needs_whole_chunks || a.K % bk == 0;
}

bool is_k128(int cfg) {
    return cfg == qg::TILE_128x128_K128 || cfg == qg::TILE_256x128_W8_K128 || cfg == qg::TILE_256x256_W8_K128 ||
           cfg == qg::TILE_64x128_K128;
}

// The 64-byte-stage configuration of the same tile shape (of the nearest
// shape that has one, for 64x128).
int k64_of(int cfg) {
    switch (cfg) {
        case qg::TILE_128x128_K128: return qg::TILE_128x128;
        case qg::TILE_64x128_K128: return qg::TILE_128x128;
        case qg::TILE_256x128_W8_K128: return qg::TILE_256x128_W8;
        case qg::TILE_256x256_W8_K128: return qg::TILE_256x256_W8;
        default: return cfg;
    }
}

hipError_t launch_tiled(const qg::Int8GemmArgs& a, int cfg, bool bkm, bool vec, int epi, int zp,
                        hipStream_t s, const char** name) {
    static const char* dma_names[qg::NUM_TILE_CFGS] = {
        "int8_dma_256x256", "int8_dma_256x128s3", "int8_dma_128x128",
        "int8_dma_128x128s3", "int8_dma_256x256w8", "int8_dma_256x128w8",
        "int8_dma_128x128k128", "int8_dma_256x128w8k128", "int8_dma_256x256w8k128", "int8_dma_64x128k128"};
    // A 128-byte-stage configuration whose K is not whole stages, where bytes
    // past K would reach a sum, runs its 64-byte-stage sibling.
    if (is_k128(cfg) && !dma_ok(a, bkm, vec, epi, 128) && dma_ok(a, bkm, vec, epi, 64)) cfg = k64_of(cfg);
    if (dma_ok(a, bkm, vec, epi, is_k128(cfg) ? 128 : 64)) {
        *name = dma_names[cfg];
        qg::Int8GemmArgs d = a;
        d.stage_out = stage_output(cfg, a.K, epi);
        switch (cfg) {
            case qg::TILE_256x256: return qg::launch_dma_256x256(d, bkm, epi, zp, s);
            case qg::TILE_256x128_S3: return qg::launch_dma_256x128s3(d, bkm, epi, zp, s);
            case qg::TILE_128x128: return qg::launch_dma_128x128(d, bkm, epi, zp, s);
            case qg::TILE_128x128_S3: return qg::launch_dma_128x128s3(d, bkm, epi, zp, s);
            case qg::TILE_256x256_W8: return qg::launch_dma_256x256w8(d, bkm, epi, zp, s);
            case qg::TILE_128x128_K128: return qg::launch_dma_128x128k128(d, bkm, epi, zp, s);
            case qg::TILE_256x128_W8_K128: return qg::launch_dma_256x128w8k128(d, bkm, epi, zp, s);
            case qg::TILE_256x256_W8_K128: return qg::launch_dma_256x256w8k128(d, bkm, epi, zp, s);
            case qg::TILE_64x128_K128: return qg::launch_dma_64x128k128(d, bkm, epi, zp, s);
            default: return qg::launch_dma_256x128w8(d, bkm, epi, zp, s);
        }
    }
    // Register-staged kernel: the byte-wise (any alignment) variants exist
    // for the 128x128 tile only.
    int shape = cfg == qg::TILE_256x256 || cfg == qg::TILE_256x256_W8 || cfg == qg::TILE_256x256_W8_K128 ? 0
              : cfg == qg::TILE_256x128_S3 || cfg == qg::TILE_256x128_W8 || cfg == qg::TILE_256x128_W8_K128 ? 1 : 2;
    if (!vec) shape = 2;
    static const char* staged_names[] = {"int8_staged_256x256", "int8_staged_256x128", "int8_staged_128x128"};
    *name = staged_names[shape];
    switch (shape) {
        case 0: return qg::launch_tiled_256x256(a, bkm, vec, epi, zp, s);
        case 1: return qg::launch_tiled_256x128(a, bkm, vec, epi, zp, s);
        default: return qg::launch_tiled_128x128(a, bkm, vec, epi, zp, s);
    }
}

}  // namespace

extern "C" {

const char* qgemm_version(void) { return "qgemm 0.1 (gfx950)"; }

qg_status qgemm_calib_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
    static_assert(qg::CALIB_READ_BLOCKS * 4 == QG_CALIB_SINK_WORDS, "sink size");
    if (buf == nullptr || sink == nullptr || bytes == 0 || bytes % 16 != 0 ||
        (reinterpret_cast<uintptr_t>(buf) & 15) != 0)
        return QG_ERR_INVALID_ARGUMENT;
    (void)hipGetLastError();
    return finish_launch(qg::launch_calib_read(buf, bytes, sink, (hipStream_t)stream), "calib_read");
}

qg_status qgemm_calib_mfma_i8(const void* operands, int iters, uint32_t* sink, void* stream,
                              int64_t* ops_out) {
    static_assert(qg::CALIB_MFMA_BLOCKS * 4 == QG_CALIB_SINK_WORDS, "sink size");
    static_assert((int64_t)qg::CALIB_MFMA_BLOCKS * 4 * 16 * 32768 == QG_CALIB_MFMA_OPS_PER_ROUND, "ops");
    if (operands == nullptr || sink == nullptr || iters < 1 || iters > (1 << 20) || ops_out == nullptr)
        return QG_ERR_INVALID_ARGUMENT;
    *ops_out = QG_CALIB_MFMA_OPS_PER_ROUND * (int64_t)iters;
    (void)hipGetLastError();
    return finish_launch(qg::launch_calib_mfma(operands, iters, sink, (hipStream_t)stream), "calib_mfma_i8");
}

qg_status qgemm_calib_mfma_i8_32x32(const void* operands, int iters, uint32_t* sink, void* stream,
                                    int64_t* ops_out) {
    if (operands == nullptr || sink == nullptr || iters < 1 || iters > (1 << 20) || ops_out == nullptr)
        return QG_ERR_INVALID_ARGUMENT;
    *ops_out = QG_CALIB_MFMA_OPS_PER_ROUND * (int64_t)iters;
    (void)hipGetLastError();
    return finish_launch(qg::launch_calib_mfma32(operands, iters, sink, (hipStream_t)stream),
                         "calib_mfma_i8_32x32");
}

qg_status qgemm_calib_mfma_f32(const void* operands, int iters, uint32_t* sink, void* stream,
                               int64_t* flops_out) {
    static_assert((int64_t)qg::CALIB_MFMA_BLOCKS * 4 * 16 * 2048 == QG_CALIB_MFMA_F32_FLOPS_PER_ROUND, "flops");
    if (operands == nullptr || sink == nullptr || iters < 1 || iters > (1 << 20) || flops_out == nullptr)
        return QG_ERR_INVALID_ARGUMENT;
    *flops_out = QG_CALIB_MFMA_F32_FLOPS_PER_ROUND * (int64_t)iters;
    (void)hipGetLastError();
    return finish_launch(qg::launch_calib_mfma_f32(operands, iters, sink, (hipStream_t)stream), "calib_mfma_f32");
}

qg_status qgemm_calib_mfma_bf16(const void* operands, int iters, uint32_t* sink, void* stream,
                                int64_t* flops_out) {
    static_assert((int64_t)qg::CALIB_MFMA_BLOCKS * 4 * 16 * 16384 == QG_CALIB_MFMA_BF16_FLOPS_PER_ROUND, "flops");
    if (operands == nullptr || sink == nullptr || iters < 1 || iters > (1 << 20) || flops_out == nullptr)
        return QG_ERR_INVALID_ARGUMENT;
    *flops_out = QG_CALIB_MFMA_BF16_FLOPS_PER_ROUND * (int64_t)iters;
    (void)hipGetLastError();
    return finish_launch(qg::launch_calib_mfma_bf16(operands, iters, sink, (hipStream_t)stream), "calib_mfma_bf16");
}

const char* qgemm_last_kernel(void) { return g_last_kernel; }

const char* qgemm_status_string(qg_status s) {
    switch (s) {
        case QG_OK: return "ok";
        case QG_ERR_INVALID_ARGUMENT: return "invalid argument";
        case QG_ERR_UNSUPPORTED: return "unsupported";
        case QG_ERR_WORKSPACE: return "workspace too small";
        case QG_ERR_HIP: return "HIP launch error";
    }
    return "unknown status";
}

// Splits of K for the decode kernel, and the steps each split covers.
// QGEMM_SPLITS asks for a split count (tests and tuning).
static void a8w8_skinny_plan(int64_t M, int64_t N, int64_t K, int* splits, int* steps) {
    (void)M;
    const int forced = env_int("QGEMM_SPLITS", 0);
    int per = qg::skinny_split_steps((int)N, (int)K);
    if (forced > 0) {
        const int total = (int)((K + 63) / 64);
        per = (total + forced - 1) / forced;
        per = ((per + 7) / 8) * 8;
    }
    *steps = per;
    *splits = qg::skinny_splits_for((int)N, (int)K, per);
    // More column tiles than the fixed ticket header holds: one split over
    // all of K (the natural plan already gives one split from 256 tiles on).
    if (*splits > 1 && (N + 255) / 256 > qg::SKINNY_MAX_TICKETS) {
        *steps = (int)(((K + 63) / 64 + 7) / 8) * 8;
        *splits = 1;
    }
}

static int a8w8_skinny_splits(int64_t M, int64_t N, int64_t K) {
    int s, per;
    a8w8_skinny_plan(M, N, K, &s, &per);
    return s;
}

static bool a8w8_is_skinny(int64_t M, int b_trans) {
    if (env_is("QGEMM_FORCE_KERNEL", "tiled")) return false;
    if (env_is("QGEMM_FORCE_KERNEL", "skinny")) return !b_trans && M <= SKINNY_MAX_M;
    return !b_trans && M <= SKINNY_MAX_M;
}

// Column slabs for W as [N,K] (each workgroup owns tn output columns over all
// of K: whole weight lines per workgroup and no split-K exchange): the slab
// width for a decode-shaped product, or 0 when it does not take this kernel.
// It needs N / 16 >= 256 workgroups to occupy the chip; 16-column slabs up
// to 8 rows or below N = 8192, 32-column slabs (A fragments reused over two
// column fragments) otherwise.  QGEMM_FORCE_KERNEL=slab takes it whenever
// the shape allows, =skinny or =tiled never; QGEMM_SLAB_TN picks the width.
static int slab_width(const qg::Int8GemmArgs& a, bool b_trans) {
    if (!b_trans || env_is("QGEMM_FORCE_KERNEL", "tiled") || env_is("QGEMM_FORCE_KERNEL", "skinny")) return 0;
    const int forced = env_int("QGEMM_SLAB_TN", 0);
    const int tn = forced > 0 ? forced : ((a.M <= 8 || a.N < 8192) ? 16 : 32);
    if (!qg::slab_shape_ok(a, tn)) return 0;
    if (env_is("QGEMM_FORCE_KERNEL", "slab")) return tn;
    return a.N >= 16 * 256 ? tn : 0;
}

// Split of K for the tiled A8W8 kernel (128x128 tiles, 128-byte stages):
// an output of at most 128 tiles leaves most of the 256 CUs idle, so K is cut
// into up to 8 splits of at least 1024 rows (whole stages) that together
// give about one workgroup per CU.  max_splits caps the count (the static
// scratch of the workspace-free entry point); QGEMM_TILE_SPLITS asks for one.
static void a8w8_tiled_split_plan(int64_t M, int64_t N, int64_t K, int max_splits, int* splits, int* steps) {
    *splits = 1;
    *steps = 0;
    const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
    if (tiles > qg::SKINNY_MAX_TICKETS / 2) return;
    int64_t S = env_int("QGEMM_TILE_SPLITS", 0);
    if (S <= 0) S = std::min<int64_t>(std::min<int64_t>(256 / tiles, K / 1024), 8);
    S = std::min<int64_t>(S, max_splits);
    if (S < 2) return;
    const int64_t stages = (K + 127) / 128;
    const int64_t per = (stages + S - 1) / S;
    const int64_t n = (stages + per - 1) / per;
    if (n < 2) return;
    *splits = (int)n;
    *steps = (int)(per * 2);
}

static size_t a8w8_tiled_split_bytes(int64_t M, int64_t N, int splits) {
    if (splits <= 1) return 0;
    const size_t tiles = (size_t)((M + 127) / 128) * (size_t)((N + 127) / 128);
    return qg::SKINNY_TICKET_BYTES + tiles * (size_t)splits * 128 * 128 * 4;
}

// MatMulInteger rows (batches folded) that the decode kernel takes when a
// workspace is given: at most 16, over whole 64-row steps of K.
static bool mmi_is_skinny(int64_t M, int64_t K) {
    return a8w8_is_skinny(M, 0) && K % 64 == 0;
}

// MatMulInteger's split partials: the tile plus each lane's row and column
// sums (4 + 4 ints for 64x64 waves: 8 KiB per 128x128 tile).
static size_t mmi_tiled_split_bytes(int64_t M, int64_t N, int splits) {
    if (splits <= 1) return 0;
    const size_t tiles = (size_t)((M + 127) / 128) * (size_t)((N + 127) / 128);
    return qg::SKINNY_TICKET_BYTES + tiles * (size_t)splits * (128 * 128 * 4 + 8192);
}

// The W8A32 decode kernel's shapes (the kernel's view: M x N outputs,
// contraction K): the bf16 split path, at most 64 rows, 16-byte aligned
// operand rows; the forward also needs N % 16 == 0 (its weight rows are
// read 16 outputs at a time).  QGEMM_FORCE_KERNEL=tiled turns it off.
static bool w8a32_skinny_ok(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* W, int64_t ldw,
                            bool wt) {
    if (!w8a32_split() || M > qg::SKINNY_W8A32_MAX_M || env_is("QGEMM_FORCE_KERNEL", "tiled")) return false;
    const bool no_ptrs = A == nullptr && W == nullptr;   // sizing only (qgemm_workspace_bytes)
    return (no_ptrs || (aligned16(A) && aligned16(W))) && lda % 4 == 0 && K % 4 == 0 && ldw % 16 == 0 &&
           (wt || N % 16 == 0);
}

// The input gradient's slab form (each workgroup owns 32 outputs, i.e. W
// rows, over the whole contraction; no workspace) for at most 8 rows across
// at least 8192 outputs.  Graph-timed at N = K = 8192: 17.3 / 17.4 / 18.7 /
// 20.6 us at M = 1 / 2 / 4 / 8 against 20.8 / 21.3 at M = 1 / 4 on the
// split decode kernel; at 16 rows 25.7 against 23.1 (every workgroup reads
// and splits all of dC).  QGEMM_FORCE_KERNEL=slab takes it whenever the shape allows.
static bool w8a32_grad_slab(const qg::W8A32Args& a) {
    if (!w8a32_split() || env_is("QGEMM_FORCE_KERNEL", "tiled") || env_is("QGEMM_FORCE_KERNEL", "skinny")) return false;
    if (!qg::w8a32_grad_slab_ok(a)) return false;
    return env_is("QGEMM_FORCE_KERNEL", "slab") || (a.M <= 8 && a.N >= 8192);
}

size_t qgemm_workspace_bytes(int op, int64_t batch, int64_t M, int64_t N, int64_t K) {
    if (op == QG_OP_DYNAMIC_QUANTIZE_LINEAR) return N < 0 ? 0 : (size_t)qg::dql_partials(N) * 8;
    if (op == QG_OP_W8A32 || op == QG_OP_W8A32_INPUT_GRAD) {
        if (!dims_ok(M, N, K) || !w8a32_split()) return 0;
        // the kernel's view: the input gradient's outputs are dA's K columns
        const int64_t rows = M, outs = op == QG_OP_W8A32 ? N : K, red = op == QG_OP_W8A32 ? K : N;
        const int forced = env_int("QGEMM_W8A32_SPLITS", 0);
        int splits, split_k;
        qg::w8a32_split_plan(rows, outs, red, red, forced, &splits, &split_k);
        size_t bytes = qg::w8a32_split_bytes(rows, outs, splits);
        // decode shapes take the decode kernel when their rows are aligned,
        // the tiled one otherwise: enough for either
        const bool wt = op == QG_OP_W8A32_INPUT_GRAD;
        if (w8a32_skinny_ok(rows, outs, red, nullptr, red, nullptr, wt ? red : outs, wt)) {
            qg::w8a32_skinny_plan(rows, outs, red, forced, &splits, &split_k);
            bytes = std::max(bytes, qg::w8a32_skinny_bytes(rows, outs, splits));
        }
        return bytes;
    }
    if (op == QG_OP_MATMUL_INTEGER) {
        // sized for the batch folded into M (contiguous A / Y batches, shared B)
        if (batch < 1 || batch >= 65536 || !dims_ok(M, N, K) || batch * M >= ((int64_t)1 << 30)) return 0;
        int splits, steps;
        if (mmi_is_skinny(batch * M, K)) {
            a8w8_skinny_plan(batch * M, N, K, &splits, &steps);
            return qg::skinny_workspace_bytes((int)(batch * M), (int)N, splits, true);
        }
        if (K % 128 != 0) return 0;   // the split kernel's sums need whole 128-byte stages
        a8w8_tiled_split_plan(batch * M, N, K, 8, &splits, &steps);
        return mmi_tiled_split_bytes(batch * M, N, splits);
    }
    if (op != QG_OP_A8W8 || !dims_ok(M, N, K)) return 0;
    if (a8w8_is_skinny(M, 0)) return qg::skinny_workspace_bytes((int)M, (int)N, a8w8_skinny_splits(M, N, K));
    int splits, steps;
    a8w8_tiled_split_plan(M, N, K, 8, &splits, &steps);
    return a8w8_tiled_split_bytes(M, N, splits);
}

// W8A32 in the kernel's view: M x N outputs, contraction K (the input
// gradient passes dA's columns as N and the forward N as K).  A workspace
// lets the 128x128 split tiles divide the contraction among workgroups.
static qg_status w8a32_run(qg::W8A32Args& a, bool vec_a, bool vec_w, bool wt, void* workspace, size_t workspace_bytes,
                           void* stream, const char* op) {
    if (workspace != nullptr && (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return QG_ERR_INVALID_ARGUMENT;
    // At most 64 rows with 16-byte operand rows: the decode kernel (blocks
    // of 16 rows), the contraction split across workgroups when a workspace
    // is given.  Rows 17-64 measured against the split 128x128 tiles at
    // N = K = 8192: 25-38 against 96 us (forward), 34-57 against 98 us
    // (gradient); at 4096^2 12.6-16.6 against 33-36 us.
    if (wt && w8a32_grad_slab(a)) {
        const char* name = "";
        (void)hipGetLastError();
        const hipError_t e = qg::launch_w8a32_grad_slab(a, (hipStream_t)stream, &name);
        log_dispatch(op, name, 1, a.M, a.N, a.K, 1);
        return finish_launch(e, name);
    }
    if (w8a32_skinny_ok(a.M, a.N, a.K, a.A, a.lda, a.W, a.ldw, wt)) {
        int splits, split_k;
        qg::w8a32_skinny_plan(a.M, a.N, a.K, env_int("QGEMM_W8A32_SPLITS", 0), &splits, &split_k);
        if (workspace == nullptr) {
            qg::w8a32_skinny_plan(a.M, a.N, a.K, 1, &splits, &split_k);
        } else if (qg::w8a32_skinny_bytes(a.M, a.N, splits) > workspace_bytes) {
            return QG_ERR_WORKSPACE;
        }
        a.workspace = splits > 1 ? workspace : nullptr;
        a.splits = splits;
        a.split_k = split_k;
        const char* name = "";
        (void)hipGetLastError();
        const hipError_t e = qg::launch_w8a32_skinny(a, wt, (hipStream_t)stream, &name);
        log_dispatch(op, name, 1, a.M, a.N, a.K, splits);
        return finish_launch(e, name);
    }
    int splits = 1, split_k = 0;
    if (w8a32_split() && workspace != nullptr) {
        qg::w8a32_split_plan(a.M, a.N, a.K, a.lda, env_int("QGEMM_W8A32_SPLITS", 0), &splits, &split_k);
        if (qg::w8a32_split_bytes(a.M, a.N, splits) > workspace_bytes) return QG_ERR_WORKSPACE;
    }
    a.workspace = splits > 1 ? workspace : nullptr;
    a.splits = splits;
    a.split_k = split_k;
    const char* name = "";
    (void)hipGetLastError();
    const hipError_t e = w8a32_split() ? qg::launch_w8a32_split(a, vec_a, vec_w, wt, (hipStream_t)stream, &name)
                                         : qg::launch_w8a32(a, vec_a, vec_w, wt, (hipStream_t)stream, &name);
    log_dispatch(op, name, 1, a.M, a.N, a.K, splits);
    return finish_launch(e, name);
}

qg_status qgemm_w8a32_ws(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const int8_t* W,
                         int64_t ldw, float scale, int32_t zero_point, float* C, int64_t ldc, void* workspace,
                         size_t workspace_bytes, void* stream) {
    if (empty_output(M, N, K)) return empty_call();
    if (!dims_ok(M, N, K)) return QG_ERR_INVALID_ARGUMENT;
    if (A == nullptr || W == nullptr || C == nullptr) return QG_ERR_INVALID_ARGUMENT;
    if (lda < K || ldw < N || ldc < N) return QG_ERR_INVALID_ARGUMENT;
    if (!std::isfinite(scale)) return QG_ERR_INVALID_ARGUMENT;
    if ((K + 64) * ldw >= SPAN_LIMIT || (128 * lda + K + 64) * 4 >= SPAN_LIMIT) return QG_ERR_UNSUPPORTED;

    qg::W8A32Args a{};
    a.M = (int)M; a.N = (int)N; a.K = (int)K;
    a.A = A; a.lda = lda; a.W = W; a.ldw = ldw;
    a.scale = scale; a.zp = zero_point; a.C = C; a.ldc = ldc;
    const bool vec_a = aligned16(A) && lda % 4 == 0 && K % 4 == 0;
    const bool vec_w = (reinterpret_cast<uintptr_t>(W) & 3u) == 0 && ldw % 4 == 0 && N % 4 == 0;
    return w8a32_run(a, vec_a, vec_w, false, workspace, workspace_bytes, stream, "w8a32");
}

qg_status qgemm_w8a32(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const int8_t* W,
                      int64_t ldw, float scale, int32_t zero_point, float* C, int64_t ldc, void* stream) {
    return qgemm_w8a32_ws(M, N, K, A, lda, W, ldw, scale, zero_point, C, ldc, nullptr, 0, stream);
}

qg_status qgemm_w8a32_input_grad_ws(int64_t M, int64_t N, int64_t K, const float* dC, int64_t lddc,
                                    const int8_t* W, int64_t ldw, float scale, int32_t zero_point, float* dA,
                                    int64_t ldda, void* workspace, size_t workspace_bytes, void* stream) {
    if (empty_output(M, K, N)) return empty_call();      // dA is [M, K]; N is the reduction
    if (!dims_ok(M, N, K)) return QG_ERR_INVALID_ARGUMENT;
    if (dC == nullptr || W == nullptr || dA == nullptr) return QG_ERR_INVALID_ARGUMENT;
    if (lddc < N || ldw < N || ldda < K) return QG_ERR_INVALID_ARGUMENT;
    if (!std::isfinite(scale)) return QG_ERR_INVALID_ARGUMENT;
    if ((K + 256) * ldw >= SPAN_LIMIT || (128 * lddc + N + 64) * 4 >= SPAN_LIMIT) return QG_ERR_UNSUPPORTED;

    // The kernel's view: outputs = the K columns of dA, contraction = N.
    qg::W8A32Args a{};
    a.M = (int)M; a.N = (int)K; a.K = (int)N;
    a.A = dC; a.lda = lddc; a.W = W; a.ldw = ldw;
    a.scale = scale; a.zp = zero_point; a.C = dA; a.ldc = ldda;
    const bool vec_a = aligned16(dC) && lddc % 4 == 0 && N % 4 == 0;
    const bool vec_w = aligned16(W) && ldw % 16 == 0;
    return w8a32_run(a, vec_a, vec_w, true, workspace, workspace_bytes, stream, "w8a32_input_grad");
}

qg_status qgemm_w8a32_input_grad(int64_t M, int64_t N, int64_t K, const float* dC, int64_t lddc,
                                 const int8_t* W, int64_t ldw, float scale, int32_t zero_point, float* dA,
                                 int64_t ldda, void* stream) {
    return qgemm_w8a32_input_grad_ws(M, N, K, dC, lddc, W, ldw, scale, zero_point, dA, ldda, nullptr, 0, stream);
}

}  // extern "C"

namespace {

// A8W8 with an optional int32 accumulator input (acc_in == NULL: none).
// lib_scratch: the split-K workspace is the library's static scratch of the
// current device (workspace / workspace_bytes are ignored).
qg_status a8w8_impl(int64_t M, int64_t N, int64_t K, const int8_t* A, int64_t lda, const int8_t* W,
                    int64_t ldw, int b_trans, const int32_t* acc_in, int64_t ld_acc, const float* act_scale,
                    int64_t act_scale_len, const float* weight_scale, int64_t weight_scale_len, void* out,
                    qg_dtype out_dtype, int64_t ldo, void* workspace, size_t workspace_bytes, void* stream,
                    const char* op, bool lib_scratch = false) {
    if (empty_output(M, N, K)) return empty_call();
    if (!dims_ok(M, N, K)) return QG_ERR_INVALID_ARGUMENT;
    if (A == nullptr || W == nullptr || act_scale == nullptr || weight_scale == nullptr || out == nullptr)
        return QG_ERR_INVALID_ARGUMENT;
    if (b_trans != 0 && b_trans != 1) return QG_ERR_INVALID_ARGUMENT;
    if (lda < K || ldo < N || ldw < (b_trans ? K : N)) return QG_ERR_INVALID_ARGUMENT;
    if (act_scale_len != 1 && act_scale_len != M) return QG_ERR_INVALID_ARGUMENT;
    if (weight_scale_len != 1 && weight_scale_len != N) return QG_ERR_INVALID_ARGUMENT;
    if (out_dtype != QG_FP32 && out_dtype != QG_BF16) return QG_ERR_INVALID_ARGUMENT;
    // The decode kernel's tickets take atomics and its partials 16-byte
    // coherent stores: a workspace must start on a 256-byte boundary.
    if (!lib_scratch && workspace != nullptr && (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return QG_ERR_INVALID_ARGUMENT;
    if (256 * lda + K + 256 >= SPAN_LIMIT || (b_trans ? 256 * ldw + K + 256 : (K + 256) * ldw) >= SPAN_LIMIT)
        return QG_ERR_UNSUPPORTED;

    qg::Int8GemmArgs a{};
    a.M = (int)M; a.N = (int)N; a.K = (int)K; a.batch = 1;
    a.A = A; a.lda = lda; a.a_bstride = 0;
    a.B = W; a.ldb = ldw; a.b_bstride = 0;
    a.a_flip = 0; a.b_flip = 0;
    a.out = out; a.ldo = ldo; a.o_bstride = 0;
    a.act_scale = act_scale; a.as_stride = act_scale_len == 1 ? 0 : 1;
    a.weight_scale = weight_scale; a.ws_stride = weight_scale_len == 1 ? 0 : 1;
    a.acc_in = acc_in; a.ld_acc = ld_acc;
    const int epi = out_dtype == QG_FP32 ? qg::EPI_F32 : qg::EPI_BF16;
    const bool vec = aligned16(A) && aligned16(W) && lda % 16 == 0 && ldw % 16 == 0 && K % 16 == 0 &&
                     (b_trans || N % 16 == 0);

    const char* name = "";
    hipError_t e;
    // Decode rows with W as [N,K] across a wide N: column slabs, no workspace.
    if (const int tn = slab_width(a, b_trans != 0)) {
        (void)hipGetLastError();
        e = qg::launch_a8w8_slab(a, tn, epi, (hipStream_t)stream, &name);
        log_dispatch(op, name, 1, M, N, K, 1);
        return finish_launch(e, name);
    }
    // Decode shapes: W as [K,N], or as [N,K] with 16-byte aligned rows (each
    // weight row then already holds its column's k-bytes).
    const bool skinny_bkm = b_trans != 0 && vec && a8w8_is_skinny(M, 0);
    if (a8w8_is_skinny(M, b_trans) || skinny_bkm) {
        int splits, per;
        a8w8_skinny_plan(M, N, K, &splits, &per);
        const size_t need = qg::skinny_workspace_bytes((int)M, (int)N, splits);
        if (lib_scratch) {
            workspace = nullptr;
            if (need > qg::SKINNY_SCRATCH_BYTES) return QG_ERR_WORKSPACE;
        } else if (need > 0 && workspace == nullptr) {
            // no workspace: one split covering all of K
            per = (int)(((K + 63) / 64 + 7) / 8) * 8;
            splits = 1;
        } else if (need > workspace_bytes) {
            return QG_ERR_WORKSPACE;
        }
        (void)hipGetLastError();
        if (lib_scratch && need > 0 && qg::skinny_scratch((hipStream_t)stream, &workspace) != hipSuccess)
            return QG_ERR_HIP;
        a.workspace = workspace;
        a.splits = splits;
        a.split_steps = per;
        e = qg::launch_a8w8_skinny(a, vec, epi, (hipStream_t)stream, &name, skinny_bkm);
        log_dispatch(op, name, 1, M, N, K, splits);
    } else {
        const int cfg = pick_tile(1, M, N, K);
        // Few output tiles and a long K (128x128 tiles with 128-byte stages):
        // the three-stage kernel, K split across workgroups when the output
        // has at most 128 tiles and a workspace holds the partial sums.
        const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
        const bool deep = cfg == qg::TILE_128x128_K128 && dma_ok(a, b_trans != 0, vec, epi, 128) &&
                          tiles <= qg::SKINNY_MAX_TICKETS && K >= 2048;
        int splits = 1, per = 0;
        if (deep && (lib_scratch || workspace != nullptr)) {
            const int cap = lib_scratch
                ? (int)std::min<int64_t>(8, (int64_t)((qg::SKINNY_SCRATCH_BYTES - qg::SKINNY_TICKET_BYTES) /
                                                      ((size_t)tiles * 128 * 128 * 4)))
                : 8;
            a8w8_tiled_split_plan(M, N, K, cap, &splits, &per);
            // From a caller's workspace: the plan qgemm_workspace_bytes sized;
            // a shorter workspace is an error, as for the decode kernel (a
            // [N,K] weight at M <= 16 is sized as a decode shape: it splits
            // only when the workspace holds the plan).
            const size_t need = a8w8_tiled_split_bytes(M, N, splits);
            if (!lib_scratch && need > workspace_bytes) {
                if (a8w8_is_skinny(M, 0)) splits = 1;
                else return QG_ERR_WORKSPACE;
            }
        }
        (void)hipGetLastError();
        if (deep) {
            if (splits > 1 && lib_scratch && qg::skinny_scratch((hipStream_t)stream, &workspace) != hipSuccess)
                return QG_ERR_HIP;
            qg::Int8GemmArgs d = a;
            d.workspace = splits > 1 ? workspace : nullptr;
            d.splits = splits;
            d.split_steps = splits > 1 ? per : (int)(((K + 127) / 128) * 2);
            d.stage_out = stage_output(cfg, K, epi);
            // at most 64 rows: 64x128 tiles, the same tile count (and plan)
            if (M <= 64) {
                name = splits > 1 ? "int8_dma_64x128k128_splitk" : "int8_dma_64x128k128x3";
                e = qg::launch_dma_64x128k128_split(d, b_trans != 0, epi, 0, (hipStream_t)stream);
            } else {
                name = splits > 1 ? "int8_dma_128x128k128_splitk" : "int8_dma_128x128k128x3";
                e = qg::launch_dma_128x128k128_split(d, b_trans != 0, epi, 0, (hipStream_t)stream);
            }
        } else {
            e = launch_tiled(a, cfg, b_trans != 0, vec, epi, 0, (hipStream_t)stream, &name);
        }
        log_dispatch(op, name, 1, M, N, K, splits);
    }
    return finish_launch(e, name);
}

}  // namespace

extern "C" {

qg_status qgemm_a8w8(int64_t M, int64_t N, int64_t K, const int8_t* A, int64_t lda, const int8_t* W,
                     int64_t ldw, int b_trans, const float* act_scale, int64_t act_scale_len,
                     const float* weight_scale, int64_t weight_scale_len, void* out, qg_dtype out_dtype,
                     int64_t ldo, void* workspace, size_t workspace_bytes, void* stream) {
    return a8w8_impl(M, N, K, A, lda, W, ldw, b_trans, nullptr, 0, act_scale, act_scale_len, weight_scale,
                     weight_scale_len, out, out_dtype, ldo, workspace, workspace_bytes, stream, "a8w8");
}

static_assert(QG_A8W8_NOALLOC_SCRATCH_BYTES == qg::SKINNY_SCRATCH_BYTES, "scratch size in the header");

qg_status qgemm_a8w8_noalloc(int64_t M, int64_t N, int64_t K, const int8_t* A, int64_t lda, const int8_t* W,
                             int64_t ldw, int b_trans, const float* act_scale, int64_t act_scale_len,
                             const float* weight_scale, int64_t weight_scale_len, void* out, qg_dtype out_dtype,
                             int64_t ldo, void* stream) {
    return a8w8_impl(M, N, K, A, lda, W, ldw, b_trans, nullptr, 0, act_scale, act_scale_len, weight_scale,
                     weight_scale_len, out, out_dtype, ldo, nullptr, 0, stream, "a8w8_noalloc", true);
}

qg_status qgemm_a8w8_acc(int64_t M, int64_t N, int64_t K, const int8_t* A, int64_t lda, const int8_t* W,
                         int64_t ldw, int b_trans, const int32_t* acc_in, int64_t ld_acc,
                         const float* act_scale, int64_t act_scale_len, const float* weight_scale,
                         int64_t weight_scale_len, void* out, qg_dtype out_dtype, int64_t ldo,
                         void* workspace, size_t workspace_bytes, void* stream) {
    if (empty_output(M, N, K)) return empty_call();
    if (!dims_ok(M, N, K)) return QG_ERR_INVALID_ARGUMENT;
    if (acc_in == nullptr || ld_acc < N) return QG_ERR_INVALID_ARGUMENT;
    if ((M - 1) * ld_acc + N >= SPAN_LIMIT / 4) return QG_ERR_UNSUPPORTED;
    return a8w8_impl(M, N, K, A, lda, W, ldw, b_trans, acc_in, ld_acc, act_scale, act_scale_len, weight_scale,
                     weight_scale_len, out, out_dtype, ldo, workspace, workspace_bytes, stream, "a8w8_acc");
}

}  // extern "C"

namespace {

// MatMulInteger with a scalar activation zero point (a_zp_rows == NULL) or
// one per row (device values of a_dtype, a_zp_len 1 or M).
qg_status matmul_integer_impl(int64_t batch, int64_t M, int64_t N, int64_t K, const void* A, qg_dtype a_dtype,
                              int64_t lda, int64_t a_batch_stride, const void* B, qg_dtype b_dtype, int64_t ldb,
                              int64_t b_batch_stride, int32_t a_zero_point, const void* a_zp_rows,
                              int64_t a_zp_len, const void* b_zero_point, int64_t b_zero_point_len, int32_t* Y,
                              int64_t ldy, int64_t y_batch_stride, void* workspace, size_t workspace_bytes,
                              void* stream) {
    if (empty_output(M, N, K, batch)) return empty_call();
    if (!dims_ok(M, N, K) || batch < 1 || batch >= 65536) return QG_ERR_INVALID_ARGUMENT;
    if (A == nullptr || B == nullptr || Y == nullptr) return QG_ERR_INVALID_ARGUMENT;
    // A dtype outside the enumeration is invalid; fp32 / bf16 / int32
    // operands are well-formed forms the page does not lower (unsupported).
    if (a_dtype < QG_FP32 || a_dtype > QG_UINT8 || b_dtype < QG_FP32 || b_dtype > QG_UINT8)
        return QG_ERR_INVALID_ARGUMENT;
    if ((a_dtype != QG_UINT8 && a_dtype != QG_INT8) || (b_dtype != QG_UINT8 && b_dtype != QG_INT8))
        return QG_ERR_UNSUPPORTED;
    if (lda < K || ldb < N || ldy < N) return QG_ERR_INVALID_ARGUMENT;
    if (a_batch_stride < 0 || b_batch_stride < 0 || y_batch_stride < 0) return QG_ERR_INVALID_ARGUMENT;
    if (batch > 1) {
        if (a_batch_stride != 0 && a_batch_stride < (M - 1) * lda + K) return QG_ERR_INVALID_ARGUMENT;
        if (b_batch_stride != 0 && b_batch_stride < (K - 1) * ldb + N) return QG_ERR_INVALID_ARGUMENT;
        if (y_batch_stride < (M - 1) * ldy + N) return QG_ERR_INVALID_ARGUMENT;
    }
    const bool a_u8 = a_dtype == QG_UINT8, b_u8 = b_dtype == QG_UINT8;
    if (a_u8 ? (a_zero_point < 0 || a_zero_point > 255) : (a_zero_point < -128 || a_zero_point > 127))
        return QG_ERR_INVALID_ARGUMENT;
    if (b_zero_point != nullptr && b_zero_point_len != 1 && b_zero_point_len != N)
        return QG_ERR_INVALID_ARGUMENT;
    if (b_zero_point == nullptr && b_zero_point_len != 0 && b_zero_point_len != 1 && b_zero_point_len != N)
        return QG_ERR_INVALID_ARGUMENT;
    if (256 * lda + K + 256 >= SPAN_LIMIT || (K + 256) * ldb >= SPAN_LIMIT) return QG_ERR_UNSUPPORTED;
    // split-K tickets take atomics and partials 16-byte coherent stores
    if (workspace != nullptr && (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return QG_ERR_INVALID_ARGUMENT;

    qg::Int8GemmArgs a{};
    a.M = (int)M; a.N = (int)N; a.K = (int)K; a.batch = (int)batch;
    a.A = reinterpret_cast<const int8_t*>(A); a.lda = lda; a.a_bstride = a_batch_stride;
    a.B = reinterpret_cast<const int8_t*>(B); a.ldb = ldb; a.b_bstride = b_batch_stride;
    a.a_flip = a_u8 ? 0x80808080u : 0u;
    a.b_flip = b_u8 ? 0x80808080u : 0u;
    a.out = Y; a.ldo = ldy; a.o_bstride = y_batch_stride;
    a.b_zp = b_zero_point;
    a.b_zp_stride = (b_zero_point != nullptr && b_zero_point_len == N && N > 1) ? 1 : 0;
    a.b_zp_u8 = b_u8 ? 1 : 0;
    a.ca = (a_u8 ? 128 : 0) - a_zero_point;
    a.sb = b_u8 ? 128 : 0;
    if (a_zp_rows != nullptr) {
        a.a_zp = a_zp_rows;
        a.a_zp_stride = (a_zp_len == M && M > 1) ? 1 : 0;
        a.a_zp_rows = (int)M;   // row index modulo M, also once the batch is folded into M
        a.a_zp_u8 = a_u8 ? 1 : 0;
        a.sa = a_u8 ? 128 : 0;
    }
    // Fold the batch into M when B is shared and A / Y batches are contiguous
    // row blocks: one [batch*M, K] x [K, N] product with the same B.
    if (batch > 1 && b_batch_stride == 0 && a_batch_stride == M * lda && y_batch_stride == M * ldy &&
        batch * M < ((int64_t)1 << 30)) {
        a.M = (int)(batch * M);
        a.batch = 1;
    }
    // Row sums of A are needed when some cb[n] = sb - zb[n] may be non-zero;
    // column sums of B when some ca[m] may be.
    const bool need_rowsum = b_zero_point != nullptr || b_u8;
    const bool need_colsum = a.ca != 0 || a_zp_rows != nullptr;
    const int zp = (need_rowsum ? 1 : 0) | (need_colsum ? 2 : 0);
    const bool vec = aligned16(A) && aligned16(B) && lda % 16 == 0 && ldb % 16 == 0 && K % 16 == 0 &&
                     N % 16 == 0 && (a.batch == 1 || (a_batch_stride % 16 == 0 && b_batch_stride % 16 == 0));
    // At most 16 rows with a workspace: the decode kernel, which streams B
    // once with K split across workgroups (its row and column sums travel
    // with the partial tiles).
    if (a.batch == 1 && vec && workspace != nullptr && mmi_is_skinny(a.M, K)) {
        int splits, per;
        a8w8_skinny_plan(a.M, N, K, &splits, &per);
        if (qg::skinny_workspace_bytes(a.M, (int)N, splits, true) > workspace_bytes) return QG_ERR_WORKSPACE;
        a.workspace = workspace;
        a.splits = splits;
        a.split_steps = per;
        const char* name = "";
        (void)hipGetLastError();
        const hipError_t e = qg::launch_a8w8_skinny(a, true, qg::EPI_I32, (hipStream_t)stream, &name);
        log_dispatch("matmul_integer", name, 1, a.M, N, K, splits);
        return finish_launch(e, name);
    }
    const int cfg = pick_tile(a.batch, a.M, N, K);
    // Few output tiles and a long K: the three-stage kernel, K split across
    // workgroups (partial tiles and row / column sums in the workspace) when
    // the output has at most 128 tiles and a workspace is given.
    const int64_t tiles = (((int64_t)a.M + 127) / 128) * ((N + 127) / 128);
    const bool deep = a.batch == 1 && cfg == qg::TILE_128x128_K128 && dma_ok(a, false, vec, qg::EPI_I32, 128) &&
                      tiles <= qg::SKINNY_MAX_TICKETS && K >= 2048;
    int splits = 1, per = 0;
    if (deep && workspace != nullptr) {
        a8w8_tiled_split_plan(a.M, N, K, 8, &splits, &per);
        if (mmi_tiled_split_bytes(a.M, N, splits) > workspace_bytes) return QG_ERR_WORKSPACE;
    }
    const char* name = "";
    hipError_t e;
    (void)hipGetLastError();
    if (deep) {
        qg::Int8GemmArgs d = a;
        d.workspace = splits > 1 ? workspace : nullptr;
        d.splits = splits;
        d.split_steps = splits > 1 ? per : (int)(((K + 127) / 128) * 2);
        d.stage_out = stage_output(cfg, K, qg::EPI_I32);
        if (a.M <= 64) {   // 64x128 tiles, the same tile count (and plan)
            name = splits > 1 ? "int8_dma_64x128k128_splitk" : "int8_dma_64x128k128x3";
            e = qg::launch_dma_64x128k128_split(d, false, qg::EPI_I32, zp, (hipStream_t)stream);
        } else {
            name = splits > 1 ? "int8_dma_128x128k128_splitk" : "int8_dma_128x128k128x3";
            e = qg::launch_dma_128x128k128_split(d, false, qg::EPI_I32, zp, (hipStream_t)stream);
        }
    } else {
        e = launch_tiled(a, cfg, false, vec, qg::EPI_I32, zp, (hipStream_t)stream, &name);
    }
    log_dispatch("matmul_integer", name, a.batch, a.M, N, K, splits);
    return finish_launch(e, name);
}

}  // namespace

extern "C" {

qg_status matmul_integer(int64_t batch, int64_t M, int64_t N, int64_t K, const void* A, qg_dtype a_dtype,
                         int64_t lda, int64_t a_batch_stride, const void* B, qg_dtype b_dtype, int64_t ldb,
                         int64_t b_batch_stride, int32_t a_zero_point, const void* b_zero_point,
                         int64_t b_zero_point_len, int32_t* Y, int64_t ldy, int64_t y_batch_stride,
                         void* workspace, size_t workspace_bytes, void* stream) {
    return matmul_integer_impl(batch, M, N, K, A, a_dtype, lda, a_batch_stride, B, b_dtype, ldb, b_batch_stride,
                               a_zero_point, nullptr, 0, b_zero_point, b_zero_point_len, Y, ldy,
                               y_batch_stride, workspace, workspace_bytes, stream);
}

qg_status matmul_integer_row_zp(int64_t batch, int64_t M, int64_t N, int64_t K, const void* A,
                                qg_dtype a_dtype, int64_t lda, int64_t a_batch_stride, const void* B,
                                qg_dtype b_dtype, int64_t ldb, int64_t b_batch_stride, const void* a_zero_point,
                                int64_t a_zero_point_len, const void* b_zero_point, int64_t b_zero_point_len,
                                int32_t* Y, int64_t ldy, int64_t y_batch_stride, void* workspace,
                                size_t workspace_bytes, void* stream) {
    if (empty_output(M, N, K, batch)) return empty_call();
    if (a_zero_point == nullptr || (a_zero_point_len != 1 && a_zero_point_len != M))
        return QG_ERR_INVALID_ARGUMENT;
    const int32_t za0 = a_dtype == QG_UINT8 ? 128 : 0;   // in range; the kernel reads the real values
    return matmul_integer_impl(batch, M, N, K, A, a_dtype, lda, a_batch_stride, B, b_dtype, ldb, b_batch_stride,
                               za0, a_zero_point, a_zero_point_len, b_zero_point, b_zero_point_len, Y, ldy,
                               y_batch_stride, workspace, workspace_bytes, stream);
}

}  // extern "C"

extern "C" {

qg_status dynamic_quantize_linear(int64_t n, const float* x, uint8_t* y, float* y_scale, uint8_t* y_zero_point,
                                  void* workspace, size_t workspace_bytes, void* stream) {
    if (n < 0 || y_scale == nullptr || y_zero_point == nullptr || workspace == nullptr)
        return QG_ERR_INVALID_ARGUMENT;
    if (n > 0 && (x == nullptr || y == nullptr)) return QG_ERR_INVALID_ARGUMENT;
    if ((reinterpret_cast<uintptr_t>(workspace) & 7u) != 0) return QG_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < (size_t)qg::dql_partials(n) * 8) return QG_ERR_WORKSPACE;
    const bool vec = aligned16(x) && aligned16(y);
    (void)hipGetLastError();
    const hipError_t e = qg::launch_dynamic_quantize(x, n, y, y_scale, y_zero_point, workspace, vec,
                                                     (hipStream_t)stream);
    log_dispatch("dynamic_quantize_linear", "dql_minmax+dql_quantize", 1, 1, n, 1, qg::dql_partials(n));
    return finish_launch(e, "dql_minmax+dql_quantize");
}

}  // extern "C"

namespace {

// ConvInteger geometry and the path it takes: the implicit GEMM where its
// plan fits (workspace: packed w, row sums, padded channel-minor x), else
// im2col + the MatMulInteger GEMM (workspace: [packed w][pad to 256][col]).
struct ConvPlan {
    qg::ConvGeom g;
    size_t wp_bytes, col_off, total;
    bool implicit;
    qg::ConvImplicitPlan ip;
};

// Fills `plan` from the call's sizes; false if they do not describe a
// convolution this library runs (every value must also fit the kernels'
// 32-bit index arithmetic).
bool conv_plan(int64_t N, int64_t C, int64_t H, int64_t W, int64_t M, int64_t kH, int64_t kW, int64_t group,
               const int64_t* pads, const int64_t* strides, const int64_t* dilations, ConvPlan* plan) {
    const int64_t lim = (int64_t)1 << 30;
    if (pads == nullptr || strides == nullptr || dilations == nullptr) return false;
    if (N < 1 || C < 1 || H < 1 || W < 1 || M < 1 || kH < 1 || kW < 1 || group < 1) return false;
    if (N >= 65536 || C >= lim || H >= lim || W >= lim || M >= lim || kH >= lim || kW >= lim) return false;
    if (C % group != 0 || M % group != 0) return false;
    for (int i = 0; i < 4; ++i)
        if (pads[i] < 0 || pads[i] >= lim) return false;
    for (int i = 0; i < 2; ++i)
        if (strides[i] < 1 || strides[i] >= lim || dilations[i] < 1 || dilations[i] >= lim) return false;
    const int64_t eh = dilations[0] * (kH - 1) + 1, ew = dilations[1] * (kW - 1) + 1;
    if (H + pads[0] + pads[2] < eh || W + pads[1] + pads[3] < ew) return false;
    const int64_t OH = (H + pads[0] + pads[2] - eh) / strides[0] + 1;
    const int64_t OW = (W + pads[1] + pads[3] - ew) / strides[1] + 1;
    const int64_t Cg = C / group, Mg = M / group, Kg = Cg * kH * kW;
    const int64_t Kp = (Kg + 63) / 64 * 64, P = OH * OW, Pp = (P + 15) / 16 * 16;
    if (Kg >= lim || P >= lim || N * C * H * W >= ((int64_t)1 << 40)) return false;
    // grid sizes of the staging kernels: N*(C + group) workgroups, or one
    // lane per 16 column bytes
    if (N * (C + group) >= ((int64_t)1 << 31) || N * group * Kp * Pp >= ((int64_t)1 << 42)) return false;
    qg::ConvGeom& g = plan->g;
    g.N = (int)N; g.C = (int)C; g.H = (int)H; g.W = (int)W; g.M = (int)M; g.kH = (int)kH; g.kW = (int)kW;
    g.group = (int)group; g.Cg = (int)Cg; g.Mg = (int)Mg; g.Kg = (int)Kg; g.Kp = (int)Kp;
    g.OH = (int)OH; g.OW = (int)OW; g.P = (int)P; g.Pp = (int)Pp;
    g.pt = (int)pads[0]; g.pl = (int)pads[1]; g.sh = (int)strides[0]; g.sw = (int)strides[1];
    g.dh = (int)dilations[0]; g.dw = (int)dilations[1];
    plan->wp_bytes = (size_t)(group * Mg * Kp);
    plan->col_off = (plan->wp_bytes + 255) / 256 * 256;
    plan->total = plan->col_off + (size_t)N * group * Kp * Pp;
    // QGEMM_CONV=im2col keeps the column-matrix path (tests and comparisons)
    plan->implicit = !env_is("QGEMM_CONV", "im2col") && qg::conv_implicit_plan(g, &plan->ip);
    if (plan->implicit) plan->total = plan->ip.total;
    return true;
}

}  // namespace

extern "C" {

size_t conv_integer_workspace_bytes(int64_t N, int64_t C, int64_t H, int64_t W, int64_t M, int64_t kH, int64_t kW,
                                    int64_t group, const int64_t* pads, const int64_t* strides,
                                    const int64_t* dilations) {
    ConvPlan plan;
    if (!conv_plan(N, C, H, W, M, kH, kW, group, pads, strides, dilations, &plan)) return 0;
    return plan.total;
}

qg_status conv_integer(int64_t N, int64_t C, int64_t H, int64_t W, const void* x, qg_dtype x_dtype, int64_t M,
                       int64_t kH, int64_t kW, const void* w, qg_dtype w_dtype, int64_t group, const int64_t* pads,
                       const int64_t* strides, const int64_t* dilations, int32_t x_zero_point,
                       const void* w_zero_point, int64_t w_zero_point_len, int32_t* y, void* workspace,
                       size_t workspace_bytes, void* stream) {
    ConvPlan plan;
    if (!conv_plan(N, C, H, W, M, kH, kW, group, pads, strides, dilations, &plan)) return QG_ERR_INVALID_ARGUMENT;
    if (x == nullptr || w == nullptr || y == nullptr || workspace == nullptr) return QG_ERR_INVALID_ARGUMENT;
    if ((x_dtype != QG_UINT8 && x_dtype != QG_INT8) || (w_dtype != QG_UINT8 && w_dtype != QG_INT8))
        return QG_ERR_INVALID_ARGUMENT;
    const bool x_u8 = x_dtype == QG_UINT8, w_u8 = w_dtype == QG_UINT8;
    if (x_u8 ? (x_zero_point < 0 || x_zero_point > 255) : (x_zero_point < -128 || x_zero_point > 127))
        return QG_ERR_INVALID_ARGUMENT;
    if (w_zero_point == nullptr ? w_zero_point_len != 0 : (w_zero_point_len != 1 && w_zero_point_len != M))
        return QG_ERR_INVALID_ARGUMENT;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return QG_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < plan.total) return QG_ERR_WORKSPACE;
    const qg::ConvGeom& g = plan.g;
    if (plan.implicit) {
        // One launch when x's rows are 16-byte aligned (QGEMM_CONV=twopass
        // keeps the padded-copy pass for comparisons).
        const bool fused = !env_is("QGEMM_CONV", "twopass") && qg::conv_fused_ok(g, plan.ip, x, w);
        const char* name = fused ? "conv_fused" : "conv_implicit";
        (void)hipGetLastError();
        const hipError_t e = qg::launch_conv_implicit(g, plan.ip, x, x_u8, x_zero_point, w, w_u8, w_zero_point,
                                                      (int)w_zero_point_len, workspace, y, fused, (hipStream_t)stream);
        log_dispatch("conv_integer", name, N, M, (int64_t)g.P, g.Kg, g.group);
        return finish_launch(e, name);
    }
    // 32-bit buffer offsets inside one GEMM operand: a packed group of w and
    // one image's column matrix.
    if ((int64_t)g.Kp * g.Pp + 256 >= SPAN_LIMIT || (int64_t)g.Mg * g.Kp + 256 >= SPAN_LIMIT)
        return QG_ERR_UNSUPPORTED;

    uint8_t* wp = reinterpret_cast<uint8_t*>(workspace);
    uint8_t* col = wp + plan.col_off;
    (void)hipGetLastError();
    hipError_t e = qg::launch_conv_stage(g, x, (uint8_t)(x_zero_point & 0xff), w, w_zero_point,
                                         (int)w_zero_point_len, wp, col, (hipStream_t)stream);
    if (e != hipSuccess) return QG_ERR_HIP;

    // One batched MatMulInteger per group: A = packed w of the group (shared
    // by every image), B = the images' column matrices, Y = y's channels of
    // the group, NCHW.
    const bool vec = g.P % 16 == 0;
    const char* name = "";
    for (int gi = 0; gi < g.group; ++gi) {
        qg::Int8GemmArgs a{};
        a.M = g.Mg; a.N = g.P; a.K = g.Kp; a.batch = g.N;
        a.A = reinterpret_cast<const int8_t*>(wp + (int64_t)gi * g.Mg * g.Kp); a.lda = g.Kp; a.a_bstride = 0;
        a.B = reinterpret_cast<const int8_t*>(col + (int64_t)gi * g.Kp * g.Pp); a.ldb = g.Pp;
        a.b_bstride = (int64_t)g.group * g.Kp * g.Pp;
        a.a_flip = w_u8 ? 0x80808080u : 0u;
        a.b_flip = x_u8 ? 0x80808080u : 0u;
        a.out = y + (int64_t)gi * g.Mg * g.P; a.ldo = g.P; a.o_bstride = (int64_t)g.M * g.P;
        a.b_zp = nullptr; a.b_zp_stride = 0; a.b_zp_u8 = 0;
        a.sb = (x_u8 ? 128 : 0) - x_zero_point;   // cb[n] = sb: the activation zero point, constant
        if (w_zero_point != nullptr) {
            const bool per_channel = w_zero_point_len == M && M > 1;
            a.a_zp = reinterpret_cast<const uint8_t*>(w_zero_point) + (per_channel ? (int64_t)gi * g.Mg : 0);
            a.a_zp_stride = per_channel ? 1 : 0;
            a.a_zp_rows = g.Mg;
            a.a_zp_u8 = w_u8 ? 1 : 0;
            a.sa = w_u8 ? 128 : 0;
            a.ca = 0;
        } else {
            a.ca = w_u8 ? 128 : 0;
        }
        const bool need_rowsum = a.sb != 0;
        const bool need_colsum = a.ca != 0 || a.a_zp != nullptr;
        const int zp = (need_rowsum ? 1 : 0) | (need_colsum ? 2 : 0);
        const int cfg = pick_tile(a.batch, a.M, a.N, a.K);
        e = launch_tiled(a, cfg, false, vec, qg::EPI_I32, zp, (hipStream_t)stream, &name);
        if (e != hipSuccess) return QG_ERR_HIP;
    }
    log_dispatch("conv_integer", name, N, M, (int64_t)g.P, g.Kg, g.group);
    static thread_local char label[64];
    std::snprintf(label, sizeof label, "conv_im2col+%s", name);
    return finish_launch(hipSuccess, label);
}

}  // extern "C"

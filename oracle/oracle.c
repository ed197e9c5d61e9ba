/*
 * CPU oracle for the quantised matrix multiplies -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this library.  The product path (the HIP library and its Python
 * binding) never links, imports or calls it.  It shares no source, header,
 * table or helper with the HIP path.
 *
 * Everything here is the plain definition written out as loops: integer sums
 * in int64, floating-point references in double, each epilogue step in the
 * order the pages give.  No blocking, no fusion, no reordering of
 * floating-point work beyond the loop nest shown (integer sums are exact in
 * any order).  Compile with -ffp-contract=off so that no multiply is fused
 * into an add behind our back.
 *
 * Sources (page titles; sections named as on the page):
 *  [P1] "feat(PULPOpen): matmul that dequantises an int8 weight in-kernel",
 *       intro paragraph and section "The kernel" (the identity
 *       sum_k a_k (b_k - zp) scale = scale (sum a_k b_k - zp sum a_k)).
 *  [P4] "perf(pulpopen/gap9): share L3 storage between byte-identical
 *       constants", intro (a frozen weight is read by the forward op and by
 *       its gradient, dL/dx needs W).
 *  [P2] "Feature/a8w8 matmul dequant fusion", the walkthrough's sequence
 *       diagram (int8 matmul -> int32 accumulator -> cast to FP32 -> row scale
 *       by act_scale -> column scale by weight_scale -> cast to out_dtype),
 *       the Codex review (rank-1 [M]/[N] scales mean rows/columns) and the
 *       "What Changed" list (INT32 accumulator, FP32/BF16 outputs).
 *  [P5] "feat(onnx-to-hip): lower quantized integer conv and matmul",
 *       section "What", DynamicQuantizeLinear paragraph, MatMulInteger
 *       paragraph (ranks 2-4, zero points, shared B) and the accumulator paragraph (f32 accumulation only while
 *       65025*K fits the 24-bit mantissa, otherwise int64 accumulation stored
 *       as a wrapping int32), and the ConvInteger paragraph (rank-3 NCL and
 *       rank-4 NCHW, scalar activation zero point, weight zero point scalar
 *       or one per output channel, groups).
 */
#include <math.h>
#include <fenv.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Number of OpenMP threads the oracle's parallel loops use. */
int oracle_threads(void) { return omp_get_max_threads(); }

/* Sets that number (the benchmark times some calls on one thread). */
void oracle_set_threads(int n) { if (n >= 1) omp_set_num_threads(n); }

/* ---------------------------------------------------------------------- */
/* Helpers that are part of the definition                                 */
/* ---------------------------------------------------------------------- */

/* int64 -> int32 by two's-complement wrap ([P5] "What": "storing a wrapping
 * int32").  Done through uint32 so the conversion is defined C. */
static int32_t wrap_i32(int64_t v) {
    uint32_t u = (uint32_t)((uint64_t)v & 0xffffffffu);
    int32_t r;
    memcpy(&r, &u, sizeof r);
    return r;
}

/* IEEE-754 binary32 -> bfloat16, round to nearest, ties to even, written
 * from the definition on the bit pattern: keep the top 16 bits, add half an
 * ulp of the kept part, with ties going to the even kept value.  NaN stays a
 * quiet NaN of the same sign.  ([P2] out_dtype BF16 "cast".) */
uint16_t oracle_f32_to_bf16(float f) {
    uint32_t b;
    memcpy(&b, &f, sizeof b);
    if ((b & 0x7f800000u) == 0x7f800000u && (b & 0x007fffffu) != 0)
        return (uint16_t)((b >> 16) | 0x0040u);
    uint32_t kept_lsb = (b >> 16) & 1u;
    uint32_t rounded = b + 0x7fffu + kept_lsb;
    return (uint16_t)(rounded >> 16);
}

/* ---------------------------------------------------------------------- */
/* Row updates used by the loops below                                     */
/* ---------------------------------------------------------------------- */

/* The dequantised weight element of [P1]'s Dequant node, (w - zp) * scale,
 * in double: w - zp is an integer of at most 9 bits and scale has 24, so the
 * product is exact.  Its magnitude |w - zp| * |scale| scales the tolerance. */
static inline double dequant(int8_t w, int32_t zp, double scale) {
    return ((double)w - (double)zp) * scale;
}

/* y[i] = y[i] + a * dequant(w[i]) and yb[i] = yb[i] + |a| * |dequant(w[i])|
 * for i < n: one rounded multiply, then one rounded add per element (no
 * fused multiply-add: -ffp-contract=off).  Compiled for several instruction
 * sets and picked at run time; every clone performs the same IEEE
 * operations on each element. */
__attribute__((target_clones("avx512f", "avx2", "default")))
static void row_axpy_dequant(double* y, double* yb, double a, const int8_t* w, int32_t zp, double scale,
                             int64_t n) {
    const double abs_a = fabs(a), abs_scale = fabs(scale);
    for (int64_t i = 0; i < n; ++i) {
        const double centred = (double)w[i] - (double)zp;
        y[i] = y[i] + a * (centred * scale);
        yb[i] = yb[i] + abs_a * (fabs(centred) * abs_scale);
    }
}

/* row[i] += a * b[i] for i < n, with a and b[i] 8-bit integers: the product
 * is exact in int32 and the sum is kept in int64. */
__attribute__((target_clones("avx512f", "avx2", "default")))
static void row_axpy_i8(int64_t* row, int32_t a, const int8_t* b, int64_t n) {
    for (int64_t i = 0; i < n; ++i) row[i] += (int64_t)(a * (int32_t)b[i]);
}

/* ---------------------------------------------------------------------- */
/* W8A32 ([P1]): naive dequantise-then-matmul                              */
/* ---------------------------------------------------------------------- */

/* The Dequant node of [P1]'s intro, materialised: Wd = (W - zp) * scale,
 * then the fp32 matmul A @ Wd -- here carried out in double so that R is the
 * exact result up to double rounding.  `bound` receives
 * |scale| * sum_k |A[m,k]| * |W[k,n] - zp|, the scale of the tolerance.
 * A: [M,K] (lda), W: [K,N] (ldw), R and bound: [M,N] dense. */
void oracle_w8a32(int64_t M, int64_t N, int64_t K,
                  const float* A, int64_t lda,
                  const int8_t* W, int64_t ldw,
                  float scale, int32_t zero_point,
                  double* R, double* bound) {
    /* Row m of R is built up one k at a time (k ascending), so every output
     * sees exactly the sequence s = s + A[m,k] * Wd[k,n], k = 0 .. K-1, with
     * Wd[k,n] = dequant(W[k,n]) formed as the row is read. */
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        double* s = (double*)calloc((size_t)N, sizeof(double));
        double* b = (double*)calloc((size_t)N, sizeof(double));
        for (int64_t k = 0; k < K; ++k)
            row_axpy_dequant(s, b, (double)A[m * lda + k], W + k * ldw, zero_point, (double)scale, N);
        for (int64_t n = 0; n < N; ++n) {
            R[m * N + n] = s[n];
            if (bound) bound[m * N + n] = b[n];
        }
        free(s);
        free(b);
    }
}

/* Input gradient of the W8A32 matmul.  [P1]'s intro: the frozen int8
 * weight has two consumers, the forward matmul and its gradient; [P4]'s
 * intro: dL/dx needs W.  With the forward C = A @ Wd, Wd = (W - zp) * scale,
 * the gradient with respect to A is dA = dC @ Wd^T, here in double:
 *   R[m,k] = sum_n dC[m,n] * (W[k,n] - zp) * scale
 * and bound[m,k] = |scale| * sum_n |dC[m,n]| * |W[k,n] - zp|.
 * dC: [M,N] (ldd), W: [K,N] (ldw) -- the forward weight as stored --,
 * R and bound: [M,K] dense. */
void oracle_w8a32_input_grad(int64_t M, int64_t N, int64_t K,
                             const float* dC, int64_t ldd,
                             const int8_t* W, int64_t ldw,
                             float scale, int32_t zero_point,
                             double* R, double* bound) {
    /* W transposed (a copy of its bytes, WT[n,k] = W[k,n]), so that the
     * weight values one n contributes to row m of R are contiguous. */
    int8_t* WT = (int8_t*)malloc((size_t)(K * N));
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n) WT[n * K + k] = W[k * ldw + n];
    /* Row m of R is built up one n at a time (n ascending): every output sees
     * s = s + dC[m,n] * Wd[k,n], n = 0 .. N-1. */
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        double* s = (double*)calloc((size_t)K, sizeof(double));
        double* b = (double*)calloc((size_t)K, sizeof(double));
        for (int64_t n = 0; n < N; ++n)
            row_axpy_dequant(s, b, (double)dC[m * ldd + n], WT + n * K, zero_point, (double)scale, K);
        for (int64_t k = 0; k < K; ++k) {
            R[m * K + k] = s[k];
            if (bound) bound[m * K + k] = b[k];
        }
        free(s);
        free(b);
    }
    free(WT);
}

/* ---------------------------------------------------------------------- */
/* A8W8 ([P2]): int8 x int8 -> int32 -> fp32 -> *act_scale -> *weight_scale */
/* ---------------------------------------------------------------------- */

static float a8w8_epilogue(int32_t acc, float as, float ws) {
    float f = (float)acc;    /* cast: int32 -> fp32, round to nearest even */
    f = f * as;              /* row scale, rounded to fp32                 */
    f = f * ws;              /* column scale, rounded to fp32              */
    return f;
}

/* W is [K,N] (ldw) when b_trans == 0 and [N,K] (ldw) when b_trans == 1.
 * act_scale has length 1 or M, weight_scale length 1 or N.
 * Outputs ([M,N] dense) may each be NULL. */
void oracle_a8w8(int64_t M, int64_t N, int64_t K,
                 const int8_t* A, int64_t lda,
                 const int8_t* W, int64_t ldw, int b_trans,
                 const float* act_scale, int64_t as_len,
                 const float* weight_scale, int64_t ws_len,
                 int32_t* acc_out, float* out_f32, uint16_t* out_bf16) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        int64_t* row = (int64_t*)calloc((size_t)N, sizeof(int64_t));
        for (int64_t k = 0; k < K; ++k) {
            int64_t a = A[m * lda + k];
            if (!b_trans) {
                row_axpy_i8(row, (int32_t)a, W + k * ldw, N);
                continue;
            }
            for (int64_t n = 0; n < N; ++n) row[n] += a * (int64_t)W[n * ldw + k];
        }
        float as = act_scale[as_len == 1 ? 0 : m];
        for (int64_t n = 0; n < N; ++n) {
            int32_t acc = wrap_i32(row[n]);
            float f = a8w8_epilogue(acc, as, weight_scale[ws_len == 1 ? 0 : n]);
            if (acc_out) acc_out[m * N + n] = acc;
            if (out_f32) out_f32[m * N + n] = f;
            if (out_bf16) out_bf16[m * N + n] = oracle_f32_to_bf16(f);
        }
        free(row);
    }
}

/* Same as oracle_a8w8 at `count` chosen output positions (rows[i], cols[i]);
 * results go to index i of each (nullable) output. */
void oracle_a8w8_at(int64_t M, int64_t N, int64_t K,
                    const int8_t* A, int64_t lda,
                    const int8_t* W, int64_t ldw, int b_trans,
                    const float* act_scale, int64_t as_len,
                    const float* weight_scale, int64_t ws_len,
                    int64_t count, const int64_t* rows, const int64_t* cols,
                    int32_t* acc_out, float* out_f32, uint16_t* out_bf16) {
    (void)M; (void)N;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        int64_t m = rows[i], n = cols[i];
        int64_t s = 0;
        for (int64_t k = 0; k < K; ++k) {
            int64_t b = b_trans ? W[n * ldw + k] : W[k * ldw + n];
            s += (int64_t)A[m * lda + k] * b;
        }
        int32_t acc = wrap_i32(s);
        float f = a8w8_epilogue(acc, act_scale[as_len == 1 ? 0 : m],
                                weight_scale[ws_len == 1 ? 0 : n]);
        if (acc_out) acc_out[i] = acc;
        if (out_f32) out_f32[i] = f;
        if (out_bf16) out_bf16[i] = oracle_f32_to_bf16(f);
    }
}

/* A8W8 with an int32 accumulator input ([P2] "Summary" and "What Changed":
 * the matmul-dequant-acc op takes an INT32 accumulator input and lowers to
 * tile.matmul_acc / tile.gemv_acc, which add the int8 product into that
 * accumulator, followed by the same cast and scale chain):
 *   acc[m,n] = wrap32(acc_in[m,n] + sum_k A[m,k] W[k,n])
 * then the a8w8 epilogue.  acc_in is [M,N] with row stride ld_acc. */
void oracle_a8w8_acc(int64_t M, int64_t N, int64_t K,
                     const int8_t* A, int64_t lda,
                     const int8_t* W, int64_t ldw, int b_trans,
                     const int32_t* acc_in, int64_t ld_acc,
                     const float* act_scale, int64_t as_len,
                     const float* weight_scale, int64_t ws_len,
                     int32_t* acc_out, float* out_f32, uint16_t* out_bf16) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        int64_t* row = (int64_t*)calloc((size_t)N, sizeof(int64_t));
        for (int64_t n = 0; n < N; ++n) row[n] = acc_in[m * ld_acc + n];
        for (int64_t k = 0; k < K; ++k) {
            int64_t a = A[m * lda + k];
            if (!b_trans) {
                row_axpy_i8(row, (int32_t)a, W + k * ldw, N);
                continue;
            }
            for (int64_t n = 0; n < N; ++n) row[n] += a * (int64_t)W[n * ldw + k];
        }
        float as = act_scale[as_len == 1 ? 0 : m];
        for (int64_t n = 0; n < N; ++n) {
            int32_t acc = wrap_i32(row[n]);
            float f = a8w8_epilogue(acc, as, weight_scale[ws_len == 1 ? 0 : n]);
            if (acc_out) acc_out[m * N + n] = acc;
            if (out_f32) out_f32[m * N + n] = f;
            if (out_bf16) out_bf16[m * N + n] = oracle_f32_to_bf16(f);
        }
        free(row);
    }
}

/* ---------------------------------------------------------------------- */
/* MatMulInteger ([P5])                                                    */
/* ---------------------------------------------------------------------- */

static int64_t load_8bit(const void* base, int is_u8, int64_t idx) {
    return is_u8 ? (int64_t)((const uint8_t*)base)[idx]
                 : (int64_t)((const int8_t*)base)[idx];
}

/* Y[b,m,n] = wrap32( sum_k (A[b,m,k] - a_zp) * (B[b,k,n] - b_zp[n or 0]) ).
 * A: batch x [M,K] with row stride lda and batch stride a_bstride (0 means
 * one A shared by every batch); B: batch x [K,N] with ldb and b_bstride
 * (0 = one shared matrix); zero points already widened to int32; b_zp may be
 * NULL (absent = 0) or hold 1 or N values.  Y: batch x [M,N] (ldy,
 * y_bstride). */
void oracle_matmul_integer(int64_t batch, int64_t M, int64_t N, int64_t K,
                           const void* A, int a_is_u8, int64_t lda, int64_t a_bstride,
                           const void* B, int b_is_u8, int64_t ldb, int64_t b_bstride,
                           int32_t a_zp, const int32_t* b_zp, int64_t b_zp_len,
                           int32_t* Y, int64_t ldy, int64_t y_bstride) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t bt = 0; bt < batch; ++bt) {
        for (int64_t m = 0; m < M; ++m) {
            int64_t* row = (int64_t*)calloc((size_t)N, sizeof(int64_t));
            for (int64_t k = 0; k < K; ++k) {
                int64_t a = load_8bit(A, a_is_u8, bt * a_bstride + m * lda + k) - a_zp;
                for (int64_t n = 0; n < N; ++n) {
                    int64_t zb = b_zp ? b_zp[b_zp_len == 1 ? 0 : n] : 0;
                    int64_t b = load_8bit(B, b_is_u8, bt * b_bstride + k * ldb + n) - zb;
                    row[n] += a * b;
                }
            }
            for (int64_t n = 0; n < N; ++n)
                Y[bt * y_bstride + m * ldy + n] = wrap_i32(row[n]);
            free(row);
        }
    }
}

/* MatMulInteger with one activation zero point per row ([P5] "What": a
 * per-row zero point is accepted when M is static; it is the value
 * subtracted from every element of that row of A, in every batch):
 *   Y[b,m,n] = wrap32( sum_k (A[b,m,k] - a_zp[m]) * (B[b',k,n] - zb[n]) )
 * a_zp has a_zp_len == 1 or M entries. */
void oracle_matmul_integer_rows(int64_t batch, int64_t M, int64_t N, int64_t K,
                                const void* A, int a_is_u8, int64_t lda, int64_t a_bstride,
                                const void* B, int b_is_u8, int64_t ldb, int64_t b_bstride,
                                const int32_t* a_zp, int64_t a_zp_len,
                                const int32_t* b_zp, int64_t b_zp_len,
                                int32_t* Y, int64_t ldy, int64_t y_bstride) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t bt = 0; bt < batch; ++bt) {
        for (int64_t m = 0; m < M; ++m) {
            int64_t* row = (int64_t*)calloc((size_t)N, sizeof(int64_t));
            const int64_t za = a_zp[a_zp_len == 1 ? 0 : m];
            for (int64_t k = 0; k < K; ++k) {
                int64_t a = load_8bit(A, a_is_u8, bt * a_bstride + m * lda + k) - za;
                for (int64_t n = 0; n < N; ++n) {
                    int64_t zb = b_zp ? b_zp[b_zp_len == 1 ? 0 : n] : 0;
                    int64_t b = load_8bit(B, b_is_u8, bt * b_bstride + k * ldb + n) - zb;
                    row[n] += a * b;
                }
            }
            for (int64_t n = 0; n < N; ++n)
                Y[bt * y_bstride + m * ldy + n] = wrap_i32(row[n]);
            free(row);
        }
    }
}

/* Same sum at `count` positions (bts[i], rows[i], cols[i]) -> Y[i]. */
void oracle_matmul_integer_at(int64_t K,
                              const void* A, int a_is_u8, int64_t lda, int64_t a_bstride,
                              const void* B, int b_is_u8, int64_t ldb, int64_t b_bstride,
                              int32_t a_zp, const int32_t* b_zp, int64_t b_zp_len,
                              int64_t count, const int64_t* bts, const int64_t* rows,
                              const int64_t* cols, int32_t* Y) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        int64_t bt = bts[i], m = rows[i], n = cols[i];
        int64_t zb = b_zp ? b_zp[b_zp_len == 1 ? 0 : n] : 0;
        int64_t s = 0;
        for (int64_t k = 0; k < K; ++k) {
            int64_t a = load_8bit(A, a_is_u8, bt * a_bstride + m * lda + k) - a_zp;
            int64_t b = load_8bit(B, b_is_u8, bt * b_bstride + k * ldb + n) - zb;
            s += a * b;
        }
        Y[i] = wrap_i32(s);
    }
}

/* The f32-accumulator form [P5] selects while 65025*K fits the 24-bit
 * mantissa: the same centred products, summed one after another in fp32,
 * the total converted to int32.  Used only to check the accumulator bound;
 * one dot product of length K (a: stride 1, b: stride ldb). */
int32_t oracle_dot_f32acc(int64_t K, const void* a, int a_is_u8,
                          const void* b, int b_is_u8, int64_t ldb,
                          int32_t a_zp, int32_t b_zp) {
    float s = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
        float p = (float)((load_8bit(a, a_is_u8, k) - a_zp) *
                          (load_8bit(b, b_is_u8, k * ldb) - b_zp));
        s = s + p;
    }
    return (int32_t)s;
}

/* ---------------------------------------------------------------------- */
/* DynamicQuantizeLinear, uint8 ([P5])                                    */
/* ---------------------------------------------------------------------- */

/* [P5] "What", DynamicQuantizeLinear paragraph: reduce the input to its
 * minimum and maximum, scale = (max - min) / 255 with a zero range selecting
 * scale 1, a zero point rounded with ties to even, then quantize; the
 * review's all-zero case gives scale 1, zero point 0 and an all-zero output.
 * Readings where the page is silent:
 *  - the range is widened to include 0 (min <= 0 <= max), the semantics of
 *    the ONNX operator the page lowers: a real 0 then quantizes exactly to
 *    the zero point, and the zero point needs no clamping;
 *  - every step is fp32 arithmetic (the page reduces f32), each division
 *    rounded to nearest even; a scale that comes out as 0 takes the
 *    zero-range value 1;
 *  - quantizing rounds x / scale to the nearest integer with ties to even,
 *    adds the zero point and saturates to [0, 255].
 * y: n bytes; scale_out and zp_out: one value each. */
void oracle_dynamic_quantize_linear(int64_t n, const float* x, uint8_t* y,
                                    float* scale_out, int32_t* zp_out) {
    float mn = 0.0f, mx = 0.0f;        /* the range always includes 0 */
    for (int64_t i = 0; i < n; ++i) {
        if (x[i] < mn) mn = x[i];
        if (x[i] > mx) mx = x[i];
    }
    const int saved = fegetround();
    fesetround(FE_TONEAREST);
    volatile float range = mx - mn;    /* volatile: keep each fp32 rounding */
    volatile float scale = range / 255.0f;
    if (scale == 0.0f) scale = 1.0f;
    volatile float q0 = mn / scale;
    volatile float zf = rintf(0.0f - q0);   /* ties to even */
    int32_t zp = (int32_t)zf;
    if (zp < 0) zp = 0;
    if (zp > 255) zp = 255;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        float q = x[i] / scale;
        int64_t v = (int64_t)rintf(q) + zp;
        y[i] = (uint8_t)(v < 0 ? 0 : (v > 255 ? 255 : v));
    }
    fesetround(saved);
    *scale_out = scale;
    *zp_out = zp;
}

/* ---------------------------------------------------------------------- */
/* ConvInteger ([P5])                                                     */
/* ---------------------------------------------------------------------- */

/* [P5] "What", ConvInteger paragraph, with the grouped, padded, strided case
 * of its GPU numeric tests: an integer convolution of x [N, C, H, W] with
 * w [M, C/group, kH, kW], each operand minus its zero point, summed exactly
 * and stored as a wrapping int32 (the accumulator paragraph):
 *
 *   y[n, m, oh, ow] = wrap32( sum_{c < C/group, kh < kH, kw < kW}
 *       (x[n, g*(C/group) + c, ih, iw] - x_zp) * (w[m, c, kh, kw] - w_zp[m]) )
 *   g = m / (M/group),  ih = oh*sh - pt + kh*dh,  iw = ow*sw - pl + kw*dw,
 *   OH = (H + pt + pb - dh*(kH - 1) - 1) / sh + 1, likewise OW.
 *
 * Reading where the page is silent: a tap outside the input contributes
 * nothing, i.e. the input is padded with its own zero point (the page's
 * lowering subtracts the zero point first and then convolves with zero
 * padding, which is the same thing).  w_zp: w_zp_len 0 (none: all zero),
 * 1 (scalar) or M (one per output channel).  A rank-3 NCL convolution is the
 * H = kH = 1 case.  y: [N, M, OH, OW] int32. */
void oracle_conv_integer(int64_t N, int64_t C, int64_t H, int64_t W,
                         const void* x, int x_is_u8,
                         int64_t M, int64_t kH, int64_t kW,
                         const void* w, int w_is_u8, int64_t group,
                         int64_t pt, int64_t pl, int64_t pb, int64_t pr,
                         int64_t sh, int64_t sw, int64_t dh, int64_t dw,
                         int32_t x_zp, const int32_t* w_zp, int64_t w_zp_len,
                         int32_t* y) {
    const int64_t Cg = C / group, Mg = M / group;
    const int64_t OH = (H + pt + pb - dh * (kH - 1) - 1) / sh + 1;
    const int64_t OW = (W + pl + pr - dw * (kW - 1) - 1) / sw + 1;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            const int64_t g = m / Mg;
            const int64_t zw = w_zp_len == 0 ? 0 : (w_zp_len == 1 ? w_zp[0] : w_zp[m]);
            for (int64_t oh = 0; oh < OH; ++oh) {
                for (int64_t ow = 0; ow < OW; ++ow) {
                    int64_t s = 0;
                    for (int64_t c = 0; c < Cg; ++c) {
                        for (int64_t kh = 0; kh < kH; ++kh) {
                            for (int64_t kw = 0; kw < kW; ++kw) {
                                const int64_t ih = oh * sh - pt + kh * dh;
                                const int64_t iw = ow * sw - pl + kw * dw;
                                if (ih < 0 || ih >= H || iw < 0 || iw >= W) continue;
                                const int64_t xv = load_8bit(x, x_is_u8, ((n * C + g * Cg + c) * H + ih) * W + iw);
                                const int64_t wv = load_8bit(w, w_is_u8, ((m * Cg + c) * kH + kh) * kW + kw);
                                s += (xv - x_zp) * (wv - zw);
                            }
                        }
                    }
                    y[((n * M + m) * OH + oh) * OW + ow] = wrap_i32(s);
                }
            }
        }
    }
}

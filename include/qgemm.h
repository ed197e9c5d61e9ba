/*
 * qgemm: quantised matrix multiplies for AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Every tensor pointer is a DEVICE pointer owned by the caller; the
 * library allocates no memory and keeps no state apart from a per-thread
 * record of the last kernel it launched and the static scratch array per
 * GPU of qgemm_a8w8_noalloc.  Matrices are row-major with an
 * explicit leading dimension (elements between consecutive rows).  Every
 * compute call is asynchronous on `stream` (a hipStream_t; NULL is the null
 * stream): it validates its arguments on the host, clears any pending HIP
 * error, launches, and reports the launch status.  Failures during execution
 * surface at the caller's next synchronisation.  Outputs must not overlap
 * inputs.  Calls on different streams may run concurrently from several host
 * threads, provided they do not share a workspace.
 *
 * Errors (qg_status):
 *   QG_ERR_INVALID_ARGUMENT  a bad size, leading dimension, pointer, dtype,
 *                            scale length or zero point; nothing launched.
 *   QG_ERR_UNSUPPORTED       a well-formed form this library does not
 *                            implement (listed per call); nothing launched.
 *   QG_ERR_WORKSPACE         a workspace smaller than qgemm_workspace_bytes()
 *                            was passed; nothing launched.
 *   QG_ERR_HIP               the kernel launch itself failed.
 * Following the launch convention of "feat(onnx-to-hip): lower quantized
 * integer conv and matmul" ("What", last paragraph), a HIP error already
 * pending before the call is cleared and does not fail the call.
 *
 * Empty outputs: a matrix-multiply call (qgemm_w8a32, qgemm_w8a32_input_grad,
 * qgemm_a8w8, qgemm_a8w8_acc, matmul_integer, matmul_integer_row_zp) whose
 * output has no elements (a zero M or N, or a zero batch) checks only that
 * no size is negative or past the limits, launches nothing and returns
 * QG_OK; its pointers may then be NULL and qgemm_last_kernel() reads
 * "none".  An empty reduction (K = 0; N = 0 for the W8A32 input gradient)
 * under a non-empty output is QG_ERR_INVALID_ARGUMENT.
 */
#ifndef QGEMM_H
#define QGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QG_OK = 0,
    QG_ERR_INVALID_ARGUMENT = 1,
    QG_ERR_UNSUPPORTED = 2,
    QG_ERR_WORKSPACE = 3,
    QG_ERR_HIP = 4
} qg_status;

typedef enum {
    QG_FP32 = 0,
    QG_BF16 = 1,
    QG_INT32 = 2,
    QG_INT8 = 3,
    QG_UINT8 = 4
} qg_dtype;

/* Operation ids for qgemm_workspace_bytes. */
enum { QG_OP_W8A32 = 0, QG_OP_A8W8 = 1, QG_OP_MATMUL_INTEGER = 2, QG_OP_DYNAMIC_QUANTIZE_LINEAR = 3,
       QG_OP_W8A32_INPUT_GRAD = 4 };

/*
 * W8A32: fp32 activations times an int8 weight with a per-tensor scale and
 * zero point ("feat(PULPOpen): matmul that dequantises an int8 weight
 * in-kernel", section "The kernel"):
 *
 *   C[m,n] = sum_k A[m,k] * (W[k,n] - zero_point) * scale
 *          = scale * (sum_k A[m,k] W[k,n] - zero_point * sum_k A[m,k])
 *
 * evaluated in the second (factorised) form; the dequantised weight is
 * never formed.  zero_point == 0 drops the correction.  The sum
 * sum_k A[m,k] W[k,n] runs on the bf16 matrix cores with every A value split
 * exactly into three bfloat16 parts (hi + lo + lo2 == A[m,k]; the int8 weight
 * is exact in bfloat16), so each product is exact and only the fp32
 * accumulation rounds; sum_k A[m,k] and the epilogue are fp32.  The
 * environment variable QGEMM_W8A32=fp32 (read per call) selects the fp32
 * matrix cores instead.
 *   A: fp32 [M,K], row stride lda >= K.    W: int8 [K,N], row stride ldw >= N.
 *   C: fp32 [M,N], row stride ldc >= N.    scale: finite fp32 (host value).
 *   zero_point: any int32 (host value).
 * Requires M, N, K >= 1.  QG_ERR_UNSUPPORTED if K*ldw or M*lda*4 reaches 2^31
 * bytes.  The result is not bit-defined (summation order is the kernel's);
 * it is within 1e-5 * |scale| * sum_k |A[m,k]| * |W[k,n] - zp| of the exact
 * value for the library's workloads.  The split is exact for A values of
 * magnitude 2^-103 and above (and zero); smaller ones may lose their bits
 * below 2^-126.  An infinite A value gives NaN in its output row on the
 * split path, and on both paths when zero_point != 0 (the factorised form
 * subtracts zero_point * inf from an infinite sum).
 */
qg_status qgemm_w8a32(int64_t M, int64_t N, int64_t K,
                      const float* A, int64_t lda,
                      const int8_t* W, int64_t ldw,
                      float scale, int32_t zero_point,
                      float* C, int64_t ldc,
                      void* stream);

/*
 * qgemm_w8a32 with a workspace (same operation, arguments and accuracy;
 * qgemm_w8a32 is this call with NULL / 0).  workspace: NULL, or device
 * memory of at least qgemm_workspace_bytes(QG_OP_W8A32, 1, M, N, K) bytes,
 * 256-byte aligned (else QG_ERR_INVALID_ARGUMENT), zero-filled before its
 * first use.  At most 16 rows with 16-byte aligned rows of A and W
 * (lda % 4 == 0, K % 4 == 0, ldw % 16 == 0, N % 16 == 0) run a decode
 * kernel that streams W once, 256 columns per workgroup, K divided among
 * workgroups (one ticket per 256 columns; without a workspace, one split).
 * Other outputs of at most 256 tiles of 128 x 128 (e.g. M <= 512 at
 * N = 8192) divide K among up to 8 workgroups per tile, about two per CU
 * (one ticket per tile).  The first 1024 bytes hold the tickets, the rest each split's fp32
 * partial sums and partial row sums.  The last split to finish adds the
 * partials in split order, so results do not depend on timing and repeat
 * bit for bit; they differ from the unsplit call's only in the order of the
 * fp32 additions.  Tickets return to zero when a call completes, so one
 * workspace serves later calls on the same stream of any shape; calls that
 * overlap in time must not share one.  QG_ERR_WORKSPACE: a workspace smaller
 * than the split needs.
 */
qg_status qgemm_w8a32_ws(int64_t M, int64_t N, int64_t K,
                         const float* A, int64_t lda,
                         const int8_t* W, int64_t ldw,
                         float scale, int32_t zero_point,
                         float* C, int64_t ldc,
                         void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * Input gradient of the W8A32 matmul: the frozen int8 weight's second
 * consumer ("feat(PULPOpen): matmul that dequantises an int8 weight
 * in-kernel", intro; "perf(pulpopen/gap9): share L3 storage between
 * byte-identical constants", intro: dL/dx needs W).  For the forward
 * C = A @ ((W - zp) * scale) with W [K,N]:
 *
 *   dA[m,k] = sum_n dC[m,n] * (W[k,n] - zero_point) * scale
 *           = scale * (sum_n dC[m,n] W[k,n] - zero_point * sum_n dC[m,n])
 *
 * evaluated in the factorised form as qgemm_w8a32 evaluates it (the exact
 * three-way bf16 split of dC on the bf16 matrix cores, or the fp32 matrix
 * cores with QGEMM_W8A32=fp32), the dequantised weight never formed, W read
 * in its forward layout.
 *   dC: fp32 [M,N], row stride lddc >= N.   W: int8 [K,N], row stride ldw >= N.
 *   dA: fp32 [M,K], row stride ldda >= K.    scale, zero_point: as qgemm_w8a32.
 * Requires M, N, K >= 1.  QG_ERR_UNSUPPORTED if K*ldw or M*lddc*4 reaches
 * 2^31 bytes.  Accuracy as qgemm_w8a32, with the sum over n:
 * within 1e-5 * |scale| * sum_n |dC[m,n]| * |W[k,n] - zp| of the exact value.
 */
qg_status qgemm_w8a32_input_grad(int64_t M, int64_t N, int64_t K,
                                 const float* dC, int64_t lddc,
                                 const int8_t* W, int64_t ldw,
                                 float scale, int32_t zero_point,
                                 float* dA, int64_t ldda,
                                 void* stream);

/*
 * qgemm_w8a32_input_grad with a workspace, sized by
 * qgemm_workspace_bytes(QG_OP_W8A32_INPUT_GRAD, 1, M, N, K) with this call's
 * M, N, K; it divides the sum over n as qgemm_w8a32_ws divides the sum over
 * k (at most 16 rows with 16-byte aligned rows of dC and W: the decode
 * kernel; else dA of at most 256 tiles of 128 x 128), with the same rules.
 * At most 8 rows across K >= 8192 outputs (16-byte aligned rows, N % 4 ==
 * 0) take a form in which each workgroup owns whole rows of W over all of
 * n; it leaves the workspace untouched.
 */
qg_status qgemm_w8a32_input_grad_ws(int64_t M, int64_t N, int64_t K,
                                    const float* dC, int64_t lddc,
                                    const int8_t* W, int64_t ldw,
                                    float scale, int32_t zero_point,
                                    float* dA, int64_t ldda,
                                    void* workspace, size_t workspace_bytes,
                                    void* stream);

/*
 * A8W8 matmul with fused dequantisation ("Feature/a8w8 matmul dequant
 * fusion": sequence diagram and "What Changed"):
 *
 *   acc[m,n] = sum_k A[m,k] * W[k,n]          exact, int32 (wraps mod 2^32)
 *   out[m,n] = cast_out( (((float)acc) * act_scale[m]) * weight_scale[n] )
 *
 * with each fp32 step rounded to nearest even in exactly this order, and the
 * bf16 cast rounding to nearest even.  Results are bit-exact.
 *   A: int8 [M,K], row stride lda >= K.
 *   W: int8 [K,N] with row stride ldw >= N (b_trans == 0), or
 *      int8 [N,K] with row stride ldw >= K (b_trans == 1).
 *   act_scale: fp32, act_scale_len == M (one per row) or 1 (one for all).
 *     A rank-1 [M] scale always scales ROWS, also when M == N.
 *   weight_scale: fp32, weight_scale_len == N (per column) or 1.
 *   out: out_dtype QG_FP32 or QG_BF16, [M,N], row stride ldo >= N.
 *   workspace: NULL, or device memory of at least
 *     qgemm_workspace_bytes(QG_OP_A8W8, 1, M, N, K) bytes, 256-byte aligned
 *     (else QG_ERR_INVALID_ARGUMENT), zero-filled before its first use.
 *     Decode shapes split K across workgroups, and so do tiled shapes whose
 *     output has at most 128 tiles of 128 x 128 when K allows two or more
 *     splits of at least 1024 (e.g. M = 17 .. 256 at N = K = 8192): the
 *     first 1024 bytes hold one ticket counter per 256 columns (decode) or
 *     per output tile (tiled), a header of fixed size whatever the shape,
 *     the rest the exact int32 partial sums.  Every call returns the
 *     tickets to zero when it completes, so the same workspace serves the
 *     next call on the same stream, of this or any other shape, without
 *     clearing; calls that overlap in time must not share one.  With NULL,
 *     both run unsplit (decode shapes as a single-pass kernel).  A [N,K]
 *     weight (b_trans == 1) at M <= 16 whose rows are not 16-byte aligned
 *     runs the tiled kernel, which splits only when the workspace passed
 *     holds its plan (the size returned is the decode kernel's).
 * Decode shapes (M <= 16, W as [K,N], or as [N,K] with 16-byte aligned rows
 * and K % 16 == 0) run a bandwidth-bound kernel that streams W once; all
 * other shapes run the tiled matrix-core kernel.  With W as [N,K] and
 * N >= 4096 the decode kernel owns whole columns over all of K (no split,
 * the workspace is not touched); otherwise it splits K as described above.
 * QG_ERR_UNSUPPORTED if an operand's byte span reaches 2^31 (for W as
 * [N,K], the span of 256 of its rows: the kernels address it a tile of rows
 * at a time, so the whole weight may be larger).
 */
qg_status qgemm_a8w8(int64_t M, int64_t N, int64_t K,
                     const int8_t* A, int64_t lda,
                     const int8_t* W, int64_t ldw, int b_trans,
                     const float* act_scale, int64_t act_scale_len,
                     const float* weight_scale, int64_t weight_scale_len,
                     void* out, qg_dtype out_dtype, int64_t ldo,
                     void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * qgemm_a8w8 for callers that cannot allocate device memory: code under
 * stream capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same operation, arguments, results (bit for bit) and errors as qgemm_a8w8,
 * without the workspace arguments; it allocates nothing.  Shapes that
 * split K use a scratch array the library holds in static device memory,
 * QG_A8W8_NOALLOC_SCRATCH_BYTES on each GPU it runs on (held until the
 * process ends).  A decode shape whose split-K workspace
 * (qgemm_workspace_bytes(QG_OP_A8W8, ...)) would exceed that returns
 * QG_ERR_WORKSPACE with nothing launched (no shape of the default plan
 * does); a tiled shape takes as many splits as fit in it (e.g. 2 instead
 * of 4 for 64 output tiles), or none.  The first call on a device looks up that device's copy and
 * clears its ticket words with a small kernel on `stream`; every call
 * leaves them at zero again.  All calls on one GPU share its array, which
 * keeps the last call's partial sums: calls that overlap in time on one GPU
 * (several streams or host threads) race, so the caller serialises them.
 * `stream` must belong to the calling thread's current device.
 */
#define QG_A8W8_NOALLOC_SCRATCH_BYTES ((size_t)1024 + ((size_t)8 << 20))
qg_status qgemm_a8w8_noalloc(int64_t M, int64_t N, int64_t K,
                             const int8_t* A, int64_t lda,
                             const int8_t* W, int64_t ldw, int b_trans,
                             const float* act_scale, int64_t act_scale_len,
                             const float* weight_scale, int64_t weight_scale_len,
                             void* out, qg_dtype out_dtype, int64_t ldo,
                             void* stream);

/*
 * A8W8 with an int32 accumulator input ("Feature/a8w8 matmul dequant
 * fusion", "Summary" and "What Changed": the matmul-dequant-acc op takes an
 * INT32 accumulator input and lowers to matmul_acc / gemv_acc, which add the
 * int8 product into it, before the same cast and scale chain):
 *
 *   acc[m,n] = acc_in[m,n] + sum_k A[m,k] * W[k,n]    exact, wraps mod 2^32
 *   out[m,n] = cast_out( (((float)acc) * act_scale[m]) * weight_scale[n] )
 *
 * Bit-exact.  acc_in: int32 [M,N], row stride ld_acc >= N, device memory,
 * read only (it may not overlap `out`).  Every other argument, the
 * workspace (size from qgemm_workspace_bytes(QG_OP_A8W8, ...)) and the
 * errors are those of qgemm_a8w8; in addition QG_ERR_INVALID_ARGUMENT for a
 * NULL acc_in or ld_acc < N, QG_ERR_UNSUPPORTED if acc_in spans 2^31 bytes.
 * The int32 accumulator of one K chunk (matmul_integer with int8 operands
 * and zero points 0 computes it) fed into the call for the next chunk gives
 * the result over the whole K.
 */
qg_status qgemm_a8w8_acc(int64_t M, int64_t N, int64_t K,
                         const int8_t* A, int64_t lda,
                         const int8_t* W, int64_t ldw, int b_trans,
                         const int32_t* acc_in, int64_t ld_acc,
                         const float* act_scale, int64_t act_scale_len,
                         const float* weight_scale, int64_t weight_scale_len,
                         void* out, qg_dtype out_dtype, int64_t ldo,
                         void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * MatMulInteger ("feat(onnx-to-hip): lower quantized integer conv and
 * matmul", section "What", MatMulInteger and accumulator paragraphs):
 *
 *   Y[b,m,n] = wrap32( sum_k (A[b,m,k] - a_zero_point) * (B[b,k,n] - zb[n]) )
 *
 * summed exactly and stored as a wrapping (two's-complement) int32, the
 * result the page's int64 accumulation gives for any K.  Bit-exact.
 *   A: a_dtype QG_UINT8 or QG_INT8 (QG_FP32, QG_BF16, QG_INT32: a form the
 *      page does not lower, QG_ERR_UNSUPPORTED; likewise for b_dtype),
 *      `batch` matrices [M,K], row stride
 *      lda >= K, batch stride a_batch_stride (0: one A used by every batch,
 *      the page's size-1 batch expanded without a copy).
 *   B: b_dtype QG_UINT8 or QG_INT8, [K,N], row stride ldb >= N, batch stride
 *      b_batch_stride (0: one shared matrix, never copied per batch).
 *   a_zero_point: scalar, within a_dtype's range.
 *   b_zero_point: device pointer to b_dtype values, NULL (all zero), or
 *      b_zero_point_len == 1 (scalar) or N (one per column).
 *   Y: int32, `batch` matrices [M,N], row stride ldy >= N, batch stride
 *      y_batch_stride >= (M-1)*ldy + N when batch > 1.
 *   workspace: NULL, or device memory of at least
 *     qgemm_workspace_bytes(QG_OP_MATMUL_INTEGER, batch, M, N, K) bytes,
 *     256-byte aligned (else QG_ERR_INVALID_ARGUMENT), zero-filled before
 *     its first use.  With batches folded into M: at most 16 rows with K a
 *     multiple of 64 run the decode kernel (B streamed once, K split across
 *     workgroups; one ticket per 256 output columns); other outputs of at
 *     most 128 tiles of 128 x 128 whose K allows two or more splits of at
 *     least 1024 split K on the tiled kernel (one ticket per output tile).
 *     The first 1024 bytes hold the tickets, the rest each split's exact
 *     int32 partial tile with its partial row and column sums.  Tickets return to zero when a call
 *     completes, so one workspace serves later calls on the same stream of
 *     any shape; calls that overlap in time must not share one.  With NULL
 *     the tiled kernel runs unsplit (also for decode shapes);
 *     QG_ERR_WORKSPACE when a workspace is given but smaller than the split
 *     needs.
 * Requires batch, M, N, K >= 1.  QG_ERR_UNSUPPORTED: an operand byte span
 * that reaches 2^31.  (Per-row activation zero points: matmul_integer_row_zp.
 * Ranks outside 2-4 are rejected by the Python binding, which maps ONNX
 * ranks to batch.)
 */
qg_status matmul_integer(int64_t batch, int64_t M, int64_t N, int64_t K,
                         const void* A, qg_dtype a_dtype, int64_t lda, int64_t a_batch_stride,
                         const void* B, qg_dtype b_dtype, int64_t ldb, int64_t b_batch_stride,
                         int32_t a_zero_point,
                         const void* b_zero_point, int64_t b_zero_point_len,
                         int32_t* Y, int64_t ldy, int64_t y_batch_stride,
                         void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * MatMulInteger with one activation zero point per row of A (same page,
 * "What": a per-row zero point is accepted when M is static):
 *
 *   Y[b,m,n] = wrap32( sum_k (A[b,m,k] - a_zp[m]) * (B[b,k,n] - zb[n]) )
 *
 * a_zero_point: device pointer to a_zero_point_len (1 or M) values of
 * a_dtype; row m of every batch uses value m.  Everything else as in
 * matmul_integer; QG_ERR_INVALID_ARGUMENT for a NULL a_zero_point or
 * another length.  Bit-exact.
 */
qg_status matmul_integer_row_zp(int64_t batch, int64_t M, int64_t N, int64_t K,
                                const void* A, qg_dtype a_dtype, int64_t lda, int64_t a_batch_stride,
                                const void* B, qg_dtype b_dtype, int64_t ldb, int64_t b_batch_stride,
                                const void* a_zero_point, int64_t a_zero_point_len,
                                const void* b_zero_point, int64_t b_zero_point_len,
                                int32_t* Y, int64_t ldy, int64_t y_batch_stride,
                                void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * DynamicQuantizeLinear to uint8 ("feat(onnx-to-hip): lower quantized
 * integer conv and matmul", section "What", DynamicQuantizeLinear paragraph),
 * the step that produces MatMulInteger's uint8 activations and their zero
 * point:
 *
 *   lo = min(0, min_i x[i])      hi = max(0, max_i x[i])
 *   scale = (hi - lo) / 255,  replaced by 1 when it is 0
 *   zp = clamp(round_half_even(0 - lo / scale), 0, 255)
 *   y[i] = clamp(round_half_even(x[i] / scale) + zp, 0, 255)
 *
 * every step an fp32 operation rounded to nearest even (the division
 * correctly rounded).  The page fixes the scale, the zero-range case and the
 * ties-to-even zero point; widening the range to include 0 and saturating
 * are the ONNX operator's definition the page lowers.  Bit-exact.
 *   x: n fp32 values, contiguous, finite (NaN or Inf is outside the contract).
 *   y: n uint8 values, contiguous.  n == 0 is allowed: scale 1, zp 0.
 *   y_scale: device pointer to one fp32; y_zero_point: device pointer to one
 *     uint8.  They may feed matmul_integer_row_zp directly (a_zero_point_len
 *     1) with no host round trip.
 *   workspace: device memory of at least
 *     qgemm_workspace_bytes(QG_OP_DYNAMIC_QUANTIZE_LINEAR, 1, 1, n, 1)
 *     bytes (at most 2 KiB), 8-byte aligned; needs no initialisation and
 *     holds nothing after the call.  Calls that overlap in time must not
 *     share one.
 * Two kernels on `stream`: a min/max pass, then a quantize pass.
 * QG_ERR_INVALID_ARGUMENT for n < 0 or a NULL pointer (x and y may be NULL
 * when n == 0); QG_ERR_WORKSPACE for a short workspace.
 */
qg_status dynamic_quantize_linear(int64_t n, const float* x, uint8_t* y,
                                  float* y_scale, uint8_t* y_zero_point,
                                  void* workspace, size_t workspace_bytes,
                                  void* stream);

/*
 * ConvInteger ("feat(onnx-to-hip): lower quantized integer conv and matmul",
 * section "What", ConvInteger paragraph; the grouped, padded, strided case of
 * its GPU numeric tests):
 *
 *   y[n, m, oh, ow] = wrap32( sum_{c < C/group, kh, kw}
 *       (x[n, g*(C/group) + c, oh*sh - pt + kh*dh, ow*sw - pl + kw*dw] - x_zp)
 *       * (w[m, c, kh, kw] - w_zp[m]) ),   g = m / (M/group)
 *
 * summed exactly and stored as a wrapping int32 (the page's int64-then-wrap
 * result for any reduction length).  A tap outside the input contributes
 * nothing: the input is padded with its own zero point (the page's lowering
 * subtracts the zero point, then convolves with zero padding).  Bit-exact.
 *   x: x_dtype QG_UINT8 or QG_INT8, [N, C, H, W] contiguous.  A rank-3 NCL
 *      input is H = 1 (kH = 1, pads[0] = pads[2] = 0).
 *   w: w_dtype QG_UINT8 or QG_INT8, [M, C/group, kH, kW] contiguous.
 *   group >= 1 divides C and M.
 *   pads: host int64[4] = {top, left, bottom, right} >= 0;
 *   strides, dilations: host int64[2] = {h, w} >= 1.
 *   OH = (H + top + bottom - dilations[0]*(kH-1) - 1) / strides[0] + 1 >= 1,
 *   OW likewise.
 *   x_zero_point: scalar within x_dtype's range.
 *   w_zero_point: device pointer to w_dtype values, NULL (all zero,
 *      w_zero_point_len 0), or w_zero_point_len 1 (scalar) or M (one per
 *      output channel).
 *   y: int32 [N, M, OH, OW] contiguous.
 *   workspace: device memory of at least conv_integer_workspace_bytes(...)
 *      bytes, 256-byte aligned, no initialisation needed; it receives the
 *      packed weight and the column matrices.  Calls that overlap in time
 *      must not share one.
 * Kernels on `stream`: a weight pack, an im2col gather, and one batched int8
 * matrix-core GEMM per group.  Requires N < 65536.  QG_ERR_INVALID_ARGUMENT:
 * a bad size, dtype, zero point, pointer or alignment; QG_ERR_WORKSPACE: a
 * short workspace; QG_ERR_UNSUPPORTED: one image's column matrix or one
 * group's weight spans 2^31 bytes.
 */
qg_status conv_integer(int64_t N, int64_t C, int64_t H, int64_t W,
                       const void* x, qg_dtype x_dtype,
                       int64_t M, int64_t kH, int64_t kW,
                       const void* w, qg_dtype w_dtype,
                       int64_t group,
                       const int64_t* pads, const int64_t* strides, const int64_t* dilations,
                       int32_t x_zero_point,
                       const void* w_zero_point, int64_t w_zero_point_len,
                       int32_t* y,
                       void* workspace, size_t workspace_bytes,
                       void* stream);

/* Workspace bytes conv_integer needs for these sizes (0: sizes invalid). */
size_t conv_integer_workspace_bytes(int64_t N, int64_t C, int64_t H, int64_t W,
                                    int64_t M, int64_t kH, int64_t kW, int64_t group,
                                    const int64_t* pads, const int64_t* strides,
                                    const int64_t* dilations);

/* Workspace bytes the fastest kernel for this shape wants (0: none).  For
 * QG_OP_DYNAMIC_QUANTIZE_LINEAR, N is the element count n. */
size_t qgemm_workspace_bytes(int op, int64_t batch, int64_t M, int64_t N, int64_t K);

/* Static text for a status code. */
const char* qgemm_status_string(qg_status s);

/* Name of the kernel the calling thread's last successful call launched
 * (static text; "" before the first launch).  It lets a test or benchmark
 * assert which kernel actually ran: "feat(PULPOpen): matmul that dequantises
 * an int8 weight in-kernel" retracts its own measurement in a later comment
 * because the intended int8 kernel was never emitted, and the fp32 kernel
 * that ran instead read the int8 weight as float. */
const char* qgemm_last_kernel(void);

/* Library version string. */
const char* qgemm_version(void);

/*
 * Calibration (diagnostics for the roofline figures; no part of the
 * quantised matmuls).  They measure the ceilings the kernels above are held
 * to on the machine at hand.  Both write QG_CALIB_SINK_WORDS uint32 words to
 * the device buffer `sink` (only so that the work is kept) and are
 * asynchronous on `stream`.
 *
 * qgemm_calib_read: reads `bytes` bytes of device memory at `buf` once,
 *   each workgroup one contiguous share as non-temporal 16-byte vectors.  buf 16-byte aligned, bytes a
 *   positive multiple of 16; otherwise QG_ERR_INVALID_ARGUMENT.
 * qgemm_calib_mfma_i8: runs `iters` (1 .. 2^20) rounds of int8 matrix-core
 *   multiplies (v_mfma_i32_16x16x64_i8, 16 independent per wave per round)
 *   on operands read once from `operands`, a device buffer of 4096 bytes;
 *   the operand bytes set how much the data paths toggle and hence the clock
 *   the chip holds.  *ops_out (host) receives the int8 operations performed
 *   (2 per multiply-add): QG_CALIB_MFMA_OPS_PER_ROUND * iters.
 * qgemm_calib_mfma_i8_32x32: the same int8 work (same operands, same
 *   *ops_out) with v_mfma_i32_32x32x32_i8, which does twice the operations
 *   of the 16x16x64 form per operand byte read.
 * qgemm_calib_mfma_f32: the same with fp32 matrix-core multiplies
 *   (v_mfma_f32_16x16x4_f32, the W8A32 kernels' instruction) on 1024 fp32
 *   operands (4096 bytes) that should lie in [-1, 1];
 *   *flops_out (host) receives QG_CALIB_MFMA_F32_FLOPS_PER_ROUND * iters.
 * qgemm_calib_mfma_bf16: the same with bf16 matrix-core multiplies
 *   (v_mfma_f32_16x16x32_bf16, the instruction of the W8A32 kernels' exact
 *   bf16 split) on 2048 bf16 operands (4096 bytes) that should lie in
 *   [-1, 1]; *flops_out (host) receives
 *   QG_CALIB_MFMA_BF16_FLOPS_PER_ROUND * iters.
 */
#define QG_CALIB_SINK_WORDS 8192
#define QG_CALIB_MFMA_OPS_PER_ROUND 4294967296LL
#define QG_CALIB_MFMA_F32_FLOPS_PER_ROUND 268435456LL
#define QG_CALIB_MFMA_BF16_FLOPS_PER_ROUND 2147483648LL
qg_status qgemm_calib_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);
qg_status qgemm_calib_mfma_i8(const void* operands, int iters, uint32_t* sink, void* stream,
                              int64_t* ops_out);
qg_status qgemm_calib_mfma_i8_32x32(const void* operands, int iters, uint32_t* sink, void* stream,
                                    int64_t* ops_out);
qg_status qgemm_calib_mfma_f32(const void* operands, int iters, uint32_t* sink, void* stream,
                               int64_t* flops_out);
qg_status qgemm_calib_mfma_bf16(const void* operands, int iters, uint32_t* sink, void* stream,
                                int64_t* flops_out);

#ifdef __cplusplus
}
#endif

#endif /* QGEMM_H */

"""MI355X-native quantised matrix multiplies.

The C-ABI library ``libqgemm.so`` (HIP kernels for gfx950) does the work;
this package is its thin Python binding, with the same call names:

* ``qgemm_w8a32(A, W, scale, zero_point=0)``: fp32 x int8 weight with a
  per-tensor scale and zero point, dequantisation folded into the epilogue
  (bf16 matrix cores on an exact three-way split of A; QGEMM_W8A32=fp32
  selects the fp32 matrix cores).
* ``qgemm_w8a32_input_grad(dC, W, scale, zero_point=0)``: its gradient
  with respect to the activations, W in its forward layout.
* ``qgemm_a8w8(A, W, act_scale, weight_scale, out_dtype=torch.float32)``:
  int8 x int8 with int32 accumulation, per-row and per-column fp32 scales,
  fp32 or bf16 output.
* ``qgemm_a8w8_acc(acc_in, A, W, act_scale, weight_scale, ...)``: the same
  with an int32 accumulator input added before the cast.
* ``qgemm_a8w8_noalloc(A, W, act_scale, weight_scale, ...)``: qgemm_a8w8
  for callers that cannot allocate (its decode scratch is a static array).
* ``matmul_integer(A, B, a_zero_point=0, b_zero_point=None)``: ONNX
  MatMulInteger, int32 output, shared weight never copied; per-row
  activation zero points go to ``matmul_integer_row_zp``.
* ``conv_integer(x, w, x_zero_point, w_zero_point, pads, strides,
  dilations, group)``: ONNX ConvInteger (NCHW / NCL), int32 output.
* ``dynamic_quantize_linear(x)``: ONNX DynamicQuantizeLinear to uint8,
  returning (y, scale, zero_point) on the device.

``calib_read``, ``calib_mfma_i8``, ``calib_mfma_f32`` and ``calib_mfma_bf16``
measure the machine's HBM read and int8, fp32 and bf16 matrix-core ceilings
for the roofline figures.
"""
from ._binding import (  # noqa: F401
    LIB_PATH,
    QG_OP_A8W8,
    QG_OP_MATMUL_INTEGER,
    QG_OP_DYNAMIC_QUANTIZE_LINEAR,
    QG_OP_W8A32,
    QG_OP_W8A32_INPUT_GRAD,
    QGemmError,
    calib_mfma_bf16,
    calib_mfma_f32,
    calib_mfma_i8,
    calib_read,
    conv_integer,
    dynamic_quantize_linear,
    last_kernel,
    matmul_integer,
    matmul_integer_row_zp,
    qgemm_a8w8,
    qgemm_a8w8_acc,
    qgemm_a8w8_noalloc,
    qgemm_w8a32,
    qgemm_w8a32_input_grad,
    status_string,
    version,
    workspace_bytes,
)

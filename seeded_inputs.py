"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers: it holds none of the operators'
arithmetic, and both the oracle and the HIP path receive its arrays as
inputs.  Distributions follow the workloads the operators are measured on:

* W8A32: activations ~ N(0, 1) in fp32; int8 weight uniform over
  [-128, 127]; a per-tensor scale and integer zero point given by the caller.
* A8W8: int8 activations and weights uniform over [-127, 127]; fp32 row and
  column scales uniform over [0.001, 0.05).
* MatMulInteger: uint8 activations uniform over [0, 255]; int8 weight uniform
  over [-128, 127]; per-column int8 weight zero points uniform over [-8, 8].
* ConvInteger: uint8 activations uniform over [0, 255]; int8 weight uniform
  over [-128, 127]; per-output-channel int8 weight zero points uniform over
  [-8, 8] (the MatMulInteger recipe on a convolution's operands).
* DynamicQuantizeLinear: fp32 activations ~ N(mean, std) of the shape of
  MatMulInteger's activations, which it produces.

Every generator takes an explicit seed and uses numpy's PCG64 generator, so a
given (shape, seed) always yields the same bytes.
"""
import numpy as np


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def randint(g, shape, lo, hi, dtype):
    """Integers uniform over [lo, hi] inclusive."""
    return g.integers(lo, hi, size=shape, dtype=dtype, endpoint=True)


def w8a32_inputs(M, N, K, seed):
    g = rng(seed)
    A = g.standard_normal((M, K), dtype=np.float32)
    W = randint(g, (K, N), -128, 127, np.int8)
    return A, W


def a8w8_inputs(M, N, K, seed, lo=-127, hi=127):
    g = rng(seed)
    A = randint(g, (M, K), lo, hi, np.int8)
    W = randint(g, (K, N), lo, hi, np.int8)
    act_scale = g.uniform(0.001, 0.05, size=M).astype(np.float32)
    weight_scale = g.uniform(0.001, 0.05, size=N).astype(np.float32)
    return A, W, act_scale, weight_scale


def matmul_integer_inputs(batch, M, N, K, seed, a_dtype=np.uint8, b_dtype=np.int8,
                          shared_b=True):
    g = rng(seed)
    a_lo, a_hi = (0, 255) if a_dtype == np.uint8 else (-128, 127)
    b_lo, b_hi = (0, 255) if b_dtype == np.uint8 else (-128, 127)
    A = randint(g, (batch, M, K), a_lo, a_hi, a_dtype)
    B = randint(g, (K, N) if shared_b else (batch, K, N), b_lo, b_hi, b_dtype)
    if b_dtype == np.int8:
        zb = randint(g, (N,), -8, 8, np.int8)
    else:
        zb = randint(g, (N,), 120, 136, np.uint8)
    return A, B, zb


def dql_inputs(shape, seed, mean=0.0, std=1.0):
    g = rng(seed)
    x = g.standard_normal(shape, dtype=np.float32)
    return (x * np.float32(std) + np.float32(mean)).astype(np.float32)


def conv_integer_inputs(N, C, H, W, M, kH, kW, seed, group=1):
    g = rng(seed)
    x = randint(g, (N, C, H, W), 0, 255, np.uint8)
    w = randint(g, (M, C // group, kH, kW), -128, 127, np.int8)
    zw = randint(g, (M,), -8, 8, np.int8)
    return x, w, zw

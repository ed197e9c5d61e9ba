"""Helpers for the GPU parity tests: device transfer and comparisons."""
import os
import sys

import numpy as np
import pytest
import torch


def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def to_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev())


def bf16_bits(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def case(msg):
    """Name the case on stderr before touching the GPU (survives a crash)."""
    sys.stderr.write(f"[case] {msg}\n")
    sys.stderr.flush()


def ulp_diff_f32(a, b):
    """|a - b| in units in the last place, via the ordered integer map."""
    ai = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    bi = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    ai = np.where(ai < 0, np.int64(-2 ** 31) - ai, ai)
    bi = np.where(bi < 0, np.int64(-2 ** 31) - bi, bi)
    return np.abs(ai - bi)


def ulp_diff_bf16(a, b):
    return ulp_diff_f32((np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32),
                        (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)) >> 16


class env:
    """Temporarily set environment variables (read by the library per call)."""

    def __init__(self, **kw):
        self.kw = kw

    def __enter__(self):
        self.old = {k: os.environ.get(k) for k in self.kw}
        for k, v in self.kw.items():
            os.environ[k] = str(v)

    def __exit__(self, *a):
        for k, v in self.old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


# W8A32 runs on the bf16 matrix cores with an exact three-way split of its
# fp32 operand (the default) or on the fp32 matrix cores (QGEMM_W8A32=fp32);
# the parity tests run both.
W8A32_PATHS = ("bf16x3", "fp32")


def w8a32_kernel(path, rows, outs, grad=False, k=0):
    """Kernel name the library reports for a W8A32 call of `rows` x `outs`
    outputs over a contraction of `k` on `path`, through the binding (which
    passes a workspace): for the gradient with at most 8 rows across 8192
    outputs or more, the slab kernel; the decode kernel for at most 64 rows, else 256 x
    256 split tiles from 129 of them on, else 128 x 128 tiles, the
    contraction divided among workgroups when there are at most 256 of
    those and it allows two or more pieces of 512."""
    if path == "fp32":
        return "w8a32_input_grad_128x128" if grad else "w8a32_tiled_128x128"
    # the gradient's slab form: at most 8 rows across at least 8192 outputs
    forced = os.environ.get("QGEMM_FORCE_KERNEL")
    if grad and k % 16 == 0 and forced not in ("tiled", "skinny") and \
            ((rows <= 8 and outs >= 8192) or (forced == "slab" and rows <= 16)):
        return "w8a32_input_grad_slab"
    # contiguous operands: the weight's rows (N bytes) 16-byte aligned when
    # N % 16 == 0; N is `outs` forward and the contraction `k` for the gradient
    if rows <= 64 and k % 4 == 0 and (k if grad else outs) % 16 == 0 and \
            os.environ.get("QGEMM_FORCE_KERNEL") != "tiled":
        return "w8a32_input_grad_skinny" if grad else "w8a32_skinny"
    if ((rows + 255) // 256) * ((outs + 255) // 256) > 128:
        tile = "256x256"
    else:
        tile = "128x128"
        tiles = ((rows + 127) // 128) * ((outs + 127) // 128)
        splits = int(os.environ.get("QGEMM_W8A32_SPLITS", "0")) or min(512 // tiles, k // 512, 8)
        if tiles <= 256 and splits >= 2:
            chunks = (k + 31) // 32
            per = (chunks + splits - 1) // splits
            if (chunks + per - 1) // per >= 2:
                tile += "_splitk"
    return f"w8a32_input_grad_bf16x3_{tile}" if grad else f"w8a32_bf16x3_{tile}"


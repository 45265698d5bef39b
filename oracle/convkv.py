"""ConvKV temporal-conv memory, fp64.

SoulX-LiveAct page, section 技术内核, ConvKV Memory bullet: older frames are
compressed along time by a 1D convolution (ratio up to 5:1) into memory of
fixed length.  Readings: depthwise per head and channel, valid (no padding),
stride = kernel, no bias; separate weights for K and V; K is compressed
before any RoPE (positions are reset afterwards); tap i multiplies the i-th
oldest frame of its group.

    mem[j, h, s, c] = sum_{i < kernel} w[h, c, i] * frames[j * stride + i, h, s, c]
"""
from __future__ import annotations

import numpy as np


def conv_memory(frames, w, stride: int | None = None) -> np.ndarray:
    """frames [n_in, H, S, D] oldest first, w [H, D, kernel] -> memory [n_out, H, S, D] fp64."""
    frames = np.asarray(frames, np.float64)
    w = np.asarray(w, np.float64)
    kernel = w.shape[-1]
    stride = kernel if stride is None else stride
    n_in = frames.shape[0]
    n_out = (n_in - kernel) // stride + 1 if n_in >= kernel else 0
    out = np.zeros((n_out,) + frames.shape[1:], np.float64)
    for j in range(n_out):
        for i in range(kernel):
            out[j] += w[:, None, :, i] * frames[j * stride + i]
    return out

"""3D rotary position embedding, fp64.

The pages say only that ConvKV resets RoPE positions (SoulX-LiveAct page,
section 技术内核, ConvKV Memory bullet) and give no RoPE convention.  The
reading taken, the plainest standard one:
  * head channels split into three contiguous groups [t | h | w] of sizes
    (D_t, D_h, D_w), each even, summing to D (all zero = no RoPE);
  * within a group of size D_a at channel offset o_a, pair i = (o_a+2i,
    o_a+2i+1) is rotated by angle pos_a * theta**(-2i / D_a):
        (u, u') -> (u cos phi - u' sin phi, u sin phi + u' cos phi);
  * theta = 10000, no scaling; applied to Q and K, never to V.
"""
from __future__ import annotations

import numpy as np


def rope_frequencies(dim: int, theta: float = 10000.0) -> np.ndarray:
    """omega_i = theta ** (-2 i / dim), i < dim / 2, fp64."""
    i = np.arange(dim // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * i / dim)


def apply_rope(x, pos_t, pos_h, pos_w, split, theta: float = 10000.0) -> np.ndarray:
    """Rotate x [N, H, D] (any float) at per-token positions; returns fp64 [N, H, D]."""
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    if sum(split) == 0:
        return out
    D = x.shape[-1]
    if sum(split) != D or any(s % 2 for s in split):
        raise ValueError("RoPE split must be even parts summing to head_dim")
    off = 0
    for size, pos in zip(split, (pos_t, pos_h, pos_w)):
        if size:
            omega = rope_frequencies(size, theta)
            phi = np.asarray(pos, np.float64)[:, None] * omega[None, :]        # [N, size/2]
            c = np.cos(phi)[:, None, :]
            s = np.sin(phi)[:, None, :]
            u0 = x[:, :, off + 0:off + size:2]
            u1 = x[:, :, off + 1:off + size:2]
            out[:, :, off + 0:off + size:2] = u0 * c - u1 * s
            out[:, :, off + 1:off + size:2] = u0 * s + u1 * c
        off += size
    return out

"""Softmax attention over the bounded context, fp64.

LiveAnimate page, section 方法: the bidirectional DiT is turned into a
block-causal generator in which each block depends only on the reference and
already generated blocks; at inference, attention reads the PR-Sink context.
Readings: inside the context there is no mask (the current block attends to
itself in full); scale 1/sqrt(D) unless given; no bias, no dropout.

    o_i = sum_j exp(z_ij - max_j z_ij) v_j / sum_j exp(z_ij - max_j z_ij),
    z_ij = scale * q_i . k_j
"""
from __future__ import annotations

import numpy as np


def softmax_weights(q, k, scale: float) -> np.ndarray:
    """Weights [Nq, Nk] of one head, fp64."""
    z = (np.asarray(q, np.float64) @ np.asarray(k, np.float64).T) * scale
    z -= z.max(axis=1, keepdims=True)
    p = np.exp(z)
    return p / p.sum(axis=1, keepdims=True)


def attention(q, k, v, scale: float | None = None, heads=None, rows=None) -> np.ndarray:
    """o [Nq, H, D] for q [Nq, H, D], k, v [Nk, H, D]; fp64.

    ``heads``/``rows`` restrict the work to a subset (others are left zero).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    Nq, H, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.zeros((Nq, H, v.shape[-1]), np.float64)
    hs = range(H) if heads is None else heads
    rs = np.arange(Nq) if rows is None else np.asarray(rows)
    for h in hs:
        for c0 in range(0, len(rs), 256):            # query chunks bound the [chunk, Nk] buffer
            r = rs[c0:c0 + 256]
            p = softmax_weights(q[r, h, :], k[:, h, :], scale)
            out[r, h, :] = p @ v[:, h, :]
    return out


def masked_attention(q, k_all, v_all, mask, scale: float | None = None, heads=None) -> np.ndarray:
    """Dense attention of q over all keys with a boolean mask [Nq, Nk_all] (True = visible)."""
    q = np.asarray(q, np.float64)
    k_all = np.asarray(k_all, np.float64)
    v_all = np.asarray(v_all, np.float64)
    Nq, H, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.zeros((Nq, H, D), np.float64)
    for h in (range(H) if heads is None else heads):
        z = (q[:, h, :] @ k_all[:, h, :].T) * scale
        z = np.where(mask, z, -np.inf)
        z -= z.max(axis=1, keepdims=True)
        p = np.exp(z)
        p /= p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ v_all[:, h, :]
    return out

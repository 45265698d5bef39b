"""QKV projection of a block's hidden states, fp64 (test infrastructure).

The LiveAnimate page (section 方法) reaches its frame rate with operator
fusion, and the SoulX-LiveAct page (section 上手实践) offers a fused-QKV build;
neither writes the operation out.  Reading taken here: an attention layer's q,
k and v are the plain linear projection of the block's hidden states,

    [q | k | v] = x W^T + b,

with x [T, C], W [3*heads*head_dim, C] whose rows are the q heads' features,
then the k heads', then the v heads' (head-major, a head's head_dim rows
together), and an optional bias b [3*heads*head_dim].  A fused path must
equal the unfused path fed with these q, k and v.

With bf16 activations the unfused path receives q, k and v in bf16, so the
projection's results are rounded to bf16 (nearest, ties to even) where they
leave it: ``qkv_projection(..., round_bf16=True)``.
"""
from __future__ import annotations

import numpy as np


def bf16_round(x) -> np.ndarray:
    """Nearest bf16 value (8 significant bits, ties to even) of each finite
    element, computed from its fp64 value; returned as fp64."""
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)                                 # x = m * 2^e, |m| in [0.5, 1)
    return np.ldexp(np.round(np.ldexp(m, 8)), e - 8)  # numpy rounds halves to even


def qkv_projection(x, w, b, heads: int, head_dim: int, round_bf16: bool = False):
    """q, k, v, each [T, heads, head_dim] fp64 (rounded to bf16 values when
    round_bf16)."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    n = heads * head_dim
    if w.shape != (3 * n, x.shape[1]):
        raise ValueError(f"w has shape {w.shape}, expected {(3 * n, x.shape[1])}")
    y = x @ w.T                                        # a library matmul, one step
    if b is not None:
        y = y + np.asarray(b, np.float64)[None, :]
    if round_bf16:
        y = bf16_round(y)
    T = x.shape[0]
    return tuple(y[:, i * n:(i + 1) * n].reshape(T, heads, head_dim) for i in range(3))

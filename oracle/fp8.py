"""FP8 (OCP E4M3) quantisation of attention keys and queries, fp64 (test infrastructure).

The SoulX-LiveAct page (section 关键信息速览, and its 上手实践 deployment notes)
runs attention in FP8 but fixes no scheme.  Reading taken here, for the PR-Sink
cache mode with an FP8 key cache:

  * K after RoPE is stored as E4M3 with one power-of-two scale per (head,
    64-token tile of a block).
  * Q after RoPE, times softmax_scale * log2(e), is quantised the same way with
    one scale per (query token, head).
  * Q K^T uses the quantised values.  V, the softmax and P V are unchanged.

E4M3 (OCP "fn" variant): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
bits, no infinities; the largest finite magnitude is 448 and subnormals are
m * 2^-9 (m = 1..7).  Rounding is to nearest, ties to even.

Power-of-two scale of a group whose largest magnitude is a > 0: the smallest
integer e with a * 2^-e <= 448 (e = 0 for an all-zero group), clamped to
[-120, 120].  Dividing by 2^e is exact, so every value is rounded once, and
dequantisation x8 * 2^e is exact in fp64.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
SCALE_LIMIT = 120


def e4m3_round(x) -> np.ndarray:
    """Nearest E4M3 value of each element (ties to even), as fp64.

    Elements must lie within [-448, 448] (the scale rule guarantees it)."""
    x = np.asarray(x, np.float64)
    if np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("value outside the E4M3 range")
    a = np.abs(x)
    # quantum of the binade: 2^(E - 3) for normal values (E = floor(log2 a)),
    # 2^-9 for the subnormal range a < 2^-6
    _, ex = np.frexp(np.where(a > 0, a, 1.0))          # a = f * 2^ex, f in [0.5, 1)
    e_floor = ex - 1
    quantum = np.where(a >= 2.0 ** -6, np.ldexp(1.0, e_floor - 3), 2.0 ** -9)
    n = np.round(a / quantum)                          # numpy rounds halves to even
    return np.copysign(n * quantum, x)


def pow2_exponents(amax) -> np.ndarray:
    """Smallest integer e with amax * 2^-e <= 448, elementwise (0 where amax =
    0), clamped to [-120, 120]."""
    a = np.asarray(amax, np.float64)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))          # a = f * 2^ex, f in [0.5, 1)
    e = (ex - 1) - 8                                   # a * 2^-e in [256, 512)
    e = np.where(a * np.ldexp(1.0, -e) > E4M3_MAX, e + 1, e)
    e = np.where(a > 0, e, 0)
    return np.clip(e, -SCALE_LIMIT, SCALE_LIMIT).astype(np.int64)


def pow2_exponent(amax: float) -> int:
    return int(pow2_exponents(np.array([amax]))[0])


def quantize_keys(k_rot) -> np.ndarray:
    """Dequantised E4M3 K [T, H, D] of one block: one scale per (64-token
    tile, head)."""
    k = np.asarray(k_rot, np.float64)
    T, H, D = k.shape
    nt = (T + 63) // 64
    pad = np.zeros((nt * 64, H, D))
    pad[:T] = k
    amax = np.abs(pad).reshape(nt, 64, H, D).max(axis=(1, 3))          # [nt, H]
    sc = np.ldexp(1.0, pow2_exponents(amax))                            # [nt, H]
    sc_tok = np.repeat(sc, 64, axis=0)[:T][:, :, None]                  # [T, H, 1]
    return e4m3_round(k / sc_tok) * sc_tok


def quantize_queries(q_scaled) -> np.ndarray:
    """Dequantised E4M3 Q [T, H, D] (rotated, times softmax_scale * log2 e):
    one scale per (token, head)."""
    q = np.asarray(q_scaled, np.float64)
    sc = np.ldexp(1.0, pow2_exponents(np.abs(q).max(axis=2)))[:, :, None]
    return e4m3_round(q / sc) * sc

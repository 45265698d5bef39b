"""FP8 (OCP E4M3) quantisation inside attention, fp64 (test infrastructure).

The SoulX-LiveAct page (section 关键信息速览, and its 上手实践 deployment notes,
which offer an FP8 KV cache) runs attention in FP8 but fixes no scheme.
Reading taken here:

  * FP8 key cache: K after RoPE is stored as E4M3 with one power-of-two scale
    per (head, 64-token tile of a context segment, counted from the segment's
    first token).
  * Q after RoPE, times softmax_scale * log2(e), is quantised the same way with
    one scale per (query token, head).  The base-2 logits are the products of
    these E4M3 values; P = 2^(logit - row max) is the softmax's numerator.
  * Q K^T uses the quantised values.  With the key cache alone, V, the
    softmax and P V are unchanged.
  * FP8 KV cache (``attention_fp8_pv``): V is stored as E4M3 with the key
    cache's tile rule (one power-of-two scale per head and 64-token tile of a
    segment, over all channels), and the softmax numerator P_j = 2^(z_j) (z
    the base-2 logit, so P_j = exp of the natural logit) is held as E4M3 with
    the same rule applied to each query row over its whole context: one
    power-of-two scale 2^e per row, the smallest with max_j P_j * 2^-e <= 448.
    o = sum_j P~_j v_j / sum_j P_j; the denominator sums the unrounded P.
    (The codes are those of 2^(z_j - e): a whole-number shift of z, not a
    shift by the row max itself, which would change every code.)

  * Comparing a library's FP8-KV output with this reading: the library forms
    the logits with the FP8 matrix product, whose sum of E4M3 products is not
    exact, so a P whose exact value lies within that error of a rounding
    boundary between two E4M3 codes has two valid codes, and no CPU reading
    can know which one the matrix core's rounding picks.
    ``attention_fp8_pv_slack`` bounds how far each output may move from such
    codes; outputs are compared beyond that slack (zero for a row with no
    such P).

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


def quantize_values(v) -> np.ndarray:
    """Dequantised E4M3 V [T, H, D] of one context segment: the key cache's
    tile rule (one scale per 64-token tile and head, over all channels)."""
    return quantize_keys(v)


def numerators_e4m3(z):
    """For base-2 logits z [N, Nk]: P = 2^z held as E4M3 with one
    power-of-two scale 2^e per row (the tile rule of ``pow2_exponents`` on the
    row's largest P = 2^max z).  Returns (P~ 2^-e, P 2^-e): the common factor
    2^-e keeps both in range and cancels in a ratio."""
    z = np.asarray(z, np.float64)
    P = np.exp2(z)                                     # logits well inside fp64's exponent range
    e = pow2_exponents(P.max(axis=1))[:, None]
    p = np.ldexp(P, -e)                                # exact: a power-of-two scaling
    return e4m3_round(p), p


# Bound on the FP8 matrix product's accumulation error in a logit, relative to
# sum_i |q_i k_i|: the exact product of two E4M3 values fits fp32, but the
# matrix core's sum of them is not exact.  Measured on MI355X (scaled E4M3
# matrix product, 128-term dot products of random E4M3 operands): at most
# 3.2e-5 of sum |q_i k_i|; the bound takes twice that, 2^-14.
FP8_PRODUCT_REL_ERR = 2.0 ** -14


def attention_fp8_pv_slack(q, k, v, rel=FP8_PRODUCT_REL_ERR, rows=None):
    """``attention_fp8_pv`` together with how far each output may move where
    the FP8 product's own rounding decides a P code.

    The logit z_j = q . k_j that the product delivers lies within
    b_j = rel * sum_i |q_i k_ij| of the exact one, so P_j (held as E4M3 under
    the row's power-of-two scale, ``numerators_e4m3``) may be rounded from any
    value in [p_j 2^-b_j, p_j 2^b_j].  Rounding is monotone, so the codes it
    can take run from round(p_j 2^-b_j) to round(p_j 2^b_j); a P away from
    every rounding boundary has one code, a P within b_j of a boundary two.
    The output o = sum_j P~_j v_j / sum_j P_j then moves by at most
    sum_j (round(p_j 2^b_j) - round(p_j 2^-b_j)) |v_j| / sum_j p_j per channel
    (the denominator sums unrounded P, which moves continuously and is left
    out).  Returns (o, slack), both [Nq, H, D] fp64."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    Nq, H, D = q.shape
    out = np.zeros((Nq, H, v.shape[-1]), np.float64)
    slack = np.zeros_like(out)
    rs = np.arange(Nq) if rows is None else np.asarray(rows)
    for h in range(H):
        for c0 in range(0, len(rs), 256):
            r = rs[c0:c0 + 256]
            z = q[r, h, :] @ k[:, h, :].T
            pq, p = numerators_e4m3(z)
            b = rel * (np.abs(q[r, h, :]) @ np.abs(k[:, h, :]).T)
            # Only a P whose interval reaches a rounding boundary beside its
            # code needs rounding again.  Above a code c the next code is one
            # quantum of c's binade up (none above 448); below, one quantum
            # down, or half a quantum where c is a power of two (taken there
            # also at 2^-6, where the true gap is wider); 2^-9 in the subnormal
            # range.  The boundaries lie half a gap from c, and the tests are
            # inclusive, so no P with two codes is missed.
            hi_end, lo_end = p * np.exp2(b), p * np.exp2(-b)
            frac, ex = np.frexp(np.where(pq > 0, pq, 1.0))
            quantum = np.where(pq >= 2.0 ** -6, np.ldexp(1.0, ex - 4), 2.0 ** -9)
            gap_up = np.where(pq >= E4M3_MAX, np.inf, quantum)
            gap_dn = np.where(pq <= 0.0, np.inf, np.where((frac == 0.5) & (pq >= 2.0 ** -6), 0.5 * quantum, quantum))
            near = (hi_end >= pq + 0.5 * gap_up) | (lo_end <= pq - 0.5 * gap_dn)
            step = np.zeros_like(p)
            if near.any():
                step[near] = (e4m3_round(np.minimum(hi_end[near], E4M3_MAX)) -
                              e4m3_round(lo_end[near]))
            l = p.sum(axis=1, keepdims=True)
            out[r, h, :] = (pq @ v[:, h, :]) / l
            slack[r, h, :] = (step @ np.abs(v[:, h, :])) / l
    return out, slack


def attention_fp8_pv(q, k, v, rows=None) -> np.ndarray:
    """o [Nq, H, D] for (already quantised) q and k and a quantised v, with
    base-2 logits z = q . k: P = 2^z held as E4M3 with one power-of-two
    scale per row (``numerators_e4m3``), o = sum_j P~_j v_j / sum_j P_j (the
    unrounded sum), fp64.  ``rows`` restricts the work to a subset of query
    rows (others zero)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    Nq, H, D = q.shape
    out = np.zeros((Nq, H, v.shape[-1]), np.float64)
    rs = np.arange(Nq) if rows is None else np.asarray(rows)
    for h in range(H):
        for c0 in range(0, len(rs), 256):
            r = rs[c0:c0 + 256]
            z = q[r, h, :] @ k[:, h, :].T
            pq, p = numerators_e4m3(z)
            out[r, h, :] = (pq @ v[:, h, :]) / p.sum(axis=1, keepdims=True)
    return out

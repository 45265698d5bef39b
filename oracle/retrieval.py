"""Pose retrieval for the dynamic sink, computed exactly.

LiveAnimate page, section 方法 (Dynamic Sink bullet) and section 局限 (the
retrieval is by pose similarity): the dynamic sink holds historical blocks
whose pose resembles the current one.  The page does not name the measure;
the reading taken is cosine similarity between the current block's pose and
each bank block's pose, top-k, ranked by (cosine descending, stream id
ascending) so exact ties go to the lower id.  A zero-norm vector scores 0,
and so does a pose holding a non-finite value (Inf or NaN: its cosine has no
value).  Fewer candidates than k: return all of them.

Exactness: every fp32 value is an integer multiple of 2**-149, so scaling by
2**149 turns the poses into Python integers and all dot products are exact.
cos(q, b) = d / (|q| |b|) is ranked through the strictly increasing map
x -> x|x|, i.e. by the exact rational d|d| / (|b|^2) (the common positive
factor 1/|q|^2 dropped).
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

_SCALE = 2.0 ** 149


def _as_ints(v):
    """The pose as exact integers, or None if it holds Inf or NaN."""
    a = np.asarray(v, dtype=np.float32).astype(np.float64)
    if not np.all(np.isfinite(a)):
        return None
    return [int(x) for x in a * _SCALE]                 # exact: power-of-two scaling


def exact_keys(query, bank: list) -> list:
    """Exact ranking key for each (id, pose) in ``bank``: Fraction d|d| / |b|^2;
    0 for zero norms and for non-finite poses."""
    q = _as_ints(query)
    qq = 0 if q is None else sum(x * x for x in q)
    keys = []
    for _, pose in bank:
        b = _as_ints(pose)
        bb = 0 if b is None else sum(x * x for x in b)
        if qq == 0 or bb == 0:
            keys.append(Fraction(0))
            continue
        d = sum(x * y for x, y in zip(q, b))
        keys.append(Fraction(d * abs(d), bb))
    return keys


def retrieve(query, bank: list, k: int) -> list:
    """Top-min(k, len(bank)) stream ids of ``bank`` = [(id, pose[P] fp32), ...]."""
    keys = exact_keys(query, bank)
    order = sorted(range(len(bank)), key=lambda i: (-keys[i], bank[i][0]))
    return [bank[i][0] for i in order[:min(k, len(bank))]]


def boundary_gap(query, bank: list, k: int):
    """Relative exact gap between the k-th and (k+1)-th ranked keys (None if no boundary).

    Used by tests to reject generator streams whose ranking would hinge on a
    difference below fp64 resolution (exact ties, gap 0, are legitimate).
    """
    if len(bank) <= k or k == 0:
        return None
    keys = sorted(exact_keys(query, bank), reverse=True)
    a, b = keys[k - 1], keys[k]
    if a == b:
        return Fraction(0)
    den = max(abs(a), abs(b))
    return abs(a - b) / den


def fp64_cosines(query, poses) -> np.ndarray:
    """Plain fp64 cosines (an independent check used by the tests on tie-free data)."""
    q = np.asarray(query, np.float64)
    P = np.asarray(poses, np.float64)
    nq = np.linalg.norm(q)
    nb = np.linalg.norm(P, axis=1)
    with np.errstate(invalid="ignore", divide="ignore"):
        c = (P @ q) / (nb * nq)
    c[(nb == 0) | (nq == 0)] = 0.0
    return c

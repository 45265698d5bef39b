"""Whole-block references: schedule -> retrieval -> RoPE -> attention (-> ConvKV memory).

A *provider* hands the oracle the stream's inputs, exactly as the GPU path got
them: ``provider.qkv(layer, block, step) -> (q, k, v)`` each [T, H, D];
``provider.pose(block) -> [P]``; ``provider.conv_weights(layer) -> (wk, wv)``;
``provider.reference(layer) -> (k, v)`` each [R * grid_h * grid_w, H, D].
The oracle keeps no cache: a context block's K/V are asked for again when
needed, which keeps memory flat and the code short.

Readings (beyond those stated in the modules used here):
  * PR-Sink positions are absolute: token (f, y, x) of block b sits at
    t = b * frames + f.  Cached keys keep the position they were written at.
  * The block's retrieval uses its own pose, once, before its first step; all
    layers and steps share the result.
  * With several sampling steps per block (LiveAnimate page, section 方法:
    three steps), a committed block contributes the K/V of its last step.
  * ConvKV context order is [memory frames, window blocks oldest first,
    current block]; temporal positions run 0, 1, 2, ... over those frames.
  * The ConvKV memory frame is cached like every other K and V, in the
    cache's element type: a bf16 cache (dtypes "bf16", "bf16_fp8k",
    "bf16_fp8kv") holds the conv output rounded to bf16 (nearest, ties to
    even); the FP8 caches quantise that held value.
  * An FP8 key cache (dtype "bf16_fp8k", either policy): the rotated K of
    each context segment and Q are quantised to E4M3 as ``fp8`` states (K in
    64-token tiles counted from the segment's first token) before Q K^T; V
    and the softmax are unchanged.  For ConvKV the memory frames, window
    blocks and current block are the segments (the SoulX-LiveAct page runs
    its ConvKV attention in FP8, sections 关键信息速览 and 上手实践).
  * An FP8 KV cache (dtype "bf16_fp8kv"): as the key cache, and V of each
    segment quantised with the same tile rule, and P rounded to E4M3 against
    the exact row max before P V (``fp8.attention_fp8_pv``; the same page's
    上手实践 notes offer an FP8 KV cache).  ``attend(..., with_slack=True)``
    also returns how far each output may move where the FP8 product's own
    rounding decides a P code (``fp8.attention_fp8_pv_slack``).
  * PR-Sink with reference_frames = R > 0 (the LiveAnimate page, section 方法,
    conditions every block on the reference image; the Live Avatar page's
    abstract recalibrates appearance from a cached reference image): the R
    reference frames are a permanent first context segment at temporal
    positions 0..R-1, and generated frame f of block b moves to t = R + b *
    frames + f.  R = 0 is the plain reading above.
  * PR-Sink with positions = "relative" (the alternative to absolute
    positions: the SoulX-LiveAct page, section 技术内核, restarts RoPE over
    the retained context for ConvKV): the context's blocks keep their temporal
    order with the gaps between them removed -- the i-th context block by
    stream id (static, retrieved, window, current) has its frame f at
    t = R + i * frames + f.  Keys are rotated per block at these positions,
    not once at append.
  * PR-Sink with bank_policy = "pose": the bank follows
    ``iter_prsink_pose_bank`` (pose-aware replacement) instead of FIFO.
  * ConvKV with positions = "absolute" (the literal alternative of the same
    passage: only the memory's positions restart): memory frame j at t = j,
    window and current blocks at their absolute t = b * frames + f.
"""
from __future__ import annotations

import numpy as np

from . import fp8
from .attention import attention
from .convkv import conv_memory
from .projection import bf16_round
from .retrieval import retrieve
from .rope import apply_rope
from .schedule import convkv_schedule, iter_prsink_pose_bank, prsink_schedule, token_positions


def _scale(cfg):
    s = cfg.get("softmax_scale", 0.0) or 0.0
    return float(s) if s > 0 else 1.0 / np.sqrt(cfg["head_dim"])


class _Base:
    def __init__(self, cfg: dict, provider):
        self.cfg = cfg
        self.p = provider
        F, gh, gw = cfg["frames"], cfg["grid_h"], cfg["grid_w"]
        self.F = F
        self.T = F * gh * gw
        self.Tf = gh * gw
        self.f_tok, self.y_tok, self.x_tok = token_positions(F, gh, gw)
        self.split = tuple(cfg["rope"])
        self.theta = float(cfg.get("theta", 10000.0))
        self.R = int(cfg.get("reference_frames", 0) or 0)
        self.relative = cfg.get("positions", "absolute") == "relative"

    def _rot(self, x, t_of_frame, heads, tok=None):
        """Rotate x [N, H, D] (tokens ``tok`` of a block, default all) with t = t_of_frame(f)."""
        tok = np.arange(x.shape[0]) if tok is None else tok
        xs = np.asarray(x)[:, heads, :]
        t = np.array([t_of_frame(f) for f in self.f_tok[tok]], np.float64)
        return apply_rope(xs, t, self.y_tok[tok], self.x_tok[tok], self.split, self.theta)

    def _attend(self, q_rot, ks, vs, heads, rows, with_slack=False):
        if self.cfg["dtype"] in ("bf16_fp8k", "bf16_fp8kv"):
            return self._attend_fp8(q_rot, ks, vs, rows, with_slack)
        k = np.concatenate(ks, axis=0)
        v = np.concatenate([np.asarray(x, np.float64) for x in vs], axis=0)
        o_sub = attention(q_rot, k, v, _scale(self.cfg), rows=rows)
        return (o_sub, np.zeros_like(o_sub)) if with_slack else o_sub

    def _attend_fp8(self, q_rot, ks, vs, rows, with_slack=False):
        """FP8 key (and value) cache: base-2 logits from E4M3 Q (one scale per
        row) and E4M3 K (one scale per 64-token tile of each context segment);
        quantising Q row by row lets the unrequested rows stay zero.  With the
        FP8 KV cache, V is quantised per segment tile too and P rounded to
        E4M3 against the exact row max."""
        log2e = 1.0 / np.log(2.0)
        s = _scale(self.cfg)
        rs = np.arange(self.T) if rows is None else np.asarray(rows)
        q2 = np.zeros_like(q_rot)
        q2[rs] = fp8.quantize_queries(q_rot[rs] * (s * log2e))
        k = np.concatenate([fp8.quantize_keys(x) for x in ks], axis=0)
        if self.cfg["dtype"] == "bf16_fp8kv":
            v = np.concatenate([fp8.quantize_values(x) for x in vs], axis=0)
            if with_slack:
                return fp8.attention_fp8_pv_slack(q2, k, v, rows=rows)
            return fp8.attention_fp8_pv(q2, k, v, rows=rows)
        v = np.concatenate([np.asarray(x, np.float64) for x in vs], axis=0)
        # exp(q2 . k / log2 e) = 2^(q2 . k): the base-2 logits
        o = attention(q2 / log2e, k, v, 1.0, rows=rows)
        return (o, np.zeros_like(o)) if with_slack else o


class PRSinkReference(_Base):
    """Static sink + pose-retrieved dynamic sinks + rolling window + current block."""

    def schedule(self, m: int) -> dict:
        c = self.cfg
        if c.get("bank_policy", "fifo") == "pose":
            if not hasattr(self, "_pose_bank"):
                self._pose_bank = []
                self._pose_iter = iter_prsink_pose_bank(self.p.pose, c["window"], c["bank"], c["static"])
            while len(self._pose_bank) <= m:           # advances only as far as block m
                self._pose_bank.append(next(self._pose_iter))
            return self._pose_bank[m]
        return prsink_schedule(m, c["window"], c["bank"], c["static"])

    def selection(self, m: int) -> list:
        c = self.cfg
        sch = self.schedule(m)
        if c["dynamic_k"] == 0 or not sch["bank"]:
            return []
        pq = self.p.pose(m)
        return retrieve(pq, [(b, self.p.pose(b)) for b in sch["bank"]], c["dynamic_k"])

    def context(self, m: int, selection=None) -> list:
        """[(kind, block id, tokens, t0)] in order static, dynamic, window, current."""
        sch = self.schedule(m)
        sel = self.selection(m) if selection is None else selection
        F, T = self.F, self.T
        t = self.block_t0
        if self.relative:       # consecutive frames in stream-id order, after the reference
            ids = sorted(set(sch["static"]) | set(sel) | set(sch["window"]) | {m})
            rank = {b: i for i, b in enumerate(ids)}
            t = lambda b: self.R + rank[b] * F
        segs = [("reference", -1, self.R * self.Tf, 0)] if self.R > 0 else []
        segs += [("static", b, T, t(b)) for b in sch["static"]]
        segs += [("dynamic", b, T, t(b)) for b in sel]
        segs += [("window", b, T, t(b)) for b in sch["window"]]
        segs.append(("current", m, T, t(m)))
        return segs

    def block_t0(self, b: int) -> int:
        """Absolute temporal position of block b's first frame (after the reference frames)."""
        return self.R + b * self.F

    def context_kv(self, m: int, layer: int, step: int, heads, selection=None):
        """Rotated K and raw V of every context segment, each [T, len(heads), D] fp64."""
        last = self.cfg["steps"] - 1
        out = []
        for kind, b, _, t0 in self.context(m, selection):
            if kind == "reference":
                k, v = self.p.reference(layer)
                f, y, x = token_positions(self.R, self.cfg["grid_h"], self.cfg["grid_w"])
                kr = apply_rope(np.asarray(k)[:, heads, :], f.astype(np.float64), y, x, self.split, self.theta)
            else:
                s = step if kind == "current" else last
                _, k, v = self.p.qkv(layer, b, s)
                kr = self._rot(k, lambda f, t0=t0: t0 + f, heads)
            out.append((kind, b, kr, np.asarray(v, np.float64)[:, heads, :]))
        return out

    def attend(self, m: int, layer: int, step: int, heads=None, rows=None, selection=None, with_slack=False):
        """Output [T, len(heads), D] fp64 of block m at (layer, step).  With
        ``with_slack``, (output, slack): how far each output may move where the
        FP8 product's rounding decides a P code (``fp8.attention_fp8_pv_slack``;
        zeros for the dtypes without an FP8 P)."""
        H = self.cfg["heads"]
        heads = list(range(H)) if heads is None else list(heads)
        if selection is None:
            selection = self.selection(m)
        t0 = self.context(m, selection)[-1][3]
        q, _, _ = self.p.qkv(layer, m, step)
        q_rot = self._rot(q, lambda f: t0 + f, heads)
        kv = self.context_kv(m, layer, step, heads, selection)
        return self._attend(q_rot, [x[2] for x in kv], [x[3] for x in kv], heads, rows, with_slack)


class ConvKVReference(_Base):
    """Conv-compressed memory + rolling window + current block, context-relative RoPE."""

    def schedule(self, m: int) -> dict:
        c = self.cfg
        if c["conv_stride"] != c["conv_kernel"]:
            raise ValueError("the oracle follows the stride == kernel reading")
        return convkv_schedule(m, self.F, c["window"], c["conv_kernel"], c["memory_frames"])

    def positions(self, m: int):
        """(t0 of each window block, t0 of the current block)."""
        sch = self.schedule(m)
        if self.cfg.get("positions") == "absolute":
            return [b * self.F for b in sch["window"]], m * self.F
        return sch["t0"]["window"], sch["t0"]["current"]

    def context(self, m: int) -> list:
        sch = self.schedule(m)
        tw, tc = self.positions(m)
        segs = [("memory", j, self.Tf, j) for j in range(len(sch["memory"]))]
        segs += [("window", b, self.T, t0) for b, t0 in zip(sch["window"], tw)]
        segs.append(("current", m, self.T, tc))
        return segs

    def _frame(self, layer: int, e: int, heads):
        """Raw K and V [Tf, len(heads), D] of evicted frame number e (last step's)."""
        b, f = divmod(e, self.F)
        _, k, v = self.p.qkv(layer, b, self.cfg["steps"] - 1)
        sl = slice(f * self.Tf, (f + 1) * self.Tf)
        return (np.asarray(k, np.float64)[sl][:, heads, :], np.asarray(v, np.float64)[sl][:, heads, :])

    def memory(self, m: int, layer: int, heads):
        """Raw memory K and V as cached, each [n_mem, Tf, len(heads), D] fp64."""
        sch = self.schedule(m)
        if not sch["memory"]:
            return None, None
        wk, wv = self.p.conv_weights(layer)
        wk = np.asarray(wk, np.float64)[heads]
        wv = np.asarray(wv, np.float64)[heads]
        mk, mv = [], []
        for group in sch["memory"]:
            fk, fv = zip(*[self._frame(layer, e, heads) for e in group])
            # [kernel, Tf, H, D] -> [kernel, H, Tf, D] for conv_memory
            fk = np.stack(fk).transpose(0, 2, 1, 3)
            fv = np.stack(fv).transpose(0, 2, 1, 3)
            mk.append(conv_memory(fk, wk)[0].transpose(1, 0, 2))
            mv.append(conv_memory(fv, wv)[0].transpose(1, 0, 2))
        mk, mv = np.stack(mk), np.stack(mv)
        if self.cfg["dtype"] != "f32":          # held in the cache's bf16
            mk, mv = bf16_round(mk), bf16_round(mv)
        return mk, mv

    def context_kv(self, m: int, layer: int, step: int, heads):
        """Rotated K and raw V of every context segment (memory frames: Tf tokens)."""
        sch = self.schedule(m)
        last = self.cfg["steps"] - 1
        out = []
        mk, mv = self.memory(m, layer, heads)
        tok_frame0 = np.arange(self.Tf)                          # a memory frame has frame-0 layout
        for j in range(len(sch["memory"])):
            kr = self._rot(mk[j], lambda f, j=j: j, list(range(len(heads))), tok=tok_frame0)
            out.append(("memory", j, kr, mv[j]))
        tw, t0 = self.positions(m)
        for b, tb in zip(sch["window"], tw):
            _, k, v = self.p.qkv(layer, b, last)
            kr = self._rot(k, lambda f, tb=tb: tb + f, heads)
            out.append(("window", b, kr, np.asarray(v, np.float64)[:, heads, :]))
        _, k, v = self.p.qkv(layer, m, step)
        kr = self._rot(k, lambda f: t0 + f, heads)
        out.append(("current", m, kr, np.asarray(v, np.float64)[:, heads, :]))
        return out

    def attend(self, m: int, layer: int, step: int, heads=None, rows=None, with_slack=False):
        """Output [T, len(heads), D] fp64 of block m at (layer, step); with
        ``with_slack``, (output, slack) as for PR-Sink."""
        H = self.cfg["heads"]
        heads = list(range(H)) if heads is None else list(heads)
        t0 = self.positions(m)[1]
        q, _, _ = self.p.qkv(layer, m, step)
        q_rot = self._rot(q, lambda f: t0 + f, heads)
        kv = self.context_kv(m, layer, step, heads)
        return self._attend(q_rot, [x[2] for x in kv], [x[3] for x in kv], heads, rows, with_slack)

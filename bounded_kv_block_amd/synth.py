"""Seeded synthetic workloads for bounded-KV block attention.

This module only *draws inputs*: block shapes, Q/K/V tensors, pose streams and
ConvKV weights.  It holds none of the method's arithmetic (no schedule, no
retrieval, no RoPE, no attention, no compression), so both the HIP path and
the CPU oracle can take their inputs from it without sharing any code.

The shapes follow the pages' workloads: 512x512 and 720x416 latent grids
(SoulX-LiveAct page, section 关键信息速览), blocks of latent frames with a
3-block rolling window and 3 sampling steps (LiveAnimate page, sections 方法
and 实验设计), and a roughly three-minute stream (LiveAnimate page, 实验设计).
The pages publish no dataset we can use; every tensor here is drawn from
N(0, 1) with a seed derived from (workload seed, layer, block, step, tensor).

Seeds: ``numpy.random.SeedSequence([seed, layer, block, step, tensor_id])``
with tensor ids Q=0, K=1, V=2, pose noise=3, keyframes=4, conv weights=5,
pose schedule=6.  bf16 workloads draw fp32 and round to nearest-even bf16,
so the values both sides see are exactly representable in bf16.
"""
from __future__ import annotations

import copy
import numpy as np

(TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_POSE, TENSOR_KEYFRAMES, TENSOR_CONV, TENSOR_SCHED, TENSOR_HIDDEN,
 TENSOR_WQKV, TENSOR_BQKV, TENSOR_REF) = range(11)

# Workload shapes.  Keys mirror the C-ABI config struct field names.
_BASE = dict(mode="pr_sink", dtype="bf16", layers=1, steps=1, heads=40, head_dim=128,
             frames=3, grid_h=32, grid_w=32, window=3, static=1, dynamic_k=2, bank=56,
             pose_dim=128, rope=(44, 42, 42), theta=10000.0, conv_kernel=5, conv_stride=5,
             memory_frames=1, blocks=60, seed=2, pose_kind="walk", keyframes=16, model_dim=5120, reference_frames=0,
             positions="default", bank_policy="fifo")

WORKLOADS = {
    # tiny fp32 stream: 2 heads x 64, 2 frames of 8x8, top-1 over 32-d poses,
    # bank of 8 evicted blocks, no RoPE, 12 blocks.
    "tiny_fp32": dict(_BASE, dtype="f32", heads=2, head_dim=64, frames=2, grid_h=8, grid_w=8,
                      dynamic_k=1, bank=8, pose_dim=32, rope=(0, 0, 0), blocks=12, seed=1,
                      pose_kind="repeat4"),
    # 512x512-shaped bf16 PR-Sink: 40 x 128, 3 frames of 32x32 = 3072 queries,
    # 7-block context = 21504 keys, top-2 over 128-d poses, bank of 56.
    "prsink_512": dict(_BASE),
    # the same with the FP8 key cache (K as E4M3 with per-tile scales)
    "prsink_512_fp8k": dict(_BASE, dtype="bf16_fp8k"),
    # the same with the FP8 KV cache (K and V as E4M3, P V on FP8 MFMA)
    "prsink_512_fp8kv": dict(_BASE, dtype="bf16_fp8kv"),
    # the same with one reference frame (1024 tokens) as a permanent sink
    "prsink_512_ref": dict(_BASE, reference_frames=1),
    # the same with context-relative RoPE positions (keys re-rotated per block)
    "prsink_512_rel": dict(_BASE, positions="relative"),
    # the same with a bank of 8 and pose-aware replacement (the entering block
    # displaces the member with the most similar pose)
    "prsink_512_posebank": dict(_BASE, bank=8, bank_policy="pose"),
    # the same driven from hidden states: q, k, v projected in the fused path
    # from x [3072, 5120] (40 heads x 128 = 5120, a 14B-class DiT's width)
    "prsink_512_qkv": dict(_BASE, qkv=True),
    # the same with the FP8 key cache (K quantised in the projection's epilogue)
    "prsink_512_qkv_fp8k": dict(_BASE, qkv=True, dtype="bf16_fp8k"),
    # 720x416-shaped bf16: 3 frames of 26x45 = 3510 queries, 40 layers x 3 steps,
    # commit after the third step, bank of 16.
    "prsink_720x416": dict(_BASE, grid_h=26, grid_w=45, layers=40, steps=3, bank=16, seed=3),
    # long stream: 512x512 shapes for 1080 blocks, 24 keyframes revisited in
    # random order so the dynamic sink swaps often, bank of 64.
    "prsink_long": dict(_BASE, bank=64, blocks=1080, seed=4, pose_kind="jump", keyframes=24),
    # ConvKV variant: no sinks; older history compressed 5:1 into one
    # 1024-token memory frame; 200 blocks.
    "convkv_512": dict(_BASE, mode="convkv", static=0, dynamic_k=0, bank=0, pose_dim=0,
                       blocks=200, seed=5, pose_kind="none"),
    # the same with the FP8 key cache (the rotated context quantised as it is gathered)
    "convkv_512_fp8k": dict(_BASE, mode="convkv", dtype="bf16_fp8k", static=0, dynamic_k=0, bank=0, pose_dim=0,
                            blocks=200, seed=5, pose_kind="none"),
    # the same with the FP8 KV cache
    "convkv_512_fp8kv": dict(_BASE, mode="convkv", dtype="bf16_fp8kv", static=0, dynamic_k=0, bank=0, pose_dim=0,
                             blocks=200, seed=5, pose_kind="none"),
    # 720x416 with the FP8 KV cache
    "prsink_720x416_fp8kv": dict(_BASE, grid_h=26, grid_w=45, layers=40, steps=3, bank=16, seed=3,
                                 dtype="bf16_fp8kv"),
    # the same with only the memory's positions restarted (window and current absolute)
    "convkv_512_abs": dict(_BASE, mode="convkv", static=0, dynamic_k=0, bank=0, pose_dim=0,
                           blocks=200, seed=5, pose_kind="none", positions="absolute"),
}


def workload(name: str, **overrides) -> dict:
    """A copy of a named workload with overrides applied."""
    cfg = copy.deepcopy(WORKLOADS[name])
    cfg.update(overrides)
    cfg["name"] = name
    return cfg


def tokens_per_block(cfg: dict) -> int:
    return cfg["frames"] * cfg["grid_h"] * cfg["grid_w"]


def _rng(cfg: dict, layer: int, block: int, step: int, tensor: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([int(cfg["seed"]), int(layer), int(block), int(step), int(tensor)])))


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns fp32 holding bf16 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def qkv(cfg: dict, layer: int, block: int, step: int = 0):
    """Q, K, V of one block as fp32 numpy arrays [T, H, D] (bf16-exact for bf16 workloads)."""
    shape = (tokens_per_block(cfg), cfg["heads"], cfg["head_dim"])
    out = []
    for tid in (TENSOR_Q, TENSOR_K, TENSOR_V):
        x = _rng(cfg, layer, block, step, tid).standard_normal(shape, dtype=np.float32)
        out.append(x if cfg["dtype"] == "f32" else round_to_bf16(x))
    return tuple(out)


def conv_weights(cfg: dict, layer: int):
    """Depthwise temporal-conv weights w^K, w^V, each [H, D, kernel] fp32, N(0, 1/kernel)."""
    kern = cfg["conv_kernel"]
    rng = _rng(cfg, layer, 0, 0, TENSOR_CONV)
    shape = (cfg["heads"], cfg["head_dim"], kern)
    sd = np.float32(1.0 / np.sqrt(kern))
    wk = (rng.standard_normal(shape, dtype=np.float32) * sd).astype(np.float32)
    wv = (rng.standard_normal(shape, dtype=np.float32) * sd).astype(np.float32)
    return wk, wv


def poses(cfg: dict, n_blocks: int | None = None) -> np.ndarray:
    """Pose embeddings [n_blocks, P] fp32 for the workload's pose stream.

    kinds:
      repeat4 -- i.i.d. N(0, I) except every block n with n % 4 == 3, which
                 copies the pose of one earlier block plus 0.01 N(0, I) noise.
                 The source is block 0 for n = 3 and otherwise drawn uniformly
                 from earlier blocks at least 4 back (not block 0, not a copy
                 block, not a previous source), so exactly one retrievable block
                 is near each copy.
      walk     -- keyframes k_j ~ N(0, I); j_0 = 0, j_{n+1} = j_n + U{-1,0,1} mod K;
                 pose = keyframe + 0.01 N(0, I).
      jump     -- K keyframes; segments jump to a uniformly chosen other
                 keyframe and dwell U{1..4} blocks; pose = keyframe + 0.01 N(0, I).
      none     -- no poses (ConvKV).
    """
    n = cfg["blocks"] if n_blocks is None else n_blocks
    P = cfg["pose_dim"]
    kind = cfg["pose_kind"]
    if kind == "none" or P == 0:
        return np.zeros((n, 0), np.float32)
    out = np.empty((n, P), np.float32)
    if kind == "repeat4":
        sources_used = []
        for b in range(n):
            base = _rng(cfg, 0, b, 0, TENSOR_POSE).standard_normal(P, dtype=np.float32)
            if b % 4 == 3:
                cands = [c for c in range(1, b - 3) if c % 4 != 3 and c not in sources_used]
                if cands:
                    pick = _rng(cfg, 0, b, 0, TENSOR_SCHED).integers(0, len(cands))
                    src = cands[int(pick)]
                else:
                    src = 0
                sources_used.append(src)
                out[b] = out[src] + np.float32(0.01) * base
            else:
                out[b] = base
        return out
    K = cfg["keyframes"]
    key = _rng(cfg, 0, 0, 0, TENSOR_KEYFRAMES).standard_normal((K, P), dtype=np.float32)
    sched = _rng(cfg, 0, 0, 0, TENSOR_SCHED)
    idx = np.empty(n, np.int64)
    if kind == "walk":
        j = 0
        for b in range(n):
            idx[b] = j
            j = (j + int(sched.integers(-1, 2))) % K
    elif kind == "jump":
        j, left = 0, int(sched.integers(1, 5))
        for b in range(n):
            if left == 0:
                j = (j + 1 + int(sched.integers(0, K - 1))) % K
                left = int(sched.integers(1, 5))
            idx[b] = j
            left -= 1
    else:
        raise ValueError(f"unknown pose kind {kind!r}")
    for b in range(n):
        noise = _rng(cfg, 0, b, 0, TENSOR_POSE).standard_normal(P, dtype=np.float32)
        out[b] = key[idx[b]] + np.float32(0.01) * noise
    return out


def repeat_sources(cfg: dict, n_blocks: int | None = None) -> dict:
    """For ``repeat4`` streams: {copy block: source block}, recomputed from the same seeds."""
    n = cfg["blocks"] if n_blocks is None else n_blocks
    out, used = {}, []
    for b in range(n):
        if b % 4 == 3:
            cands = [c for c in range(1, b - 3) if c % 4 != 3 and c not in used]
            if cands:
                src = cands[int(_rng(cfg, 0, b, 0, TENSOR_SCHED).integers(0, len(cands)))]
            else:
                src = 0
            used.append(src)
            out[b] = src
    return out


# ---- device-side generation (large workloads) --------------------------------
def _torch_seed(cfg: dict, layer: int, block: int, step: int, tensor: int) -> int:
    ss = np.random.SeedSequence([int(cfg["seed"]), int(layer), int(block), int(step), int(tensor)])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def qkv_device(cfg: dict, layer: int, block: int, step: int = 0, device="cuda"):
    """Q, K, V [T, H, D] drawn on ``device`` with torch's seeded generator.

    For large workloads, where drawing on the host would dominate a test.  The
    values differ from :func:`qkv` (another generator) but are just as
    deterministic; a test copies them to the host to hand them to the oracle.
    """
    import torch
    shape = (tokens_per_block(cfg), cfg["heads"], cfg["head_dim"])
    dt = torch.float32 if cfg["dtype"] == "f32" else torch.bfloat16
    out = []
    for tid in (TENSOR_Q, TENSOR_K, TENSOR_V):
        g = torch.Generator(device=device)
        g.manual_seed(_torch_seed(cfg, layer, block, step, tid))
        out.append(torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(dt))
    return tuple(out)


# ---- hidden states and QKV projection weights (fused-projection path) -------
def hidden(cfg: dict, layer: int, block: int, step: int = 0) -> np.ndarray:
    """Hidden states x [T, model_dim] fp32 holding bf16 values, N(0, 1)."""
    shape = (tokens_per_block(cfg), cfg["model_dim"])
    return round_to_bf16(_rng(cfg, layer, block, step, TENSOR_HIDDEN).standard_normal(shape, dtype=np.float32))


def qkv_weights(cfg: dict, layer: int):
    """W [3*H*D, model_dim] ~ N(0, 1/model_dim) and bias [3*H*D] ~ N(0, 0.01),
    both fp32 holding bf16 values (so q, k, v come out about N(0, 1))."""
    n = 3 * cfg["heads"] * cfg["head_dim"]
    C = cfg["model_dim"]
    w = _rng(cfg, layer, 0, 0, TENSOR_WQKV).standard_normal((n, C), dtype=np.float32) / np.float32(np.sqrt(C))
    b = _rng(cfg, layer, 0, 0, TENSOR_BQKV).standard_normal(n, dtype=np.float32) * np.float32(0.1)
    return round_to_bf16(w), round_to_bf16(b)


def hidden_device(cfg: dict, layer: int, block: int, step: int = 0, device="cuda"):
    """hidden() drawn on the device with torch's seeded generator (bf16)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(cfg, layer, block, step, TENSOR_HIDDEN))
    shape = (tokens_per_block(cfg), cfg["model_dim"])
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def qkv_weights_device(cfg: dict, layer: int, device="cuda"):
    """qkv_weights() drawn on the device with torch's seeded generator (bf16)."""
    import torch
    n = 3 * cfg["heads"] * cfg["head_dim"]
    C = cfg["model_dim"]
    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(cfg, layer, 0, 0, TENSOR_WQKV))
    w = torch.randn((n, C), generator=g, device=device, dtype=torch.float32) / float(np.sqrt(C))
    g.manual_seed(_torch_seed(cfg, layer, 0, 0, TENSOR_BQKV))
    b = torch.randn(n, generator=g, device=device, dtype=torch.float32) * 0.1
    return w.to(torch.bfloat16), b.to(torch.bfloat16)


# ---- reference frames (reference-sink variant) --------------------------------
def reference(cfg: dict, layer: int):
    """K, V [reference_frames * grid_h * grid_w, H, D] of the reference frames
    (fp32 holding bf16 values for bf16 workloads), N(0, 1)."""
    shape = (cfg["reference_frames"] * cfg["grid_h"] * cfg["grid_w"], cfg["heads"], cfg["head_dim"])
    g = _rng(cfg, layer, 0, 0, TENSOR_REF)
    k = g.standard_normal(shape, dtype=np.float32)
    v = g.standard_normal(shape, dtype=np.float32)
    if cfg["dtype"] != "f32":
        k, v = round_to_bf16(k), round_to_bf16(v)
    return k, v

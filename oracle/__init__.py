"""CPU oracle for bounded-KV block attention (test infrastructure only).

A plain, slow, fp64 numpy implementation of what the hot path computes:
block schedule (static sink, rolling window, FIFO bank of evicted blocks),
exact pose retrieval, 3D RoPE, softmax attention over the bounded context,
and the ConvKV temporal-conv memory.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP path
(``bounded_kv_block_amd``) and never imports it; both take their inputs from
the seeded generators in ``bounded_kv_block_amd.synth``, which hold none of
the method's arithmetic.

Sources (pages, by title and section):
  * LiveAnimate: 实时稳定长时流式人体动画 -- section 方法 (PR-Sink: static
    sink, dynamic sink by pose retrieval, rolling window of three blocks),
    section 实验设计 (block-causal generator, 3 steps), section 关键发现
    (constant cache size), section 局限 (retrieval by pose similarity).
  * Soul App开源实时数字人生成框架SoulX-LiveAct详解 -- section 技术内核,
    ConvKV Memory bullet (exact recent KV, older history compressed by a 1D
    conv up to 5:1 into fixed-length memory, RoPE positions reset); sections
    关键信息速览 and 上手实践 (FP8 attention in deployment; the E4M3 key cache
    scheme in ``fp8`` is this package's reading; the fused-QKV build, read in
    ``projection`` as the plain linear projection of the hidden states).

Where the pages leave a step open, the reading taken is stated in the
function that implements it.  Every function is pinned by a CPU test against
closed forms, library routines, hand-derived fixtures or brute force.
"""
from .schedule import (prsink_schedule, simulate_prsink, simulate_prsink_pose_bank, convkv_schedule,
                       simulate_convkv, token_positions)
from .retrieval import retrieve, exact_keys, fp64_cosines, boundary_gap
from .rope import rope_frequencies, apply_rope
from .attention import attention, masked_attention, softmax_weights
from .convkv import conv_memory
from .stream import PRSinkReference, ConvKVReference
from .projection import qkv_projection
from . import fp8

__all__ = [
    "qkv_projection",
    "prsink_schedule", "simulate_prsink", "simulate_prsink_pose_bank", "convkv_schedule", "simulate_convkv",
    "token_positions", "retrieve", "exact_keys", "fp64_cosines", "boundary_gap",
    "rope_frequencies", "apply_rope", "attention", "masked_attention", "softmax_weights",
    "conv_memory", "PRSinkReference", "ConvKVReference", "fp8",
]

"""Head sharding on one GPU: the path shards over heads with nothing
exchanged inside it.  A stream run through one cache of all heads and
through G caches of H/G heads each (fed the matching head slices of q, k, v,
and the same poses) gives the same retrieved ids on every shard and
bit-identical outputs: each (head, query tile) unit computes the same thing
whichever launch runs it."""
import numpy as np
import pytest

from bounded_kv_block_amd import bkv, synth
from gpu_helpers import Run

pytestmark = pytest.mark.gpu


def _sharded(cfg, G, blocks, host_inputs=True):
    import torch
    H = cfg["heads"]
    full = Run(cfg, host_inputs)
    shards = [bkv.Cache(dict(cfg, heads=H // G)) for _ in range(G)]
    for m in range(blocks):
        pose = full.pose_dev(m)
        full.cache.retrieve(pose)
        for c in shards:
            c.retrieve(pose)
        sel = full.cache.selection()
        assert all(c.selection() == sel for c in shards), m
        q, k, v = full.qkv_dev(0, m, 0)
        out = full.cache.attend(0, q, k, v)
        for g, c in enumerate(shards):
            hs = slice(g * H // G, (g + 1) * H // G)
            part = c.attend(0, q[:, hs].contiguous(), k[:, hs].contiguous(), v[:, hs].contiguous())
            assert torch.equal(part, out[:, hs]), (m, g)
        full.cache.commit()
        for c in shards:
            c.commit()
        if not host_inputs:
            full.drop({m + 1})


def test_head_shards_bit_identical_small():
    """8 heads in 2 and in 4 shards, 180-token blocks, top-2 over a bank of 4,
    12 blocks (bf16), and the same with the FP8 key cache."""
    cfg = synth.workload("prsink_512", heads=8, grid_h=6, grid_w=10, bank=4, blocks=12, pose_dim=16, keyframes=5)
    _sharded(cfg, 2, 12)
    _sharded(cfg, 4, 12)
    _sharded(dict(cfg, dtype="bf16_fp8k", name="prsink_512_fp8k"), 2, 12)


def test_head_shards_bit_identical_prsink_512():
    """The 512x512 shape at full size, 40 heads as 2 shards of 20 (the share
    one of two GPUs would hold), 9 blocks."""
    cfg = synth.workload("prsink_512", blocks=9)
    _sharded(cfg, 2, 9, host_inputs=False)

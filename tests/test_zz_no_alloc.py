"""The allocation-free attend (bkv_attend_static_scratch) against bkv_attend
through the C-ABI: the same stream on two handles, one driven by each entry
point, gives bit-identical outputs on every block -- first a 1800-query,
40-head stream (320 units: the split launch cuts the 64 remaining units
into 4 key parts, 256 part states in the static array), then a smaller
1600-query, 44-head one (308 units: 52 remaining, 4 parts, 208 states), so
the second reads only what it wrote over the first's leftovers.  Then the
FP8 KV cache and ConvKV on the first shape, whose split launches use the same
array."""
import numpy as np
import pytest

from bounded_kv_block_amd import synth
from gpu_helpers import Run

pytestmark = pytest.mark.gpu


def _pair(cfg):
    a, b = Run(cfg, host_inputs=False), Run(cfg, host_inputs=False)
    for m in range(cfg["blocks"]):
        a.open(m)
        b.open(m)
        q, k, v = a.qkv_dev(0, m, 0)
        oa = a.cache.attend(0, q, k, v)
        ob = b.cache.attend_static_scratch(0, q, k, v)
        assert bool((oa == ob).all()), (cfg["name"], m)
        a.cache.commit()
        b.cache.commit()
        a.drop({m + 1})
    assert a.cache.stats()["split_attends"] == cfg["blocks"] == b.cache.stats()["split_attends"]


def test_static_scratch_attend_matches_attend_two_calls():
    _pair(synth.workload("prsink_512", frames=2, grid_h=30, grid_w=30, blocks=7))
    _pair(synth.workload("prsink_512", heads=44, frames=2, grid_h=20, grid_w=40, blocks=7))
    _pair(synth.workload("prsink_512_fp8kv", frames=2, grid_h=30, grid_w=30, blocks=7))
    _pair(synth.workload("convkv_512", frames=2, grid_h=30, grid_w=30, blocks=9))

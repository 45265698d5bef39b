"""Two handles on two HIP streams, their calls interleaved on one host
thread: each stream's outputs equal those of the same handle run alone (the
library keeps no state outside the handle and its workspace, and every
device operation goes to the caller's stream)."""
import numpy as np
import pytest

from bounded_kv_block_amd import synth
from gpu_helpers import Run

pytestmark = pytest.mark.gpu


def _alone(cfg):
    run = Run(cfg)
    outs = []
    for m in range(cfg["blocks"]):
        run.open(m)
        outs.append(run.attend(m, 0, 0).clone())
        run.cache.commit()
    return outs


def test_two_streams_interleaved():
    import torch
    a_cfg = synth.workload("prsink_512", heads=4, grid_h=6, grid_w=10, bank=4, blocks=10, pose_dim=16,
                           keyframes=4)
    b_cfg = synth.workload("convkv_512", dtype="bf16_fp8k", heads=2, grid_h=4, grid_w=6, blocks=10)
    want_a, want_b = _alone(a_cfg), _alone(b_cfg)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    with torch.cuda.stream(sa):
        ra = Run(a_cfg)
    with torch.cuda.stream(sb):
        rb = Run(b_cfg)
    torch.cuda.synchronize()
    got_a, got_b = [], []
    for m in range(10):
        with torch.cuda.stream(sa):
            ra.open(m)
        with torch.cuda.stream(sb):
            rb.open(m)
        with torch.cuda.stream(sa):
            got_a.append(ra.attend(m, 0, 0))
        with torch.cuda.stream(sb):
            got_b.append(rb.attend(m, 0, 0))
        with torch.cuda.stream(sa):
            ra.cache.commit()
        with torch.cuda.stream(sb):
            rb.cache.commit()
    torch.cuda.synchronize()
    for m in range(10):
        assert torch.equal(got_a[m], want_a[m]), m
        assert torch.equal(got_b[m], want_b[m]), m

"""GPU parity at the configuration limits: a bank of 256 blocks (the largest
accepted), 1024-d poses, top-8 retrieval, a window of 8 and two reference
frames -- a 19-segment context -- over a 275-block stream of 16-token
blocks.  Retrieved ids are checked against the oracle's exact ranking on
sampled blocks (every block retrieves on the GPU), outputs within 2e-2."""
import numpy as np
import pytest

import oracle
from bounded_kv_block_amd import synth
from gpu_helpers import TOL, Run, max_err

pytestmark = pytest.mark.gpu


def test_largest_bank_pose_and_context():
    cfg = synth.workload("prsink_512_ref", heads=2, frames=1, grid_h=4, grid_w=4, window=8, dynamic_k=8,
                         bank=256, pose_dim=1024, keyframes=40, blocks=275, reference_frames=2)
    run = Run(cfg)
    ref = oracle.PRSinkReference(cfg, run)
    check = set(range(0, 275, 17)) | set(range(262, 275))
    P = synth.poses(cfg, cfg["blocks"])
    for m in range(cfg["blocks"]):
        run.open(m)
        if m in check:
            sch = ref.schedule(m)
            g = oracle.boundary_gap(P[m], [(b, P[b]) for b in sch["bank"]], cfg["dynamic_k"])
            assert g is None or g == 0 or g > 2.0 ** -40, m
            sel = ref.selection(m)
            assert run.cache.selection() == sel, m
            ctx = run.cache.context()
            assert len(ctx) == 1 + len(sch["static"]) + len(sel) + len(sch["window"]) + 1
            assert m < 265 or len(ctx) == 19
            out = run.attend(m, 0, 0)
            err = max_err(out, ref.attend(m, 0, 0, selection=sel))
            assert err <= TOL["bf16"], (m, err)
        else:
            run.attend(m, 0, 0)
        run.cache.commit()
        run._dev.clear()
        run._host.clear()
    st = run.cache.stats()
    assert st["bank_count"] == 256

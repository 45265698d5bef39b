"""GPU retrieval through the C-ABI on constructed pose streams (FIFO bank):
exact cosine ties -- a bitwise-duplicate pose and a copy scaled by 2 -- go to
the lower stream id, as the oracle's exact ranking says (LiveAnimate page,
section 方法, Dynamic Sink bullet; section 局限, retrieval by pose
similarity); poses holding Inf or NaN score 0, also at the largest bank (256
blocks).  Retrieved ids are compared with the oracle on every block and with
the hand-derived expectation where one is stated; outputs within tolerance."""
import numpy as np
import pytest

import oracle
from bounded_kv_block_amd import synth
from gpu_helpers import TOL, Run, max_err

pytestmark = pytest.mark.gpu


class _Poses(Run):
    """A Run whose pose stream is given explicitly."""

    def __init__(self, cfg, poses):
        super().__init__(cfg)
        self._poses_np = np.asarray(poses, np.float32)


def _drive(run, expect=None, check_out=()):
    ref = oracle.PRSinkReference(run.cfg, run)
    for m in range(run.cfg["blocks"]):
        run.open(m)
        sel = ref.selection(m)
        got = run.cache.selection()
        assert got == sel, (m, got, sel)
        if expect and m in expect:
            assert got == expect[m], (m, got, expect[m])
        out = run.attend(m, 0, 0)
        if m in check_out:
            err = max_err(out, ref.attend(m, 0, 0, selection=sel))
            assert err <= TOL[run.cfg["dtype"]], (m, err)
        run.cache.commit()
        run._dev.clear()
        run._host.clear()


def test_exact_ties_go_to_the_lower_id():
    # window 1, bank 16, top-2: block b enters the bank at the commit of b + 1
    cfg = synth.workload("tiny_fp32", window=1, bank=16, dynamic_k=2, pose_dim=8, blocks=14)
    rng = np.random.default_rng(7)
    P = rng.standard_normal((14, 8)).astype(np.float32)
    P[5] = P[2]                      # bitwise duplicate of block 2
    P[6] = P[3] * np.float32(2.0)    # exact x2 copy of block 3: the same cosine to any query
    P[9] = P[2]                      # query = block 2's pose: blocks 2 and 5 tie at cosine 1
    P[10] = P[3]                     # query = block 3's pose: blocks 3 and 6 tie at cosine 1
    P[12] = P[3] * np.float32(-1.0)  # opposite of 3 (and 6): those two tie at -1, ranked last
    P[13] = P[6]                     # query = the x2 copy: 3 and 6 tie again
    expect = {9: [2, 5], 10: [3, 6], 13: [3, 6]}
    _drive(_Poses(cfg, P), expect, check_out=(9, 10, 13))


def test_non_finite_poses_score_zero_at_the_largest_bank():
    # bank of 256 (the largest accepted), 1024-d poses, top-8; some bank
    # members hold NaN or -Inf, and two queries hold +Inf / NaN (all their
    # scores are 0, so the 8 lowest ids win)
    cfg = synth.workload("prsink_512", heads=2, frames=1, grid_h=4, grid_w=4, dynamic_k=8, bank=256,
                         pose_dim=1024, blocks=263)
    rng = np.random.default_rng(11)
    P = rng.standard_normal((263, 1024)).astype(np.float32)
    P[10, 5] = np.nan
    P[40, 0] = -np.inf
    P[41] = np.nan
    P[260, 17] = np.inf
    P[262, 3] = np.nan
    run = _Poses(cfg, P)
    ref = oracle.PRSinkReference(cfg, run)
    bank_260 = ref.schedule(260)["bank"]
    assert len(bank_260) == 256
    expect = {260: sorted(bank_260)[:8], 262: sorted(ref.schedule(262)["bank"])[:8]}
    _drive(run, expect, check_out=(250, 260, 262))

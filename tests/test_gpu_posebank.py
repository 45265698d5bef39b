"""GPU parity of pose-aware bank replacement (PR-Sink, bank_policy "pose")
through the C-ABI: the bank the library keeps (seen through the retrieved
ids) equals the oracle's on every block, including exact ties and a zero
pose, and attention outputs match the oracle within max-abs 2e-2 (bf16) /
1e-5 (fp32)."""
import numpy as np
import pytest

import oracle
from bounded_kv_block_amd import synth
from conftest import ids, read_table
from gpu_helpers import TOL, Run, max_err

pytestmark = pytest.mark.gpu


def _stream(cfg, run=None, check=None, heads=None, rows=None, host_inputs=True):
    run = run or Run(cfg, host_inputs)
    ref = oracle.PRSinkReference(cfg, run)
    replaced = 0
    for m in range(cfg["blocks"]):
        run.open(m)
        sel = ref.selection(m)
        assert run.cache.selection() == sel, (m, run.cache.selection(), sel)
        sch = ref.schedule(m)
        assert run.cache.stats()["bank_count"] == len(sch["bank"])
        replaced += sch["evicted"] is not None and len(sch["bank"]) == cfg["bank"]
        out = run.attend(m, 0, 0)
        if check is None or m in check:
            want = ref.attend(m, 0, 0, heads=heads, rows=rows, selection=sel)
            err = max_err(out, want, heads, rows)
            print(f"block {m}: bank {sch['bank']} max|err| {err:.3e}", flush=True)
            assert err <= TOL[cfg["dtype"]], (m, err)
        run.cache.commit()
        if not host_inputs:
            run.drop(set(range(m - 70, m + 2)))
    return run, replaced


class _GoldenPoses(Run):
    """The hand-derived 2-D pose stream (exact ties, a zero pose)."""

    def __init__(self, cfg):
        super().__init__(cfg)
        rows = read_table("prsink_pose_bank_w1_b2_s1.txt")
        self._poses_np = np.array([[float(r[1]), float(r[2])] for r in rows], np.float32)
        self.golden = {int(r[0]): ids(r[4]) for r in rows}


def test_posebank_golden_stream():
    """Window 1, bank 2, top-2 (the retrieved set is the whole bank) over the
    hand-derived pose table: the library's bank equals the table's on every
    block, and the outputs match the oracle in fp32."""
    cfg = synth.workload("tiny_fp32", window=1, bank=2, dynamic_k=2, pose_dim=2, blocks=13, rope=(24, 20, 20),
                         bank_policy="pose")
    run = _GoldenPoses(cfg)
    _stream(cfg, run=run)
    # replay: the retrieved set of each block is its golden bank
    run.cache.reset()
    for m in range(cfg["blocks"]):
        run.open(m)
        assert sorted(run.cache.selection()) == sorted(run.golden[m]), m
        run.attend(m, 0, 0)
        run.cache.commit()


def test_posebank_bf16_small():
    """bf16, 2 heads, 3-frame blocks of 4x10, bank 3, top-2, 30 blocks of a
    pose walk over 4 keyframes: many replacements, every output checked."""
    cfg = synth.workload("prsink_512_posebank", heads=2, grid_h=4, grid_w=10, bank=3, blocks=30, pose_dim=16,
                         keyframes=4)
    P = synth.poses(cfg, cfg["blocks"])
    sim = oracle.simulate_prsink_pose_bank(cfg["blocks"], lambda b: P[b], cfg["window"], cfg["bank"], cfg["static"])
    for m, s in enumerate(sim):       # no decision hinges on a gap near fp64 resolution
        if s["evicted"] is not None and len(s["bank"]) == cfg["bank"]:
            g = oracle.boundary_gap(P[s["evicted"]], [(b, P[b]) for b in s["bank"]], 1)
            assert g is None or g == 0 or g > 2.0 ** -40, m
    _, replaced = _stream(cfg)
    assert replaced >= 20


def test_posebank_prsink_512_full_shape_sampled():
    """512x512 shapes at full size, bank 8 with pose-aware replacement, 40
    blocks: indices on every block, outputs of 2 heads on sampled rows of
    blocks 6, 20 and 39."""
    cfg = synth.workload("prsink_512_posebank", blocks=40)
    _, replaced = _stream(cfg, host_inputs=False, check={6, 20, 39}, heads=[0, 39],
                          rows=np.r_[0:64, 1500:1532, 3008:3072])
    assert replaced >= 25


@pytest.mark.parametrize("variant", [
    dict(dtype="bf16_fp8k", reference_frames=1),
    dict(positions="relative", reference_frames=2),
    dict(positions="relative", layers=2, steps=2),
])
def test_posebank_combined_with_other_variants(variant):
    """Pose-aware replacement together with the FP8 key cache and a reference
    frame, with context-relative positions and two reference frames, and with
    context-relative positions over 2 layers x 2 steps: the bank, the
    retrieved ids and every output of a 24-block stream (6x10 grid, 3 frames,
    bank 3, top-2)."""
    cfg = synth.workload("prsink_512_posebank", heads=2, grid_h=6, grid_w=10, bank=3, blocks=24, pose_dim=16,
                         keyframes=4, **variant)
    run = Run(cfg)
    ref = oracle.PRSinkReference(cfg, run)
    tol = TOL[cfg["dtype"]]
    for m in range(cfg["blocks"]):
        run.open(m)
        sel = ref.selection(m)
        assert run.cache.selection() == sel, m
        assert run.cache.stats()["bank_count"] == len(ref.schedule(m)["bank"])
        assert run.cache.context() == ref.context(m, sel), m
        for s in range(cfg["steps"]):
            for l in range(cfg["layers"]):
                out = run.attend(m, l, s)
                err = max_err(out, ref.attend(m, l, s, selection=sel))
                assert err <= tol, (m, l, s, err)
        run.cache.commit()

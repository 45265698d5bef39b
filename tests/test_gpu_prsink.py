"""GPU parity of the PR-Sink path (through the C-ABI) against the CPU oracle.

Retrieval and eviction indices must match exactly; attention outputs within
max-abs 1e-5 (fp32 path) and 2e-2 (bf16 path) of the fp64 oracle."""
import numpy as np
import pytest

import oracle
from bounded_kv_block_amd import synth
from gpu_helpers import TOL, Run, max_err, oracle_err

pytestmark = pytest.mark.gpu


def _check_block(run, ref, m, layer=0, step=0, heads=None, rows=None, out=None):
    cfg = run.cfg
    want_sel = ref.selection(m)
    got_sel = run.cache.selection()
    assert got_sel == want_sel, (m, got_sel, want_sel)
    ctx = run.cache.context()
    want_ctx = ref.context(m, want_sel)
    assert ctx == [(k, b, t, t0) for k, b, t, t0 in want_ctx], (m, ctx, want_ctx)
    if out is None:
        out = run.attend(m, layer, step)
    err = oracle_err(out, lambda **kw: ref.attend(m, layer, step, heads=heads, selection=want_sel, **kw),
                     heads, rows, TOL[cfg["dtype"]])
    print(f"block {m} layer {layer} step {step}: keys {sum(c[2] for c in ctx)} max|err| {err:.3e}", flush=True)
    assert err <= TOL[cfg["dtype"]], (m, err)
    return out


def _stream(cfg, host_inputs=True, check=None, heads=None, rows=None):
    run = Run(cfg, host_inputs)
    ref = oracle.PRSinkReference(cfg, run)
    for m in range(cfg["blocks"]):
        run.open(m)
        if check is None or m in check:
            _check_block(run, ref, m, heads=heads, rows=rows)
        else:
            assert run.cache.selection() == ref.selection(m)
            run.attend(m, 0, 0)
        run.cache.commit()
        st = run.cache.stats()
        want_ev = oracle.prsink_schedule(m, cfg["window"], cfg["bank"], cfg["static"])["evicted"]
        assert st["last_evicted"] == (-1 if want_ev is None else want_ev)
        if not host_inputs:
            run.drop(set(range(m - 70, m + 2)))
    return run


def test_tiny_fp32_stream():
    """12-block fp32 stream, 2 heads x 64, top-1 over 32-d poses: every block, every output."""
    cfg = synth.workload("tiny_fp32")
    src = synth.repeat_sources(cfg)
    run = Run(cfg)
    ref = oracle.PRSinkReference(cfg, run)
    for m in range(cfg["blocks"]):
        run.open(m)
        _check_block(run, ref, m)
        if m in (7, 11):
            assert run.cache.selection() == [src[m]]          # repeat pose -> that block
        run.cache.commit()
    st = run.cache.stats()
    assert st["block"] == 12 and st["bank_count"] == 8


def test_tiny_fp32_rope_and_d128():
    for kw in (dict(rope=(24, 20, 20)), dict(head_dim=128, rope=(44, 42, 42))):
        cfg = synth.workload("tiny_fp32", **kw)
        _stream(cfg)


def test_bf16_small_ragged():
    """bf16, 3 heads, 3 frames of 6x10 = 180 tokens (two full 64-key tiles and a
    52-key tail per segment, a ragged query tile), RoPE 44/42/42, top-2 over a
    bank of 4, 14 blocks: every output of every block."""
    cfg = synth.workload("prsink_512", heads=3, grid_h=6, grid_w=10, bank=4, blocks=14, pose_dim=16,
                         keyframes=5)
    _stream(cfg)


def test_bf16_single_token_blocks():
    """Degenerate block of one token (one key per segment, one query)."""
    cfg = synth.workload("prsink_512", heads=2, frames=1, grid_h=1, grid_w=1, bank=3, blocks=10,
                         pose_dim=8, keyframes=3, rope=(44, 42, 42))
    _stream(cfg)


def test_prsink_512_full_shape_sampled():
    """512x512-shaped workload at full size (40 x 128, 3072 queries, 21504 keys
    once warm): indices on every block, outputs sampled (2 heads, 160 query rows
    including the last) on blocks 0, 4, 6 and 9."""
    cfg = synth.workload("prsink_512", blocks=10)
    rows = np.r_[0:64, 1500:1532, 3008:3072]
    run = _stream(cfg, host_inputs=False, check={0, 4, 6, 9}, heads=[0, 39], rows=rows)
    assert run.cache.stats()["split_attends"] == 0        # 480 units: 6% idle, one unit per workgroup


def test_split_launch_key_parts_ragged_tile():
    """1800-query blocks with 40 heads: 320 (head, 256-query) units leave the
    second round of 256 workgroups 75% idle, so the attention runs its split
    launch: one full round, then the 64 remainder units (heads 32..39) each
    cut into 4 key parts whose fp32 states are merged.  Outputs of heads in
    the full round and in the remainder, rows in several query tiles incl.
    the ragged last one (8 rows), against the oracle."""
    cfg = synth.workload("prsink_512", frames=2, grid_h=30, grid_w=30, blocks=8)
    run = _stream(cfg, host_inputs=False, check={0, 4, 7}, heads=[0, 33, 39],
                  rows=np.r_[0:64, 900:964, 1736:1800])
    assert run.cache.stats()["split_attends"] == cfg["blocks"]


def test_split_launch_whole_remainder_units():
    """2560-query blocks with 40 heads: 400 units; the split launch runs one
    full round and the 144 remainder units whole (one key part each)."""
    cfg = synth.workload("prsink_512", frames=2, grid_h=32, grid_w=40, blocks=8)
    run = _stream(cfg, host_inputs=False, check={0, 7}, heads=[0, 25, 39],
                  rows=np.r_[0:64, 1536:1600, 2496:2560])
    assert run.cache.stats()["split_attends"] == cfg["blocks"]


@pytest.mark.parametrize("name", ["prsink_512", "prsink_512_fp8k"])
def test_split_launch_deterministic(name):
    """The key parts of a cut remainder unit are merged in part order by a
    launch of their own, so attending the same inputs twice in a block gives
    bit-identical outputs (1800-query blocks: 64 remainder units in 4 parts)."""
    import torch
    cfg = synth.workload(name, frames=2, grid_h=30, grid_w=30, blocks=6, steps=2)
    run = Run(cfg, host_inputs=False)
    for m in range(cfg["blocks"]):
        run.open(m)
        q, k, v = run.qkv_dev(0, m, 0)
        first = run.cache.attend(0, q, k, v).clone()
        second = run.cache.attend(0, q, k, v)
        assert torch.equal(first, second), m
        run.cache.commit()
    assert run.cache.stats()["split_attends"] == 2 * cfg["blocks"]


def test_multistep_multilayer_commit_after_last_step():
    """3 layers x 3 steps per block; the cache keeps each layer's last-step K/V."""
    cfg = synth.workload("prsink_512", heads=2, grid_h=4, grid_w=10, bank=3, blocks=9, pose_dim=16,
                         keyframes=4, layers=3, steps=3)
    run = Run(cfg)
    ref = oracle.PRSinkReference(cfg, run)
    for m in range(cfg["blocks"]):
        run.open(m)
        sel = ref.selection(m)
        assert run.cache.selection() == sel
        for s in range(3):
            for l in range(3):
                out = run.attend(m, l, s)
                want = ref.attend(m, l, s, selection=sel)
                err = max_err(out, want)
                assert err <= TOL["bf16"], (m, l, s, err)
        run.cache.commit()


def test_export_segments_match_oracle_context():
    """Stored K (rotated at absolute positions) and V of every context segment."""
    cfg = synth.workload("prsink_512", heads=2, grid_h=4, grid_w=6, bank=4, blocks=9, pose_dim=16, keyframes=4)
    run = Run(cfg)
    ref = oracle.PRSinkReference(cfg, run)
    for m in range(cfg["blocks"]):
        run.open(m)
        run.attend(m, 0, 0)
        kv = ref.context_kv(m, 0, 0, [0, 1], ref.selection(m))
        for i, (_, _, kr, v) in enumerate(kv):
            gk, gv = run.cache.export_segment(0, i)
            # K: rotation in fp32 then rounding to bf16: within one bf16 ulp
            assert np.max(np.abs(gk.float().cpu().numpy() - kr)) <= 2.0 ** -7 * np.max(np.abs(kr)) + 1e-6
            assert np.array_equal(gv.float().cpu().numpy(), v)
        run.cache.commit()


class _GrowingKeys(Run):
    """Block m's keys scaled by 1 + g m (g = 0.75 unless set; rounded to bf16, the same values
    for the device and the oracle).  Full tiles run in segment order, static
    sink first, so a row's scores rise by several powers of two from tile to
    tile and every row's running max must move within one attend.  Values
    are scaled by 1/8 (exact): scores this large turn the bf16 rounding of
    the rotated queries into errors of about 0.7% of the dominant P, which
    on N(0,1) values would pass the bound, while a missed rescale of O or l
    still moves an output by about |V|, some 0.5."""

    growth = 0.75

    def qkv(self, layer, block, step):
        key = (layer, block, step)
        if key not in self._host:
            import torch
            q, k, v = synth.qkv(self.cfg, layer, block, step)
            k = torch.from_numpy(k * np.float32(1.0 + self.growth * block)).to(torch.bfloat16).float().numpy()
            self._host[key] = (q, k, v * np.float32(0.125))
        return self._host[key]

    def qkv_dev(self, layer, block, step):
        key = (layer, block, step)
        if key not in self._dev:
            self._dev[key] = tuple(self.torch.from_numpy(a).to(self.device).to(self.dt)
                                   for a in self.qkv(layer, block, step))
        return self._dev[key]


@pytest.mark.parametrize("name", ["prsink_512", "prsink_512_fp8k", "prsink_512_fp8kv"])
def test_running_max_rescales_on_growing_scores(name):
    """The lazy running max under scores that grow from tile to tile (bf16
    and FP8 keys: the lane-sum test; FP8 KV: the lane-max test and whole
    power-of-two moves of m): 2 heads, 3 frames of 4x8 tokens (one full tile
    and a 32-key tail per segment), RoPE, top-2 of a bank of 3, 10 blocks,
    every output of every block."""
    cfg = synth.workload(name, heads=2, grid_h=4, grid_w=8, bank=3, blocks=10, pose_dim=16, keyframes=4)
    run = _GrowingKeys(cfg)
    ref = oracle.PRSinkReference(cfg, run)
    for m in range(cfg["blocks"]):
        run.open(m)
        _check_block(run, ref, m)
        run.cache.commit()


@pytest.mark.parametrize("name", ["prsink_512", "prsink_512_fp8k", "prsink_512_fp8kv"])
def test_running_max_rescales_through_overflow(name):
    """Keys scaled by 1 + 20 m: from block 3 on, the window's scores lie 150
    to 750 powers of two above the static sink tile that opens each row, so
    the first pass of exponentials over them overflows to infinity and the
    rescale must recompute P from the new max.  Scores this large put the
    softmax outside the range where the bf16 rounding of the rotated keys
    leaves near-ties to the oracle, so this is a property test: retrieval
    matches the oracle, every output is finite, and every output channel lies
    within that channel's range over the context's values, widened by 10% of
    its largest magnitude for the FP8 roundings of P and V (a missed rescale
    of O or l leaves outputs at zero or scaled by 2^100 and more)."""
    cfg = synth.workload(name, heads=2, grid_h=4, grid_w=8, bank=3, blocks=8, pose_dim=16, keyframes=4)
    run = _GrowingKeys(cfg)
    run.growth = 20.0
    ref = oracle.PRSinkReference(cfg, run)
    for m in range(cfg["blocks"]):
        run.open(m)
        sel = run.cache.selection()
        assert sel == ref.selection(m), m
        ctx = run.cache.context()                  # (kind, block, tokens, t0) per segment
        out = run.attend(m, 0, 0).float().cpu().numpy()                  # [T, H, D]
        assert np.isfinite(out).all(), m
        vs = np.stack([run.qkv(0, blk, 0)[2] for _, blk, _, _ in ctx])  # [segments, T, H, D]
        lo, hi = vs.min(axis=(0, 1)), vs.max(axis=(0, 1))                # [H, D]
        slack = 0.1 * np.abs(vs).max(axis=(0, 1, 3))[:, None]            # [H, 1]
        assert (out >= lo - slack).all() and (out <= hi + slack).all(), m
        if m >= 3:                                 # the window dominates: outputs far from zero
            assert np.abs(out).max() > 0.05 * np.abs(vs).max(), m
        run.cache.commit()

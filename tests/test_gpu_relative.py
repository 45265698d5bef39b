"""GPU parity of PR-Sink with context-relative RoPE positions (the context's
blocks at consecutive frames in stream-id order; keys re-rotated every block
by the gather kernel) through the C-ABI against the CPU oracle: indices and
segment positions exact, outputs within max-abs 1e-5 (fp32) / 2e-2 (bf16),
stored context K (rotated at its relative positions) and V within bf16
rounding."""
import numpy as np
import pytest

import oracle
from bounded_kv_block_amd import synth
from gpu_helpers import TOL, Run, max_err

pytestmark = pytest.mark.gpu


def _stream(cfg, run=None, check=None, heads=None, rows=None, host_inputs=True, export=False, layers_steps=None):
    run = run or Run(cfg, host_inputs)
    ref = oracle.PRSinkReference(cfg, run)
    tol = TOL[cfg["dtype"]]
    unordered = 0
    for m in range(cfg["blocks"]):
        run.open(m)
        sel = ref.selection(m)
        assert run.cache.selection() == sel, m
        unordered += sel != sorted(sel)
        want_ctx = ref.context(m, sel)
        got_ctx = run.cache.context()
        assert [(k, b, n, t) for k, b, n, t in got_ctx] == [(k, b, n, t) for k, b, n, t in want_ctx], m
        pairs = layers_steps or [(0, 0)]
        for s, l in pairs:
            out = run.attend(m, l, s)
            if check is None or m in check:
                want = ref.attend(m, l, s, heads=heads, rows=rows, selection=sel)
                err = max_err(out, want, heads, rows)
                print(f"block {m} layer {l} step {s}: max|err| {err:.3e}", flush=True)
                assert err <= tol, (m, l, s, err)
        if export:
            hs = list(range(cfg["heads"]))
            s, l = pairs[-1]
            for i, (_, _, kr, v) in enumerate(ref.context_kv(m, l, s, hs, sel)):
                gk, gv = run.cache.export_segment(l, i)
                gk = gk.float().cpu().numpy().astype(np.float64)
                gv = gv.float().cpu().numpy().astype(np.float64)
                if cfg["dtype"] == "f32":
                    assert np.allclose(gk, kr, atol=1e-5, rtol=0), (m, i)
                else:
                    assert np.all(np.abs(gk - kr) <= 2.0 ** -8 * np.abs(kr) + 1e-3), (m, i)
                assert np.array_equal(gv, v), (m, i)
        run.cache.commit()
        if not host_inputs:
            run.drop(set(range(m - 70, m + 2)))
    return run, unordered


def test_relative_bf16_small_ragged_with_export():
    """3 heads, 3 frames of 6x10 = 180 tokens, RoPE 44/42/42, top-2 over a
    bank of 4, 14 blocks: segment positions (retrieved blocks ranked by id on
    the device), every output, the stored K and V of every segment; the stream
    retrieves out of id order at least once."""
    cfg = synth.workload("prsink_512_rel", heads=3, grid_h=6, grid_w=10, bank=4, blocks=14, pose_dim=16,
                         keyframes=5)
    _, unordered = _stream(cfg, export=True)
    assert unordered > 0


def test_relative_f32_with_reference():
    """fp32 (head_dim 64), one reference frame ahead of the relative block
    positions, top-3 over a bank of 8, RoPE 24/20/20: every output within
    1e-5, every stored segment."""
    cfg = synth.workload("tiny_fp32", rope=(24, 20, 20), dynamic_k=3, reference_frames=1, positions="relative")
    _, unordered = _stream(cfg, export=True)
    assert unordered > 0


def test_relative_multilayer_multistep():
    """2 layers x 3 steps per block: one gather per layer and block, the
    current block's K rewritten at each step, the cache keeping each layer's
    last-step K."""
    cfg = synth.workload("prsink_512_rel", heads=2, grid_h=4, grid_w=10, bank=3, blocks=9, pose_dim=16,
                         keyframes=4, layers=2, steps=3)
    _stream(cfg, layers_steps=[(s, l) for s in range(3) for l in range(2)], export=True)


def test_relative_fused_projection():
    """The fused QKV projection path writes raw K to the slot and rotated K at
    the current block's relative position into the context buffer."""
    from test_gpu_qkv import QkvRun
    cfg = synth.workload("prsink_512_qkv", heads=2, grid_h=6, grid_w=10, bank=4, blocks=10, pose_dim=16,
                         keyframes=5, model_dim=128, positions="relative")
    _stream(cfg, run=QkvRun(cfg))


def test_relative_prsink_512_full_shape_sampled():
    """512x512 shapes at full size (21504 keys re-rotated per block):
    positions and indices on every block, outputs of 2 heads on sampled
    query rows of blocks 0, 6 and 11."""
    cfg = synth.workload("prsink_512_rel", blocks=12)
    _stream(cfg, host_inputs=False, check={0, 6, 11}, heads=[0, 39], rows=np.r_[0:64, 1500:1532, 3008:3072])

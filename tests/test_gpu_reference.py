"""GPU parity of PR-Sink with reference frames (a permanent first context
segment at temporal positions 0..R-1; generated blocks at R + b*frames + f)
through the C-ABI against the CPU oracle: indices exact, outputs within
max-abs 1e-5 (fp32) / 2e-2 (bf16, FP8 keys) of the fp64 oracle, the stored
reference K (rotated) and V within bf16 rounding; call-order errors."""
import ctypes

import numpy as np
import pytest

import oracle
from bounded_kv_block_amd import bkv, synth
from gpu_helpers import TOL, Run, max_err

pytestmark = pytest.mark.gpu


def _stream(cfg, run=None, check=None, heads=None, rows=None, host_inputs=True, export=False):
    run = run or Run(cfg, host_inputs)
    ref = oracle.PRSinkReference(cfg, run)
    tol = TOL[cfg["dtype"]]
    outs = []
    for m in range(cfg["blocks"]):
        run.open(m)
        sel = ref.selection(m)
        assert run.cache.selection() == sel, m
        ctx = run.cache.context()
        assert ctx[0] == ("reference", -1, cfg["reference_frames"] * cfg["grid_h"] * cfg["grid_w"], 0)
        assert ctx[-1][3] == cfg["reference_frames"] + m * cfg["frames"]
        run.ctx_lens = getattr(run, "ctx_lens", []) + [len(ctx)]
        out = run.attend(m, 0, 0)
        if check is None or m in check:
            want = ref.attend(m, 0, 0, heads=heads, rows=rows, selection=sel)
            err = max_err(out, want, heads, rows)
            print(f"block {m}: max|err| {err:.3e}", flush=True)
            assert err <= tol, (m, err)
        if export:
            hs = list(range(cfg["heads"]))
            kv = ref.context_kv(m, 0, 0, hs, sel)
            for i, (_, _, kr, v) in enumerate(kv):
                gk, gv = run.cache.export_segment(0, i)
                gk = gk.float().cpu().numpy().astype(np.float64)
                gv = gv.float().cpu().numpy().astype(np.float64)
                if cfg["dtype"] == "f32":
                    assert np.allclose(gk, kr, atol=1e-5, rtol=0), (m, i)
                else:
                    assert np.all(np.abs(gk - kr) <= 2.0 ** -8 * np.abs(kr) + 1e-3), (m, i)
                assert np.array_equal(gv, v), (m, i)
        outs.append(out)
        run.cache.commit()
        if not host_inputs:
            run.drop(set(range(m - 70, m + 2)))
    return run, outs


def test_reference_bf16_small_ragged_with_export():
    """One reference frame of 6x10 = 60 keys (a single partial key tile), 3
    heads, 3-frame blocks of 180 tokens, RoPE 44/42/42, top-2 over a bank of
    4, 12 blocks: every output, and the stored K and V of every segment,
    the reference included."""
    cfg = synth.workload("prsink_512_ref", heads=3, grid_h=6, grid_w=10, bank=4, blocks=12, pose_dim=16,
                         keyframes=5)
    _stream(cfg, export=True)


def test_reference_f32_two_frames():
    """fp32, head_dim 64, two reference frames of 8x8 at t = 0 and 1, RoPE
    24/20/20, the repeat-pose stream: every output within 1e-5."""
    cfg = synth.workload("tiny_fp32", rope=(24, 20, 20), reference_frames=2)
    _stream(cfg, export=True)


def test_reference_fp8k_small():
    """FP8 key cache: the reference K stored as E4M3 with per-tile scales like
    every block; 2 reference frames of 6x10 (120 keys: a full and a partial
    tile), every output within 2e-2."""
    cfg = synth.workload("prsink_512_fp8k", heads=2, grid_h=6, grid_w=10, bank=4, blocks=10, pose_dim=16,
                         keyframes=4, reference_frames=2)
    _stream(cfg)


def test_reference_largest_context():
    """Every segment kind at its limit: 3 reference frames, the static sink, 8
    retrieved blocks and a window of 8 (19 segments), single-frame blocks of
    4x4 tokens, 24 blocks, bf16."""
    cfg = synth.workload("prsink_512_ref", heads=2, frames=1, grid_h=4, grid_w=4, window=8, dynamic_k=8,
                         bank=12, blocks=24, pose_dim=16, keyframes=10, reference_frames=3)
    run, _ = _stream(cfg)
    assert max(run.ctx_lens) == 19 and run.ctx_lens[-1] == 19


def test_reference_call_order_and_reset():
    """retrieve before every layer's reference is set -> BKV_ERR_STATE; setting
    it with a block open -> BKV_ERR_STATE; a handle without reference frames
    -> BKV_ERR_UNSUPPORTED; bkv_reset keeps the reference: the replayed stream
    is bit-identical."""
    import torch
    cfg = synth.workload("prsink_512_ref", heads=2, grid_h=4, grid_w=8, bank=3, blocks=6, pose_dim=8,
                         keyframes=3, layers=2)
    c = bkv.Cache(cfg)
    k, v = (torch.from_numpy(a).cuda().to(torch.bfloat16) for a in synth.reference(cfg, 0))
    c.set_reference(0, k, v)
    pose = torch.from_numpy(synth.poses(cfg, 1)[0]).cuda()
    with pytest.raises(bkv.BkvError) as ei:
        c.retrieve(pose)
    assert ei.value.status == bkv.BKV_ERR_STATE
    with pytest.raises(bkv.BkvError) as ei:
        c.set_reference(1, k, k)
    assert ei.value.status == bkv.BKV_ERR_ARG
    c.set_reference(1, *(torch.from_numpy(a).cuda().to(torch.bfloat16) for a in synth.reference(cfg, 1)))
    c.retrieve(pose)
    with pytest.raises(bkv.BkvError) as ei:
        c.set_reference(0, k, v)
    assert ei.value.status == bkv.BKV_ERR_STATE
    plain = bkv.Cache(synth.workload("prsink_512", heads=2, grid_h=4, grid_w=8, bank=3, pose_dim=8))
    st = bkv.lib().bkv_set_reference(plain._h, 0, ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
                                     plain._s())
    assert st == bkv.BKV_ERR_UNSUPPORTED

    run = Run(cfg)
    first = []
    for m in range(cfg["blocks"]):
        run.open(m)
        first.append([run.attend(m, l, 0).clone() for l in range(2)])
        run.cache.commit()
    run.cache.reset()
    for m in range(cfg["blocks"]):
        run.open(m)
        for l in range(2):
            assert bool((run.attend(m, l, 0) == first[m][l]).all()), (m, l)
        run.cache.commit()


def test_reference_prsink_512_full_shape_sampled():
    """512x512 shapes at full size with one 32x32 reference frame (1024 keys,
    22528 keys once warm): indices on every block, outputs of 2 heads on
    sampled query rows of blocks 0, 5 and 9."""
    cfg = synth.workload("prsink_512_ref", blocks=10)
    _stream(cfg, host_inputs=False, check={0, 5, 9}, heads=[0, 39], rows=np.r_[0:64, 1500:1532, 3008:3072])

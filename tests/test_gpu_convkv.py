"""GPU parity of the ConvKV path (through the C-ABI) against the CPU oracle."""
import numpy as np
import pytest

import oracle
from bounded_kv_block_amd import synth
from gpu_helpers import TOL, Run, max_err

pytestmark = pytest.mark.gpu


def _run(cfg, host_inputs=True, check=None, heads=None, rows=None, export=False):
    run = Run(cfg, host_inputs)
    ref = oracle.ConvKVReference(cfg, run)
    H = cfg["heads"]
    for m in range(cfg["blocks"]):
        run.open(m)
        ctx = run.cache.context()
        want_ctx = ref.context(m)
        assert ctx == list(want_ctx), (m, ctx, want_ctx)
        out = run.attend(m, 0, 0)
        if check is None or m in check:
            want = ref.attend(m, 0, 0, heads=heads, rows=rows)
            err = max_err(out, want, heads, rows)
            print(f"block {m}: keys {sum(c[2] for c in ctx)} max|err| {err:.3e}", flush=True)
            assert err <= TOL[cfg["dtype"]], (m, err)
        if export:
            hs = list(range(H))
            kv = ref.context_kv(m, 0, 0, hs)
            for i, (kind, _, kr, v) in enumerate(kv):
                gk, gv = run.cache.export_segment(0, i)
                gk = gk.float().cpu().numpy()
                gv = gv.float().cpu().numpy()
                tol_k = 2.0 ** -7 * np.max(np.abs(kr)) + 1e-6
                assert np.max(np.abs(gk - kr)) <= tol_k, (m, kind)
                if kind == "memory":
                    # conv output: fp32 sums of bf16 inputs, stored in bf16
                    assert np.max(np.abs(gv - v)) <= 2.0 ** -7 * np.max(np.abs(v)) + 1e-6, (m, kind)
                else:
                    assert np.array_equal(gv, v), (m, kind)
        run.cache.commit()
        st = run.cache.stats()
        assert st["memory_count"] == len(ref.schedule(m + 1)["memory"])
        if not host_inputs:
            run.drop(set(range(m - 8, m + 2)))
    return run


def test_convkv_small_every_block():
    """bf16, 2 heads, 3 frames of 4x6 (24-token frames, 72-token blocks: ragged
    tiles), memory from block 5 on, 12 blocks; outputs and every segment's K/V."""
    cfg = synth.workload("convkv_512", heads=2, grid_h=4, grid_w=6, blocks=12)
    _run(cfg, export=True)


def test_convkv_fp32_two_memory_frames():
    cfg = synth.workload("convkv_512", dtype="f32", heads=2, head_dim=64, rope=(24, 20, 20), frames=2,
                         grid_h=4, grid_w=4, memory_frames=2, blocks=14)
    _run(cfg, export=True)


@pytest.mark.parametrize("kernel", [1, 2, 3, 8])
def test_convkv_conv_kernel_sizes(kernel):
    """Temporal conv of 1, 2, 3 and 8 taps (stride = kernel), bf16, 2 heads:
    outputs and every segment's K/V, the conv memory against the oracle's."""
    cfg = synth.workload("convkv_512", heads=2, grid_h=4, grid_w=6, conv_kernel=kernel, conv_stride=kernel,
                         blocks=8 + kernel)
    run = _run(cfg, export=True)
    assert run.cache.stats()["memory_count"] == 1


def test_convkv_odd_frame_size():
    """15-token frames (3 x 5): a V^T row of a frame is 30 bytes, so the conv
    reads and writes V^T element by element; 45-token blocks, ragged tiles."""
    cfg = synth.workload("convkv_512", heads=2, grid_h=3, grid_w=5, blocks=10)
    run = _run(cfg, export=True)
    assert run.cache.stats()["memory_count"] == 1


def test_convkv_fp32_three_taps_two_memory_frames():
    """fp32 conv (4-channel chunks) with 3 taps and two memory frames."""
    cfg = synth.workload("convkv_512", dtype="f32", heads=2, head_dim=64, rope=(24, 20, 20), frames=2,
                         grid_h=4, grid_w=4, conv_kernel=3, conv_stride=3, memory_frames=2, blocks=12)
    run = _run(cfg, export=True)
    assert run.cache.stats()["memory_count"] == 2


def test_convkv_512_full_shape_sampled():
    """512x512 ConvKV at full size: 1024-token memory + 3 windows + current =
    13312 keys from block 5; outputs sampled on blocks 0, 4, 5, 7."""
    cfg = synth.workload("convkv_512", blocks=8)
    rows = np.r_[0:64, 3008:3072]
    _run(cfg, host_inputs=False, check={0, 4, 5, 7}, heads=[0, 21], rows=rows)


# ---- only the memory's positions restarted (window and current absolute)
def test_convkv_absolute_small_every_block():
    """The memory-only reset: per-block temporal rows (memory at 0, window and
    current at absolute frame indices), reported positions, outputs and every
    segment's K/V on 14 blocks of the ragged bf16 stream."""
    cfg = synth.workload("convkv_512_abs", heads=2, grid_h=4, grid_w=6, blocks=14)
    _run(cfg, export=True)


def test_convkv_absolute_fp32_two_memory_frames():
    cfg = synth.workload("convkv_512_abs", dtype="f32", heads=2, head_dim=64, rope=(24, 20, 20), frames=2,
                         grid_h=4, grid_w=4, memory_frames=2, blocks=16)
    _run(cfg, export=True)


def test_convkv_absolute_full_shape_sampled():
    """512x512 shapes at full size, blocks 0..39 (absolute positions up to
    117): outputs of 2 heads on sampled rows of blocks 4, 5 and 39."""
    cfg = synth.workload("convkv_512_abs", blocks=40)
    _run(cfg, host_inputs=False, check={4, 5, 39}, heads=[0, 39], rows=np.r_[0:64, 1500:1532, 3008:3072])

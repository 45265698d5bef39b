"""GPU parity of the FP8 KV cache (dtype "bf16_fp8kv": K and V held as E4M3
with per-tile power-of-two scales, P held as E4M3 with one power-of-two scale
per query row, P V on the scaled FP8 matrix instruction) through the C-ABI
against the CPU oracle (the library moves its running max by whole numbers,
so its P codes are the oracle's up to values near the subnormal range).

Indices exact; the stored V equals the oracle's E4M3 quantisation bit for
bit (codes and tile scales: V is not rotated); outputs within max-abs 2e-2
of the fp64 oracle; and, reported beside it, the error against the plain
(unquantised) fp64 attention -- the accuracy cost of the FP8 reading."""
import numpy as np
import pytest

import oracle
from bounded_kv_block_amd import synth
from gpu_helpers import TOL, Run, max_err, oracle_err

pytestmark = pytest.mark.gpu


def _check_stored_values(run, kv, layer=0, memory_tol=False):
    """Every segment's stored V (E4M3 code x 2^e, exact in bf16) against the
    oracle's quantisation of that segment's V.  Memory frames (conv output
    stored in bf16 from an fp32 sum) may differ by one E4M3 step."""
    for i, (kind, _, _, v) in enumerate(kv):
        _, gv = run.cache.export_segment(layer, i)
        got = gv.float().cpu().numpy().astype(np.float64)
        if kind == "memory":
            import torch
            vb = torch.from_numpy(v).to(torch.bfloat16).double().numpy()
            want = oracle.fp8.quantize_values(vb)
            step = np.abs(want) * 2.0 ** -3 + np.max(np.abs(want)) * 2.0 ** -9
            assert np.all(np.abs(got - want) <= step), (i, kind)
            assert np.mean(got != want) < 1e-2, (i, kind)
        else:
            assert np.array_equal(got, oracle.fp8.quantize_values(v)), (i, kind)


def _stream(cfg, run=None, check=None, heads=None, rows=None, host_inputs=True, values=False, plain=False,
            plain_tol=None):
    run = run or Run(cfg, host_inputs)
    ref = oracle.PRSinkReference(cfg, run)
    ref16 = oracle.PRSinkReference(dict(cfg, dtype="bf16"), run) if plain else None
    worst = worst16 = 0.0
    for m in range(cfg["blocks"]):
        run.open(m)
        sel = ref.selection(m)
        assert run.cache.selection() == sel, m
        out = run.attend(m, 0, 0)
        if check is None or m in check:
            err = oracle_err(out, lambda **kw: ref.attend(m, 0, 0, heads=heads, selection=sel, **kw),
                             heads, rows, TOL["bf16_fp8kv"])
            worst = max(worst, err)
            msg = f"block {m}: max|err| {err:.3e}"
            if plain:
                e16 = max_err(out, ref16.attend(m, 0, 0, heads=heads, rows=rows, selection=sel), heads, rows)
                worst16 = max(worst16, e16)
                msg += f", against the unquantised fp64 attention {e16:.3e}"
            print(msg, flush=True)
            assert err <= TOL["bf16_fp8kv"], (m, err)
            if plain_tol is not None:
                assert e16 <= plain_tol, (m, e16)
        if values:
            _check_stored_values(run, ref.context_kv(m, 0, 0, list(range(cfg["heads"])), sel))
        run.cache.commit()
        if not host_inputs:
            run.drop(set(range(m - 70, m + 2)))
    if plain:
        print(f"FP8 KV cache: worst max|err| {worst:.3e} against the oracle's FP8 reading, "
              f"{worst16:.3e} against the unquantised fp64 attention", flush=True)
    return run


def test_fp8kv_small_ragged_with_values():
    """3 heads, 3 frames of 6x10 = 180 tokens (two full 64-key tiles and a
    52-key tail per segment, a ragged query tile), RoPE 44/42/42, top-2 over
    a bank of 4, 14 blocks: every output of every block, every segment's
    stored V, and (reported, not bounded: a 180-key context averages few
    values, so E4M3 rounding of V and P shows) the error against the
    unquantised attention."""
    cfg = synth.workload("prsink_512_fp8kv", heads=3, grid_h=6, grid_w=10, bank=4, blocks=14,
                         pose_dim=16, keyframes=5)
    _stream(cfg, values=True, plain=True)


def test_fp8kv_single_token_blocks():
    """Degenerate blocks of one token: one key per segment, one query."""
    cfg = synth.workload("prsink_512_fp8kv", heads=2, frames=1, grid_h=1, grid_w=1, bank=3, blocks=10,
                         pose_dim=8, keyframes=3)
    _stream(cfg, values=True)


def test_fp8kv_multistep_multilayer():
    """2 layers x 3 steps per block; the cache keeps each layer's last-step K, V."""
    cfg = synth.workload("prsink_512_fp8kv", heads=2, grid_h=4, grid_w=10, bank=3, blocks=8, pose_dim=16,
                         keyframes=4, layers=2, steps=3)
    run = Run(cfg)
    ref = oracle.PRSinkReference(cfg, run)
    for m in range(cfg["blocks"]):
        run.open(m)
        sel = ref.selection(m)
        assert run.cache.selection() == sel
        for s in range(3):
            for l in range(2):
                out = run.attend(m, l, s)
                err = oracle_err(out, lambda **kw: ref.attend(m, l, s, selection=sel, **kw), tol=TOL["bf16_fp8kv"])
                assert err <= TOL["bf16_fp8kv"], (m, l, s, err)
        run.cache.commit()


def test_fp8kv_reference_frames_and_relative_positions():
    """Context-relative PR-Sink with one reference frame and the FP8 KV cache:
    the reference's V is quantised when it is set, blocks' V at append;
    indices, outputs and stored V on 12 blocks."""
    cfg = synth.workload("prsink_512_fp8kv", heads=2, grid_h=6, grid_w=10, bank=4, blocks=12, pose_dim=16,
                         keyframes=5, positions="relative", reference_frames=1)
    _stream(cfg, values=True)


def test_fp8kv_split_launch_key_parts():
    """1800-query blocks, 40 heads: the split launch (one full round, then the
    64 remainder units cut into 4 key parts) with the FP8 KV cache."""
    cfg = synth.workload("prsink_512_fp8kv", frames=2, grid_h=30, grid_w=30, blocks=8)
    run = _stream(cfg, host_inputs=False, check={0, 4, 7}, heads=[0, 33, 39],
                  rows=np.r_[0:64, 900:964, 1736:1800])
    assert run.cache.stats()["split_attends"] == cfg["blocks"]


def test_fp8kv_prsink_512_full_shape():
    """512x512 shapes at full size with the FP8 KV cache: indices on every
    block; on the last (steady) block every head and every query against the
    oracle, and against the unquantised attention within the bf16 path's
    2e-2 (the accuracy cost of the FP8 reading at the workload's size)."""
    cfg = synth.workload("prsink_512_fp8kv", blocks=8)
    _stream(cfg, host_inputs=False, check={7}, plain=True, plain_tol=2e-2)


def _convkv_stream(cfg, check=None, heads=None, rows=None, host_inputs=True, values=False):
    run = Run(cfg, host_inputs)
    ref = oracle.ConvKVReference(cfg, run)
    for m in range(cfg["blocks"]):
        run.open(m)
        assert run.cache.context() == ref.context(m), m
        out = run.attend(m, 0, 0)
        if check is None or m in check:
            err = oracle_err(out, lambda **kw: ref.attend(m, 0, 0, heads=heads, **kw), heads, rows,
                             TOL["bf16_fp8kv"])
            print(f"block {m}: max|err| {err:.3e}", flush=True)
            assert err <= TOL["bf16_fp8kv"], (m, err)
        if values:
            _check_stored_values(run, ref.context_kv(m, 0, 0, list(range(cfg["heads"]))))
        run.cache.commit()
        if not host_inputs:
            run.drop(set(range(m - 8, m + 2)))
    return run


def test_fp8kv_convkv_small_ragged_with_values():
    """ConvKV with the FP8 KV cache: 2 heads, 3 frames of 4x6 (a 24-token
    memory frame and 72-token blocks), 12 blocks; every output and every
    segment's stored V (the memory frame's quantised after the conv)."""
    cfg = synth.workload("convkv_512_fp8kv", heads=2, grid_h=4, grid_w=6, blocks=12)
    run = _convkv_stream(cfg, values=True)
    assert run.cache.stats()["memory_count"] == 1


def test_fp8kv_convkv_two_memory_frames():
    """Two memory frames of 6x10 tokens, memory-only position reset, 16 blocks."""
    cfg = synth.workload("convkv_512_fp8kv", heads=2, grid_h=6, grid_w=10, frames=2, memory_frames=2,
                         blocks=16, positions="absolute")
    _convkv_stream(cfg, values=True)


def test_fp8kv_convkv_512_full_shape():
    """ConvKV 512x512 at full size with the FP8 KV cache: the last block (a
    1024-token memory frame, three window blocks, the current block) on every
    head and query."""
    cfg = synth.workload("convkv_512_fp8kv", blocks=7)
    _convkv_stream(cfg, host_inputs=False, check={6})

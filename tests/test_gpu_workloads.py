"""Full-size workloads on the GPU: the 720x416 multi-layer/multi-step stream,
the 1080-block long stream and the 200-block ConvKV stream, each checked
against the CPU oracle (indices on every block, outputs on sampled blocks,
heads and rows)."""
import numpy as np
import pytest

import oracle
from bounded_kv_block_amd import synth
from gpu_helpers import TOL, Run, max_err

pytestmark = pytest.mark.gpu


def test_prsink_720x416_layers_steps_sampled():
    """3 frames of 26x45 = 3510 queries (ragged: 54 full tiles + a 54-key tail
    per segment), 40 layers x 3 sampling steps per block, commit after the
    third step.  Indices on every block; on the first steady block (6) the
    outputs of layers 0, 17, 39 at steps 1 and 3 (2 heads, 128 rows incl.
    the ragged last query tile) against the oracle."""
    cfg = synth.workload("prsink_720x416", blocks=7)
    run = Run(cfg, host_inputs=False)
    ref = oracle.PRSinkReference(cfg, run)
    heads, rows = [0, 39], np.r_[0:64, 3446:3510]
    L, S = cfg["layers"], cfg["steps"]
    checked = 0
    for m in range(cfg["blocks"]):
        run.open(m)
        sel = ref.selection(m)
        assert run.cache.selection() == sel, m
        n_keys = run.cache.stats()["n_keys"]
        for s in range(S):
            for l in range(L):
                out = run.attend(m, l, s)
                if m == 6 and l in (0, 17, 39) and s in (0, 2):
                    want = ref.attend(m, l, s, heads=heads, rows=rows, selection=sel)
                    err = max_err(out, want, heads, rows)
                    print(f"block {m} layer {l} step {s}: keys {n_keys} max|err| {err:.3e}", flush=True)
                    assert err <= TOL["bf16"], (m, l, s, err)
                    checked += 1
                run._dev.clear()           # inputs are regenerated when the oracle needs them
        run.cache.commit()
        run._host.clear()
    assert checked == 6 and n_keys == 7 * 3510
    # 560 units (2.19 rounds of 256 workgroups): every attend used the split launch
    assert run.cache.stats()["split_attends"] == cfg["blocks"] * L * S


def test_prsink_long_stream_1080_blocks():
    """512x512 shapes for 1080 blocks, 24 keyframes revisited in random order
    (the dynamic sink swaps often), bank of 64: retrieval and eviction indices
    on all 1080 blocks, outputs on every 45th block, constant workspace and
    device memory, and a flat per-block latency.

    The latency is timed in a pass of its own, after an untimed pass of
    sustained load: on a fresh GPU the clock settles over the first second or
    so of such load, which moved a first pass's per-block latency by -2.1%
    on one box and +1.1% on another, with time and not with the stream's
    length (a second pass after a reset stayed within 0.2%).  The checking
    passes pause for the oracle and read indices back every block."""
    import torch
    cfg = synth.workload("prsink_long")
    run = Run(cfg, host_inputs=False)
    ref = oracle.PRSinkReference(cfg, run)
    heads, rows = [5], np.r_[0:32, 3040:3072]
    ws = run.cache.stats()["workspace_bytes"]
    mem0 = None
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    swaps = 0
    prev_sel = None
    for m in range(cfg["blocks"]):
        q, k, v = run.qkv_dev(0, m, 0)
        out = torch.empty_like(q)
        run.cache.retrieve(run.pose_dev(m))
        run.cache.attend(0, q, k, v, out)
        run.cache.commit()
        st = run.cache.stats()
        want_ev = oracle.prsink_schedule(m, cfg["window"], cfg["bank"], cfg["static"])["evicted"]
        assert st["last_evicted"] == (-1 if want_ev is None else want_ev), m
        assert st["workspace_bytes"] == ws
        if m % 45 == 44 or m < 8:
            sel = ref.selection(m)
            want = ref.attend(m, 0, 0, heads=heads, rows=rows, selection=sel)
            err = max_err(out, want, heads, rows)
            assert err <= TOL["bf16"], (m, err)
        run.drop({m + 1})
        run._host.clear()
        if m == 10:
            torch.cuda.synchronize()
            mem0 = torch.cuda.memory_allocated()
        if m > 10 and m % 100 == 0:
            assert torch.cuda.memory_allocated() == mem0
    # indices of every block: a second pass with one resident input block
    # (selections depend on poses only) against the oracle's exact ranking
    run2 = Run(cfg, host_inputs=False)
    q, k, v = run2.qkv_dev(0, 0, 0)
    out = torch.empty_like(q)
    for m in range(cfg["blocks"]):
        run2.cache.retrieve(run2.pose_dev(m))
        got = run2.cache.selection()
        want = ref.selection(m)
        assert got == want, (m, got, want)
        swaps += prev_sel is not None and got != prev_sel
        prev_sel = got
        run2.cache.attend(0, q, k, v, out)
        run2.cache.commit()
    assert swaps > 50                         # the dynamic sink really moves
    # per-block latency: an untimed pass of sustained load, then a pass timed
    # with events around each block's calls
    poses = [run2.pose_dev(m) for m in range(cfg["blocks"])]
    lat = []
    for timed in (False, True):
        run2.cache.reset()
        for m in range(cfg["blocks"]):
            if timed:
                ev[0].record()
            run2.cache.retrieve(poses[m])
            run2.cache.attend(0, q, k, v, out)
            run2.cache.commit()
            if timed:
                ev[1].record()
                torch.cuda.synchronize()
                lat.append(ev[0].elapsed_time(ev[1]))
        torch.cuda.synchronize()
    lat = np.array(lat[20:])
    slope = np.polyfit(np.arange(len(lat)), lat, 1)[0]
    p50 = float(np.percentile(lat, 50))
    print(f"per-block latency p50 {p50:.3f} ms p99 {np.percentile(lat, 99):.3f} ms slope {slope * 1000:.4f} ms/1000 blocks")
    assert abs(slope * 1000) < 0.02 * p50


def test_convkv_512_stream_200_blocks():
    """ConvKV 512x512 for 200 blocks: memory provenance (segment layout and
    positions) on every block, outputs on every 10th block and blocks <= 12."""
    cfg = synth.workload("convkv_512")
    run = Run(cfg, host_inputs=False)
    ref = oracle.ConvKVReference(cfg, run)
    heads, rows = [3], np.r_[0:32, 3040:3072]
    for m in range(cfg["blocks"]):
        run.open(m)
        assert run.cache.context() == list(ref.context(m)), m
        out = run.attend(m, 0, 0)
        if m <= 12 or m % 10 == 9:
            want = ref.attend(m, 0, 0, heads=heads, rows=rows)
            err = max_err(out, want, heads, rows)
            assert err <= TOL["bf16"], (m, err)
        run.cache.commit()
        run.drop(set(range(m - 8, m + 2)))
        run._host.clear()
    assert run.cache.stats()["memory_count"] == 1

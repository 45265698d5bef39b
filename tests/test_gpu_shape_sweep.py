"""A seeded sweep over irregular shapes: every output of every block of short
streams, through the C-ABI, against the CPU oracle.

Each case draws its shape from a fixed seed: cache policy, dtype, head count,
a block's token count (tile edges 1, 64, 65, 256, 257 and ragged values in
between), window length, static sink, top-k and bank size (k above the bank
included), RoPE split (none, the workloads' split, lopsided splits), position
reading, reference frames, bank policy, conv taps and memory frames, layers and
steps per block.  Retrieval, the block table, eviction and the memory count
must match exactly; outputs within the dtype's bound, with the FP8 KV cache
beyond the oracle's slack (P codes that the FP8 product's rounding may decide
either way are allowed their other value)."""
import numpy as np
import pytest

import oracle
from bounded_kv_block_amd import synth
from gpu_helpers import TOL, Run, oracle_err

pytestmark = pytest.mark.gpu

_TOKENS = [(1, 1, 1), (1, 8, 8), (1, 5, 13), (1, 16, 16), (1, 1, 257), (3, 7, 9), (2, 6, 11), (3, 3, 5),
           (2, 1, 1), (1, 9, 7)]
_ROPE = {64: [(0, 0, 0), (24, 20, 20), (32, 16, 16), (2, 30, 32)],
         128: [(0, 0, 0), (44, 42, 42), (64, 32, 32), (16, 56, 56), (2, 62, 64)]}


def _case(i):
    rng = np.random.default_rng([20261203, i])
    pick = lambda xs: xs[int(rng.integers(len(xs)))]
    mode = "convkv" if i % 3 == 2 else "pr_sink"
    dtype = pick(["f32", "bf16", "bf16_fp8k", "bf16_fp8kv"])
    frames, gh, gw = _TOKENS[i % len(_TOKENS)]
    T = frames * gh * gw
    D = pick([64, 128]) if dtype == "f32" else 128
    kw = dict(dtype=dtype, head_dim=D, heads=int(rng.integers(1, 6)), frames=frames, grid_h=gh, grid_w=gw,
              window=int(rng.integers(1, 5)), rope=pick(_ROPE[D]), layers=int(rng.integers(1, 3)),
              steps=int(rng.integers(1, 3)), seed=100 + i)
    if mode == "pr_sink":
        k = int(rng.integers(0, 4))
        bank = int(rng.integers(1, 7))
        kw.update(static=int(rng.integers(0, 2)), dynamic_k=k, bank=bank, pose_dim=int(rng.integers(3, 41)),
                  keyframes=4, pose_kind="walk", positions=pick(["default", "default", "relative"]),
                  reference_frames=pick([0, 0, 1, 2]), bank_policy=pick(["fifo", "fifo", "pose"]))
        kw["blocks"] = kw["static"] + kw["window"] + bank + 3
        base = "prsink_512"
    else:
        taps = int(rng.integers(1, 6))
        kw.update(conv_kernel=taps, conv_stride=taps, memory_frames=int(rng.integers(1, 3)),
                  positions=pick(["default", "absolute"]))
        kw["blocks"] = kw["window"] + 3 + -(-taps * kw["memory_frames"] // frames) + 2
        base = "convkv_512"
    cfg = synth.workload(base, **kw)
    tag = (f"{mode}-{dtype}-H{kw['heads']}-D{D}-T{T}-W{kw['window']}-L{kw['layers']}S{kw['steps']}"
           + (f"-k{kw['dynamic_k']}b{kw['bank']}s{kw['static']}-{kw['positions']}-r{kw['reference_frames']}"
              f"-{kw['bank_policy']}" if mode == "pr_sink" else
              f"-c{kw['conv_kernel']}m{kw['memory_frames']}-{kw['positions']}"))
    return tag, cfg


CASES = [_case(i) for i in range(20)]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_shape_sweep_every_output(case):
    tag, cfg = case
    print(tag, flush=True)
    run = Run(cfg)
    convkv = cfg["mode"] == "convkv"
    ref = (oracle.ConvKVReference if convkv else oracle.PRSinkReference)(cfg, run)
    worst = 0.0
    for m in range(cfg["blocks"]):
        run.open(m)
        if convkv:
            sel = None
            assert run.cache.context() == list(ref.context(m)), m
        else:
            sel = ref.selection(m)
            assert run.cache.selection() == sel, (m, run.cache.selection(), sel)
            want_ctx = ref.context(m, sel)
            assert run.cache.context() == [(k, b, t, t0) for k, b, t, t0 in want_ctx], m
        for step in range(cfg["steps"]):
            for layer in range(cfg["layers"]):
                out = run.attend(m, layer, step)
                want = ((lambda **kw: ref.attend(m, layer, step, **kw)) if convkv else
                        (lambda **kw: ref.attend(m, layer, step, selection=sel, **kw)))
                err = oracle_err(out, want, tol=TOL[cfg["dtype"]])
                worst = max(worst, err)
                assert err <= TOL[cfg["dtype"]], (m, layer, step, err)
        run.cache.commit()
        st = run.cache.stats()
        if convkv:
            assert st["memory_count"] == len(ref.schedule(m + 1)["memory"]), m
        elif cfg["bank_policy"] == "fifo":
            want_ev = oracle.prsink_schedule(m, cfg["window"], cfg["bank"], cfg["static"])["evicted"]
            assert st["last_evicted"] == (-1 if want_ev is None else want_ev), m
    print(f"{tag}: {cfg['blocks']} blocks, max|err| {worst:.3e}", flush=True)
